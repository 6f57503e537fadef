"""CPU oracle for one-sided window put/get with signals and counters.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``collective_window_put_amd`` and its HIP library) never imports, links or
calls anything here, and this package never imports the product path; the
two share only the seeded input generators in ``workloads``.

It is written to be obviously correct, not fast: plain numpy and Python, in
the order the pages describe the steps. Sources (cited by page and section):

* GIN page -- NCCL GIN device API walkthrough, lpnh.cn/news/2681042.
  Sections used: one-sided transfers (put/get), completion management
  (flush), signals and counters (rolling comparison, strong/weak signals,
  signal methods, counter methods), and the pure-GIN AlltoAll kernel.
* Symmetric-memory page -- NCCL symmetric memory examples,
  zwxr.cn/news/250719. Sections used: AllReduce example (steps 2-7 and the
  expected output for 4 GPUs), AllGather with Copy Engine (expected
  segments), and window registration (flags, 4096-byte alignment).
* GPUDirect Async survey -- 10100.com/article/158785524. Sections used: the
  motivating MoE token dispatch (opening), and section 4 on GIN's device
  API semantics (signal ordering, batch of puts with one trailing signal,
  integer signal IDs, the ring-exchange example). The MoE combine (each
  token's expert outputs brought back and mixed by its router weights) is
  read as the dispatch's inverse; the pages describe only the dispatch.

Modules:
  primitives   state model (windows, 64-bit signals, 56-bit counters) and
               sequential put/get/signal/wait/reset semantics
  definitions  plain definitions of each collective's result
  protocol     step-by-step protocol simulation under seeded or exhaustive
               rank interleavings, with deadlock detection
  ordering     relaxed-visibility model: enumerates every state the strong
               or weak signal rule allows and checks what an observer of a
               signal value may conclude

Every function is pinned by tests under ``tests/`` (``-m "not gpu"``)
against the pages' worked examples, closed forms, library routines,
brute force and invariants. Parity unpinned: none of the functions here
is left without a pin; the dispatch result and its per-entry positions are
pinned by brute force (a token may name one expert more than once: one row
per routing entry, in k order), a library stable sort and invariants only,
and the combine by hand-worked binary32 cases (product rounding, k order,
a repeated expert), a closed form checked against torch's bf16 rounding,
and the one-hot special case, since the pages give no worked example for
either. ``allgather_for_rank`` is pinned by the Symmetric-memory page's
segments and brute force over small rank counts and sizes;
``signal_increment`` by the final signals of each collective's
step-by-step protocol and the GIN page's nRanks rule.

``protocol`` computes every element value itself (its own rank-order owner
sum and its own bf16 widening and rounding, pinned against torch), so its
agreement with ``definitions`` checks the arithmetic as well as the data
movement.
"""
from . import primitives, definitions, protocol, ordering  # noqa: F401
