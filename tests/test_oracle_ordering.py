"""The relaxed-visibility model: strong signals give the prefix property, weak ones do not."""
import pytest

from oracle import ordering as O


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_strong_signal_prefix_property_holds_in_every_state(n):
    assert not O.prefix_violation_exists(n, strong=True)


@pytest.mark.parametrize("n", [2, 3, 4])
def test_weak_signal_admits_a_missing_earlier_payload(n):
    # negative test: the checker has teeth
    assert O.prefix_violation_exists(n, strong=False)


def test_single_put_weak_and_strong_agree():
    assert not O.prefix_violation_exists(1, strong=False)
    assert O.stream_states(1, True) == O.stream_states(1, False)


@pytest.mark.parametrize("sizes", [[3], [2, 2], [3, 2], [1, 3, 2]])
def test_several_contexts_each_keep_their_own_prefix(sizes):
    checked, bad = O.check_streams(sizes, strong=True)
    assert checked > 1 and bad == 0
    _, bad_w = O.check_streams(sizes, strong=False)  # weak: only counts are consistent
    assert bad_w == 0


def test_strong_signal_says_nothing_about_another_context():
    assert O.cross_context_violation_exists(2, 2)


@pytest.mark.parametrize("n,strong", [(1, True), (2, True), (3, True), (2, False), (3, False)])
def test_states_are_exactly_the_prefixes_of_legal_orders(n, strong):
    exts = list(O.linear_extensions(n, strong))
    assert len(exts) == O.count_linear_extensions(n, strong)
    prefixes = {frozenset(o[:i]) for o in exts for i in range(len(o) + 1)}
    assert prefixes == set(O.stream_states(n, strong))
    # the observer rule checked on every prefix of every order
    for o in exts:
        for i in range(len(o) + 1):
            st = frozenset(o[:i])
            assert O.observer_ok(st, n, strong)
            if strong:
                v = sum(1 for e in st if e[0] == "S")
                assert all(("D", k) in st for k in range(v))


def test_extension_counts_hand_checked():
    # one put: D before S -> 1 order; two puts weak: D0<S0, D1<S1 -> 4!/(2*2) = 6
    assert O.count_linear_extensions(1, True) == 1
    assert O.count_linear_extensions(2, False) == 6
    # two puts strong: D0<S0, D0<S1, D1<S1 -> orders of {D0,D1,S0,S1}: 6 - 1 (S1 before D1 ruled out twice...)
    assert O.count_linear_extensions(2, True) == len(list(O.linear_extensions(2, True))) == 5
