/*
 * A plain C client of libvrcomm (C11, host code only; built with gcc against
 * include/vrcomm.h and the HIP runtime's C API).
 *
 * The Symmetric page's AllReduce example: 4 ranks of 1,048,576 fp32 each,
 * rank r's buffer filled with the value r; after a sum-AllReduce every
 * element of every rank's result is 0 + 1 + 2 + 3 = 6.0, and each rank's
 * completion signal has risen by the number of ranks.
 *
 * Exit status: 0 when every element and signal is as expected, 1 on a wrong
 * value, 2 when a library or HIP call fails.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "vrcomm.h"

#define R 4
#define N (1u << 20)

#define CHECK_VR(call)                                                      \
  do {                                                                      \
    vrResult_t rc_ = (call);                                                \
    if (rc_ != VR_OK) {                                                     \
      fprintf(stderr, "%s: %s\n", #call, vr_error_string(rc_));             \
      return 2;                                                             \
    }                                                                       \
  } while (0)
#define CHECK_HIP(call)                                                     \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));            \
      return 2;                                                             \
    }                                                                       \
  } while (0)

int main(void) {
  const size_t bytes = (size_t)N * sizeof(float);
  vrCommRequirements req = {2, 1, 1, 0}; /* signals, counters, contexts, barrier slots per rank */
  vrComm_t comm;
  CHECK_VR(vr_comm_create(R, &req, NULL, 0, &comm));

  char *send, *recv;
  CHECK_HIP(hipMalloc((void**)&send, R * bytes));
  CHECK_HIP(hipMalloc((void**)&recv, R * bytes));
  float* host = (float*)malloc(bytes);
  if (!host) return 2;
  void *sb[R], *rb[R];
  for (int r = 0; r < R; ++r) {
    sb[r] = send + (size_t)r * bytes;
    rb[r] = recv + (size_t)r * bytes;
    for (size_t i = 0; i < N; ++i) host[i] = (float)r;
    CHECK_HIP(hipMemcpy(sb[r], host, bytes, hipMemcpyHostToDevice));
  }
  CHECK_HIP(hipMemset(recv, 0, R * bytes));

  vrWindow_t sw, rw;
  CHECK_VR(vr_window_register(comm, sb, bytes, VR_WIN_DEFAULT, &sw));
  CHECK_VR(vr_window_register(comm, rb, bytes, VR_WIN_DEFAULT, &rw));
  CHECK_VR(vr_allreduce(comm, sw, 0, rw, 0, N, VR_DT_F32, VR_OP_SUM, /*sig=*/1, /*flags=*/0, NULL));
  CHECK_HIP(hipDeviceSynchronize());

  vrResult_t code;
  uint32_t bits;
  CHECK_VR(vr_comm_get_async_error(comm, &code, &bits));
  if (code != VR_OK) {
    fprintf(stderr, "device error: %s (bits 0x%x)\n", vr_error_string(code), bits);
    return 2;
  }
  int bad = 0;
  for (int r = 0; r < R; ++r) {
    CHECK_HIP(hipMemcpy(host, rb[r], bytes, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < N; ++i)
      if (host[i] != 6.0f) {
        if (bad < 5) fprintf(stderr, "rank %d element %zu: %g\n", r, i, (double)host[i]);
        ++bad;
      }
    uint64_t sig;
    CHECK_VR(vr_signal_read(comm, r, 1, 64, &sig));
    if (sig != R) {
      fprintf(stderr, "rank %d signal 1: %llu, expected %d\n", r, (unsigned long long)sig, R);
      ++bad;
    }
  }
  CHECK_VR(vr_window_deregister(comm, sw));
  CHECK_VR(vr_window_deregister(comm, rw));
  CHECK_VR(vr_comm_destroy(comm));
  CHECK_HIP(hipFree(send));
  CHECK_HIP(hipFree(recv));
  free(host);
  if (bad) return 1;
  printf("ok: %d ranks x %u fp32 filled with the rank value, every element 6.0, every signal %d\n", R, N, R);
  return 0;
}
