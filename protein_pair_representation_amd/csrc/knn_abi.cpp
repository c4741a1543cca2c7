// knn_abi.cpp -- the C ABI of the kNN sparse atom-pair encoder (declared in include/knn.h).
//
// Host-side only: validates every argument, then enqueues the encoder's
// kernels on the caller's stream.  Nothing here allocates, frees or
// synchronises, and no HIP call is made before validation has passed.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/knn.h"
#include "knn_kernels.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Span {
  const void* p;
  size_t n;
};

bool overlap(Span a, Span b) {
  if (a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

}  // namespace

extern "C" {

int knn_workspace_bytes(int64_t L, size_t* bytes) {
  if (bytes == nullptr) return TA_ERR_NULL_PTR;
  if (L < 0 || L > KNN_MAX_ATOMS) return TA_ERR_BAD_SHAPE;
  *bytes = knn::workspace_layout(L).total;
  return TA_OK;
}

int knn_pair_encode(const float* x, const void* s, int64_t L, int k, const void* w_l, const void* w_m,
                    const float* w_d, int32_t* nbr, void* pair, void* ws, size_t ws_bytes, void* stream) {
  if (L < 0 || L > KNN_MAX_ATOMS || k < 1 || k > KNN_MAX_K) return TA_ERR_BAD_SHAPE;
  if (L == 0) return TA_OK;
  if (k > L - 1) return TA_ERR_BAD_SHAPE;
  const void* ptrs[] = {x, s, w_l, w_m, w_d, nbr, pair, ws};
  for (const void* p : ptrs)
    if (p == nullptr) return TA_ERR_NULL_PTR;
  for (const void* p : ptrs)
    if (!aligned16(p)) return TA_ERR_MISALIGNED;
  const size_t need = knn::workspace_layout(L).total;
  if (ws_bytes < need) return TA_ERR_WORKSPACE_TOO_SMALL;
  const size_t n = (size_t)L, kk = (size_t)k;
  const Span in[] = {{x, n * 3 * sizeof(float)},
                     {s, n * KNN_SINGLE_CHANNELS * 2},
                     {w_l, (size_t)KNN_PAIR_CHANNELS * KNN_SINGLE_CHANNELS * 2},
                     {w_m, (size_t)KNN_PAIR_CHANNELS * KNN_SINGLE_CHANNELS * 2},
                     {w_d, (size_t)KNN_PAIR_CHANNELS * 4 * sizeof(float)}};
  const Span out[] = {{nbr, n * kk * sizeof(int32_t)}, {pair, n * kk * KNN_PAIR_CHANNELS * 2}, {ws, need}};
  for (int i = 0; i < 3; ++i) {
    for (const Span& a : in)
      if (overlap(out[i], a)) return TA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(out[i], out[j])) return TA_ERR_ALIAS;
  }
  return knn::launch_encode(x, s, (int)L, k, w_l, w_m, w_d, nbr, pair, ws, (hipStream_t)stream) == hipSuccess
             ? TA_OK
             : TA_ERR_HIP;
}

}  // extern "C"
