// Internal interface between the C ABI layer and the kNN pair-encoder kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace knn {

// Workspace regions (byte offsets): per-atom single-feature halves fp32
// [L][2][16], coordinates padded to whole 64-atom chunks as float4, and one
// bounding box (lo, hi as float4) per chunk.
struct WsLayout {
  size_t ab, xp, box, total;
};

WsLayout workspace_layout(int64_t L);

// Arguments are validated by the caller: 1 <= k <= 64, k <= L - 1, pointers
// 16-byte aligned, ws at least workspace_layout(L).total bytes.
hipError_t launch_encode(const float* x, const void* s, int L, int k, const void* w_l, const void* w_m,
                         const float* w_d, int32_t* nbr, void* pair, void* ws, hipStream_t stream);

}  // namespace knn
