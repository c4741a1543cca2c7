// knn_kernels.hip -- k-nearest-neighbour sparse atom-pair encoder on gfx950.
//
// What is computed (Design-CP summary, implementation details, memory
// optimisation: the atom-pair tensor is built on the fly at the sparse indices
// of each atom's k nearest neighbours, never densely):
//  * N(l): the k atoms m != l with the smallest squared distance to atom l,
//    ascending, equal distances to the lower index.  The squared distance is
//    float32 ((dx*dx + dy*dy) + dz*dz), d = x_l - x_m, with no fused operations,
//    so the selection is exact and reproducible;
//  * p_lm = W_l s_l + W_m s_m + W_d (d_x, d_y, d_z, 1 / (1 + |d|^2)) for m in
//    N(l), c_s = 128 single channels (bf16), c_p = 16 pair channels, stored bf16.
//
// Kernels, in launch order:
//  * knn_prepare: A = s W_l^T and B = s W_m^T per atom (fp32, [L][2][16]), the
//    single-feature halves of every pair, computed once per atom on MFMA; and,
//    per chunk of 64 consecutive atoms, the coordinates copied as float4 (one
//    16-byte load per candidate later) and the chunk's axis-aligned bounding box;
//  * knn_select_encode: one wave per query atom.  Lanes 0..k-1 hold the best
//    list found so far, sorted by (d2, index); lane 63 down to k hold +inf.
//    Chunks are scanned 64 candidates at a time (one per lane).  When many
//    beat the k-th entry (the first chunks), the chunk is sorted (bitonic,
//    across lanes) and merged into the list; when few do, they are inserted
//    one by one: the insert position is the popcount of a ballot, and the
//    list moves up by a whole-wave DPP shift.
//    The query's own chunk and its two chain neighbours go first, so the k-th
//    distance is small early; every other chunk is skipped when the squared
//    distance from the query to its box exceeds the k-th distance.  That skip
//    is exact: the box bound is evaluated with the same float32 operations in
//    the same order as a candidate's distance, and correctly rounded
//    subtraction, squaring and addition are monotone, so no candidate of a
//    skipped chunk can round to a value at or below the bound.  Lane n then
//    builds pair (l, N(l)[n]); the k pairs of a query are one contiguous run
//    of 32-byte rows.
// Atoms stored along the chain (consecutive indices close in space, as in a
// protein) give tight boxes and few scanned chunks; any order gives the same
// result, only slower.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "knn_kernels.h"

namespace knn {
namespace {

constexpr int CS = 128;        // single channels
constexpr int CP = 16;         // pair channels
constexpr int CH = 64;         // atoms per chunk: one per lane
constexpr int QPB = 4;         // query waves per workgroup
constexpr int DPP_WAVE_SHR1 = 0x138;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- single-feature halves
// One wave per 32 atoms: [A | B] (32 atoms x 32 channels) = s W^T with
// W = [W_l; W_m], eight v_mfma_f32_32x32x16_bf16 over the 128 single channels
// (exact bf16 products, float32 accumulation).  Operand layout: lane q holds
// row (q & 31) of the 32x16 A-slice and column (q & 31) of the 16x32 B-slice,
// contraction slots 8 (q >> 5) + t; the result holds in lane q column (q & 31)
// and rows 8 (i / 4) + 4 (q >> 5) + (i % 4), i = 0..15.  A = W with its rows
// permuted so that lane q's 16 results are the consecutive channels
// 16 (q >> 5) + i of atom (q & 31): one 64-byte store per lane.
__device__ __forceinline__ void project_wave(const uint16_t* __restrict__ s, const uint16_t* __restrict__ w_l,
                                             const uint16_t* __restrict__ w_m, float* __restrict__ ab, int L,
                                             int atom0, int lane) {
  const int h = lane >> 5, r = lane & 31;
  const int o = 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);     // channel of result row r
  const uint16_t* wrow = o < CP ? w_l + (size_t)o * CS : w_m + (size_t)(o - CP) * CS;
  const int atom = atom0 + r;
  const uint16_t* srow = s + (size_t)(atom < L ? atom : L - 1) * CS;
  bf16x8 a[CS / 16], b[CS / 16];
#pragma unroll
  for (int u = 0; u < CS / 16; ++u) {
    a[u] = *reinterpret_cast<const bf16x8*>(wrow + 16 * u + 8 * h);
    b[u] = *reinterpret_cast<const bf16x8*>(srow + 16 * u + 8 * h);
  }
  f32x16 acc = {};
#pragma unroll
  for (int u = 0; u < CS / 16; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u], acc, 0, 0, 0);
  if (atom < L) {
    float4* dst = reinterpret_cast<float4*>(ab + (size_t)atom * 2 * CP + CP * h);
#pragma unroll
    for (int v = 0; v < 4; ++v) dst[v] = make_float4(acc[4 * v], acc[4 * v + 1], acc[4 * v + 2], acc[4 * v + 3]);
  }
}

// ---------------------------------------------------------------- chunk boxes
// One wave per chunk c of 64 atoms: the coordinates as float4 (padding atoms
// past L hold 0 and are never candidates) and the chunk's bounding box.
__device__ __forceinline__ void box_wave(const float* __restrict__ x, int L, float4* __restrict__ xp,
                                         float4* __restrict__ box, int c, int lane) {
  const int m = c * CH + lane;
  const bool ok = m < L;
  const float px = ok ? x[3 * (size_t)m] : 0.f, py = ok ? x[3 * (size_t)m + 1] : 0.f,
              pz = ok ? x[3 * (size_t)m + 2] : 0.f;
  xp[m] = make_float4(px, py, pz, 0.f);
  const float inf = __builtin_inff();
  float lx = ok ? px : inf, ly = ok ? py : inf, lz = ok ? pz : inf;
  float hx = ok ? px : -inf, hy = ok ? py : -inf, hz = ok ? pz : -inf;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    lx = fminf(lx, __shfl_xor(lx, w));
    ly = fminf(ly, __shfl_xor(ly, w));
    lz = fminf(lz, __shfl_xor(lz, w));
    hx = fmaxf(hx, __shfl_xor(hx, w));
    hy = fmaxf(hy, __shfl_xor(hy, w));
    hz = fmaxf(hz, __shfl_xor(hz, w));
  }
  if (lane == 0) {
    box[2 * c] = make_float4(lx, ly, lz, 0.f);
    box[2 * c + 1] = make_float4(hx, hy, hz, 0.f);
  }
}

// Both preparation passes in one launch: workgroup b covers atoms
// [128 b, 128 b + 128): wave w projects atoms 128 b + 32 w .. + 31, and waves 0
// and 1 also build chunks 2 b and 2 b + 1.
__global__ void __launch_bounds__(256) knn_prepare(const uint16_t* __restrict__ s, const uint16_t* __restrict__ w_l,
                                                   const uint16_t* __restrict__ w_m, float* __restrict__ ab,
                                                   const float* __restrict__ x, int L, float4* __restrict__ xp,
                                                   float4* __restrict__ box) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = 2 * blockIdx.x + wave;
  if (wave < 2 && c < (L + CH - 1) / CH) box_wave(x, L, xp, box, c, lane);
  const int atom0 = (4 * blockIdx.x + wave) * 32;
  if (atom0 < L) project_wave(s, w_l, w_m, ab, L, atom0, lane);
}

// ---------------------------------------------------------------- selection + pairs
__device__ __forceinline__ float sq_dist(float xl, float yl, float zl, float xm, float ym, float zm) {
#pragma clang fp contract(off)
  const float dx = xl - xm, dy = yl - ym, dz = zl - zm;
  return (dx * dx + dy * dy) + dz * dz;
}

// Lower bound of sq_dist(query, m) over every m in the box: per axis the gap
// lo - q or q - hi (rounded like the candidate's own difference), else 0.
__device__ __forceinline__ float box_bound(float xl, float yl, float zl, float4 lo, float4 hi) {
#pragma clang fp contract(off)
  const float gx = fmaxf(fmaxf(lo.x - xl, xl - hi.x), 0.f);
  const float gy = fmaxf(fmaxf(lo.y - yl, yl - hi.y), 0.f);
  const float gz = fmaxf(fmaxf(lo.z - zl, zl - hi.z), 0.f);
  return (gx * gx + gy * gy) + gz * gz;
}

// A list entry is the 64-bit key (bits of d2) << 32 | index: for d2 >= 0 the
// float bits order like the values, so keys order by (d2, index).
typedef unsigned long long u64;
constexpr u64 EMPTY = 0x7F800000FFFFFFFFull;     // (+inf, no atom)
constexpr int NINS = 8;                           // at most this many beaters: insert one by one

__device__ __forceinline__ u64 key_of(float d2, int m) { return ((u64)__float_as_uint(d2) << 32) | (uint32_t)m; }
__device__ __forceinline__ float key_d2(u64 key) { return __uint_as_float((uint32_t)(key >> 32)); }

__device__ __forceinline__ u64 join(uint32_t lo, uint32_t hi) { return ((u64)hi << 32) | lo; }
template <int CTRL> __device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL> __device__ __forceinline__ u64 dpp64(u64 v) {
  return join(dpp32<CTRL>((uint32_t)v), dpp32<CTRL>((uint32_t)(v >> 32)));
}
// The key of lane (lane ^ J): DPP inside a row of 16 lanes (quad permutes for
// 1 and 2; a rotation right by n gives lane i the value of lane (i - n) mod 16,
// so lane ^ 4 is a rotation by 4 or 12 and lane ^ 8 one by 8), the LDS
// crossbar across rows.
template <int J> __device__ __forceinline__ u64 xor_lane(u64 v, int lane) {
  if constexpr (J == 1) return dpp64<0xB1>(v);                 // quad_perm [1,0,3,2]
  else if constexpr (J == 2) return dpp64<0x4E>(v);            // quad_perm [2,3,0,1]
  else if constexpr (J == 4) {
    // both rotations run on every lane before the select (a DPP move inside a
    // branch would read lanes the branch switched off)
    const u64 down = dpp64<0x124>(v), up = dpp64<0x12C>(v);  // row_ror 4 / 12
    return (lane & 4) ? down : up;
  }
  else if constexpr (J == 8) return dpp64<0x128>(v);           // row_ror 8
  else return join((uint32_t)__shfl_xor((int)(uint32_t)v, J), (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), J));
}
__device__ __forceinline__ u64 shfl64(u64 v, int src) {
  return join((uint32_t)__shfl((int)(uint32_t)v, src), (uint32_t)__shfl((int)(uint32_t)(v >> 32), src));
}
__device__ __forceinline__ u64 wave_shr1(u64 v) {
  return join((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, DPP_WAVE_SHR1, 0xF, 0xF, false),
              (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), DPP_WAVE_SHR1, 0xF, 0xF, false));
}
__device__ __forceinline__ u64 readlane64(u64 v, int lane) {
  return join((uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane),
              (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane));
}

// One compare-exchange step of a bitonic network: the lower lane of each pair
// keeps the smaller key when `ascending`, the larger otherwise.
template <int J> __device__ __forceinline__ u64 exchange(u64 key, int lane, bool ascending) {
  const u64 other = xor_lane<J>(key, lane);
  const bool keep_min = ((lane & J) == 0) == ascending;
  return keep_min ? (other < key ? other : key) : (other > key ? other : key);
}

// Bitonic merge of a bitonic sequence of 2J keys per block into ascending
// (or descending) order.
template <int J> __device__ __forceinline__ u64 merge_steps(u64 key, int lane, bool ascending) {
  key = exchange<J>(key, lane, ascending);
  if constexpr (J > 1) key = merge_steps<J / 2>(key, lane, ascending);
  return key;
}

// Bitonic sort of one key per lane into ascending lane order: blocks of
// SIZE lanes sorted alternately up and down, then merged.
template <int SIZE> __device__ __forceinline__ u64 sort_steps(u64 key, int lane) {
  if constexpr (SIZE > 2) key = sort_steps<SIZE / 2>(key, lane);
  return merge_steps<SIZE / 2>(key, lane, (lane & SIZE) == 0);
}
__device__ __forceinline__ u64 sort64(u64 key, int lane) { return sort_steps<64>(key, lane); }

// The 64 smallest of two ascending lists, ascending: the elementwise minimum of
// one list and the other reversed is a bitonic sequence holding them; a
// bitonic merge sorts it.
__device__ __forceinline__ u64 merge64(u64 list, u64 batch, int lane) {
  const u64 rev = shfl64(batch, 63 - lane);
  return merge_steps<32>(rev < list ? rev : list, lane, true);
}

// The best list of one query wave: one key per lane (lanes >= k hold EMPTY);
// tk = the key in lane k - 1, the bar a candidate must beat.
struct Best {
  u64 key, tk;
};

__device__ __forceinline__ void scan_chunk(const float4* __restrict__ xp, int c, int l, int L, int k, int lane,
                                           float xl, float yl, float zl, Best& b) {
  const int m = c * CH + lane;
  const float4 p = xp[m];                            // padded to whole chunks
  const bool ok = m < L && m != l;
  const u64 ck = key_of(sq_dist(xl, yl, zl, p.x, p.y, p.z), m);
  const bool beats = ok && ck < b.tk;
  uint64_t mask = __ballot(beats);
  if (__builtin_popcountll(mask) > NINS) {           // many: sort the chunk, merge it in
    const u64 sorted = sort64(beats ? ck : EMPTY, lane);
    const u64 merged = readlane64(b.key, 0) == EMPTY ? sorted      // the list is empty
                                                     : merge64(b.key, sorted, lane);
    b.key = lane < k ? merged : EMPTY;
    b.tk = readlane64(b.key, k - 1);
    return;
  }
  while (mask) {                                     // few: insert one at a time
    const int src = __builtin_ctzll(mask);
    mask &= mask - 1;
    const u64 cand = readlane64(ck, src);
    if (!(cand < b.tk)) continue;                    // the bar moved below it
    // entries ahead of the candidate; the bar is not, so pos <= k - 1
    const int pos = __builtin_popcountll(__ballot(b.key < cand));
    const u64 up = wave_shr1(b.key);
    b.key = lane > pos ? up : (lane == pos ? cand : b.key);
    if (lane >= k) b.key = EMPTY;                    // the entry pushed out of the list
    b.tk = readlane64(b.key, k - 1);
  }
}

__global__ void __launch_bounds__(64 * QPB) knn_select_encode(const float4* __restrict__ xp,
                                                              const float4* __restrict__ box,
                                                              const float* __restrict__ ab,
                                                              const float* __restrict__ w_d, int L, int k,
                                                              int32_t* __restrict__ nbr,
                                                              uint16_t* __restrict__ pair) {
  const int lane = threadIdx.x & 63;
  const int l = blockIdx.x * QPB + (threadIdx.x >> 6);
  if (l >= L) return;                                // whole waves leave
  const float4 q = xp[l];
  const float xl = q.x, yl = q.y, zl = q.z;
  Best b{EMPTY, EMPTY};

  const int nch = (L + CH - 1) / CH;
  const int c0 = l / CH;
  scan_chunk(xp, c0, l, L, k, lane, xl, yl, zl, b);
  if (c0 > 0) scan_chunk(xp, c0 - 1, l, L, k, lane, xl, yl, zl, b);
  if (c0 + 1 < nch) scan_chunk(xp, c0 + 1, l, L, k, lane, xl, yl, zl, b);
  for (int g = 0; g < nch; g += 64) {                // 64 boxes tested at once, one per lane
    const int c = g + lane;
    const bool fresh = c < nch && (c < c0 - 1 || c > c0 + 1);
    const float lb = fresh ? box_bound(xl, yl, zl, box[2 * c], box[2 * c + 1]) : __builtin_inff();
    uint64_t mask = __ballot(fresh && lb <= key_d2(b.tk));
    while (mask) {
      const int src = __builtin_ctzll(mask);
      mask &= mask - 1;
      if (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(lb), src)) > key_d2(b.tk)) continue;
      scan_chunk(xp, g + src, l, L, k, lane, xl, yl, zl, b);
    }
  }

  if (lane >= k) return;
  // Every slot is filled when k <= L - 1 and all distances are finite; an
  // empty one (non-finite coordinates) is reported as -1 with the pair of l itself.
  const uint32_t bi = (uint32_t)b.key;
  const bool have = bi < (uint32_t)L;
  const int m = have ? (int)bi : l;
  const float4 pm = xp[m];
  const float dx = xl - pm.x, dy = yl - pm.y, dz = zl - pm.z;
  const float ph[4] = {dx, dy, dz, 1.0f / (1.0f + (have ? key_d2(b.key) : 0.f))};
  const float4* al = reinterpret_cast<const float4*>(ab + (size_t)l * 2 * CP);
  const float4* bm = reinterpret_cast<const float4*>(ab + (size_t)m * 2 * CP + CP);
  float v[CP];
#pragma unroll
  for (int u = 0; u < CP / 4; ++u) {
    const float4 a4 = al[u], b4 = bm[u];
    v[4 * u] = a4.x + b4.x;
    v[4 * u + 1] = a4.y + b4.y;
    v[4 * u + 2] = a4.z + b4.z;
    v[4 * u + 3] = a4.w + b4.w;
  }
  uint32_t packed[CP / 2];
#pragma unroll
  for (int o = 0; o < CP; ++o) {
    float acc = v[o];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = fmaf(w_d[o * 4 + j], ph[j], acc);
    const uint32_t h = __builtin_bit_cast(uint16_t, (__bf16)acc);
    packed[o / 2] = (o & 1) ? (packed[o / 2] | (h << 16)) : h;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(pair + ((size_t)l * k + lane) * CP);
  dst[0] = u32x4{packed[0], packed[1], packed[2], packed[3]};
  dst[1] = u32x4{packed[4], packed[5], packed[6], packed[7]};
  nbr[(size_t)l * k + lane] = have ? m : -1;
}

}  // namespace

WsLayout workspace_layout(int64_t L) {
  WsLayout w;
  const int64_t nch = (L + CH - 1) / CH;
  w.ab = 0;
  w.xp = (size_t)L * 2 * CP * sizeof(float);
  w.box = w.xp + (size_t)nch * CH * sizeof(float4);
  w.total = w.box + (size_t)nch * 2 * sizeof(float4);
  return w;
}

hipError_t launch_encode(const float* x, const void* s, int L, int k, const void* w_l, const void* w_m,
                         const float* w_d, int32_t* nbr, void* pair, void* ws, hipStream_t stream) {
  if (L <= 0) return hipSuccess;
  const WsLayout w = workspace_layout(L);
  char* base = static_cast<char*>(ws);
  float* ab = reinterpret_cast<float*>(base + w.ab);
  float4* xp = reinterpret_cast<float4*>(base + w.xp);
  float4* box = reinterpret_cast<float4*>(base + w.box);
  hipLaunchKernelGGL(knn_prepare, dim3((unsigned)((L + 127) / 128)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(s), static_cast<const uint16_t*>(w_l),
                     static_cast<const uint16_t*>(w_m), ab, x, L, xp, box);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(knn_select_encode, dim3((unsigned)((L + QPB - 1) / QPB)), dim3(64 * QPB), 0, stream, xp, box,
                     ab, w_d, L, k, nbr, static_cast<uint16_t*>(pair));
  return hipGetLastError();
}

}  // namespace knn
