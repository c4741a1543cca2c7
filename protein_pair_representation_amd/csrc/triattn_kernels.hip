// triattn_kernels.hip -- gfx950 (CDNA4) kernels for gated triangle self-attention.
//
//   K1 tri_project : LayerNorm fused into one MFMA GEMM per token tile,
//                    [tokens x 128] . [128 x (4*128 + 4)] -> q, k, v^T, g, pair bias.
//   tri_pack_bias  : pair bias -> per-query shifted, base-2, compute-dtype tiles.
//   K2 tri_attend  : fused attention per (line, block of 128 queries), all heads:
//                    S^T = bias + K Q^T - m (bias and running maximum both added
//                    by the MFMA itself, through selector fragments), online
//                    softmax at wavefront level, O^T += V^T P^T, then 1/l, sigmoid
//                    gate and the output projection, stored once.
//
// Operator: gated triangular attention over the pair representation (named in
// the LightNobel article, section 3.1; tokens of c_z = 128 channels, section 1.1).
// The softmax is blockwise with a running maximum and sum, so no I x I score
// matrix is stored (the on-the-fly scoring of ring attention, Design-CP summary,
// Methodology section 1).  Fusing the attention steps into one kernel to cut
// memory traffic is the approach the OpenFold-TRT summary describes (Methodology).
//
// MFMA conventions (v_mfma_f32_32x32x16_bf16, and 8x v_mfma_f32_32x32x2_f32 for
// fp32, see mma() below).  A "fragment" is the 8 operand elements one lane holds
// for a 16-deep slice of the contraction: lane l holds row (l & 31) of A (column
// of B) and contraction slots 8*(l >> 5) + t, t = 0..7.  The 32x32 fp32 result
// holds, in lane l, column (l & 31) and rows 8*(i/4) + 4*(l>>5) + (i%4), i = 0..15.
// Every tile here loads the A/B row it calls m from index rho(m); with that
// permutation lane l's 16 results cover the 16 CONSECUTIVE indices
// 16*(l>>5) + i, which makes every epilogue store and every bias load a
// contiguous 32/64-byte run, and lets the softmax output feed P.V directly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "triattn_kernels.h"

namespace triattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int CZ = 128;        // channels per token
constexpr int NH = 4;          // heads
constexpr int HD = 32;         // head width
constexpr int QB = 128;        // queries (positions) per workgroup tile
constexpr int KT = 64;         // keys per attention tile
constexpr int NTHREADS = 256;  // 4 waves
constexpr float LOG2E = 1.4426950408889634f;
// Masked / padded keys carry this bias (base-2 units): exp2 of it underflows to
// exactly 0.  It must be finite: the bias enters the scores through a product
// with a 0/1 selector, and 0 * -inf would be NaN.
constexpr float MASKED = -30000.0f;

__device__ __forceinline__ int rho(int m) { return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3); }

// Workspace pair-bias layout: fp16 (bf16 problems) or fp32, lane-interleaved tiles.  Tile
// (h, j/32, k/64) holds the 32 x 64 block a wave adds in one key step as four
// 16-key chunks; chunk g is exactly the B-operand fragments of that slice
// (lane j%32 + 32*hh holds keys 16g + 8hh + t, t = 0..7), so each chunk is one
// contiguous per-lane load: element (j, k) with k%64 = 16g + 8hh + t sits at
//   g*512 + (j%32 + 32*hh)*8 + t       inside a 2048-element tile.
// P (a multiple of 128) bounds j and k.
__device__ __forceinline__ size_t bias_tiled_index(int h, int j, int k, int P) {
  const int jb = j >> 5, jj = j & 31, kb = k >> 6, kk = k & 63;
  const int g = kk >> 4, hh = (kk >> 3) & 1, t = kk & 7;
  return ((((size_t)h * (P >> 5) + jb) * (P >> 6) + kb) << 11) + (g << 9) + ((jj + 32 * hh) << 3) + t;
}

// ---------------------------------------------------------------- element traits
// bias_t: element type of the packed pair bias (fp16 next to bf16 operands:
// 11 significant bits for the logits at the same 2 bytes; fp32 with fp32).
template <typename T> struct El;
template <> struct El<__bf16> {
  typedef bf16x8 frag;
  typedef _Float16 bias_t;
  typedef f16x8 bias_frag;
  static constexpr int bytes = 2;
};
template <> struct El<float> {
  typedef f32x8 frag;
  typedef float bias_t;
  typedef f32x8 bias_frag;
  static constexpr int bytes = 4;
};

__device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// fp32: eight K=2 products; step t contracts slot t of both lane halves.
__device__ __forceinline__ f32x16 mma(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
  for (int t = 0; t < 8; ++t) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], b[t], c, 0, 0, 0);
  return c;
}

template <typename T> __device__ __forceinline__ typename El<T>::frag to_frag(const float* v);
template <> __device__ __forceinline__ bf16x8 to_frag<__bf16>(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (__bf16)v[t];
  return r;
}
template <> __device__ __forceinline__ f32x8 to_frag<float>(const float* v) {
  f32x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = v[t];
  return r;
}

template <typename V> __device__ __forceinline__ V to_vec8(const float* v) {
  V r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = v[t];
  return r;
}

template <typename T> __device__ __forceinline__ void frag_to_f32(const typename El<T>::frag& f, float* v) {
#pragma unroll
  for (int t = 0; t < 8; ++t) v[t] = (float)f[t];
}

// Global loads/stores of 8 consecutive elements (16 B bf16, 32 B fp32).
template <typename T> __device__ __forceinline__ typename El<T>::frag gld8(const T* p) {
  return *reinterpret_cast<const typename El<T>::frag*>(p);
}
template <typename T> __device__ __forceinline__ void gst8(T* p, const typename El<T>::frag& f) {
  *reinterpret_cast<typename El<T>::frag*>(p) = f;
}

// Value held by lane l ^ 32, combined: returns op(x[l], x[l^32]) in every lane.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * LOG2E));
}

// ---------------------------------------------------------------- LDS tiles
// Rows of 16-byte units; unit u of row r lives at unit u ^ swz(r) so that the
// fragment reads of a wave (rows rho(0..31), one unit) spread over all banks.
template <int UNITS> __device__ __forceinline__ int swz(int r) {
  int f = ((r ^ (r >> 2)) & 1) | (r & 2) | ((r >> 2) & 4) | ((r << 1) & 8);
  if (UNITS == 4) f = (((r >> 2) ^ (r >> 1)) & 1) | ((r >> 3) & 2);
  return f & (UNITS - 1);
}

template <int UNITS> __device__ __forceinline__ void lds_put(u32x4* base, int r, int u, const u32x4& v) {
  base[r * UNITS + (u ^ swz<UNITS>(r))] = v;
}

// Fragment (8 elements starting at element column col8*8) of row r.
template <typename T, int UNITS>
__device__ __forceinline__ typename El<T>::frag lds_frag(const u32x4* base, int r, int col8) {
  typename El<T>::frag f;
  constexpr int U = El<T>::bytes / 2;  // 16-B units per fragment: 1 (bf16) or 2 (fp32)
  u32x4 tmp[U];
#pragma unroll
  for (int s = 0; s < U; ++s) tmp[s] = base[r * UNITS + ((col8 * U + s) ^ swz<UNITS>(r))];
  __builtin_memcpy(&f, tmp, sizeof(f));
  return f;
}

// ================================================================ K1: LN + projections
// One workgroup loops over tiles of 128 tokens (one line, 128 consecutive
// positions); each wave owns 32 tokens.  Lane l holds token rho(l & 31) of its
// wave and channels 64*(l>>5) .. +63 -- exactly the B-operand fragments of the
// eight 16-deep contraction slices, with contraction index 64*(l>>5) + 8c + t.
// The 17 output tiles of 32 channels are q0..3, k0..3, v0..3, g0..3, bias (4 used).
template <typename T>
__global__ void __launch_bounds__(NTHREADS) tri_project(ProjectArgs a) {
  constexpr bool W_IN_LDS = sizeof(T) == 2;
  constexpr int WUNITS = CZ * El<T>::bytes / 16;   // 16-B units per weight row
  constexpr int NW_ROWS = 17 * 32;
  __shared__ u32x4 w_lds[W_IN_LDS ? NW_ROWS * WUNITS : 1];
  __shared__ float ln_lds[2 * CZ];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, lr = lane & 31;
  const T* wsrc[5] = {(const T*)a.w_q, (const T*)a.w_k, (const T*)a.w_v, (const T*)a.w_g, (const T*)a.w_b};

  if (W_IN_LDS) {
    for (int idx = tid; idx < NW_ROWS * WUNITS; idx += NTHREADS) {
      int r = idx / WUNITS, u = idx % WUNITS, mt = r >> 5;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (mt < 4 * 4) v = reinterpret_cast<const u32x4*>(wsrc[mt >> 2] + (size_t)((mt & 3) * 32 + (r & 31)) * CZ)[u];
      else if ((r & 31) < NH) v = reinterpret_cast<const u32x4*>(wsrc[4] + (size_t)(r & 31) * CZ)[u];
      lds_put<WUNITS>(w_lds, r, u, v);
    }
  }
  for (int c = tid; c < 2 * CZ; c += NTHREADS) ln_lds[c] = c < CZ ? a.ln_gamma[c] : a.ln_beta[c - CZ];
  __syncthreads();

  const int pblocks = a.P / QB;
  const long ntiles = (long)a.lines * pblocks;
  const int mt0 = a.bias_only ? 16 : 0;
  const T* z = (const T*)a.z;

  for (long tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int line = (int)(tile / pblocks);
    const int pos0 = (int)(tile % pblocks) * QB + wave * 32;
    const int pos = pos0 + rho(lr);
    // ---- load the token half and normalise it
    float x[64];
    if (pos < a.I) {
      const T* zp = z + (size_t)line * a.z_line_stride + (size_t)pos * a.z_pos_stride + 64 * hh;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        typename El<T>::frag f = gld8<T>(zp + 8 * c);
        frag_to_f32<T>(f, x + 8 * c);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 64; ++t) x[t] = 0.f;
    }
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < 64; ++t) s += x[t];
    const float mean = xhalf_sum(s) * (1.0f / CZ);
    float v2 = 0.f;
#pragma unroll
    for (int t = 0; t < 64; ++t) { x[t] -= mean; v2 += x[t] * x[t]; }
    const float rstd = rsqrtf(xhalf_sum(v2) * (1.0f / CZ) + a.eps);
    typename El<T>::frag xf[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float t8[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        int ch = 64 * hh + 8 * c + t;
        t8[t] = x[8 * c + t] * rstd * ln_lds[ch] + ln_lds[CZ + ch];
      }
      xf[c] = to_frag<T>(t8);
    }

    // ---- 17 output tiles
    for (int mt = mt0; mt < 17; ++mt) {
      f32x16 acc = {};
      const bool vt_tile = mt >= 8 && mt < 12;
      const int wrow = 32 * mt + rho(lr);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        typename El<T>::frag wf;
        if constexpr (W_IN_LDS) {
          wf = lds_frag<T, WUNITS>(w_lds, wrow, 8 * hh + c);
        } else {
          const T* wp = mt < 16 ? wsrc[mt >> 2] + (size_t)((mt & 3) * 32 + rho(lr)) * CZ
                                : wsrc[4] + (size_t)(rho(lr) < NH ? rho(lr) : 0) * CZ;
          wf = gld8<T>(wp + 64 * hh + 8 * c);
        }
        acc = vt_tile ? mma(xf[c], wf, acc) : mma(wf, xf[c], acc);
      }
      const int head = mt & 3;
      if (mt < 8 || (mt >= 12 && mt < 16)) {
        // lane: token pos, channels 16*hh + i of head `head`
        float o[16];
        if (mt < 4) {
#pragma unroll
          for (int i = 0; i < 16; ++i) o[i] = acc[i] * (LOG2E * 0.17677669529663687f);  // log2(e)/sqrt(32)
        } else if (mt < 8) {
#pragma unroll
          for (int i = 0; i < 16; ++i) o[i] = acc[i];
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float bg = a.b_g ? a.b_g[head * HD + 16 * hh + i] : 0.f;
            o[i] = sigmoidf_(acc[i] + bg);
          }
        }
        T* dst = (T*)(mt < 4 ? a.q : mt < 8 ? a.k : a.g);
        T* p = dst + (((size_t)line * NH + head) * a.P + pos) * HD + 16 * hh;
        gst8<T>(p, to_frag<T>(o));
        gst8<T>(p + 8, to_frag<T>(o + 8));
      } else if (vt_tile) {
        // lane: channel e = rho(lr) of head, tokens pos0 + 16*hh + i
        float o[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] = acc[i];
        T* p = (T*)a.vt + (((size_t)line * NH + head) * HD + rho(lr)) * a.P + pos0 + 16 * hh;
        gst8<T>(p, to_frag<T>(o));
        gst8<T>(p + 8, to_frag<T>(o + 8));
      } else if (a.bias != nullptr && hh == 0 && pos < a.I) {
        // bias tile: lanes of the lower half hold channels 0..15; heads are 0..3
#pragma unroll
        for (int h = 0; h < NH; ++h)
          a.bias[((size_t)h * a.I + a.bias_row0 + line) * a.I + pos] = acc[h];
      }
    }
  }
}

// ================================================================ K2: fused attention
// Scores arrive from the MFMA already in base-2 units and already shifted by
// the running maximum: q is stored pre-multiplied by log2(e)/sqrt(d), the bias
// by log2(e), and one extra 16-deep contraction slice multiplies a unit
// fragment with a fragment holding -m (m = running maximum, rounded to the
// compute dtype so that the MFMA adds it exactly).  The softmax of a tile is
// then just p = exp2(acc), its conversion, and a row sum (dot2 on packed
// pairs).  m is only moved when a tile's partial sums exceed 2^16 (and on the
// first tile of every head): then the exact maximum is taken, O and l are
// rescaled and the tile is re-exponentiated.  In exact arithmetic any shift
// gives the same softmax; the shift only keeps exp2 in range.
constexpr float SUM_LIMIT = 65536.0f;

template <typename T> __device__ __forceinline__ typename El<T>::frag unit_frag(float v) {
  float t8[8] = {v, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  return to_frag<T>(t8);
}

// p = exp2(s) for the 32 scores of a lane, as MFMA B fragments, and their sum.
template <typename T>
__device__ __forceinline__ float exp_tile(const f32x16 (&s)[2], typename El<T>::frag (&pf)[2][2]) {
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float p[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) p[t] = fast_exp2(s[st][8 * c + t]);
      pf[st][c] = to_frag<T>(p);
      if constexpr (sizeof(T) == 2) {
        // row sum of the rounded values the P.V product uses
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          bf16x2 pr = {pf[st][c][2 * t], pf[st][c][2 * t + 1]};
          if (t & 1) l1 = __builtin_amdgcn_fdot2_f32_bf16(pr, one, l1, false);
          else l0 = __builtin_amdgcn_fdot2_f32_bf16(pr, one, l0, false);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 8; t += 2) { l0 += p[t]; l1 += p[t + 1]; }
      }
    }
  return l0 + l1;
}

// Move the running maximum to the tile's exact maximum (if larger), rescale
// the accumulators, shift the scores and re-exponentiate.  m is kept exactly
// representable in T so that the MFMA's -m slice and this code agree.
template <typename T>
__device__ __forceinline__ float rebase_tile(f32x16 (&s)[2], typename El<T>::frag (&pf)[2][2], float& m,
                                             f32x16& o, float& lsum, bool first) {
  float mx = s[0][0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
  mx = xhalf_max(mx);                        // excess of the tile maximum over m
  float mnew = first ? mx : m + fmaxf(mx, 0.f);
  mnew = (float)(T)mnew;
  const float d = mnew - m;
  if (!first) {
    const float alpha = fast_exp2(-d);
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] *= alpha;
    lsum *= alpha;
  }
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[st][i] -= d;
  m = mnew;
  return exp_tile<T>(s, pf);
}

template <typename T>
__global__ void __launch_bounds__(NTHREADS, 2) tri_attend(AttendArgs a) {
  typedef typename El<T>::frag frag;
  constexpr int KU = HD * El<T>::bytes / 16;      // units per K-tile row (32 channels)
  constexpr int VU = KT * El<T>::bytes / 16;      // units per V^T-tile row (64 keys)
  constexpr int WU = CZ * El<T>::bytes / 16;      // units per W_o row
  constexpr int KTILE_UNITS = KT * KU;
  constexpr int VTILE_UNITS = HD * VU;
  constexpr int LD_PER_THREAD = KTILE_UNITS / NTHREADS;  // same for K and V^T tiles
  __shared__ u32x4 k_lds[2][KTILE_UNITS];
  __shared__ u32x4 v_lds[2][VTILE_UNITS];
  // finished heads: per wave, query lr's gated output o[h*32 + e], unit u at u ^ (lr & (WU-1))
  __shared__ u32x4 o_lds[NTHREADS / 64][32 * WU];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, lr = lane & 31;
  const int I = a.I, P = a.P;

  // XCD-aware order: consecutive logical tiles (same line, neighbouring query
  // blocks) go to the same XCD so its L2 serves the line's keys and values.
  const int nblk = gridDim.x;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int line = bid / a.nqb, qb = bid % a.nqb;
  const int j = qb * QB + wave * 32 + lr;  // this lane's query
  const int jc = j < I ? j : I - 1;

  const T* qbase = (const T*)a.q + (size_t)line * NH * P * HD;
  const T* kbase = (const T*)a.k + (size_t)line * NH * P * HD;
  const T* vbase = (const T*)a.vt + (size_t)line * NH * HD * P;
  const T* gbase = (const T*)a.g + (size_t)line * NH * P * HD;
  const int nkt = (I + KT - 1) / KT;

  // K / V^T tile staging: thread tid moves LD_PER_THREAD 16-B units of each.
  // Addresses are a wave-uniform tile base plus a fixed 32-bit per-lane offset.
  constexpr int EPU = 16 / El<T>::bytes;  // elements per 16-B unit
  int k_off[LD_PER_THREAD], v_off[LD_PER_THREAD];
#pragma unroll
  for (int s = 0; s < LD_PER_THREAD; ++s) {
    const int idx = tid + s * NTHREADS;
    k_off[s] = (idx / KU) * HD + (idx % KU) * EPU;
    v_off[s] = (idx / VU) * P + (idx % VU) * EPU;
  }
  u32x4 kreg[LD_PER_THREAD], vreg[LD_PER_THREAD];
  auto load_tile = [&](int h, int kt) {
#pragma unroll
    for (int s = 0; s < LD_PER_THREAD; ++s) {
      int idx = tid + s * NTHREADS;
      int r = idx / KU, u = idx % KU;
      kreg[s] = reinterpret_cast<const u32x4*>(kbase + ((size_t)h * P + kt * KT + r) * HD)[u];
      int e = idx / VU, uv = idx % VU;
      vreg[s] = reinterpret_cast<const u32x4*>(vbase + ((size_t)h * HD + e) * P + kt * KT)[uv];
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int s = 0; s < LD_PER_THREAD; ++s) {
      int idx = tid + s * NTHREADS;
      lds_put<KU>(k_lds[buf], idx / KU, idx % KU, kreg[s]);
      lds_put<VU>(v_lds[buf], idx / VU, idx % VU, vreg[s]);
    }
  };
  // bias of a key tile as four B-operand fragments (keys 16g + 8hh + t of this
  // lane's query): one tiled 32 x 64 block (see bias_tiled_index), four
  // contiguous per-lane loads
  typedef typename El<T>::bias_t BT;
  typedef typename El<T>::bias_frag bfrag;
  auto load_bias = [&](const BT* btile, bfrag (&b)[4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) b[g] = *reinterpret_cast<const bfrag*>(btile + g * 512 + lane * 8);
  };
  // selector A-fragments: row m of the score tile is key rho(m); esel[g] puts a
  // 1 in contraction slot (hh, t) exactly when rho(m) = 16g + 8hh + t, so that
  // mma(esel[g], bias chunk) adds each score's own bias
  bfrag esel[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int t = rho(lr) - 16 * g - 8 * hh;
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = (u == t) ? 1.0f : 0.0f;
    esel[g] = to_vec8<bfrag>(v);
  }
  const frag e0 = unit_frag<T>(hh == 0 ? 1.0f : 0.0f);  // contraction slot (0,0) = 1

  // this wave's query block; blocks wholly beyond I reuse the last real block
  const int jb = qb * (QB / 32) + wave, jb_last = (I - 1) >> 5;
  const BT* bias0 = (const BT*)a.bias + ((size_t)(jb < jb_last ? jb : jb_last) * (P >> 6) << 11);
  const size_t bias_head = (size_t)P * P;        // elements per head; key tile stride 2048

  bfrag bias_next[4];                            // bias of the next tile, prefetched
  load_tile(0, 0);
  store_tile(0);
  load_bias(bias0, bias_next);
  __syncthreads();

  u32x4* orow_lds = o_lds[wave] + lr * WU;
  const int oswz = lr & (WU - 1);
  constexpr int FU = El<T>::bytes / 2;  // 16-B units per 8-element fragment
  int it = 0;       // flattened (head, key tile) counter; LDS buffer = it & 1
#pragma unroll 1
  for (int h = 0; h < NH; ++h) {
    frag qf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) qf[c] = gld8<T>(qbase + ((size_t)h * P + j) * HD + 16 * c + 8 * hh);
    float m = 0.f, lsum = 0.f;
    frag qm = unit_frag<T>(0.f);
    f32x16 o = {};
    const BT* brow = bias0 + h * bias_head;      // key tile kt at brow + kt * 2048

    // one key tile: scores, softmax, P.V.  FIRST: the first tile of the head,
    // which always takes the exact maximum.  bcur holds this tile's bias; the
    // next tile's is loaded into bnxt.
    auto tile = [&](int kt, auto first_tag) {
      constexpr bool FIRST = decltype(first_tag)::value;
      const int buf = it & 1;
      const bool more = kt + 1 < nkt;
      const int h_next = more ? h : (h + 1 < NH ? h + 1 : h);
      const int kt_next = more ? kt + 1 : (h + 1 < NH ? 0 : kt);
      load_tile(h_next, kt_next);
      frag kf[2][2], vf[2][2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int c = 0; c < 2; ++c) kf[st][c] = lds_frag<T, KU>(k_lds[buf], 32 * st + rho(lr), 2 * c + hh);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int c = 0; c < 2; ++c) vf[st][c] = lds_frag<T, VU>(v_lds[buf], rho(lr), 4 * st + 2 * hh + c);
      // s = bias (two selector products per 32 keys) + K Q^T - m
      f32x16 sc[2];
      const f32x16 zero = {};
#pragma unroll
      for (int st = 0; st < 2; ++st) sc[st] = mma(esel[0], bias_next[2 * st], zero);
#pragma unroll
      for (int st = 0; st < 2; ++st) sc[st] = mma(esel[1], bias_next[2 * st + 1], sc[st]);
      load_bias(brow + ((size_t)kt_next << 11) + (h_next - h) * bias_head, bias_next);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int st = 0; st < 2; ++st) sc[st] = mma(kf[st][c], qf[c], sc[st]);
#pragma unroll
      for (int st = 0; st < 2; ++st) sc[st] = mma(e0, qm, sc[st]);
      frag pf[2][2];
      float lt;
      if constexpr (FIRST) {
        lt = rebase_tile<T>(sc, pf, m, o, lsum, true);
        qm = unit_frag<T>(hh == 0 ? -m : 0.f);
      } else {
        lt = exp_tile<T>(sc, pf);
        if (__builtin_amdgcn_ballot_w64(!(lt <= SUM_LIMIT)) != 0) {
          lt = rebase_tile<T>(sc, pf, m, o, lsum, false);
          qm = unit_frag<T>(hh == 0 ? -m : 0.f);
        }
      }
      lsum += lt;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int c = 0; c < 2; ++c) o = mma(vf[st][c], pf[st][c], o);
      store_tile(buf ^ 1);
      __syncthreads();
      ++it;
    };

    tile(0, std::true_type{});
    for (int kt = 1; kt < nkt; ++kt) tile(kt, std::false_type{});

    // ---- finish head h: 1/l, gate
    const float inv = 1.0f / xhalf_sum(lsum);
    const T* gp = gbase + ((size_t)h * P + j) * HD + 16 * hh;
    float gv[16];
    frag_to_f32<T>(gld8<T>(gp), gv);
    frag_to_f32<T>(gld8<T>(gp + 8), gv + 8);
    float ov[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ov[i] = o[i] * inv * gv[i];
    // o^T fragments of head h (e = 16*hh + 8c + t) kept in LDS until the output projection
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      frag f = to_frag<T>(ov + 8 * c);
      u32x4 tmp[FU];
      __builtin_memcpy(tmp, &f, sizeof(f));
#pragma unroll
      for (int s2 = 0; s2 < FU; ++s2) orow_lds[((4 * h + 2 * hh + c) * FU + s2) ^ oswz] = tmp[s2];
    }
  }

  // ---- output projection: out^T[c][j] = sum_(h,e) W_o[c][h*32+e] o^T[h*32+e][j] + b_o[c]
  T* orow = (T*)a.out + (a.out_transposed ? ((size_t)j * I + line) : ((size_t)line * I + j)) * CZ;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = a.b_o ? a.b_o[32 * ct + 16 * hh + i] : 0.f;
    const T* wrow = (const T*)a.w_o + (size_t)(32 * ct + rho(lr)) * CZ + 16 * hh;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        frag wf = gld8<T>(wrow + 32 * h + 8 * c);   // W_o is small and stays in L2
        u32x4 tmp[FU];
#pragma unroll
        for (int s2 = 0; s2 < FU; ++s2) tmp[s2] = orow_lds[((4 * h + 2 * hh + c) * FU + s2) ^ oswz];
        frag of;
        __builtin_memcpy(&of, tmp, sizeof(of));
        acc = mma(wf, of, acc);
      }
    if (j < I) {
      float ov[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ov[i] = acc[i];
      T* p = orow + 32 * ct + 16 * hh;
      gst8<T>(p, to_frag<T>(ov));
      gst8<T>(p + 8, to_frag<T>(ov + 8));
    }
  }
}

// Bias pack: natural-log fp32 bias [H][I][I] (from K1 or the caller) into the
// attention kernel's tiled layout (fp16 for bf16 problems, fp32 for fp32).  Each query row is
// shifted by its own maximum before the base-2 scale and the rounding: the
// softmax over keys does not change under a per-query shift, and after it the
// entries that carry the weight sit near 0, where a bf16 rounding error is
// smallest.  Keys >= I get MASKED; values below MASKED (e.g. -inf, a masked
// key) are raised to it; padded query rows I..(I rounded up to 32)-1 get 0.
template <typename BT>
__global__ void __launch_bounds__(NTHREADS) tri_pack_bias(const float* __restrict__ src, BT* __restrict__ dst,
                                                          int I, int P, int rows_pad) {
  __shared__ float red[NTHREADS / 64];
  for (int r = blockIdx.x; r < NH * rows_pad; r += gridDim.x) {
    const int h = r / rows_pad, j = r % rows_pad;
    const float* s = src + ((size_t)h * I + j) * I;
    float mx = -INFINITY;
    if (j < I)
      for (int k = threadIdx.x; k < I; k += NTHREADS) mx = fmaxf(mx, s[k]);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();  // red is reused by the next row
    for (int k = threadIdx.x; k < P; k += NTHREADS) {
      float v = k < I ? (j < I ? (s[k] - mx) * LOG2E : 0.f) : MASKED;
      v = v < MASKED ? MASKED : v;  // NaN stays NaN
      dst[bias_tiled_index(h, j, k, P)] = (BT)v;
    }
  }
}

// ---------------------------------------------------------------- launchers
static int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    n = v;
  }
  return n;
}

hipError_t launch_project(const ProjectArgs& a, int dtype, hipStream_t stream) {
  const long ntiles = (long)a.lines * (a.P / QB);
  long grid = cu_count();
  if (dtype == 2) grid *= 4;  // fp32 keeps its weights in global memory: more workgroups fit
  if (grid > ntiles) grid = ntiles;
  if (grid < 1) grid = 1;
  if (dtype == 1)
    hipLaunchKernelGGL(tri_project<__bf16>, dim3((unsigned)grid), dim3(NTHREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(tri_project<float>, dim3((unsigned)grid), dim3(NTHREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_pack_bias(const float* src, void* dst, int I, int P, int dtype, hipStream_t stream) {
  const int rows_pad = (I + 31) & ~31;
  int grid = NH * rows_pad < 8 * cu_count() ? NH * rows_pad : 8 * cu_count();
  if (dtype == 1)
    hipLaunchKernelGGL(tri_pack_bias<_Float16>, dim3((unsigned)grid), dim3(NTHREADS), 0, stream, src,
                       (_Float16*)dst, I, P, rows_pad);
  else
    hipLaunchKernelGGL(tri_pack_bias<float>, dim3((unsigned)grid), dim3(NTHREADS), 0, stream, src,
                       (float*)dst, I, P, rows_pad);
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs& a, int dtype, hipStream_t stream) {
  const long nblk = (long)a.lines * a.nqb;
  if (dtype == 1)
    hipLaunchKernelGGL(tri_attend<__bf16>, dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(tri_attend<float>, dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace triattn
