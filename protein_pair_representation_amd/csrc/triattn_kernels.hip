// triattn_kernels.hip -- gfx950 (CDNA4) kernels for gated triangle self-attention.
//
//   K1 tri_project : LayerNorm fused into one MFMA GEMM per token tile,
//                    [tokens x 128] . [128 x (4*128 + 4)] -> q, k, v^T, g, pair bias.
//   K2 tri_attend  : fused attention per (line, block of 128 queries), all heads:
//                    S^T = K Q^T + bias (bias preloaded into the MFMA accumulator),
//                    online softmax at wavefront level, O^T += V^T P^T, then
//                    1/l, sigmoid gate and the output projection, stored once.
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

#include "triattn_kernels.h"

namespace triattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
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

__device__ __forceinline__ int rho(int m) { return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3); }

// ---------------------------------------------------------------- element traits
template <typename T> struct El;
template <> struct El<__bf16> {
  typedef bf16x8 frag;
  static constexpr int bytes = 2;
};
template <> struct El<float> {
  typedef f32x8 frag;
  static constexpr int bytes = 4;
};

__device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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
          for (int i = 0; i < 16; ++i) o[i] = acc[i] * 0.17677669529663687f;  // 1/sqrt(32)
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
template <typename T>
__global__ void __launch_bounds__(NTHREADS) tri_attend(AttendArgs a) {
  typedef typename El<T>::frag frag;
  constexpr int KU = HD * El<T>::bytes / 16;      // units per K-tile row (32 channels)
  constexpr int VU = KT * El<T>::bytes / 16;      // units per V^T-tile row (64 keys)
  constexpr int WU = CZ * El<T>::bytes / 16;      // units per W_o row
  constexpr int KTILE_UNITS = KT * KU;
  constexpr int VTILE_UNITS = HD * VU;
  constexpr int LD_PER_THREAD = KTILE_UNITS / NTHREADS;  // same for K and V^T tiles
  __shared__ u32x4 k_lds[2][KTILE_UNITS];
  __shared__ u32x4 v_lds[2][VTILE_UNITS];
  __shared__ u32x4 wo_lds[CZ * WU];

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

  for (int idx = tid; idx < CZ * WU; idx += NTHREADS) {
    int r = idx / WU, u = idx % WU;
    lds_put<WU>(wo_lds, r, u, reinterpret_cast<const u32x4*>((const T*)a.w_o + (size_t)r * CZ)[u]);
  }

  const T* qbase = (const T*)a.q + (size_t)line * NH * P * HD;
  const T* kbase = (const T*)a.k + (size_t)line * NH * P * HD;
  const T* vbase = (const T*)a.vt + (size_t)line * NH * HD * P;
  const T* gbase = (const T*)a.g + (size_t)line * NH * P * HD;
  const int nkt = (I + KT - 1) / KT;
  const bool ragged = (I % KT) != 0;
  const bool bias_vec = (I % 4) == 0;

  // tile loader: thread tid moves LD_PER_THREAD units of K and of V^T
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

  load_tile(0, 0);
  store_tile(0);
  __syncthreads();

  frag ofr[NH][2];  // gated, normalised head outputs: B-operand fragments of the output projection
  int it = 0;       // flattened (head, key tile) counter; LDS buffer = it & 1
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    frag qf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) qf[c] = gld8<T>(qbase + ((size_t)h * P + j) * HD + 16 * c + 8 * hh);
    float m = -1e30f, lsum = 0.f;
    f32x16 o = {};
    const float* brow = a.bias + ((size_t)h * I + jc) * I;

    for (int kt = 0; kt < nkt; ++kt, ++it) {
      const int buf = it & 1;
      const bool has_next = (kt + 1 < nkt) || (h + 1 < NH);
      if (has_next) {
        if (kt + 1 < nkt) load_tile(h, kt + 1);
        else load_tile(h + 1, 0);
      }
      // ---- scores: accumulator starts at the bias b_jk (fp32), then += K Q^T
      const int k0 = kt * KT;
      const bool tail = ragged && kt == nkt - 1;
      f32x16 s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int kb = k0 + 32 * st + 16 * hh;
        if (!tail && bias_vec) {
          const f32x4* bp = reinterpret_cast<const f32x4*>(brow + kb);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 b4 = bp[q4];
#pragma unroll
            for (int t = 0; t < 4; ++t) s[st][4 * q4 + t] = b4[t];
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) s[st][i] = (kb + i < I) ? brow[kb + i] : 0.f;
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          frag kf = lds_frag<T, KU>(k_lds[buf], 32 * st + rho(lr), 2 * c + hh);
          s[st] = mma(kf, qf[c], s[st]);
        }
        if (tail) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb + i >= I) s[st][i] = -INFINITY;
        }
      }
      // ---- online softmax (lane: one query, 32 of the tile's 64 keys)
      float mx = s[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
      mx = xhalf_max(mx);
      const float mnew = fmaxf(m, mx);
      const float alpha = fast_exp2((m - mnew) * LOG2E);
      const float mb = mnew * LOG2E;
      m = mnew;
      float psum = 0.f;
      frag pf[2][2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[i] = fast_exp2(__builtin_fmaf(s[st][i], LOG2E, -mb));
          psum += p[i];
        }
        pf[st][0] = to_frag<T>(p);
        pf[st][1] = to_frag<T>(p + 8);
      }
      lsum = lsum * alpha + psum;
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] *= alpha;
      // ---- O^T += V^T P^T, 16 keys per step
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          frag vf = lds_frag<T, VU>(v_lds[buf], rho(lr), 4 * st + 2 * hh + c);
          o = mma(vf, pf[st][c], o);
        }
      if (has_next) store_tile(buf ^ 1);
      __syncthreads();
    }
    // ---- finish head h: 1/l, gate
    const float inv = 1.0f / xhalf_sum(lsum);
    const T* gp = gbase + ((size_t)h * P + j) * HD + 16 * hh;
    float gv[16];
    frag_to_f32<T>(gld8<T>(gp), gv);
    frag_to_f32<T>(gld8<T>(gp + 8), gv + 8);
    float ov[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ov[i] = o[i] * inv * gv[i];
    ofr[h][0] = to_frag<T>(ov);
    ofr[h][1] = to_frag<T>(ov + 8);
  }

  // ---- output projection: out^T[c][j] = sum_(h,e) W_o[c][h*32+e] o^T[h*32+e][j] + b_o[c]
  T* orow = (T*)a.out + (a.out_transposed ? ((size_t)j * I + line) : ((size_t)line * I + j)) * CZ;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = a.b_o ? a.b_o[32 * ct + 16 * hh + i] : 0.f;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        frag wf = lds_frag<T, WU>(wo_lds, 32 * ct + rho(lr), 4 * h + 2 * hh + c);
        acc = mma(wf, ofr[h][c], acc);
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

hipError_t launch_attend(const AttendArgs& a, int dtype, hipStream_t stream) {
  const long nblk = (long)a.lines * a.nqb;
  if (dtype == 1)
    hipLaunchKernelGGL(tri_attend<__bf16>, dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(tri_attend<float>, dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace triattn
