// triattn_kernels.hip -- gfx950 (CDNA4) kernels for gated triangle self-attention.
//
//   K1 tri_project : LayerNorm fused into one MFMA GEMM per token tile,
//                    [tokens x 128] . [128 x (4*128 + 4)] -> q, k, v^T, g, pair bias.
//   tri_pack_bias  : pair bias -> per-query shifted, base-2 tiles in the order of
//                    the score accumulators (fp16 for bf16 problems, fp32 for fp32).
//   K2 tri_attend  : fused attention per (line pair, block of 128 queries), all
//                    heads: S^T = bias + K Q^T (- m), the bias widened into the
//                    score accumulator and a running maximum m, when one is needed,
//                    subtracted by the MFMA through a unit fragment; online softmax
//                    at wavefront level, O^T += V^T P^T, then 1/l, sigmoid gate and
//                    the output projection, stored once.  tri_attend_fast is its
//                    one-pass bf16 form without m, with the row sums on the MFMA.
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

#include <atomic>
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
constexpr int KT = 64;         // keys per attention tile
constexpr int NTHREADS = 256;  // 4 waves
constexpr float LOG2E = 1.4426950408889634f;
// Masked / padded keys carry this bias (base-2 units): exp2 of it underflows to
// exactly 0.  It must be finite: a row whose keys are all masked would otherwise
// reach a running maximum of -inf, and the MFMA that subtracts it multiplies -m by
// the zeros of a unit fragment (0 * inf is NaN).
constexpr float MASKED = -30000.0f;

// Word 3 of a raw (stride 0) gfx9 buffer resource: 32-bit data format, no
// swizzle.  Accesses at offsets >= num_records read 0 / are dropped.
constexpr int BUF_DWORD3 = 0x00020000;

__device__ __forceinline__ int rho(int m) { return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3); }

// Workspace pair-bias layout: fp16 (bf16 problems) or fp32, tiles in the order of
// the score accumulators.  Tile (h, j/32, k/64) holds the 32 x 64 block a wave adds
// in one key step; lane j%32 + 32*hh of a wave holds, for the keys 32*st .. 32*st +
// 31 of the tile, the scores of its query j and keys 32*st + 16*hh + i (i = 0..15),
// so its bias is one contiguous run of 16 elements: element (j, k) with k%64 =
// 32*st + 16*hh + i sits at
//   (st*64 + j%32 + 32*hh)*16 + i       inside a 2048-element tile,
// and a wave's 16-element runs of one half tile are 64 consecutive runs.
// P (a multiple of 128) bounds j, NB (P, or a key block's padded key count) bounds k.
__device__ __forceinline__ size_t bias_tiled_index(int h, int j, int k, int P, int NB) {
  const int jb = j >> 5, jj = j & 31, kb = k >> 6, kk = k & 63;
  const int st = kk >> 5, hh = (kk >> 4) & 1, i = kk & 15;
  return ((((size_t)h * (P >> 5) + jb) * (NB >> 6) + kb) << 11) + (((st << 6) + jj + 32 * hh) << 4) + i;
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

// The bias of keys 32*st .. 32*st + 31 of a tile (this lane's run of 16, see
// bias_tiled_index) as a score accumulator: b[2*st] and b[2*st + 1] are the run's
// two halves.
template <typename BF> __device__ __forceinline__ f32x16 bias_acc(const BF (&b)[4], int st) {
  f32x16 r;
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = (float)b[2 * st + (i >> 3)][i & 7];
  return r;
}
// the four pieces of this lane's bias in a tile (16 B each in fp16, 32 B in fp32)
template <typename BT, typename BF> __device__ __forceinline__ void load_bias_tile(const BT* btile, int lane,
                                                                                  BF (&b)[4]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) b[g] = *reinterpret_cast<const BF*>(btile + (((g >> 1) << 6) + lane) * 16 + 8 * (g & 1));
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

// The carried O / l of the key-block state: 16 consecutive values of one lane, fp16
// for bf16 problems (the bias dtype), fp32 for fp32 problems.
template <typename S> __device__ __forceinline__ void state_o_load(const S* p, float (&v)[16]);
template <> __device__ __forceinline__ void state_o_load<_Float16>(const _Float16* p, float (&v)[16]) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const f16x8 h = *reinterpret_cast<const f16x8*>(p + 8 * c);
#pragma unroll
    for (int t = 0; t < 8; ++t) v[8 * c + t] = (float)h[t];
  }
}
template <> __device__ __forceinline__ void state_o_load<float>(const float* p, float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 f = reinterpret_cast<const f32x4*>(p)[q];
#pragma unroll
    for (int t = 0; t < 4; ++t) v[4 * q + t] = f[t];
  }
}
template <typename S> __device__ __forceinline__ void state_o_store(S* p, const float (&v)[16]);
template <> __device__ __forceinline__ void state_o_store<_Float16>(_Float16* p, const float (&v)[16]) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    f16x8 h;
#pragma unroll
    for (int t = 0; t < 8; ++t) h[t] = (_Float16)v[8 * c + t];
    *reinterpret_cast<f16x8*>(p + 8 * c) = h;
  }
}
template <> __device__ __forceinline__ void state_o_store<float>(float* p, const float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    reinterpret_cast<f32x4*>(p)[q] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
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

// ---------------------------------------------------------------- quantized tokens
// Records of the token-wise quantization of the pair tensor (LightNobel article,
// section 2.2; layout of include/aaq.h): group A = 128 INT8 codes + 32 B of
// metadata (160 B), group B = 128 INT4 codes + the same metadata (96 B), group
// C = 128 INT4 codes + f32 s, u8 z (80 B).  A value is s (q - z) in fp32; in A and
// B up to 5 outliers (INT16 q_o with scale s_o, channel in the metadata) replace
// their channel's value (whose code is z, i.e. 0).
template <int ZF> struct ZRec;
template <> struct ZRec<1> { static constexpr int RB = 160, CB = 128, BITS = 8; static constexpr bool OUTL = true; };
template <> struct ZRec<2> { static constexpr int RB = 96, CB = 64, BITS = 4; static constexpr bool OUTL = true; };
template <> struct ZRec<3> { static constexpr int RB = 80, CB = 64, BITS = 4; static constexpr bool OUTL = false; };

// One lane's half token: channels 16c + 8hh + t (c, t = 0..7).  cw[c] holds their
// codes (8 bytes for INT8, 4 for INT4); m0, m1 the 32 B of metadata (m1 unused
// for group C).
template <int ZF> struct ZHalf {
  uint32_t cw[8][ZRec<ZF>::BITS == 8 ? 2 : 1];
  u32x4 m0, m1;
};

template <int ZF>
__device__ __forceinline__ void zhalf_load(ZHalf<ZF>& zh, const __attribute__((address_space(1))) uint8_t* rec,
                                           int hh) {
  typedef ZRec<ZF> R;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (R::BITS == 8) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 w = *reinterpret_cast<const __attribute__((address_space(1))) u32x2*>(rec + 16 * c + 8 * hh);
      zh.cw[c][0] = w[0];
      zh.cw[c][R::BITS == 8 ? 1 : 0] = w[1];
    } else {
      zh.cw[c][0] = *reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(rec + 8 * c + 4 * hh);
    }
  }
  zh.m0 = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(rec + R::CB);
  if (R::OUTL) zh.m1 = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(rec + R::CB + 16);
  else zh.m1 = u32x4{0u, 0u, 0u, 0u};
}

template <int ZF>
__device__ __forceinline__ void zhalf_decode(const ZHalf<ZF>& zh, int hh, float (&v)[8][8]) {
  typedef ZRec<ZF> R;
  const float s = __uint_as_float(zh.m0[0]);
  const int z = R::OUTL ? (int)(zh.m1[1] >> 24) : (int)(zh.m0[1] & 0xFFu);
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int q = R::BITS == 8 ? (int)((zh.cw[c][t >> 2] >> (8 * (t & 3))) & 0xFFu)
                                 : (int)((zh.cw[c][0] >> (4 * t)) & 0xFu);
      v[c][t] = (float)(q - z) * s;
    }
  if (R::OUTL) {
    const int nst = (int)(zh.m1[2] & 0xFFu);
    const int n = nst < 5 ? nst : 5;
    const float s_o = __uint_as_float(zh.m0[1]);
    for (int k = 0; k < n; ++k) {
      const uint32_t qw = k < 2 ? zh.m0[2] : (k < 4 ? zh.m0[3] : zh.m1[0]);
      const int qo = (int)(int16_t)((qw >> (16 * (k & 1))) & 0xFFFFu);
      const int ch = k < 2 ? (int)((zh.m1[0] >> (16 + 8 * k)) & 0xFFu) : (int)((zh.m1[1] >> (8 * (k - 2))) & 0xFFu);
      const float val = (float)qo * s_o;
      if (((ch >> 3) & 1) == hh) {
        const int c8 = ch >> 4, tt = ch & 7;
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int t = 0; t < 8; ++t)
            if (c == c8 && t == tt) v[c][t] = val;
      }
    }
  }
}

// ================================================================ K1: LN + projections
// A workgroup of WAVES waves loops over tiles of 32*WAVES tokens (one line,
// consecutive positions); each wave owns 32 of them.  Lane l holds token
// rho(l & 31) of its wave and, for contraction slice c = 0..7, channels
// 16c + 8*(l>>5) + t, t = 0..7: exactly its B-operand fragment of slice c.  The
// other half of the token sits in lane l ^ 32, so the LayerNorm statistics take
// one cross-half exchange each.  The 17 output tiles of 32 channels (q0..3,
// k0..3, v0..3, g0..3, and the pair bias with 4 of 32 rows used) are computed
// four at a time: four independent accumulator chains, so each weight-fragment
// read overlaps the MFMAs of the other three.  The next tile's tokens are loaded
// while the current one is computed.
template <typename T> struct ProjCfg;
template <> struct ProjCfg<__bf16> {
  static constexpr int WAVES = 8;          // two waves per SIMD
  static constexpr bool W_IN_LDS = true;   // 17*32 rows x 256 B = 136 KiB of LDS
};
template <> struct ProjCfg<float> {
  static constexpr int WAVES = 4;
  static constexpr bool W_IN_LDS = false;  // fp32 weights (272 KiB) are read through the caches
};

// Weight fragment of output tile mt (rows 32*mt + r, r = rho(lane & 31)),
// contraction slice c.
template <typename T, int WUNITS>
__device__ __forceinline__ typename El<T>::frag proj_wfrag(const u32x4* w_lds, const T* const* wsrc, int mt,
                                                           int r, int hh, int c) {
  if constexpr (ProjCfg<T>::W_IN_LDS) {
    return lds_frag<T, WUNITS>(w_lds, 32 * mt + r, 2 * c + hh);
  } else {
    const T* wp = mt < 16 ? wsrc[mt >> 2] + (size_t)((mt & 3) * 32 + r) * CZ : wsrc[4] + (size_t)(r < NH ? r : 0) * CZ;
    return gld8<T>(wp + 16 * c + 8 * hh);
  }
}

// NT output tiles mt0 .. mt0+NT-1 of one wave's 32 tokens.  SWAP puts the tokens
// on the A side (rows), which yields the transposed tile (v^T).
// bf16: the LayerNorm output enters as two bf16 parts, x = hi + lo (lo = the
// rounding residual of hi), each multiplied by the weights, so the products see x
// to about 2^-17 instead of bf16's 2^-9 (fp32: xl is unused).  LO = false uses hi
// alone (the gate: its share of the output error from rounding x is small).
template <typename T, int WUNITS, int NT, bool SWAP, bool LO = true>
__device__ __forceinline__ void proj_tiles(const u32x4* w_lds, const T* const* wsrc, int mt0, int r, int hh,
                                           const typename El<T>::frag* xf, const typename El<T>::frag* xl,
                                           f32x16* acc) {
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x16{};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    typename El<T>::frag wf[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) wf[j] = proj_wfrag<T, WUNITS>(w_lds, wsrc, mt0 + j, r, hh, c);
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = SWAP ? mma(xf[c], wf[j], acc[j]) : mma(wf[j], xf[c], acc[j]);
    if constexpr (sizeof(T) == 2 && LO) {
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = SWAP ? mma(xl[c], wf[j], acc[j]) : mma(wf[j], xl[c], acc[j]);
    }
  }
}

// Store of one wave's 32 x 32 output block through a per-wave LDS buffer, so that
// every global store instruction writes whole contiguous rows (1 KiB per
// instruction for q/k/g, 64-B row segments for v^T) instead of 16-B pieces.
// Lane (hh, lr) holds 16 values of block row `row` = rho(lr), columns 16*hh ..
// 16*hh+15.  Block row r lives at gbase + r * gstride (elements), columns
// contiguous.  The 16-B units of a row are XOR-swizzled by the row so that the
// per-lane writes and the row-major reads both spread over the banks.
template <typename T>
__device__ __forceinline__ int stage_swz(int r) { return ((r >> 1) & 1) | (((r >> 4) & 1) << 1); }

//
// The address and data registers of a block's stores are kept untouched until the
// next block's stores have been issued (StoreHold): a store still waiting for the
// memory pipeline then never holds up the wave's next writes to its registers
// (measured 4% faster for the bf16 projection, at 256 VGPRs).  HOLD = false
// skips it where the registers are not there (group-C records).
template <typename T> struct StoreHold {
  static constexpr int LU = HD * (int)sizeof(T) / 32;  // units a lane stores per block
  u32x4 v[LU];
  u32x4* p[LU];
  __device__ __forceinline__ StoreHold() {
#pragma unroll
    for (int i = 0; i < LU; ++i) {
      v[i] = u32x4{0u, 0u, 0u, 0u};
      p[i] = nullptr;
    }
  }
};

template <typename T, bool HOLD>
__device__ __forceinline__ void stage_store(u32x4* buf, int row, int hh, int lane, const float* o, T* gbase,
                                            size_t gstride, StoreHold<T>& hold) {
  constexpr int RU = HD * (int)sizeof(T) / 16;     // 16-B units per block row
  constexpr int LU = RU / 2;                       // units a lane holds
  constexpr int EPU = 16 / (int)sizeof(T);
  T vals[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) vals[i] = (T)o[i];
  u32x4 units[LU];
  __builtin_memcpy(units, vals, sizeof(units));
#pragma unroll
  for (int s = 0; s < LU; ++s) buf[row * RU + ((hh * LU + s) ^ stage_swz<T>(row))] = units[s];
  StoreHold<T> next;
#pragma unroll
  for (int i = 0; i < LU; ++i) {
    const int U = 64 * i + lane, r = U / RU, uu = U % RU;
    next.v[i] = buf[r * RU + (uu ^ stage_swz<T>(r))];
    next.p[i] = reinterpret_cast<u32x4*>(gbase + r * gstride + uu * EPU);
  }
  // streamed: the attention stage reads these blocks long after they leave
#pragma unroll
  for (int i = 0; i < LU; ++i) __builtin_nontemporal_store(next.v[i], next.p[i]);
  if constexpr (HOLD && sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < LU; ++i) asm volatile("" ::"v"(hold.v[i]), "v"(hold.p[i]));
  }
  hold = next;
}

// What one launch writes: q, k, v^T, g and the pair bias; the four without the
// bias (row blocks, whose bias comes from the caller); or the bias alone.
enum { PROJ_ALL = 0, PROJ_NO_BIAS = 1, PROJ_BIAS_ONLY = 2 };

template <typename T, int MODE, int ZF = 0>
__global__ void __launch_bounds__(64 * ProjCfg<T>::WAVES) tri_project(ProjectArgs a) {
  static_assert(ZF == 0 || sizeof(T) == 2, "quantized tokens feed the bf16 path");
  constexpr int WAVES = ProjCfg<T>::WAVES;
  constexpr bool W_IN_LDS = ProjCfg<T>::W_IN_LDS;
  constexpr int TP = 32 * WAVES;                   // positions per tile (divides P)
  constexpr int WUNITS = CZ * El<T>::bytes / 16;   // 16-B units per weight row
  constexpr int NW_ROWS = 17 * 32;
  typedef typename El<T>::frag frag;
  __shared__ u32x4 w_lds[W_IN_LDS ? NW_ROWS * WUNITS : 1];
  __shared__ __attribute__((aligned(64))) float par_lds[3 * CZ];  // gamma, beta, gate bias
  constexpr int SU = 32 * HD * (int)sizeof(T) / 16;                 // 16-B units of one output block
  __shared__ u32x4 st_lds[WAVES * SU];                              // per-wave store staging

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, lr = lane & 31;
  const T* wsrc[5] = {(const T*)a.w_q, (const T*)a.w_k, (const T*)a.w_v, (const T*)a.w_g, (const T*)a.w_b};
  u32x4* st_buf = st_lds + wave * SU;

  if (W_IN_LDS) {
    for (int idx = tid; idx < NW_ROWS * WUNITS; idx += 64 * WAVES) {
      int r = idx / WUNITS, u = idx % WUNITS, mt = r >> 5;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (mt < 4 * 4) v = reinterpret_cast<const u32x4*>(wsrc[mt >> 2] + (size_t)((mt & 3) * 32 + (r & 31)) * CZ)[u];
      else if ((r & 31) < NH) v = reinterpret_cast<const u32x4*>(wsrc[4] + (size_t)(r & 31) * CZ)[u];
      lds_put<WUNITS>(w_lds, r, u, v);
    }
  }
  for (int c = tid; c < 3 * CZ; c += 64 * WAVES)
    par_lds[c] = c < CZ ? a.ln_gamma[c] : c < 2 * CZ ? a.ln_beta[c - CZ] : (a.b_g ? a.b_g[c - 2 * CZ] : 0.f);
  __syncthreads();

  const int pblocks = a.P / TP;
  const int ntiles = a.lines * pblocks;  // <= 65536 * 256
  const T* z = (const T*)a.z;
  const int I1 = a.I - 1;

  // Address of this lane's raw token half in a tile.  Padding positions (>= I)
  // repeat the last token: their results are finite and never read as real data.
  auto z_addr = [&](int t) {
    t = t < ntiles ? t : ntiles - 1;
    const int line = t / pblocks;
    const int pos = (t - line * pblocks) * TP + wave * 32 + rho(lr);
    const int pc = pos < I1 ? pos : I1;
    return z + (size_t)line * a.z_line_stride + (size_t)pc * a.z_pos_stride + 8 * hh;
  };

  // The next tile's tokens are loaded one tile ahead, and the address of the
  // tile after that is formed right after those loads are issued, ahead of the
  // stores: a value live across the whole iteration cannot share registers with
  // store data, so the loads never wait for earlier stores to release them.
  typedef const __attribute__((address_space(1))) T* gptr;
  typedef const __attribute__((address_space(1))) uint8_t* rptr;
  // record of this lane's token (quantized tokens): same clamping as z_addr
  auto r_addr = [&](int t) {
    t = t < ntiles ? t : ntiles - 1;
    const int line = t / pblocks;
    const int pos = (t - line * pblocks) * TP + wave * 32 + rho(lr);
    const int pc = pos < I1 ? pos : I1;
    return (const uint8_t*)a.z + ((size_t)line * a.z_line_stride + (size_t)pc * a.z_pos_stride) * ZRec<ZF ? ZF : 1>::RB;
  };
  auto next_addr = [&](int t) { return ZF ? (uint64_t)r_addr(t) : (uint64_t)z_addr(t); };
  frag zp[8];
  ZHalf<ZF ? ZF : 1> zq;
  int tile = blockIdx.x;
  uint64_t zn = next_addr(tile);
  if (tile < ntiles) {
    if constexpr (ZF == 0) {
#pragma unroll
      for (int c = 0; c < 8; ++c) zp[c] = *reinterpret_cast<const __attribute__((address_space(1))) frag*>((gptr)zn + 16 * c);
    } else {
      zhalf_load<ZF>(zq, (rptr)zn, hh);
    }
  }
  zn = next_addr(tile + gridDim.x);
  // One tile.  The first one is peeled off the loop so that the loop is entered
  // with as many stores in flight as its back edge carries: the wait for the
  // prefetched tokens then never has to cover the previous tile's stores.
  auto tile_body = [&](int tile) {
    const int line = tile / pblocks;
    const int pos0 = (tile - line * pblocks) * TP + wave * 32;
    const int pos = pos0 + rho(lr);
    // The weight rows are loop-invariant: hidden from the optimiser so that it
    // does not hoist all 136 fragment reads (544 registers) out of the loop.
    int wr = rho(lr);
    asm volatile("" : "+v"(wr));
    frag zc[8];
    float zv[ZF ? 8 : 1][8];  // quantized tokens: this lane's half token decoded to fp32
    if constexpr (ZF == 0) {
#pragma unroll
      for (int c = 0; c < 8; ++c) zc[c] = zp[c];
#pragma unroll
      for (int c = 0; c < 8; ++c)  // (the last tile reloads itself)
        zp[c] = *reinterpret_cast<const __attribute__((address_space(1))) frag*>((gptr)zn + 16 * c);
    } else {
      const ZHalf<ZF> zcur = zq;
      zhalf_load<ZF>(zq, (rptr)zn, hh);
      zhalf_decode<ZF>(zcur, hh, zv);
    }
    zn = next_addr(tile + 2 * gridDim.x);
    asm volatile("" : "+v"(zn));
    auto zval = [&](int c, int t) -> float {
      if constexpr (ZF == 0) return (float)zc[c][t];
      else return zv[c][t];
    };

    // ---- LayerNorm: mean, then the centred second moment, then scale and shift
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int t = 0; t < 8; ++t) s += zval(c, t);
    const float mean = xhalf_sum(s) * (1.0f / CZ);
    float v2 = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float d = zval(c, t) - mean;
        v2 += d * d;
      }
    const float rstd = rsqrtf(xhalf_sum(v2) * (1.0f / CZ) + a.eps);
    frag xf[8], xl[sizeof(T) == 2 ? 8 : 1];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const f32x8 gm = *reinterpret_cast<const f32x8*>(par_lds + 16 * c + 8 * hh);
      const f32x8 bt = *reinterpret_cast<const f32x8*>(par_lds + CZ + 16 * c + 8 * hh);
      float t8[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) t8[t] = (zval(c, t) - mean) * rstd * gm[t] + bt[t];
      xf[c] = to_frag<T>(t8);
      if constexpr (sizeof(T) == 2) {
        float r8[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) r8[t] = t8[t] - (float)xf[c][t];
        xl[c] = to_frag<T>(r8);
      }
    }

    f32x16 acc[4];
    float o[16];
    StoreHold<T> hold;
    if (MODE != PROJ_BIAS_ONLY) {
      // q (times log2(e)/sqrt(d)) and k: lane = token pos, channels 16*hh + i of head h
      proj_tiles<T, WUNITS, 4, false>(w_lds, wsrc, 0, wr, hh, xf, xl, acc);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] = acc[h][i] * (LOG2E * 0.17677669529663687f);
        stage_store<T, ZF != 3>(st_buf, rho(lr), hh, lane, o, (T*)a.q + (((size_t)line * NH + h) * a.P + pos0) * HD, HD, hold);
      }
      proj_tiles<T, WUNITS, 4, false>(w_lds, wsrc, 4, wr, hh, xf, xl, acc);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] = acc[h][i];
        stage_store<T, ZF != 3>(st_buf, rho(lr), hh, lane, o, (T*)a.k + (((size_t)line * NH + h) * a.P + pos0) * HD, HD, hold);
      }
      // v^T: lane = channel rho(lr) of head h, tokens pos0 + 16*hh + i
      proj_tiles<T, WUNITS, 4, true>(w_lds, wsrc, 8, wr, hh, xf, xl, acc);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] = acc[h][i];
        stage_store<T, ZF != 3>(st_buf, rho(lr), hh, lane, o, (T*)a.vt + ((size_t)line * NH + h) * HD * a.P + pos0, a.P, hold);
      }
      // gate after the sigmoid (from hi alone)
      proj_tiles<T, WUNITS, 4, false, false>(w_lds, wsrc, 12, wr, hh, xf, xl, acc);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const f32x16 bg = *reinterpret_cast<const f32x16*>(par_lds + 2 * CZ + h * HD + 16 * hh);
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] = sigmoidf_(acc[h][i] + bg[i]);
        stage_store<T, ZF != 3>(st_buf, rho(lr), hh, lane, o, (T*)a.g + (((size_t)line * NH + h) * a.P + pos0) * HD, HD, hold);
      }
    }
    if (MODE != PROJ_NO_BIAS) {
      // pair bias: rows 0..3 of the tile, in the lanes of the lower half (i = head).
      // One buffer resource per head spans exactly this line's I entries, so
      // the upper half (pushed past the end) and positions >= I are dropped by
      // the hardware range check instead of a branch.
      proj_tiles<T, WUNITS, 1, false>(w_lds, wsrc, 16, wr, hh, xf, xl, acc);
      const int boff = (pos + hh * a.I) * 4;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        float* row = a.bias + ((size_t)h * a.I + a.bias_row0 + line) * a.I;
        __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(row, (short)0, a.I * 4, BUF_DWORD3);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[0][h]), rs, boff, 0, 0);
      }
    }
  };
  if (tile < ntiles) tile_body(tile);
#pragma unroll 1
  for (tile += gridDim.x; tile < ntiles; tile += gridDim.x) tile_body(tile);
}

// ================================================================ K2: fused attention
// Scores arrive from the MFMA in base-2 units: q is stored times log2(e)/sqrt(d)
// and the packed bias times log2(e), each query row of the bias shifted by its
// own maximum (the softmax over keys is unchanged by a per-query shift).  After
// that shift a score is bounded by |q||k|, so the tile softmax is just
// p = exp2(acc), its conversion, and a row sum (dot2 on packed pairs here; the
// one-pass bf16 kernel further down sums on the matrix core).
// A running shift m is only introduced when needed: when the first tile of a
// head has its maximum outside [-64, 64], or when a tile's partial sums pass
// 2^64 (far from fp32 overflow).  Then the exact maximum is taken, O and l are
// rescaled, and from there on one extra 16-deep contraction slice (a unit
// fragment times a fragment holding -m, m rounded to the compute dtype so the
// MFMA adds it exactly) subtracts m inside the MFMA.  In exact arithmetic any
// shift gives the same softmax; the shift only keeps exp2 in range.
constexpr float SUM_LIMIT = 1.8446744073709552e19f;  // 2^64
constexpr float FIRST_LIMIT = 64.0f;

template <typename T> __device__ __forceinline__ typename El<T>::frag unit_frag(float v) {
  float t8[8] = {v, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  return to_frag<T>(t8);
}

__device__ __forceinline__ float tile_max(const f32x16 (&s)[2]) {
  float mx = s[0][0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
  return xhalf_max(mx);
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

// The same exponentials for the unshifted form of the key loop: the row sum is
// accumulated into la / lb across tiles instead of being returned per tile.
template <typename T>
__device__ __forceinline__ void exp_tile_acc(const f32x16 (&s)[2], typename El<T>::frag (&pf)[2][2], float& la,
                                             float& lb) {
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float p[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) p[t] = fast_exp2(s[st][8 * c + t]);
      pf[st][c] = to_frag<T>(p);
      if constexpr (sizeof(T) == 2) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          bf16x2 pr = {pf[st][c][2 * t], pf[st][c][2 * t + 1]};
          if (t & 1) lb = __builtin_amdgcn_fdot2_f32_bf16(pr, one, lb, false);
          else la = __builtin_amdgcn_fdot2_f32_bf16(pr, one, la, false);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 8; t += 2) { la += p[t]; lb += p[t + 1]; }
      }
    }
}

// Rare path: move the shift m up to the tile's exact maximum, rescale O and l,
// shift the scores and re-exponentiate.  Returns the tile sum; d = the amount
// m moved (scores computed earlier with the old m must be shifted by it too).
template <typename T>
__device__ __forceinline__ float rebase_tile(f32x16 (&s)[2], typename El<T>::frag (&pf)[2][2], float& m,
                                             f32x16& o, float& lsum, float& d) {
  const float mx = tile_max(s);               // excess of the tile maximum over m
  const float mnew = (float)(T)(m + fmaxf(mx, 0.f));
  d = mnew - m;
  const float alpha = fast_exp2(-d);
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] *= alpha;
  lsum *= alpha;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[st][i] -= d;
  m = mnew;
  return exp_tile<T>(s, pf);
}

// Workgroup -> (line group, query block).  Workgroups are dealt to the 8 XCDs
// round-robin (XCD x runs blocks x, x+8, ...).  Mode 4 pairs the XCDs: XCD x
// serves the line groups congruent to x >> 1 (mod 4) and, of each, the half of
// the query blocks given by x & 1, so a line group's keys and values are read by
// two XCDs only and an XCD's bias slice is half of the bias.  Mode 2 splits the
// XCDs 4 x 2: XCD x serves the query blocks congruent to x % 4 and one half of
// the line groups, two query blocks at a time, each line group's keys and values
// read by 4 XCDs walking the lines in step.  Mode 0 takes the blocks in order,
// every query block of a line group side by side.  The launcher picks mode 4 up
// to I = 2048 (1.3% faster than mode 2 at I = 1024 and than mode 0 at I = 2048)
// and mode 0 above (3% faster than mode 2 at I = 4096); a mode whose shape does
// not divide falls back to the next (4 -> 2 -> 0).
__device__ __forceinline__ void map_block(int mode, int bid, int n_lg, int nqb, int& lg, int& qb) {
  if (mode == 4 && n_lg % 4 == 0 && nqb % 2 == 0) {
    const int x = bid & 7, slot = bid >> 3, nh = nqb >> 1;
    lg = (slot / nh) * 4 + (x >> 1);
    qb = (x & 1) * nh + slot % nh;
    return;
  }
  if (mode >= 2 && nqb % 8 == 0 && n_lg % 2 == 0) {
    const int x = bid & 7, slot = bid >> 3;
    const int alpha = x & 3, beta = x >> 2, n_half = n_lg >> 1;
    const int phase = slot / (2 * n_half), rem = slot - phase * 2 * n_half;
    lg = beta * n_half + (rem >> 1);
    qb = alpha + 4 * (2 * phase + (rem & 1));
  } else {
    lg = bid / nqb;
    qb = bid - lg * nqb;
  }
}

// Output projection of a workgroup's rows: out^T[c][j] = sum_(h,e) W_o[c][h*32+e]
// o^T[h*32+e][j] + b_o[c], from the gated head outputs in the workspace (this lane
// reads back exactly the o values it wrote).  W_o is staged into w_lds (the K/V
// staging area, free once the key loop is over) and b_o into a small LDS array, so
// that the products run back to back on register and LDS operands.
//  * Every global read (W_o, b_o, the head outputs of all rows) is issued before the
//    first wait: one memory latency for the whole projection.
//  * The lane's indices are recomputed here from an opaque copy of the thread id, and
//    every address is formed before the first load (a scheduling fence between).
//    Values kept from the start of the kernel would have been spilled over the key
//    loop, and a scratch reload counts in the same in-order vmcnt as the loads: a
//    reload between the loads makes the wave wait for all loads issued before it.
// j0 is the workgroup's first query (its waves take 32 queries each).
template <typename T, int ROWS, int NT>
__device__ __forceinline__ void out_projection(const AttendArgs& a, int line0, int j0, u32x4* w_lds) {
  typedef typename El<T>::frag frag;
  constexpr int WU = CZ * El<T>::bytes / 16;       // 16-B units per W_o row
  constexpr int WN = CZ * WU / NT;                 // W_o units staged per thread
  static_assert(CZ * WU % NT == 0 && CZ <= NT, "W_o / b_o staging split");
  __shared__ float bo_lds[CZ];
  unsigned tid = threadIdx.x;
  asm volatile("" : "+v"(tid));                    // a new value: nothing derived from it is reused
  const int lane = tid & 63, hh = lane >> 5, lr = lane & 31;
  const int j = j0 + (int)(tid >> 6) * 32 + lr;
  const int I = a.I, P = a.P;
  const size_t tok_line = (size_t)NH * P * HD;
  int wdst[WN];
#pragma unroll
  for (int k = 0; k < WN; ++k) {
    const int idx = (int)tid + k * NT, r = idx / WU, u = idx % WU;
    wdst[k] = r * WU + (u ^ swz<WU>(r));
  }
  const u32x4* wsrc = reinterpret_cast<const u32x4*>(a.w_o) + tid;
  const T* orow_ws[ROWS];
  T* orow[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int line = line0 + r < a.lines ? line0 + r : a.lines - 1;   // a missing row is loaded, not used
    orow_ws[r] = (const T*)a.o + (size_t)line * tok_line + (size_t)j * HD + 16 * hh;
    orow[r] = (T*)a.out + (a.out_transposed ? ((size_t)j * I + line) : ((size_t)line * I + j)) * CZ + 16 * hh;
  }
  const int arow = rho(lr);
  __builtin_amdgcn_sched_barrier(0);
  u32x4 wreg[WN];
#pragma unroll
  for (int k = 0; k < WN; ++k) wreg[k] = wsrc[k * NT];
  const float bo = a.b_o != nullptr && tid < CZ ? a.b_o[tid] : 0.f;
  frag of[ROWS][NH][2];
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int hd = 0; hd < NH; ++hd)
#pragma unroll
      for (int c = 0; c < 2; ++c) of[r][hd][c] = gld8<T>(orow_ws[r] + (size_t)hd * P * HD + 8 * c);
  // LDS-only barriers: every wave is done with the K/V tiles, then W_o and b_o are
  // in LDS; the head outputs stay in flight until the first product
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
  for (int k = 0; k < WN; ++k) w_lds[wdst[k]] = wreg[k];
  if (tid < CZ) bo_lds[tid] = bo;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  // column tiles outside, rows inside: a tile's W_o fragments are read from LDS once
  // and serve every row
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    frag wf[NH][2];
#pragma unroll
    for (int hd = 0; hd < NH; ++hd)
#pragma unroll
      for (int c = 0; c < 2; ++c) wf[hd][c] = lds_frag<T, WU>(w_lds, 32 * ct + arow, 4 * hd + 2 * hh + c);
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      if (line0 + r >= a.lines) break;
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = bo_lds[32 * ct + 16 * hh + i];
#pragma unroll
      for (int hd = 0; hd < NH; ++hd)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc = mma(wf[hd][c], of[r][hd][c], acc);
      if (j < I) {
        float ov[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) ov[i] = acc[i];
        T* p = orow[r] + 32 * ct;
        gst8<T>(p, to_frag<T>(ov));
        gst8<T>(p + 8, to_frag<T>(ov + 8));
      }
    }
  }
}

// ROWS consecutive lines per workgroup (each wave works on all of them for its
// 32 queries, so one bias tile serves ROWS rows), WAVES waves = 32*WAVES queries.
//
// Two forms.  UNSHIFTED (one-pass calls): every head runs with m = 0 and no test
// inside a key tile; a workgroup that meets a head needing a shift (its first key
// tile's maximum outside [-64, 64], or a row sum past 2^64) sets its flag in
// a.redo at the end and skips the output projection (the shifted form rewrites
// its gated head outputs in o).  The shifted form (lazy m as described above)
// then runs only the flagged workgroups of the same grid when a.redo is given,
// and every workgroup otherwise (key-block calls).  The two forms are separate
// kernels so that each is compiled with only its own registers.  For bf16 the
// unshifted form is tri_attend_fast (below); this template's unshifted form
// serves fp32.
template <typename T, int ROWS, int WAVES, int MIN_WAVES_PER_SIMD, bool UNSHIFTED>
__global__ void __launch_bounds__(WAVES * 64, MIN_WAVES_PER_SIMD) tri_attend(AttendArgs a) {
  typedef typename El<T>::frag frag;
  typedef typename El<T>::bias_t BT;
  typedef typename El<T>::bias_frag bfrag;
  constexpr int NT = WAVES * 64;
  constexpr int KU = HD * El<T>::bytes / 16;      // units per K-tile row (32 channels)
  constexpr int VU = KT * El<T>::bytes / 16;      // units per V^T-tile row (64 keys)
  constexpr int KTILE_UNITS = KT * KU;
  constexpr int VTILE_UNITS = HD * VU;
  constexpr int ROW_UNITS = KTILE_UNITS + VTILE_UNITS;
  constexpr int STAGE_UNITS = ROWS * ROW_UNITS;
  static_assert(STAGE_UNITS % NT == 0, "staging must split evenly over the threads");
  constexpr int LDT = STAGE_UNITS / NT;            // 16-B units staged per thread per tile
  constexpr int EPU = 16 / El<T>::bytes;           // elements per 16-B unit
  constexpr int QBW = 32 * WAVES;                  // queries per workgroup
  __shared__ u32x4 kv_lds[2][STAGE_UNITS];         // [buffer][row][K tile | V^T tile]
  __shared__ int redo_flag;                        // UNSHIFTED: some wave needs the shifted form

  if constexpr (!UNSHIFTED) {
    if (a.redo != nullptr && a.redo[blockIdx.x] == 0) return;   // done by the unshifted form
  }
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, lr = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar addressing
  const int I = a.I, P = a.P;
  const int n_lg = (a.lines + ROWS - 1) / ROWS;
  int lg, qb;
  map_block(a.xcd_mode, blockIdx.x, n_lg, a.nqb, lg, qb);
  const int line0 = lg * ROWS;
  const int j = qb * QBW + wave * 32 + lr;         // this lane's query
  const int kt0 = a.kt0, nbt = a.nbt;             // key tiles kt0 .. kt0+nbt-1

  // line of row r (rows past the last line repeat it and are never stored)
  auto line_of = [&](int r) { return line0 + r < a.lines ? line0 + r : a.lines - 1; };
  const size_t tok_line = (size_t)NH * P * HD;     // q, g and o elements per line
  const int KP = a.kv_P;                           // positions of k / v^T
  const size_t kv_line = (size_t)NH * KP * HD;     // k and v^T elements per line

  // staging: thread tid moves LDT units; slot s covers unit (s % SPR)*NT + tid of
  // row s / SPR, a K unit or a V^T unit for every thread alike (KTILE_UNITS is a
  // multiple of NT), so each load is a scalar base plus a fixed per-lane offset.
  static_assert(KTILE_UNITS % NT == 0 && VTILE_UNITS % NT == 0, "staging slots must not straddle K and V^T");
  constexpr int SPR = ROW_UNITS / NT;              // slots per row
  constexpr int SPK = KTILE_UNITS / NT;            // of which K slots
  uint32_t g_off[LDT];                             // per-lane byte offset inside the tile
  int l_off[LDT];
#pragma unroll
  for (int s = 0; s < LDT; ++s) {
    const int r = s / SPR, w = (s % SPR) * NT + tid;
    if ((s % SPR) < SPK) {
      const int row = w / KU, u = w % KU;
      g_off[s] = (uint32_t)(row * HD + u * EPU) * sizeof(T);
      l_off[s] = r * ROW_UNITS + row * KU + (u ^ swz<KU>(row));
    } else {
      const int ww = w - KTILE_UNITS, e = ww / VU, u = ww % VU;
      g_off[s] = (uint32_t)(e * KP + u * EPU) * sizeof(T);
      l_off[s] = r * ROW_UNITS + KTILE_UNITS + e * VU + (u ^ swz<VU>(e));
    }
  }
  u32x4 sreg[LDT];
  auto load_tile = [&](int h, int kt) {
#pragma unroll
    for (int s = 0; s < LDT; ++s) {
      const int r = s / SPR;
      const bool is_k = (s % SPR) < SPK;
      const T* base = is_k ? (const T*)a.k + line_of(r) * kv_line + ((size_t)h * KP + kt * KT) * HD
                           : (const T*)a.vt + line_of(r) * kv_line + (size_t)h * HD * KP + kt * KT;
      sreg[s] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + g_off[s]);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int s = 0; s < LDT; ++s) kv_lds[buf][l_off[s]] = sreg[s];
  };

  // bias of a key tile: this lane's runs of one tiled 32 x 64 block (see bias_tiled_index)
  auto load_bias = [&](const BT* btile, bfrag (&b)[4]) { load_bias_tile<BT, bfrag>(btile, lane, b); };
  const frag e0 = unit_frag<T>(hh == 0 ? 1.0f : 0.0f);  // contraction slot (0,0) = 1
  const f32x16 zero = {};

  // this wave's 32-query block; blocks wholly beyond I reuse the last real block
  const int jb = qb * WAVES + wave, jb_last = (I - 1) >> 5;
  const BT* bias0 = (const BT*)a.bias + ((size_t)(jb < jb_last ? jb : jb_last) * a.bias_kt << 11);
  const size_t bias_head = (size_t)P * a.bias_kt * KT;   // elements per head; key tile stride 2048

  // step g = h * nbt + kt walks the key tiles kt0 + kt of every head; the step
  // after (h, kt) is (h, kt + 1), the next head's first tile, or past the end
  // the last tile again (loaded, unused)
  auto next_tile = [&](int h, int kt, int& hn, int& ktn) {
    hn = h;
    ktn = kt + 1;
    if (ktn == nbt) {
      hn = h + 1;
      ktn = 0;
    }
    if (hn == NH) {
      hn = NH - 1;
      ktn = nbt - 1;
    }
  };
  bfrag bias_next[4];
  if (tid == 0) redo_flag = 0;
  bool bad = false;                                // UNSHIFTED: this lane saw a head that needs a shift
  if (nbt > 0) {
    load_tile(0, kt0);
    store_tile(0);
    load_bias(bias0 + ((size_t)kt0 << 11), bias_next);
    __syncthreads();
  }

  // q of head h; heads after the first are loaded during the previous head's last
  // tile, once its score products have read q
  frag qf[ROWS][2];
  auto load_q = [&](int h) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const T* qrow = (const T*)a.q + line_of(r) * tok_line + ((size_t)h * P + j) * HD + 8 * hh;
      qf[r][0] = gld8<T>(qrow);
      qf[r][1] = gld8<T>(qrow + 16);
    }
  };
  load_q(0);
#pragma unroll 1
  for (int h = 0; h < NH; ++h) {
    frag qm[ROWS];
    float m[ROWS], lsum[ROWS];
    bool mact[ROWS];                               // wave-uniform: some lane of the row has m != 0
    f32x16 o[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      qm[r] = unit_frag<T>(0.f);
      m[r] = 0.f;
      mact[r] = false;
      lsum[r] = 0.f;
      o[r] = zero;
      if (!UNSHIFTED && a.state_in) {
        // carried state: shift m (true units), sum l (held by the lower half) and
        // O / l (stored normalised, in the bias dtype; O = (O / l) * l).  This call's
        // scores carry its bias's shift c, so it runs with m' = m - c rounded to the
        // compute dtype (the MFMA subtracts m' exactly); O and l are rescaled by the
        // rounding residual 2^((m - c) - m').
        const size_t sq = ((size_t)line_of(r) * NH + h) * P + j;
        const float2 ml = *reinterpret_cast<const float2*>(a.state_ml + 2 * sq);
        const float mt = ml.x - (a.bias_shift ? a.bias_shift[(size_t)h * P + j] : 0.f);
        const float me = (float)(T)mt;
        const float alpha = fast_exp2(mt - me);
        float on[16];                              // the carried O / l
        state_o_load<BT>(reinterpret_cast<const BT*>(a.state_o) + sq * HD + 16 * hh, on);
        const float sc = ml.y * alpha;
#pragma unroll
        for (int t = 0; t < 16; ++t) o[r][t] = on[t] * sc;
        m[r] = me;
        lsum[r] = hh == 0 ? ml.y * alpha : 0.f;
        qm[r] = unit_frag<T>(hh == 0 ? -me : 0.f);
        mact[r] = __builtin_amdgcn_ballot_w64(me != 0.f) != 0;
      }
    }

    // One key tile for all rows.  The bias of the tile, converted once, is the
    // accumulator input of every row's K Q^T; -m is a last 16-deep slice.
    // FIRST: the first tile of the head.
    auto tile = [&](int kt, auto first_tag) {
      constexpr bool FIRST = decltype(first_tag)::value;
      const int g = h * nbt + kt, buf = g & 1;
      int hn, ktn;
      next_tile(h, kt, hn, ktn);
      load_tile(hn, kt0 + ktn);                             // stage the next tile
      f32x16 sbias[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) sbias[st] = bias_acc(bias_next, st);
      load_bias(bias0 + hn * bias_head + ((size_t)(kt0 + ktn) << 11), bias_next);
      // scores of every row first, so that the exponentials of row r run on the
      // VALU while the matrix core still works on row r+1 (and P.V of row r
      // overlaps the exponentials of row r+1)
      f32x16 sc[ROWS][2];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const u32x4* kl = kv_lds[buf] + r * ROW_UNITS;
        frag kf[2][2];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int c = 0; c < 2; ++c) kf[st][c] = lds_frag<T, KU>(kl, 32 * st + rho(lr), 2 * c + hh);
#pragma unroll
        for (int st = 0; st < 2; ++st) sc[r][st] = mma(kf[st][0], qf[r][0], sbias[st]);
#pragma unroll
        for (int st = 0; st < 2; ++st) sc[r][st] = mma(kf[st][1], qf[r][1], sc[r][st]);
        if (mact[r]) {
#pragma unroll
          for (int st = 0; st < 2; ++st) sc[r][st] = mma(e0, qm[r], sc[r][st]);
        }
      }
      if (kt == nbt - 1 && h + 1 < NH) load_q(h + 1);   // the next head's q (this head's is read)
      if (FIRST && !a.state_in) {                     // (a carried shift stands)
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          // first tile: shift only if its maximum is far from 0
          const float mx = tile_max(sc[r]);
          const float mf = (mx > FIRST_LIMIT || mx < -FIRST_LIMIT) ? (float)(T)mx : 0.f;
          if (__builtin_amdgcn_ballot_w64(mf != 0.f) != 0) {
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
              for (int i = 0; i < 16; ++i) sc[r][st][i] -= mf;
            m[r] = mf;
            qm[r] = unit_frag<T>(hh == 0 ? -mf : 0.f);
            mact[r] = true;
          }
        }
      }
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const u32x4* vl = kv_lds[buf] + r * ROW_UNITS + KTILE_UNITS;
        frag pf[2][2];
        float lt = exp_tile<T>(sc[r], pf);
        if (__builtin_amdgcn_ballot_w64(!(lt <= SUM_LIMIT)) != 0) {
          float d;
          lt = rebase_tile<T>(sc[r], pf, m[r], o[r], lsum[r], d);
          qm[r] = unit_frag<T>(hh == 0 ? -m[r] : 0.f);
          mact[r] = true;
        }
        lsum[r] += lt;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            frag vf = lds_frag<T, VU>(vl, rho(lr), 4 * st + 2 * hh + c);
            o[r] = mma(vf, pf[st][c], o[r]);
          }
      }
      store_tile(buf ^ 1);
      __syncthreads();
    };

    // The unshifted form of a key tile: the same products and exponentials with
    // m = 0 and no test inside the tile, so the scheduler can interleave one row's
    // products with the other row's exponentials.  It leaves the conditions under
    // which the shifted form would have introduced a shift in `bad` (the first
    // tile's maximum outside [-64, 64], or a row sum past 2^64 -- a tile sum past
    // it makes the running sum pass it too, as every term is >= 0; NaN counts).
    auto tile_unshifted = [&](int kt, auto first_tag, float (&la)[ROWS], float (&lb)[ROWS]) {
      constexpr bool FIRST = decltype(first_tag)::value;
      const int g = h * nbt + kt, buf = g & 1;
      int hn, ktn;
      next_tile(h, kt, hn, ktn);
      load_tile(hn, kt0 + ktn);
      f32x16 sbias[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) sbias[st] = bias_acc(bias_next, st);
      load_bias(bias0 + hn * bias_head + ((size_t)(kt0 + ktn) << 11), bias_next);
      f32x16 sc[ROWS][2];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const u32x4* kl = kv_lds[buf] + r * ROW_UNITS;
        frag kf[2][2];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int c = 0; c < 2; ++c) kf[st][c] = lds_frag<T, KU>(kl, 32 * st + rho(lr), 2 * c + hh);
#pragma unroll
        for (int st = 0; st < 2; ++st) sc[r][st] = mma(kf[st][0], qf[r][0], sbias[st]);
#pragma unroll
        for (int st = 0; st < 2; ++st) sc[r][st] = mma(kf[st][1], qf[r][1], sc[r][st]);
      }
      if (kt == nbt - 1 && h + 1 < NH) load_q(h + 1);   // the next head's q (this head's is read)
      if constexpr (FIRST) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          const float mx = tile_max(sc[r]);
          bad = bad || mx > FIRST_LIMIT || mx < -FIRST_LIMIT;
        }
      }
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const u32x4* vl = kv_lds[buf] + r * ROW_UNITS + KTILE_UNITS;
        frag pf[2][2];
        exp_tile_acc<T>(sc[r], pf, la[r], lb[r]);
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            frag vf = lds_frag<T, VU>(vl, rho(lr), 4 * st + 2 * hh + c);
            o[r] = mma(vf, pf[st][c], o[r]);
          }
      }
      if constexpr (sizeof(T) == 2 && ROWS == 2) {
        // issue order: the bias and row-0 score products, then each of row 1's
        // score products and row 0's P.V products beside 16 VALU instructions
        // (the exponentials, conversions and sums of the other row), then row
        // 1's P.V products
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
      store_tile(buf ^ 1);
      __syncthreads();
    };

    if constexpr (UNSHIFTED) {
      float la[ROWS], lb[ROWS];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) la[r] = lb[r] = 0.f;
      tile_unshifted(0, std::true_type{}, la, lb);
      for (int kt = 1; kt < nbt; ++kt) tile_unshifted(kt, std::false_type{}, la, lb);
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        lsum[r] = la[r] + lb[r];
        bad = bad || !(lsum[r] <= SUM_LIMIT);
      }
    } else {
      if (nbt > 0) tile(0, std::true_type{});
      for (int kt = 1; kt < nbt; ++kt) tile(kt, std::false_type{});
    }

    if (!UNSHIFTED && a.state_out) {
      // ---- key-block mode: carry (m, l, O / l) to the next block (O / l is 0 where no
      // key has weight yet)
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        if (line0 + r >= a.lines) break;
        const size_t sq = ((size_t)(line0 + r) * NH + h) * P + j;
        const float lt = xhalf_sum(lsum[r]);
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        float on[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) on[t] = o[r][t] * inv;
        state_o_store<BT>(reinterpret_cast<BT*>(a.state_o) + sq * HD + 16 * hh, on);
        const float mt = m[r] + (a.bias_shift ? a.bias_shift[(size_t)h * P + j] : 0.f);
        if (hh == 0) *reinterpret_cast<float2*>(a.state_ml + 2 * sq) = make_float2(mt, lt);
      }
      continue;
    }
    // ---- finish head h: 1/l, gate; o^T (e = 16*hh + i) to the workspace.  The
    // gates of all rows are loaded before the first store (a store keeps the compiler
    // from hoisting a later row's loads above it): one memory latency per head
    frag gf[ROWS][2];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const size_t tok = line_of(r) * tok_line + ((size_t)h * P + j) * HD + 16 * hh;
      gf[r][0] = gld8<T>((const T*)a.g + tok);
      gf[r][1] = gld8<T>((const T*)a.g + tok + 8);
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const float inv = 1.0f / xhalf_sum(lsum[r]);
      const size_t tok = line_of(r) * tok_line + ((size_t)h * P + j) * HD + 16 * hh;
      float gv[16];
      frag_to_f32<T>(gf[r][0], gv);
      frag_to_f32<T>(gf[r][1], gv + 8);
      float ov[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ov[i] = o[r][i] * inv * gv[i];
      gst8<T>((T*)a.o + tok, to_frag<T>(ov));
      gst8<T>((T*)a.o + tok + 8, to_frag<T>(ov + 8));
    }
  }

  if constexpr (UNSHIFTED) {
    // the workgroup's decision: any lane of any wave that needs a shift
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) redo_flag = 1;
    __syncthreads();
    const bool redo = redo_flag != 0;
    if (tid == 0) a.redo[blockIdx.x] = redo ? 1 : 0;
    if (redo) return;                              // the shifted form redoes this workgroup
  }
  static_assert(2 * STAGE_UNITS >= CZ * CZ * El<T>::bytes / 16, "W_o must fit in the K/V staging area");
  if (!a.state_out) out_projection<T, ROWS, NT>(a, line0, qb * QBW, &kv_lds[0][0]);
}

// ================================================================ K2: bf16 one-pass form
// The bf16 unshifted form, built for the issue rates of gfx950: v_exp_f32 issues
// about once per 9 cycles per SIMD and overlaps poorly with the matrix core, plain
// VALU work overlaps it fully, and a wave waits for a load only where it uses it.
//  * The key loop is one continuous pipeline of chunks of 32 keys x 32 queries
//    (key tile kt, row r, half st: chunk 4 kt + 2 r + st).  While the VALU
//    exponentiates chunk c, the matrix core computes the scores of chunk c + 1 and
//    the P.V and row-sum products of chunk c - 1, across key-tile boundaries, so a
//    tile has no start-up or drain phase (only a head's first and last tiles do).
//  * K/V tiles go through a ring of three LDS slots: tile t + 2 is loaded at the
//    top of tile t and stored into its slot at the end, so tile t + 1 is already in
//    LDS while tile t runs (its first scores are computed in tile t's last phase).
//  * The bias of tile t + 2 is loaded at the top of tile t as well (two tiles of
//    latency), and each chunk's bias is converted into its score accumulator.
//  * Row sums come from the matrix core (v_mfma_f32_16x16x32_bf16 with a 0/1
//    operand, below) instead of 32 dot products per tile on the VALU.
//  * A head's last tile loads, in its last phase, the next head's q and this head's
//    gates, so the head epilogue and the next head's first scores find them there.
// Semantics, workgroup grid, redo flags and epilogue are those of tri_attend's
// unshifted form.

// Row sums on the matrix core.  v_mfma_f32_16x16x32_bf16 takes, in lane l, row
// (l & 15) of A and column (l & 15) of B over contraction slots 8*(l >> 4) + t,
// and returns, in lane l, column (l & 15), rows 4*(l >> 4) + i (i = 0..3).  A P
// fragment (lane l: query l & 31, eight keys) fed as B puts query n in column n
// for slot groups 0 and 2 and query n + 16 for groups 1 and 3.  With A = 1 where
// the slot group's parity equals the row half (row >= 8), row m < 8 of column n
// sums the fragment's 16 keys of query n and row m >= 8 those of query n + 16.
__device__ __forceinline__ bf16x8 rowsum_selector(int lane) {
  const __bf16 v = (((lane >> 4) & 1) == ((lane >> 3) & 1)) ? (__bf16)1.0f : (__bf16)0.0f;
  return bf16x8{v, v, v, v, v, v, v, v};
}
// Lane whose row-sum registers hold the sums of query q (0..31): q < 16 in lanes
// 0..31 (column q), q >= 16 in lanes 32..63 (column q - 16).
__device__ __forceinline__ int rowsum_lane(int q) { return q < 16 ? q : q + 16; }

__device__ __forceinline__ f32x4 mma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

#define TA_SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
#define TA_FENCE() __builtin_amdgcn_sched_barrier(0)

template <int MIN_WAVES_PER_SIMD>
__global__ void __launch_bounds__(256, MIN_WAVES_PER_SIMD) tri_attend_fast(AttendArgs a) {
  typedef __bf16 T;
  typedef bf16x8 frag;
  typedef _Float16 BT;
  typedef f16x8 bfrag;
  constexpr int ROWS = 2, WAVES = 4, NT = WAVES * 64;
  constexpr int KU = HD * 2 / 16;                 // 16-B units per K-tile row (32 channels)
  constexpr int VU = KT * 2 / 16;                 // 16-B units per V^T-tile row (64 keys)
  constexpr int KTILE_UNITS = KT * KU;
  constexpr int VTILE_UNITS = HD * VU;
  constexpr int ROW_UNITS = KTILE_UNITS + VTILE_UNITS;
  constexpr int STAGE_UNITS = ROWS * ROW_UNITS;   // one key tile of both rows: 16 KiB
  constexpr int NSLOT = 3;                        // LDS ring
  constexpr int LDT = STAGE_UNITS / NT;           // 16-B units staged per thread per tile
  constexpr int EPU = 8;                          // bf16 elements per 16-B unit
  constexpr int QBW = 32 * WAVES;                 // queries per workgroup
  static_assert(STAGE_UNITS % NT == 0 && KTILE_UNITS % NT == 0 && VTILE_UNITS % NT == 0, "staging split");
  __shared__ u32x4 kv_lds[NSLOT * STAGE_UNITS];
  __shared__ int redo_flag;

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, lr = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int I = a.I, P = a.P;
  const int n_lg = (a.lines + ROWS - 1) / ROWS;
  int lg, qb;
  map_block(a.xcd_mode, blockIdx.x, n_lg, a.nqb, lg, qb);
  const int line0 = lg * ROWS;
  const int j = qb * QBW + wave * 32 + lr;        // this lane's query
  const int kt0 = a.kt0, nbt = a.nbt;             // nbt >= 1 (one-pass calls)
  auto line_of = [&](int r) { return line0 + r < a.lines ? line0 + r : a.lines - 1; };
  const size_t tok_line = (size_t)NH * P * HD;

  // K/V staging (as in tri_attend: each slot a scalar base plus a per-lane offset)
  constexpr int SPR = ROW_UNITS / NT;
  constexpr int SPK = KTILE_UNITS / NT;
  uint32_t g_off[LDT];
  int l_off[LDT];
#pragma unroll
  for (int s = 0; s < LDT; ++s) {
    const int r = s / SPR, w = (s % SPR) * NT + tid;
    if ((s % SPR) < SPK) {
      const int row = w / KU, u = w % KU;
      g_off[s] = (uint32_t)(row * HD + u * EPU) * sizeof(T);
      l_off[s] = r * ROW_UNITS + row * KU + (u ^ swz<KU>(row));
    } else {
      const int ww = w - KTILE_UNITS, e = ww / VU, u = ww % VU;
      g_off[s] = (uint32_t)(e * P + u * EPU) * sizeof(T);
      l_off[s] = r * ROW_UNITS + KTILE_UNITS + e * VU + (u ^ swz<VU>(e));
    }
  }
  u32x4 sreg[LDT];
  auto load_tile = [&](int h, int kt) {
#pragma unroll
    for (int s = 0; s < LDT; ++s) {
      const int r = s / SPR;
      const bool is_k = (s % SPR) < SPK;
      const T* base = is_k ? (const T*)a.k + line_of(r) * tok_line + ((size_t)h * P + kt * KT) * HD
                           : (const T*)a.vt + line_of(r) * tok_line + (size_t)h * HD * P + kt * KT;
      sreg[s] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + g_off[s]);
    }
  };
  auto store_tile = [&](int slot) {
    u32x4* dst = kv_lds + slot * STAGE_UNITS;
#pragma unroll
    for (int s = 0; s < LDT; ++s) dst[l_off[s]] = sreg[s];
  };
  const int jb = qb * WAVES + wave, jb_last = (I - 1) >> 5;
  const BT* bias0 = (const BT*)a.bias + ((size_t)(jb < jb_last ? jb : jb_last) * a.bias_kt << 11);
  const size_t bias_head = (size_t)P * a.bias_kt * KT;
  auto load_bias = [&](int h, int kt, bfrag (&b)[4]) {
    load_bias_tile<BT, bfrag>(bias0 + h * bias_head + ((size_t)kt << 11), lane, b);
  };
  const frag rsel = rowsum_selector(lane);
  const int rs_src = rowsum_lane(lr);
  const f32x16 zero = {};

  // steps: g = h * nbt + kt walks the key tiles of every head in order; (h2, kt2)
  // is step g + 2, whose bias and K/V are loaded during step g; past the last step
  // it stays on the last one (loaded, unused)
  auto advance = [&](int& hx, int& ktx) {
    if (++ktx == nbt) {
      ktx = 0;
      ++hx;
    }
    if (hx == NH) {
      hx = NH - 1;
      ktx = nbt - 1;
    }
  };
  int h2 = 0, kt2 = 0;
  int slot_cur = 0, slot_nxt = 1, slot_wr = 2;    // ring slots of steps g, g + 1, g + 2
  if (tid == 0) redo_flag = 0;
  bool bad = false;
  bfrag b_cur[4], b_nxt[4];                       // bias of steps g and g + 1
  {
    load_bias(0, kt0, b_cur);
    load_tile(0, kt0);
    store_tile(0);
    advance(h2, kt2);
    load_bias(h2, kt0 + kt2, b_nxt);
    load_tile(h2, kt0 + kt2);
    store_tile(1);
    advance(h2, kt2);
    __syncthreads();
  }

  // chunk c = 2 r + st of a tile: row r, keys 32 st .. 32 st + 31
  auto kfr = [&](const u32x4* lds, int c, frag (&kf)[2]) {
    const u32x4* kl = lds + (c >> 1) * ROW_UNITS;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) kf[cc] = lds_frag<T, KU>(kl, 32 * (c & 1) + rho(lr), 2 * cc + hh);
  };
  auto vfr = [&](const u32x4* lds, int c, frag (&vf)[2]) {
    const u32x4* vl = lds + (c >> 1) * ROW_UNITS + KTILE_UNITS;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) vf[cc] = lds_frag<T, VU>(vl, rho(lr), 4 * (c & 1) + 2 * hh + cc);
  };

  // q of head h: this lane's query on both rows.  Heads after the first are loaded in
  // the last phase of the previous head's last tile, where q is no longer read
  frag qf[ROWS][2];
  auto load_q = [&](int h) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const T* qrow = (const T*)a.q + line_of(r) * tok_line + ((size_t)h * P + j) * HD + 8 * hh;
      qf[r][0] = gld8<T>(qrow);
      qf[r][1] = gld8<T>(qrow + 16);
    }
  };
  load_q(0);
#pragma unroll 1
  for (int h = 0; h < NH; ++h) {
    f32x16 o[ROWS];
    f32x4 lacc[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      o[r] = zero;
      lacc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // scores of chunk c: the tile's bias (converted into the accumulator) + K Q^T
    auto score = [&](int c, const frag (&kf)[2], const bfrag (&b)[4]) {
      const int r = c >> 1;
      return mma(kf[1], qf[r][1], mma(kf[0], qf[r][0], bias_acc(b, c & 1)));
    };
    auto pv = [&](int c, const frag (&vf)[2], const frag (&pf)[2]) {
      const int r = c >> 1;
      o[r] = mma(vf[0], pf[0], o[r]);
      lacc[r] = mma16(rsel, pf[0], lacc[r]);
      o[r] = mma(vf[1], pf[1], o[r]);
      lacc[r] = mma16(rsel, pf[1], lacc[r]);
    };
    // carried from one tile to the next: the scores of the next tile's chunk 0,
    // and P and the V^T fragments of this tile's chunk 3
    f32x16 s_first;
    frag pf_last[2], vf_last[2];
    frag gf[ROWS][2];                              // the head's gates, loaded in its last tile

    auto tile = [&](auto first_tag, auto last_tag) {
      constexpr bool FIRST = decltype(first_tag)::value;   // first key tile of the head
      constexpr bool LAST = decltype(last_tag)::value;     // last key tile of the head
      bfrag b_far[4];                              // bias of step g + 2
      // the gates' addresses are formed before the tile's loads are issued: a base the
      // register allocator spilled is then reloaded with no prefetch in flight (a
      // scratch reload among the prefetches would make the wave wait for all of them)
      const T* gp[ROWS];
      if constexpr (LAST) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) gp[r] = (const T*)a.g + line_of(r) * tok_line + ((size_t)h * P + j) * HD + 16 * hh;
        TA_FENCE();
      }
      // K/V first: the wait for them at the end of the tile then leaves these
      // bias loads in flight (first used in the last phase of the next tile)
      load_tile(h2, kt0 + kt2);
      TA_FENCE();
      load_bias(h2, kt0 + kt2, b_far);
      TA_FENCE();
      const u32x4* cur = kv_lds + slot_cur * STAGE_UNITS;
      const u32x4* nxt = kv_lds + slot_nxt * STAGE_UNITS;
      float mxr[ROWS] = {-INFINITY, -INFINITY};
      auto expo = [&](int c, const f32x16& s, frag (&pf)[2]) {
        if constexpr (FIRST) {
          float mx = s[0];
#pragma unroll
          for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
          mxr[c >> 1] = fmaxf(mxr[c >> 1], mx);
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          float p[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) p[t] = fast_exp2(s[8 * cc + t]);
          pf[cc] = to_frag<T>(p);
        }
      };
      frag kfa[2], kfb[2], vfa[2], vfb[2], pf0[2], pf1[2], pf2[2];
      if constexpr (FIRST) {                       // fill: the scores of chunk 0
        kfr(cur, 0, kfa);
        s_first = score(0, kfa, b_cur);
        TA_FENCE();
      }
      // phase 0: scores of chunk 1, P.V of the previous tile's chunk 3 | exponentials of chunk 0
      kfr(cur, 1, kfa);
      vfr(cur, 0, vfa);
      const f32x16 s1 = score(1, kfa, b_cur);
      if constexpr (!FIRST) pv(3, vf_last, pf_last);
      expo(0, s_first, pf0);
      TA_SGB(0x100, 4);
#pragma unroll
      for (int i = 0; i < (FIRST ? 2 : 6); ++i) { TA_SGB(0x008, 1); TA_SGB(0x002, FIRST ? 12 : 4); }
      TA_FENCE();
      // phase 1: scores of chunk 2, P.V of chunk 0 | exponentials of chunk 1
      kfr(cur, 2, kfb);
      vfr(cur, 1, vfb);
      const f32x16 s2 = score(2, kfb, b_cur);
      pv(0, vfa, pf0);
      expo(1, s1, pf1);
      TA_SGB(0x100, 4);
#pragma unroll
      for (int i = 0; i < 6; ++i) { TA_SGB(0x008, 1); TA_SGB(0x002, 4); }
      TA_FENCE();
      // phase 2: scores of chunk 3, P.V of chunk 1 | exponentials of chunk 2
      kfr(cur, 3, kfa);
      vfr(cur, 2, vfa);
      const f32x16 s3 = score(3, kfa, b_cur);
      pv(1, vfb, pf1);
      expo(2, s2, pf2);
      TA_SGB(0x100, 4);
#pragma unroll
      for (int i = 0; i < 6; ++i) { TA_SGB(0x008, 1); TA_SGB(0x002, 6); }
      TA_FENCE();
      // phase 3: scores of the next tile's chunk 0, P.V of chunk 2 | exponentials of chunk 3
      if constexpr (LAST) {
        if (h + 1 < NH) load_q(h + 1);             // the next head's q (this head's is done)
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {           // this head's gates, used after the tile
          gf[r][0] = gld8<T>(gp[r]);
          gf[r][1] = gld8<T>(gp[r] + 8);
        }
      }
      if constexpr (!LAST) kfr(nxt, 0, kfb);
      vfr(cur, 3, vf_last);
      if constexpr (!LAST) s_first = score(0, kfb, b_nxt);
      pv(2, vfa, pf2);
      expo(3, s3, pf_last);
      TA_SGB(0x100, LAST ? 2 : 4);
#pragma unroll
      for (int i = 0; i < (LAST ? 4 : 6); ++i) { TA_SGB(0x008, 1); TA_SGB(0x002, LAST ? 6 : 6); }
      TA_FENCE();
      if constexpr (LAST) pv(3, vf_last, pf_last);  // drain: the head's last chunk
      if constexpr (FIRST) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          const float mx = xhalf_max(mxr[r]);
          bad = bad || mx > FIRST_LIMIT || mx < -FIRST_LIMIT;
        }
      }
      store_tile(slot_wr);                          // K/V of step g + 2
      // LDS-only fence: __syncthreads() would also wait for every global load in
      // flight (vmcnt(0)), the bias of step g + 2 included
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        b_cur[g] = b_nxt[g];
        b_nxt[g] = b_far[g];
      }
      advance(h2, kt2);
      const int s0 = slot_cur;
      slot_cur = slot_nxt;
      slot_nxt = slot_wr;
      slot_wr = s0;
    };

    if (nbt == 1) {
      tile(std::true_type{}, std::true_type{});
    } else {
      tile(std::true_type{}, std::false_type{});
      // three tiles per round: the three bias sets and the carried fragments then
      // rotate by register naming instead of 48 VGPR moves per tile (the compiler
      // does not unroll a loop with a barrier and a runtime trip count itself)
      int kt = 1;
      for (; kt + 3 <= nbt - 1; kt += 3) {
        tile(std::false_type{}, std::false_type{});
        tile(std::false_type{}, std::false_type{});
        tile(std::false_type{}, std::false_type{});
      }
      for (; kt < nbt - 1; ++kt) tile(std::false_type{}, std::false_type{});
      tile(std::false_type{}, std::true_type{});
    }

    // ---- finish head h: row sums, 1/l, gate; o^T (e = 16*hh + i) to the workspace
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const float lsum = __shfl(lacc[r][0], rs_src);
      bad = bad || !(lsum <= SUM_LIMIT);
      const float inv = 1.0f / lsum;
      const size_t tok = line_of(r) * tok_line + ((size_t)h * P + j) * HD + 16 * hh;
      float gv[16];
      frag_to_f32<T>(gf[r][0], gv);
      frag_to_f32<T>(gf[r][1], gv + 8);
      float ov[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ov[i] = o[r][i] * inv * gv[i];
      gst8<T>((T*)a.o + tok, to_frag<T>(ov));
      gst8<T>((T*)a.o + tok + 8, to_frag<T>(ov + 8));
    }
  }

  if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) redo_flag = 1;
  __syncthreads();
  const bool redo = redo_flag != 0;
  if (tid == 0) a.redo[blockIdx.x] = redo ? 1 : 0;
  if (redo) return;
  static_assert(NSLOT * STAGE_UNITS >= CZ * CZ * 2 / 16, "W_o must fit in the K/V staging area");
  out_projection<T, ROWS, NT>(a, line0, qb * QBW, kv_lds);
}

// Bias pack: natural-log fp32 bias [H][Q][K] (from K1 or the caller: Q query rows,
// K keys; Q = K = I for a whole problem, K = a key block's size for a block) into
// the attention kernel's tiled layout (fp16 for bf16 problems, fp32 for fp32) of P
// query positions by NB key positions.  Each query row is shifted by its own
// maximum before the base-2 scale and the rounding: the softmax over keys does not
// change under a per-query shift, and after it the entries that carry the weight
// sit near 0, where the absolute rounding error of fp16 (or fp32) is smallest; the shift
// (base 2) goes to `shift` when the caller needs it (key blocks).  Keys >= K get
// MASKED; values below MASKED (e.g. -inf, a masked key) are raised to it; padded
// query rows Q..(Q rounded up to 32)-1 get 0 and a zero shift.
// One wave per row (four rows per workgroup at once): the row maximum is a wave
// reduction, with no barrier, and the second pass over the row reads what the first
// one brought into the caches.  Four consecutive keys per lane: one 16-B read when
// the row is 16-B aligned, and one contiguous run of the tiled layout to write.
template <typename BT>
__global__ void __launch_bounds__(NTHREADS) tri_pack_bias(const float* __restrict__ src, BT* __restrict__ dst,
                                                          int Q, int K, int P, int NB, int rows_pad,
                                                          float* __restrict__ shift) {
  constexpr int WPB = NTHREADS / 64;  // rows in flight per workgroup
  const int lane = threadIdx.x & 63;
  const int nrows = NH * rows_pad;
  for (int r = blockIdx.x * WPB + (threadIdx.x >> 6); r < nrows; r += gridDim.x * WPB) {
    const int h = r / rows_pad, j = r % rows_pad;
    const float* s = src + ((size_t)h * Q + (j < Q ? j : 0)) * K;
    const bool vec = (reinterpret_cast<uintptr_t>(s) & 15) == 0;
    auto load4 = [&](int k0, float (&v)[4]) {
      if (vec && k0 + 3 < K) {
        const float4 f = *reinterpret_cast<const float4*>(s + k0);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = k0 + t < K ? s[k0 + t] : -INFINITY;
      }
    };
    float mx = -INFINITY;
    if (j < Q) {
#pragma unroll 4
      for (int c = lane; c < ((K + 3) >> 2); c += 64) {
        float v[4];
        load4(c << 2, v);
        mx = fmaxf(mx, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (shift != nullptr && lane == 0) shift[(size_t)h * P + j] = j < Q ? mx * LOG2E : 0.f;
#pragma unroll 4
    for (int c = lane; c < (NB >> 2); c += 64) {
      const int k0 = c << 2;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (j < Q) load4(k0, v);
      BT out4[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float x = k0 + t < K ? (j < Q ? (v[t] - mx) * LOG2E : 0.f) : MASKED;
        x = x < MASKED ? MASKED : x;  // NaN stays NaN
        out4[t] = (BT)x;
      }
      BT* d = dst + bias_tiled_index(h, j, k0, P, NB);
      if constexpr (sizeof(BT) == 2) {
        uint2 w;
        __builtin_memcpy(&w, out4, 8);
        *reinterpret_cast<uint2*>(d) = w;
      } else {
        u32x4 w;
        __builtin_memcpy(&w, out4, 16);
        *reinterpret_cast<u32x4*>(d) = w;
      }
    }
  }
}

// ---------------------------------------------------------------- launchers
// CUs of the current device, cached per device; concurrent first calls may both
// query the device and store the same value (relaxed atomics, no data race).
static int cu_count() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_project(const ProjectArgs& a, int dtype, hipStream_t stream) {
  // Persistent: bf16 holds its weights in LDS (one workgroup per CU); fp32 reads
  // them through the caches, so several workgroups share a CU.
  const int waves = dtype == 1 ? ProjCfg<__bf16>::WAVES : ProjCfg<float>::WAVES;
  const long ntiles = (long)a.lines * (a.P / (32 * waves));
  long grid = dtype == 1 ? cu_count() : 4L * cu_count();
  if (grid > ntiles) grid = ntiles;
  if (grid < 1) grid = 1;
  const int mode = a.bias_only ? PROJ_BIAS_ONLY : a.bias != nullptr ? PROJ_ALL : PROJ_NO_BIAS;
  const dim3 g((unsigned)grid), b(64 * waves);
  if (dtype == 1 && a.zfmt != 0) {
#define TRIATTN_LAUNCH_Q(ZF)                                                                              \
  if (mode == PROJ_ALL) hipLaunchKernelGGL((tri_project<__bf16, PROJ_ALL, ZF>), g, b, 0, stream, a);      \
  else if (mode == PROJ_NO_BIAS) hipLaunchKernelGGL((tri_project<__bf16, PROJ_NO_BIAS, ZF>), g, b, 0, stream, a); \
  else hipLaunchKernelGGL((tri_project<__bf16, PROJ_BIAS_ONLY, ZF>), g, b, 0, stream, a);
    if (a.zfmt == 1) { TRIATTN_LAUNCH_Q(1) }
    else if (a.zfmt == 2) { TRIATTN_LAUNCH_Q(2) }
    else { TRIATTN_LAUNCH_Q(3) }
#undef TRIATTN_LAUNCH_Q
  } else if (dtype == 1) {
    if (mode == PROJ_ALL) hipLaunchKernelGGL((tri_project<__bf16, PROJ_ALL>), g, b, 0, stream, a);
    else if (mode == PROJ_NO_BIAS) hipLaunchKernelGGL((tri_project<__bf16, PROJ_NO_BIAS>), g, b, 0, stream, a);
    else hipLaunchKernelGGL((tri_project<__bf16, PROJ_BIAS_ONLY>), g, b, 0, stream, a);
  } else {
    if (mode == PROJ_ALL) hipLaunchKernelGGL((tri_project<float, PROJ_ALL>), g, b, 0, stream, a);
    else if (mode == PROJ_NO_BIAS) hipLaunchKernelGGL((tri_project<float, PROJ_NO_BIAS>), g, b, 0, stream, a);
    else hipLaunchKernelGGL((tri_project<float, PROJ_BIAS_ONLY>), g, b, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_pack_bias(const float* src, void* dst, int Q, int K, int P, int NB, float* shift, int dtype,
                            hipStream_t stream) {
  const int rows_pad = (Q + 31) & ~31;
  const int wgs = (NH * rows_pad + NTHREADS / 64 - 1) / (NTHREADS / 64);  // one wave per row
  const int grid = wgs < 16 * cu_count() ? wgs : 16 * cu_count();
  if (dtype == 1)
    hipLaunchKernelGGL(tri_pack_bias<_Float16>, dim3((unsigned)grid), dim3(NTHREADS), 0, stream, src,
                       (_Float16*)dst, Q, K, P, NB, rows_pad, shift);
  else
    hipLaunchKernelGGL(tri_pack_bias<float>, dim3((unsigned)grid), dim3(NTHREADS), 0, stream, src,
                       (float*)dst, Q, K, P, NB, rows_pad, shift);
  return hipGetLastError();
}

#ifndef TRIATTN_ROWS
#define TRIATTN_ROWS 2
#endif
#ifndef TRIATTN_MINW
#define TRIATTN_MINW 2  // waves per SIMD the bf16 attention kernel (shifted form) is compiled for
#endif
#ifndef TRIATTN_WAVES
#define TRIATTN_WAVES 4
#endif
#ifndef TRIATTN_MINW_FAST
#define TRIATTN_MINW_FAST 2  // waves per SIMD of the bf16 one-pass kernel
#endif

size_t attend_redo_flags(int lines, int I) {
  constexpr int R = TRIATTN_ROWS, W = TRIATTN_WAVES;
  return (size_t)((lines + R - 1) / R) * (size_t)((I + 32 * W - 1) / (32 * W));
}

hipError_t launch_attend(const AttendArgs& args, int dtype, hipStream_t stream) {
  constexpr int R = TRIATTN_ROWS, W = TRIATTN_WAVES;
  AttendArgs a = args;
  a.nqb = (a.I + 32 * W - 1) / (32 * W);
  a.xcd_mode = a.I <= 2048 ? 4 : 0;
  const long nblk = (long)((a.lines + R - 1) / R) * a.nqb;
  const bool one_pass = !a.state_in && !a.state_out && a.redo != nullptr && a.nbt > 0;
  if (!one_pass) a.redo = nullptr;
  const dim3 g((unsigned)nblk), b(W * 64);
  // bf16: the one-pass kernel and the shifted form at two waves per SIMD; fp32
  // (twice the fragment registers): one
  if (dtype == 1) {
    if (one_pass) hipLaunchKernelGGL((tri_attend_fast<TRIATTN_MINW_FAST>), g, b, 0, stream, a);
    hipLaunchKernelGGL((tri_attend<__bf16, R, W, TRIATTN_MINW, false>), g, b, 0, stream, a);
  } else {
    if (one_pass) hipLaunchKernelGGL((tri_attend<float, R, W, 1, true>), g, b, 0, stream, a);
    hipLaunchKernelGGL((tri_attend<float, R, W, 1, false>), g, b, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace triattn
