// Internal interface between the C ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace triattn {

// K1: LayerNorm + projections of `lines` x `P` tokens (positions >= I are padding).
// Token (line, pos) is read at z + line * z_line_stride + pos * z_pos_stride (elements).
struct ProjectArgs {
  const void* z;
  int64_t z_line_stride, z_pos_stride;
  const float* ln_gamma;
  const float* ln_beta;
  float eps;
  const void *w_q, *w_k, *w_v, *w_g, *w_b;
  const float* b_g;
  void *q, *k, *vt, *g;   // workspace regions (unused when bias_only)
  float* bias;            // plain fp32 [H][I][I] (natural-log units), or nullptr
  int bias_row0;          // bias row of line 0
  int I, P, lines;
  int bias_only;
  // 0: z holds tokens of the compute dtype (strides in elements); 1, 2, 3: z holds
  // token-wise quantized records of group A, B, C (strides in records; bf16 only)
  int zfmt;
};

// K2: fused attention over `lines` lines of `I` keys; P (the padded position
// count) must be a multiple of 256.
struct AttendArgs {
  const void *q, *k, *vt, *g;
  void* o;                // workspace: gated, normalised head outputs, same layout as q
  // packed bias (tri_pack_bias, bias_tiled_index: 32-query x 64-key tiles in the
  // order of the score accumulators), base-2 units, shifted per query row, keys
  // >= I at -30000; fp16 for bf16 problems, fp32 for fp32 problems
  const void* bias;
  const void* w_o;
  const float* b_o;       // or nullptr
  void* out;
  int I, P, lines;
  int nqb;                // query blocks (set by launch_attend from the block width)
  int xcd_mode;           // workgroup placement over the XCDs (set by launch_attend)
  int out_transposed;     // 1: out[j][line], 0: out[line][j]
  // key range: tiles kt0 .. kt0+nbt-1 of 64 keys (the whole row: 0, ceil(I/64))
  int kt0, nbt;
  // carried softmax state (key-block mode): O / l [lines][H][P][d] in the bias dtype
  // (fp16 for bf16 problems, fp32 for fp32) and (m, l) [lines][H][P][2] fp32
  void* state_o;
  float* state_ml;
  int state_in;           // 1: start every head from the state instead of empty
  int state_out;          // 1: store the state at the end of every head (no gate, no output projection)
  // one-pass calls: one flag per workgroup (attend_redo_flags), written by the
  // unshifted form, read by the shifted form; nullptr: the shifted form only
  int* redo;
  // positions of the k / vt arrays (their per-line, per-head stride): P for the
  // workspace, the block's padded key count for a caller's key block
  int kv_P;
  // key tiles per 32-query row of tiles in the packed bias (P / 64, or the block's)
  int bias_kt;
  // key-block calls on a caller's block: the per-(head, query) shift (base 2) the
  // block's bias was packed with, [H][P]; the carried maximum is kept in true
  // units across blocks.  nullptr: no shift
  const float* bias_shift;
};

hipError_t launch_project(const ProjectArgs& a, int dtype, hipStream_t stream);
hipError_t launch_attend(const AttendArgs& a, int dtype, hipStream_t stream);
// number of int32 flags launch_attend needs in AttendArgs::redo for `lines` lines of I keys
size_t attend_redo_flags(int lines, int I);
// tiled dst(h, j, k) = max((src[h][j][k] - max_k src[h][j][k]) * log2(e), -30000), fp16
// for bf16 problems (dtype 1) and fp32 for fp32 problems, for Q query rows of K keys
// (src row stride K); keys >= K -30000, query rows >= Q zero.  dst holds P query positions by NB key positions (NB a multiple of 64).
// shift (or nullptr) receives max_k src[h][j][k] * log2(e), [H][P] (0 past Q).
hipError_t launch_pack_bias(const float* src, void* dst, int Q, int K, int P, int NB, float* shift, int dtype,
                            hipStream_t stream);

}  // namespace triattn
