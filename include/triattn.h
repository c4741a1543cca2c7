/*
 * triattn.h -- C ABI of libtriattn.so: pair-biased (gated) triangle self-attention
 * over the pair representation Z (I x I x c_z) on AMD Instinct MI355X (gfx950).
 *
 * The operator.  The pair representation is an I x I array of c_z-vectors
 * ("tokens"), c_z = 128 (LightNobel article, section 1.1).  Triangular attention
 * is the pair-tensor operator the LightNobel article singles out in section 3.1;
 * the pages never print its equations, and this library computes the standard
 * gated form (eps 1e-5, biased variance, softmax scale 1/sqrt(d)):
 *
 *   x_ij   = LayerNorm(z_ij) * gamma + beta
 *   q,k,v  = x W_q^T, x W_k^T, x W_v^T          split into H heads of width d
 *   b_jk^h = x_jk . W_b[h]                       pair bias, one scalar per head
 *   g_ij   = sigmoid(x_ij W_g^T + b_g)
 *   start: o_ij^h = sum_k softmax_k(q_ij^h.k_ik^h/sqrt(d) + b_jk^h) v_ik^h
 *   end:   o_ij^h = sum_k softmax_k(q_ij^h.k_kj^h/sqrt(d) + b_ki^h) v_kj^h
 *   out_ij = (g_ij * o_ij) W_o^T + b_o
 *
 * The softmax over keys is evaluated blockwise with a running maximum and sum,
 * so no I x I score matrix is ever stored (the on-the-fly scoring of ring
 * attention, Design-CP summary, Methodology section 1).  The row-block entry
 * point is one device's share under 1D row sharding (Design-CP summary,
 * Methodology section 1): a block of query rows with its own keys and values
 * and the whole pair bias held locally.
 *
 * Conventions shared by every entry point
 *  - All pointers are DEVICE pointers unless stated, 16-byte aligned, dense
 *    row-major (C order).  "cdt" = the compute dtype of the problem
 *    (TA_BF16: bfloat16, TA_F32: float32).
 *  - Weights follow torch.nn.Linear: W[out][in], y = x W^T.
 *  - The caller owns every buffer (inputs, weights, outputs, workspace).
 *    The library never allocates, frees or synchronises; it only enqueues
 *    kernels on `stream` (a hipStream_t; NULL = the default stream) and returns.
 *  - Every argument is validated on the host before anything is enqueued; on
 *    error nothing is launched and no output is touched.  Execution errors of
 *    an enqueued kernel surface at the caller's next synchronisation.
 *  - Calls are thread-safe; calls that share a workspace must be ordered by the
 *    caller (same stream or events).  The only global state is a cache of each
 *    device's CU count and, for triangle_attn_start_noalloc, a static device
 *    array per GPU (calls of that entry point that overlap on one GPU race).
 *  - Supported shapes: c_z = 128, heads * head_dim = 128, head_dim = 32, any
 *    1 <= I <= 65536 (ragged tails handled), 1 <= rows <= I.
 */
#ifndef TRIATTN_H
#define TRIATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TRIATTN_ABI_VERSION 7

/* Compute dtypes. */
enum { TA_BF16 = 1, TA_F32 = 2 };

/* Variants (workspace sizing, stage entry points). */
enum { TA_START = 0, TA_END = 1, TA_ROWS = 2 };

/* Return codes: 0 = success, negative = error (nothing was enqueued). */
enum {
  TA_OK = 0,
  TA_ERR_NULL_PTR = -1,          /* a required pointer is NULL */
  TA_ERR_BAD_SHAPE = -2,         /* I < 1, rows < 1, rows > I (or != I for start/end), I too large, row0 out of range */
  TA_ERR_UNSUPPORTED = -3,       /* c_z, heads, head_dim other than 128, 4, 32 */
  TA_ERR_BAD_DTYPE = -4,         /* dtype not TA_BF16 / TA_F32 */
  TA_ERR_WORKSPACE_TOO_SMALL = -5,
  TA_ERR_MISALIGNED = -6,        /* a pointer is not 16-byte aligned */
  TA_ERR_ALIAS = -7,             /* out overlaps an input or the workspace (out == z is allowed) */
  TA_ERR_HIP = -8,               /* a kernel launch was rejected by the HIP runtime */
  TA_ERR_BAD_VARIANT = -9,
  TA_ERR_BAD_EPS = -10,          /* ln_eps not finite and > 0 */
  TA_ERR_BAD_GROUP = -11,        /* AAQ group not A, B or C (include/aaq.h) */
  TA_ERR_TOO_LARGE = -12         /* the problem needs more than the static workspace of
                                    triangle_attn_start_noalloc */
};

/* Problem description (host memory). */
typedef struct ta_problem {
  int32_t I;         /* side of the pair tensor: keys per attention row */
  int32_t rows;      /* query rows computed: I for start/end; 1..I for the row block */
  int32_t c_z;       /* channels per token (128) */
  int32_t heads;     /* H (4) */
  int32_t head_dim;  /* d (32) */
  int32_t dtype;     /* TA_BF16 or TA_F32 */
  float ln_eps;      /* LayerNorm epsilon, e.g. 1e-5 */
} ta_problem;

/* Weights of one triangle-attention block (host struct of device pointers). */
typedef struct ta_weights {
  const float* ln_gamma; /* fp32 [c_z] LayerNorm scale (required) */
  const float* ln_beta;  /* fp32 [c_z] LayerNorm shift (required) */
  const void* w_q;       /* cdt [H*d][c_z] */
  const void* w_k;       /* cdt [H*d][c_z] */
  const void* w_v;       /* cdt [H*d][c_z] */
  const void* w_g;       /* cdt [H*d][c_z] gate projection */
  const void* w_b;       /* cdt [H][c_z]   pair-bias projection */
  const float* b_g;      /* fp32 [H*d] gate bias, or NULL for zero */
  const void* w_o;       /* cdt [c_z][H*d] output projection */
  const float* b_o;      /* fp32 [c_z] output bias, or NULL for zero */
} ta_weights;

/* Byte offsets of the intermediates inside a workspace, and their layouts.
 * L = lines (rows of Z for start/rows, columns of Z for end), P = positions
 * padded to a multiple of 256 (padding holds finite values).
 *   q    cdt  [L][H][P][d]   query multiplied by log2(e)/sqrt(d)
 *   k    cdt  [L][H][P][d]
 *   vt   cdt  [L][H][d][P]   value, transposed per head
 *   g    cdt  [L][H][P][d]   gate after the sigmoid
 *   o    cdt  [L][H][P][d]   attention output of each head, normalised and
 *                            gated (written by the attention stage)
 *   bias bdt  H*P*P          the packed bias the attention kernel reads (bdt =
 *                            fp16 for TA_BF16, fp32 for TA_F32): per
 *                            query row shifted by its maximum over keys, times
 *                            log2(e), in tiles of 32 queries x 64 keys (2048
 *                            elements; tile (h, j/32, k/64) at
 *                            ((h*P/32 + j/32)*P/64 + k/64)*2048); inside a tile,
 *                            with k%64 = 32st + 16hh + i, element (j, k) is at
 *                            (st*64 + j%32 + 32*hh)*16 + i (the order of the
 *                            attention kernel's score accumulators: every lane
 *                            reads one run of 16).  Keys >= I hold
 *                            -30000 (exp2 of it is 0), query rows >= I filler.
 *                            The end variant holds the transposed bias b_ki at
 *                            (h, i, k); the row block holds the caller's bias.
 *   bias_f32 fp32 [H][I][I]  start/end only: the pair bias as K1 computes it,
 *                            bias_f32[h][line][pos] = b^h of token (line, pos),
 *                            natural-log units (absent, (size_t)-1, for rows)
 *   redo int32 [ceil(L/2) * ceil(I/128)]  one flag per attention workgroup
 *                            (2 lines x 128 queries): set when one of its heads
 *                            needs a softmax shift, so that only these
 *                            workgroups run the shifted form of the kernel
 * For the end variant line = column j of Z and position = row i.
 * The attention kernel works in base 2 on shifted logits: exp2(q.k + bias - m)
 * is the softmax numerator exp(q.k/sqrt(d) + b) up to a factor common to the
 * query's row, which the normalisation removes.                              */
typedef struct ta_ws_layout {
  size_t q, k, vt, g, o, bias, bias_f32, redo; /* byte offsets */
  size_t total;             /* bytes required */
  int32_t lines, positions; /* L and padded P */
} ta_ws_layout;

/* ABI version of the loaded library (TRIATTN_ABI_VERSION). */
int triangle_attn_abi_version(void);

/* Static description of an error code. */
const char* triangle_attn_strerror(int code);

/* Workspace size and layout for `variant` (TA_START, TA_END, TA_ROWS).
 * Host-only; never touches the device.  Returns TA_OK or a validation error. */
int triangle_attn_workspace_layout(const ta_problem* prob, int variant, ta_ws_layout* layout);

/* Starting-node triangle attention (equations above).
 *   z   cdt [I][I][c_z]  input pair tensor
 *   out cdt [I][I][c_z]  result (the update only: z is not added); out == z is allowed
 *   ws  workspace of at least triangle_attn_workspace_layout(TA_START).total bytes
 * Requires prob->rows == prob->I. */
int triangle_attn_start(const ta_problem* prob, const ta_weights* w, const void* z, void* out,
                        void* ws, size_t ws_bytes, void* stream);

/* Ending-node triangle attention: attention runs down the columns of Z with
 * bias b_ki.  Same arguments as triangle_attn_start; end(Z) equals
 * start(Z^T)^T for the same weights. */
int triangle_attn_end(const ta_problem* prob, const ta_weights* w, const void* z, void* out,
                      void* ws, size_t ws_bytes, void* stream);

/* Row block (one device's share under 1D row sharding).
 *   prob->I     full side (keys per row), prob->rows = R query rows
 *   z_rows cdt  [R][I][c_z]   R consecutive rows of Z
 *   bias   fp32 [H][I][I]     the whole pair bias, bias[h][j][k] = b_jk^h (e.g. built
 *                             with triangle_attn_pair_bias); rows are independent,
 *                             so the global offset of the block is not needed.
 *                             A key can be masked with -inf (any value below
 *                             -2.0e4 acts as -2.0e4: its softmax weight is 0)
 *   out    cdt  [R][I][c_z]
 *   ws     at least triangle_attn_workspace_layout(TA_ROWS).total bytes */
int triangle_attn_start_rows(const ta_problem* prob, const ta_weights* w, const void* z_rows,
                             const float* bias, void* out, void* ws, size_t ws_bytes,
                             void* stream);

/* Pair bias of a block of rows: bias[h][row0 + r][k] = b^h(z_rows[r][k]) for
 * r < prob->rows, written into a whole [H][I][I] fp32 array (other rows are
 * untouched).  Uses the same kernel and accumulation order as the bias
 * computed inside triangle_attn_start, so the two agree bit for bit.
 * Requires 0 <= row0 and row0 + rows <= I. */
int triangle_attn_pair_bias(const ta_problem* prob, const ta_weights* w, const void* z_rows,
                            int32_t row0, float* bias, void* stream);

/* Stage 1 alone: LayerNorm + projections of `variant` into the workspace
 * (layout above).  z is [I][I][c_z] for start/end, [R][I][c_z] for rows. */
int triangle_attn_project(const ta_problem* prob, int variant, const ta_weights* w,
                          const void* z, void* ws, size_t ws_bytes, void* stream);

/* Stage 2 alone: fused attention + gate + output projection from a workspace
 * filled by triangle_attn_project with the same problem and variant.  `bias`
 * is required for TA_ROWS (natural-log units, [H][I][I]; it is first packed,
 * shifted per query and scaled by log2(e), into the workspace) and must be NULL
 * otherwise (the workspace already holds it).  Writes the workspace's `o`
 * and `redo` regions (and, for TA_ROWS, its packed bias).  Enqueues two
 * kernels: the attention without a softmax shift, then the shifted form for the
 * workgroups the first one flagged (the others return at once). */
int triangle_attn_attend(const ta_problem* prob, int variant, const ta_weights* w,
                         const float* bias, void* out, void* ws, size_t ws_bytes,
                         void* stream);

/* Key-block stage: the per-device step of attention whose keys and values
 * arrive in blocks (the 2D grid sharding of the Design-CP summary,
 * Methodology section 1, passes K/V blocks around; the softmax over keys is
 * then merged from partial states, as ring attention computes scores on the
 * fly).  For every (line, head, query) of the workspace a state is carried:
 * the shift m (base-2 units) and the sum l of exp2(score - m), in fp32, and the
 * normalised output O / l, where O = sum exp2(score - m) v, in the dtype of the
 * packed bias: fp16 for TA_BF16 problems (O / l is a convex combination of value
 * vectors, so it lies within their range; values beyond +-65504 are not
 * representable in this state), fp32 for TA_F32.  A call folds keys
 * [key0, key0 + nkeys) into it.  Blocks may come in any order; once every key
 * has been folded exactly once, triangle_attn_attend_finalize gives what
 * triangle_attn_attend gives (up to rounding).
 *   key0    a multiple of 64, 0 <= key0 < I
 *   nkeys   >= 1, key0 + nkeys <= I, a multiple of 64 unless key0 + nkeys == I
 *   first   non-zero: the state is started afresh (its content is ignored); for
 *           TA_ROWS the caller's fp32 bias [H][I][I] is packed into the
 *           workspace by this call (bias required).  Zero: the state carries the
 *           earlier blocks, bias is ignored (may be NULL)
 *   state   triangle_attn_state_bytes() bytes, 16-byte aligned: O / l
 *           [L][H][P][d] (fp16 for TA_BF16, fp32 for TA_F32), then at the next
 *           256-byte boundary (m, l) fp32 [L][H][P][2] (L, P as in the layout),
 *           then at the next one fp32 [H][P] of scratch for caller-held blocks
 *   ws      filled by triangle_attn_project with the same problem and variant */
int triangle_attn_state_bytes(const ta_problem* prob, int variant, size_t* bytes);
int triangle_attn_attend_block(const ta_problem* prob, int variant, const ta_weights* w,
                               const float* bias, int32_t key0, int32_t nkeys, int32_t first,
                               void* state, void* ws, size_t ws_bytes, void* stream);

/* Key-block stage on a block the caller holds: the ring step of that sharding.
 * The device keeps its queries (q and the gate, in `ws`, from
 * triangle_attn_project) and receives one block of keys and values at a time,
 * e.g. the k and v^T regions another device's triangle_attn_project wrote for
 * its key positions, together with the bias of this device's queries against
 * those keys.  One call folds the block into the carried state exactly as
 * triangle_attn_attend_block does for a key range of the workspace; blocks may
 * come in any order, and once every key has been folded exactly once
 * triangle_attn_attend_finalize gives what triangle_attn_attend gives (up to
 * rounding).  To fold several blocks in one call (the state is read and written
 * once per call), place them side by side in one buffer.
 *   k_blk        compute dtype [L][H][kv_positions][d]: key position p of line
 *                l, head h; positions >= nkeys are padding (finite values)
 *   vt_blk       compute dtype [L][H][d][kv_positions]: the values, transposed
 *   kv_positions positions of k_blk / vt_blk per (line, head): a multiple of 64,
 *                nkeys <= kv_positions <= P (P of the workspace layout)
 *   bias_blk     fp32 [H][I][nkeys], natural-log units: bias_blk[h][q][k] is
 *                added to the score of query position q against key k of the
 *                block (for TA_END: b_kq, as in the transposed problem).  It
 *                is packed into the workspace, shifted per query by its maximum
 *                over the block, and the shift is carried into the state's m
 *   nkeys        keys in the block, 1 <= nkeys <= I
 *   first        non-zero: the state is started afresh; zero: it carries earlier
 *                blocks (folded by this entry point; states of
 *                triangle_attn_attend_block, whose m is relative to the whole
 *                row's bias maximum, are not to be mixed with these)
 *   state, ws    as for triangle_attn_attend_block; this call overwrites the
 *                workspace's packed-bias region (scratch between calls)
 * Errors: TA_ERR_NULL_PTR, TA_ERR_MISALIGNED, TA_ERR_BAD_SHAPE (nkeys or
 * kv_positions out of range), TA_ERR_ALIAS (state or ws overlapping a block or
 * each other), TA_ERR_WORKSPACE_TOO_SMALL; nothing is enqueued on error. */
int triangle_attn_attend_kv_block(const ta_problem* prob, int variant, const ta_weights* w,
                                  const void* k_blk, const void* vt_blk, int32_t kv_positions,
                                  const float* bias_blk, int32_t nkeys, int32_t first,
                                  void* state, void* ws, size_t ws_bytes, void* stream);

/* The last step of a ring: folds the last caller-held block into the carried
 * state and finishes the rows (o = O / l, gate, output projection) into `out`,
 * in one launch: what triangle_attn_attend_kv_block followed by
 * triangle_attn_attend_finalize computes, without writing the state and reading
 * it back.  The state is read (unless `first`, which makes this block
 * the only one) and is not updated, except for its scratch tail.  Arguments as
 * for triangle_attn_attend_kv_block, plus out as in triangle_attn_attend (rows x
 * I x c_z in the compute dtype, or transposed for TA_END); it also writes the
 * workspace's o region.
 * Errors: those of triangle_attn_attend_kv_block; TA_ERR_NULL_PTR for a NULL out,
 * TA_ERR_ALIAS for out overlapping a block, the state, the workspace or a weight. */
int triangle_attn_attend_kv_block_final(const ta_problem* prob, int variant, const ta_weights* w,
                                        const void* k_blk, const void* vt_blk, int32_t kv_positions,
                                        const float* bias_blk, int32_t nkeys, int32_t first,
                                        void* state, void* out, void* ws, size_t ws_bytes,
                                        void* stream);

/* triangle_attn_start without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid it).  The workspace is a static
 * device array of TRIATTN_NOALLOC_SCRATCH_BYTES (256 MiB) that every GPU the
 * library runs on holds until the process ends; its address is looked up once
 * per device, on the first call there.  Problems whose workspace (the layout of
 * triangle_attn_workspace_layout for TA_START) exceeds it are rejected with
 * TA_ERR_TOO_LARGE before anything is enqueued: I up to about 400 in bf16, about
 * 290 in fp32.  All calls on one GPU share that GPU's array and leave their
 * intermediates in it: calls that overlap in time on one GPU (several host
 * threads, or several streams without ordering between the calls) race and
 * give undefined results; calls ordered on one stream are safe.  Nothing needs
 * to start at zero: every region the kernels read is written earlier in the same
 * call.  Other arguments and errors as for triangle_attn_start (TA_ERR_HIP also
 * when the array's address cannot be obtained). */
#define TRIATTN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int triangle_attn_start_noalloc(const ta_problem* prob, const ta_weights* w, const void* z,
                                void* out, void* stream);

/* Finish a key-block accumulation: o = O / l (as carried), sigmoid gate, output
 * projection, out as in triangle_attn_attend.  Writes the workspace's `o` region. */
int triangle_attn_attend_finalize(const ta_problem* prob, int variant, const ta_weights* w,
                                  const void* state, void* out, void* ws, size_t ws_bytes,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TRIATTN_H */
