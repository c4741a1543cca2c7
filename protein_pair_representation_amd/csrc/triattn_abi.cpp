// triattn_abi.cpp -- the C ABI of libtriattn.so (declared in include/triattn.h).
//
// Host-side only: validates every argument, sizes the workspace, and enqueues
// the two kernels on the caller's stream.  Nothing here allocates, frees or
// synchronises, and no HIP call is made before validation has passed.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/aaq.h"
#include "../../include/triattn.h"
#include "aaq_kernels.h"
#include "triattn_kernels.h"

namespace {

constexpr int kCz = 128, kHeads = 4, kHeadDim = 32, kPosAlign = 256, kMaxI = 65536, kKeyTile = 64;

size_t esize(int dtype) { return dtype == TA_BF16 ? 2 : 4; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Span {
  const void* p;
  size_t n;
};
bool overlap(Span a, Span b) {
  if (a.p == nullptr || b.p == nullptr || a.n == 0 || b.n == 0) return false;
  uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

int check_problem(const ta_problem* p, int variant) {
  if (p == nullptr) return TA_ERR_NULL_PTR;
  if (variant != TA_START && variant != TA_END && variant != TA_ROWS) return TA_ERR_BAD_VARIANT;
  if (p->dtype != TA_BF16 && p->dtype != TA_F32) return TA_ERR_BAD_DTYPE;
  if (p->c_z != kCz || p->heads != kHeads || p->head_dim != kHeadDim) return TA_ERR_UNSUPPORTED;
  if (p->I < 1 || p->I > kMaxI || p->rows < 1 || p->rows > p->I) return TA_ERR_BAD_SHAPE;
  if (variant != TA_ROWS && p->rows != p->I) return TA_ERR_BAD_SHAPE;
  if (!(p->ln_eps > 0.0f) || !isfinite(p->ln_eps)) return TA_ERR_BAD_EPS;
  return TA_OK;
}

void layout_of(const ta_problem* p, int variant, ta_ws_layout* l) {
  const size_t lines = (size_t)(variant == TA_ROWS ? p->rows : p->I);
  const size_t P = ((size_t)p->I + kPosAlign - 1) / kPosAlign * kPosAlign;
  const size_t region = align256(lines * kHeads * P * kHeadDim * esize(p->dtype));
  l->lines = (int32_t)lines;
  l->positions = (int32_t)P;
  l->q = 0;
  l->k = region;
  l->vt = 2 * region;
  l->g = 3 * region;
  l->o = 4 * region;
  // every variant: the packed bias the attention kernel reads (tiled)
  l->bias = 5 * region;
  const size_t packed = align256((size_t)kHeads * P * P * esize(p->dtype));
  size_t end;
  if (variant == TA_ROWS) {  // the caller supplies the fp32 bias
    l->bias_f32 = (size_t)-1;
    end = l->bias + packed;
  } else {                   // K1 writes the fp32 bias here, then it is packed
    l->bias_f32 = l->bias + packed;
    end = l->bias_f32 + align256((size_t)kHeads * p->I * p->I * sizeof(float));
  }
  // per-workgroup flags of the attention kernel's unshifted form
  l->redo = end;
  l->total = end + align256(triattn::attend_redo_flags((int)lines, p->I) * sizeof(int32_t));
}

int check_weights(const ta_weights* w) {
  if (w == nullptr) return TA_ERR_NULL_PTR;
  const void* req[] = {w->ln_gamma, w->ln_beta, w->w_q, w->w_k, w->w_v, w->w_g, w->w_b, w->w_o};
  for (const void* q : req)
    if (q == nullptr) return TA_ERR_NULL_PTR;
  const void* all[] = {w->ln_gamma, w->ln_beta, w->w_q, w->w_k, w->w_v, w->w_g, w->w_b, w->w_o, w->b_g, w->b_o};
  for (const void* q : all)
    if (q != nullptr && !aligned16(q)) return TA_ERR_MISALIGNED;
  return TA_OK;
}

// Out must not overlap any input, weight or the workspace (out == z exactly is fine).
int check_out_alias(const ta_problem* p, const ta_weights* w, Span out, Span z, Span ws, Span bias) {
  const size_t es = esize(p->dtype);
  const Span wspans[] = {{w->ln_gamma, kCz * 4}, {w->ln_beta, kCz * 4}, {w->w_q, (size_t)kCz * kCz * es},
                         {w->w_k, (size_t)kCz * kCz * es}, {w->w_v, (size_t)kCz * kCz * es},
                         {w->w_g, (size_t)kCz * kCz * es}, {w->w_b, (size_t)kHeads * kCz * es},
                         {w->b_g, kCz * 4}, {w->w_o, (size_t)kCz * kCz * es}, {w->b_o, kCz * 4}};
  for (const Span& s : wspans) {
    if (overlap(out, s) || overlap(ws, s)) return TA_ERR_ALIAS;
  }
  if (overlap(out, ws) || overlap(out, bias) || overlap(ws, z) || overlap(ws, bias)) return TA_ERR_ALIAS;
  if (out.p != z.p && overlap(out, z)) return TA_ERR_ALIAS;
  return TA_OK;
}

triattn::ProjectArgs project_args(const ta_problem* p, int variant, const ta_weights* w, const void* z,
                                  void* ws, const ta_ws_layout& l) {
  triattn::ProjectArgs a;
  memset(&a, 0, sizeof(a));
  a.z = z;
  if (variant == TA_END) {  // line = column j, position = row i
    a.z_line_stride = kCz;
    a.z_pos_stride = (int64_t)p->I * kCz;
  } else {
    a.z_line_stride = (int64_t)p->I * kCz;
    a.z_pos_stride = kCz;
  }
  a.ln_gamma = w->ln_gamma;
  a.ln_beta = w->ln_beta;
  a.eps = p->ln_eps;
  a.w_q = w->w_q;
  a.w_k = w->w_k;
  a.w_v = w->w_v;
  a.w_g = w->w_g;
  a.w_b = w->w_b;
  a.b_g = w->b_g;
  char* base = (char*)ws;
  a.q = base + l.q;
  a.k = base + l.k;
  a.vt = base + l.vt;
  a.g = base + l.g;
  a.bias = variant == TA_ROWS ? nullptr : (float*)(base + l.bias_f32);
  a.bias_row0 = 0;
  a.I = p->I;
  a.P = l.positions;
  a.lines = l.lines;
  a.bias_only = 0;
  return a;
}

triattn::AttendArgs attend_args(const ta_problem* p, int variant, const ta_weights* w, const float* bias,
                                void* out, void* ws, const ta_ws_layout& l) {
  triattn::AttendArgs a;
  memset(&a, 0, sizeof(a));
  const char* base = (const char*)ws;
  a.q = base + l.q;
  a.k = base + l.k;
  a.vt = base + l.vt;
  a.g = base + l.g;
  a.o = (void*)(base + l.o);
  (void)bias;  // the row-block bias is first packed into the workspace (pack_bias)
  a.bias = (const void*)(base + l.bias);
  a.w_o = w->w_o;
  a.b_o = w->b_o;
  a.out = out;
  a.I = p->I;
  a.P = l.positions;
  a.lines = l.lines;
  a.out_transposed = variant == TA_END ? 1 : 0;
  a.kt0 = 0;
  a.nbt = (p->I + kKeyTile - 1) / kKeyTile;  // every key
  a.redo = (int*)(base + l.redo);            // used by one-pass calls only
  a.kv_P = l.positions;
  a.bias_kt = l.positions / kKeyTile;
  a.bias_shift = nullptr;
  return a;
}

// State of the key-block stage: O / l [L][H][P][d] in the bias dtype (fp16 for bf16
// problems, fp32 for fp32), then (m, l) [L][H][P][2] fp32, then the per-(head, query)
// shift [H][P] fp32 of the last caller-held block's packed bias (written by that
// call's pack, read by its attention launch); each region starts at a 256-B boundary.
void state_sizes(const ta_ws_layout& l, int dtype, size_t* o_bytes, size_t* total, size_t* shift_off = nullptr) {
  const size_t oes = dtype == TA_BF16 ? 2 : 4;     // O / l in the bias dtype: fp16 or fp32
  *o_bytes = align256((size_t)l.lines * kHeads * l.positions * kHeadDim * oes);
  const size_t sh = *o_bytes + align256((size_t)l.lines * kHeads * l.positions * 2 * sizeof(float));
  if (shift_off) *shift_off = sh;
  *total = sh + align256((size_t)kHeads * l.positions * sizeof(float));
}

int enqueue(hipError_t e) { return e == hipSuccess ? TA_OK : TA_ERR_HIP; }

// fp32 bias (the caller's for the row block, K1's otherwise) -> the packed
// tiled bias the attention kernel reads.
int pack_bias(const ta_problem* p, int variant, const float* caller_bias, void* ws, const ta_ws_layout& l,
              hipStream_t s) {
  const float* src = variant == TA_ROWS ? caller_bias : (const float*)((char*)ws + l.bias_f32);
  return enqueue(triattn::launch_pack_bias(src, (char*)ws + l.bias, p->I, p->I, l.positions, l.positions, nullptr,
                                           p->dtype, s));
}

// Shared implementation of start / end / rows.
int run_full(const ta_problem* p, int variant, const ta_weights* w, const void* z, const float* bias,
             void* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_problem(p, variant);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if (z == nullptr || out == nullptr || ws == nullptr) return TA_ERR_NULL_PTR;
  if (variant == TA_ROWS && bias == nullptr) return TA_ERR_NULL_PTR;
  if (!aligned16(z) || !aligned16(out) || !aligned16(ws) || (bias && !aligned16(bias))) return TA_ERR_MISALIGNED;
  ta_ws_layout l;
  layout_of(p, variant, &l);
  if (ws_bytes < l.total) return TA_ERR_WORKSPACE_TOO_SMALL;
  const size_t tok_bytes = (size_t)p->rows * p->I * kCz * esize(p->dtype);
  const Span bspan = {bias, bias ? (size_t)kHeads * p->I * p->I * sizeof(float) : 0};
  if ((rc = check_out_alias(p, w, {out, tok_bytes}, {z, tok_bytes}, {ws, l.total}, bspan))) return rc;

  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();  // clear a stale error so that only our launches are reported
  triattn::ProjectArgs pa = project_args(p, variant, w, z, ws, l);
  if ((rc = enqueue(triattn::launch_project(pa, p->dtype, s)))) return rc;
  if ((rc = pack_bias(p, variant, bias, ws, l, s))) return rc;
  triattn::AttendArgs aa = attend_args(p, variant, w, bias, out, ws, l);
  return enqueue(triattn::launch_attend(aa, p->dtype, s));
}

// Static workspace of triangle_attn_start_noalloc: one copy per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: only the per-device address from hipGetSymbolAddress is ever used.
static __device__ __align__(256) unsigned char scratch[TRIATTN_NOALLOC_SCRATCH_BYTES];
static_assert(sizeof(scratch) == TRIATTN_NOALLOC_SCRATCH_BYTES, "scratch size");

// Address of `scratch` on the current device, looked up once per device (with that
// device current, as this function is called).  nullptr if the runtime fails.
void* scratch_on_current_device() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

}  // namespace

extern "C" {

int triangle_attn_abi_version(void) { return TRIATTN_ABI_VERSION; }

const char* triangle_attn_strerror(int code) {
  switch (code) {
    case TA_OK: return "success";
    case TA_ERR_NULL_PTR: return "a required pointer is NULL";
    case TA_ERR_BAD_SHAPE: return "bad shape (I, rows or row0 out of range)";
    case TA_ERR_UNSUPPORTED: return "unsupported c_z / heads / head_dim (need 128 / 4 / 32)";
    case TA_ERR_BAD_DTYPE: return "dtype must be TA_BF16 or TA_F32";
    case TA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case TA_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case TA_ERR_ALIAS: return "output overlaps an input, a weight or the workspace";
    case TA_ERR_HIP: return "HIP runtime rejected a kernel launch";
    case TA_ERR_BAD_VARIANT: return "unknown variant";
    case TA_ERR_BAD_EPS: return "ln_eps must be finite and positive";
    case TA_ERR_BAD_GROUP: return "AAQ group must be AAQ_GROUP_A, _B or _C";
    case TA_ERR_TOO_LARGE:
      return "problem needs more than the 256 MiB static workspace of triangle_attn_start_noalloc";
    default: return "unknown error code";
  }
}

int triangle_attn_workspace_layout(const ta_problem* prob, int variant, ta_ws_layout* layout) {
  int rc = check_problem(prob, variant);
  if (rc) return rc;
  if (layout == nullptr) return TA_ERR_NULL_PTR;
  layout_of(prob, variant, layout);
  return TA_OK;
}

int triangle_attn_start(const ta_problem* prob, const ta_weights* w, const void* z, void* out, void* ws,
                        size_t ws_bytes, void* stream) {
  return run_full(prob, TA_START, w, z, nullptr, out, ws, ws_bytes, stream);
}

int triangle_attn_start_noalloc(const ta_problem* prob, const ta_weights* w, const void* z, void* out,
                                void* stream) {
  int rc = check_problem(prob, TA_START);
  if (rc) return rc;
  ta_ws_layout l;
  layout_of(prob, TA_START, &l);
  if (l.total > TRIATTN_NOALLOC_SCRATCH_BYTES) return TA_ERR_TOO_LARGE;
  if ((rc = check_weights(w))) return rc;
  if (z == nullptr || out == nullptr) return TA_ERR_NULL_PTR;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return TA_ERR_HIP;
  return run_full(prob, TA_START, w, z, nullptr, out, ws, TRIATTN_NOALLOC_SCRATCH_BYTES, stream);
}

int triangle_attn_end(const ta_problem* prob, const ta_weights* w, const void* z, void* out, void* ws,
                      size_t ws_bytes, void* stream) {
  return run_full(prob, TA_END, w, z, nullptr, out, ws, ws_bytes, stream);
}

int triangle_attn_start_rows(const ta_problem* prob, const ta_weights* w, const void* z_rows, const float* bias,
                             void* out, void* ws, size_t ws_bytes, void* stream) {
  return run_full(prob, TA_ROWS, w, z_rows, bias, out, ws, ws_bytes, stream);
}

int triangle_attn_pair_bias(const ta_problem* prob, const ta_weights* w, const void* z_rows, int32_t row0,
                            float* bias, void* stream) {
  int rc = check_problem(prob, TA_ROWS);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if (z_rows == nullptr || bias == nullptr) return TA_ERR_NULL_PTR;
  if (row0 < 0 || (int64_t)row0 + prob->rows > prob->I) return TA_ERR_BAD_SHAPE;
  if (!aligned16(z_rows) || !aligned16(bias)) return TA_ERR_MISALIGNED;
  const size_t bias_bytes = (size_t)kHeads * prob->I * prob->I * sizeof(float);
  const size_t tok_bytes = (size_t)prob->rows * prob->I * kCz * esize(prob->dtype);
  if ((rc = check_out_alias(prob, w, {bias, bias_bytes}, {z_rows, tok_bytes}, {nullptr, 0}, {nullptr, 0})))
    return rc;
  if (overlap({bias, bias_bytes}, {z_rows, tok_bytes})) return TA_ERR_ALIAS;
  ta_ws_layout l;
  layout_of(prob, TA_ROWS, &l);
  triattn::ProjectArgs a = project_args(prob, TA_ROWS, w, z_rows, nullptr, l);
  a.q = a.k = a.vt = a.g = nullptr;
  a.bias = bias;
  a.bias_row0 = row0;
  a.bias_only = 1;
  (void)hipGetLastError();
  return enqueue(triattn::launch_project(a, prob->dtype, (hipStream_t)stream));
}

int triangle_attn_project(const ta_problem* prob, int variant, const ta_weights* w, const void* z, void* ws,
                          size_t ws_bytes, void* stream) {
  int rc = check_problem(prob, variant);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if (z == nullptr || ws == nullptr) return TA_ERR_NULL_PTR;
  if (!aligned16(z) || !aligned16(ws)) return TA_ERR_MISALIGNED;
  ta_ws_layout l;
  layout_of(prob, variant, &l);
  if (ws_bytes < l.total) return TA_ERR_WORKSPACE_TOO_SMALL;
  const size_t tok_bytes = (size_t)prob->rows * prob->I * kCz * esize(prob->dtype);
  if ((rc = check_out_alias(prob, w, {ws, l.total}, {z, tok_bytes}, {nullptr, 0}, {nullptr, 0}))) return rc;
  if (overlap({ws, l.total}, {z, tok_bytes})) return TA_ERR_ALIAS;
  (void)hipGetLastError();
  triattn::ProjectArgs a = project_args(prob, variant, w, z, ws, l);
  if ((rc = enqueue(triattn::launch_project(a, prob->dtype, (hipStream_t)stream)))) return rc;
  if (variant == TA_ROWS) return TA_OK;  // the row block's bias arrives with the attention stage
  return pack_bias(prob, variant, nullptr, ws, l, (hipStream_t)stream);
}

int triangle_attn_project_aaq(const ta_problem* prob, int variant, const ta_weights* w, const void* records,
                              int group, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_problem(prob, variant);
  if (rc) return rc;
  if (prob->dtype != TA_BF16) return TA_ERR_BAD_DTYPE;
  const int rb = aaq::record_bytes(group);
  if (rb < 0) return TA_ERR_BAD_GROUP;
  if ((rc = check_weights(w))) return rc;
  if (records == nullptr || ws == nullptr) return TA_ERR_NULL_PTR;
  if (!aligned16(records) || !aligned16(ws)) return TA_ERR_MISALIGNED;
  ta_ws_layout l;
  layout_of(prob, variant, &l);
  if (ws_bytes < l.total) return TA_ERR_WORKSPACE_TOO_SMALL;
  const size_t rec_bytes = (size_t)prob->rows * prob->I * rb;
  if ((rc = check_out_alias(prob, w, {ws, l.total}, {records, rec_bytes}, {nullptr, 0}, {nullptr, 0}))) return rc;
  if (overlap({ws, l.total}, {records, rec_bytes})) return TA_ERR_ALIAS;
  (void)hipGetLastError();
  triattn::ProjectArgs a = project_args(prob, variant, w, records, ws, l);
  a.zfmt = group + 1;
  a.z_line_stride /= kCz;  // in records
  a.z_pos_stride /= kCz;
  if ((rc = enqueue(triattn::launch_project(a, prob->dtype, (hipStream_t)stream)))) return rc;
  if (variant == TA_ROWS) return TA_OK;
  return pack_bias(prob, variant, nullptr, ws, l, (hipStream_t)stream);
}

int triangle_attn_attend(const ta_problem* prob, int variant, const ta_weights* w, const float* bias, void* out,
                         void* ws, size_t ws_bytes, void* stream) {
  int rc = check_problem(prob, variant);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if (out == nullptr || ws == nullptr) return TA_ERR_NULL_PTR;
  if (variant == TA_ROWS && bias == nullptr) return TA_ERR_NULL_PTR;
  if (variant != TA_ROWS && bias != nullptr) return TA_ERR_BAD_VARIANT;
  if (!aligned16(out) || !aligned16(ws) || (bias && !aligned16(bias))) return TA_ERR_MISALIGNED;
  ta_ws_layout l;
  layout_of(prob, variant, &l);
  if (ws_bytes < l.total) return TA_ERR_WORKSPACE_TOO_SMALL;
  const size_t tok_bytes = (size_t)prob->rows * prob->I * kCz * esize(prob->dtype);
  const Span bspan = {bias, bias ? (size_t)kHeads * prob->I * prob->I * sizeof(float) : 0};
  if ((rc = check_out_alias(prob, w, {out, tok_bytes}, {nullptr, 0}, {ws, l.total}, bspan))) return rc;
  (void)hipGetLastError();
  if (variant == TA_ROWS && (rc = pack_bias(prob, variant, bias, ws, l, (hipStream_t)stream))) return rc;
  triattn::AttendArgs a = attend_args(prob, variant, w, bias, out, ws, l);
  return enqueue(triattn::launch_attend(a, prob->dtype, (hipStream_t)stream));
}

int triangle_attn_state_bytes(const ta_problem* prob, int variant, size_t* bytes) {
  int rc = check_problem(prob, variant);
  if (rc) return rc;
  if (bytes == nullptr) return TA_ERR_NULL_PTR;
  ta_ws_layout l;
  layout_of(prob, variant, &l);
  size_t ob;
  state_sizes(l, prob->dtype, &ob, bytes);
  return TA_OK;
}

int triangle_attn_attend_block(const ta_problem* prob, int variant, const ta_weights* w, const float* bias,
                               int32_t key0, int32_t nkeys, int32_t first, void* state, void* ws,
                               size_t ws_bytes, void* stream) {
  int rc = check_problem(prob, variant);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if (state == nullptr || ws == nullptr) return TA_ERR_NULL_PTR;
  const bool pack = variant == TA_ROWS && first != 0;
  if (pack && bias == nullptr) return TA_ERR_NULL_PTR;
  if (!aligned16(state) || !aligned16(ws) || (pack && !aligned16(bias))) return TA_ERR_MISALIGNED;
  const int I = prob->I;
  if (key0 < 0 || key0 >= I || key0 % kKeyTile != 0 || nkeys < 1 || nkeys > I - key0 ||
      (nkeys % kKeyTile != 0 && key0 + nkeys != I))
    return TA_ERR_BAD_SHAPE;
  ta_ws_layout l;
  layout_of(prob, variant, &l);
  if (ws_bytes < l.total) return TA_ERR_WORKSPACE_TOO_SMALL;
  size_t ob, sb;
  state_sizes(l, prob->dtype, &ob, &sb);
  const Span bspan = {pack ? bias : nullptr, pack ? (size_t)kHeads * I * I * sizeof(float) : 0};
  if ((rc = check_out_alias(prob, w, {state, sb}, {nullptr, 0}, {ws, l.total}, bspan))) return rc;
  (void)hipGetLastError();
  if (pack && (rc = pack_bias(prob, variant, bias, ws, l, (hipStream_t)stream))) return rc;
  triattn::AttendArgs a = attend_args(prob, variant, w, nullptr, nullptr, ws, l);
  a.kt0 = key0 / kKeyTile;
  a.nbt = (nkeys + kKeyTile - 1) / kKeyTile;
  a.state_o = state;
  a.state_ml = (float*)((char*)state + ob);
  a.state_in = first ? 0 : 1;
  a.state_out = 1;
  return enqueue(triattn::launch_attend(a, prob->dtype, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// One caller-held key block: pack its bias (shift into the state's tail), then the
// shifted attention form folds it into the state (out == nullptr) or, for the last
// block, folds it and finishes the rows into out without writing the state.
int kv_block(const ta_problem* prob, int variant, const ta_weights* w, const void* k_blk, const void* vt_blk,
             int32_t kv_positions, const float* bias_blk, int32_t nkeys, int32_t first, void* state, void* out,
             void* ws, size_t ws_bytes, void* stream) {
  int rc = check_problem(prob, variant);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if (k_blk == nullptr || vt_blk == nullptr || bias_blk == nullptr || state == nullptr || ws == nullptr)
    return TA_ERR_NULL_PTR;
  if (!aligned16(k_blk) || !aligned16(vt_blk) || !aligned16(bias_blk) || !aligned16(state) || !aligned16(ws) ||
      (out != nullptr && !aligned16(out)))
    return TA_ERR_MISALIGNED;
  ta_ws_layout l;
  layout_of(prob, variant, &l);
  // a block has 1..I keys, stored at kv_positions >= nkeys positions (a multiple of the
  // key tile, at most the workspace's P: its packed bias reuses the workspace's region)
  if (nkeys < 1 || nkeys > prob->I || kv_positions < nkeys || kv_positions % kKeyTile != 0 ||
      kv_positions > l.positions)
    return TA_ERR_BAD_SHAPE;
  if (ws_bytes < l.total) return TA_ERR_WORKSPACE_TOO_SMALL;
  size_t ob, sb, shift_off;
  state_sizes(l, prob->dtype, &ob, &sb, &shift_off);
  const size_t es = esize(prob->dtype);
  const size_t kv_bytes = (size_t)l.lines * kHeads * kv_positions * kHeadDim * es;
  const Span kspan = {k_blk, kv_bytes}, vspan = {vt_blk, kv_bytes};
  const Span bspan = {bias_blk, (size_t)kHeads * prob->I * nkeys * sizeof(float)};
  const Span wspan = {ws, l.total}, sspan = {state, sb};
  const Span ospan = {out, out ? (size_t)prob->rows * prob->I * kCz * es : 0};
  // state, workspace and out are written: none may overlap anything else
  const Span ins[] = {kspan, vspan, bspan};
  for (const Span& x : ins)
    if (overlap(x, wspan) || overlap(x, sspan) || overlap(x, ospan)) return TA_ERR_ALIAS;
  if ((rc = check_out_alias(prob, w, sspan, {nullptr, 0}, wspan, ospan))) return rc;
  if (out != nullptr && (rc = check_out_alias(prob, w, ospan, {nullptr, 0}, wspan, sspan))) return rc;
  (void)hipGetLastError();
  char* base = (char*)ws;
  float* shift = (float*)((char*)state + shift_off);
  if ((rc = enqueue(triattn::launch_pack_bias(bias_blk, base + l.bias, prob->I, nkeys, l.positions, kv_positions,
                                              shift, prob->dtype, (hipStream_t)stream))))
    return rc;
  triattn::AttendArgs a = attend_args(prob, variant, w, nullptr, out, ws, l);
  a.k = k_blk;
  a.vt = vt_blk;
  a.kv_P = kv_positions;
  a.bias_kt = kv_positions / kKeyTile;
  a.bias_shift = shift;
  a.kt0 = 0;
  a.nbt = (nkeys + kKeyTile - 1) / kKeyTile;
  a.redo = nullptr;  // the shifted form only: it reads k / v^T at kv_positions
  a.state_o = state;
  a.state_ml = (float*)((char*)state + ob);
  a.state_in = first ? 0 : 1;
  a.state_out = out == nullptr ? 1 : 0;
  return enqueue(triattn::launch_attend(a, prob->dtype, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int triangle_attn_attend_kv_block(const ta_problem* prob, int variant, const ta_weights* w, const void* k_blk,
                                  const void* vt_blk, int32_t kv_positions, const float* bias_blk, int32_t nkeys,
                                  int32_t first, void* state, void* ws, size_t ws_bytes, void* stream) {
  return kv_block(prob, variant, w, k_blk, vt_blk, kv_positions, bias_blk, nkeys, first, state, nullptr, ws,
                  ws_bytes, stream);
}

int triangle_attn_attend_kv_block_final(const ta_problem* prob, int variant, const ta_weights* w,
                                        const void* k_blk, const void* vt_blk, int32_t kv_positions,
                                        const float* bias_blk, int32_t nkeys, int32_t first, void* state,
                                        void* out, void* ws, size_t ws_bytes, void* stream) {
  if (out == nullptr) return TA_ERR_NULL_PTR;
  return kv_block(prob, variant, w, k_blk, vt_blk, kv_positions, bias_blk, nkeys, first, state, out, ws,
                  ws_bytes, stream);
}

int triangle_attn_attend_finalize(const ta_problem* prob, int variant, const ta_weights* w, const void* state,
                                  void* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_problem(prob, variant);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if (state == nullptr || out == nullptr || ws == nullptr) return TA_ERR_NULL_PTR;
  if (!aligned16(state) || !aligned16(out) || !aligned16(ws)) return TA_ERR_MISALIGNED;
  ta_ws_layout l;
  layout_of(prob, variant, &l);
  if (ws_bytes < l.total) return TA_ERR_WORKSPACE_TOO_SMALL;
  size_t ob, sb;
  state_sizes(l, prob->dtype, &ob, &sb);
  const size_t tok_bytes = (size_t)prob->rows * prob->I * kCz * esize(prob->dtype);
  if ((rc = check_out_alias(prob, w, {out, tok_bytes}, {nullptr, 0}, {ws, l.total}, {state, sb}))) return rc;
  (void)hipGetLastError();
  triattn::AttendArgs a = attend_args(prob, variant, w, nullptr, out, ws, l);
  a.nbt = 0;  // no keys: gate and output projection of the carried state
  a.state_o = const_cast<void*>(state);
  a.state_ml = (float*)((const char*)state + ob);
  a.state_in = 1;
  a.state_out = 0;
  return enqueue(triattn::launch_attend(a, prob->dtype, (hipStream_t)stream));
}

}  // extern "C"
