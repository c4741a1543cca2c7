// aaq_abi.cpp -- the C ABI of the AAQ codec (declared in include/aaq.h).
//
// Host-side only: validates every argument, then enqueues one kernel on the
// caller's stream.  Nothing here allocates, frees or synchronises, and no HIP
// call is made before validation has passed.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/aaq.h"
#include "aaq_kernels.h"

namespace {

constexpr int64_t kMaxTokens = (int64_t)1 << 40;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Common checks; on success *rb is the record size and *tb the token size in bytes.
int check(const void* tokens, int dtype, int64_t n, int group, const void* records, int* rb, size_t* tb) {
  const int r = aaq::record_bytes(group);
  if (r < 0) return TA_ERR_BAD_GROUP;
  if (dtype != TA_BF16 && dtype != TA_F32) return TA_ERR_BAD_DTYPE;
  if (n < 0 || n > kMaxTokens) return TA_ERR_BAD_SHAPE;
  *rb = r;
  *tb = (size_t)AAQ_CHANNELS * (dtype == TA_BF16 ? 2 : 4);
  if (n == 0) return TA_OK;
  if (tokens == nullptr || records == nullptr) return TA_ERR_NULL_PTR;
  if (!aligned16(tokens) || !aligned16(records)) return TA_ERR_MISALIGNED;
  if (overlap(tokens, (size_t)n * *tb, records, (size_t)n * (size_t)r)) return TA_ERR_ALIAS;
  return TA_OK;
}

}  // namespace

extern "C" {

int aaq_record_bytes(int group) {
  const int r = aaq::record_bytes(group);
  return r < 0 ? TA_ERR_BAD_GROUP : r;
}

int aaq_encode(const void* x, int dtype, int64_t n, int group, void* records, void* stream) {
  int rb = 0;
  size_t tb = 0;
  const int rc = check(x, dtype, n, group, records, &rb, &tb);
  if (rc != TA_OK || n == 0) return rc;
  return aaq::launch_encode(x, dtype, n, group, records, (hipStream_t)stream) == hipSuccess ? TA_OK : TA_ERR_HIP;
}

int aaq_decode(const void* records, int group, int64_t n, void* y, int dtype, void* stream) {
  int rb = 0;
  size_t tb = 0;
  const int rc = check(y, dtype, n, group, records, &rb, &tb);
  if (rc != TA_OK || n == 0) return rc;
  return aaq::launch_decode(records, group, n, y, dtype, (hipStream_t)stream) == hipSuccess ? TA_OK : TA_ERR_HIP;
}

}  // extern "C"
