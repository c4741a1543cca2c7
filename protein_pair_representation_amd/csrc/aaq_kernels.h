// Internal interface between the C ABI layer and the AAQ codec kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aaq {

// Record geometry of the three groups (LightNobel article, section 2.2.3).
// group 0 = A (INT8 + outliers), 1 = B (INT4 + outliers), 2 = C (INT4).
int record_bytes(int group);

// Encode n tokens of 128 channels (x: bf16 when dtype == 1, fp32 when 2) into
// n records of record_bytes(group) bytes.  Arguments are validated by the caller.
hipError_t launch_encode(const void* x, int dtype, int64_t n, int group, void* rec, hipStream_t stream);

// Decode n records into n tokens of 128 channels (y: bf16 when dtype == 1, fp32 when 2).
hipError_t launch_decode(const void* rec, int group, int64_t n, void* y, int dtype, hipStream_t stream);

}  // namespace aaq
