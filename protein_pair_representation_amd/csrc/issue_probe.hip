// issue_probe.hip -- issue costs of the attention loop's instruction mix on gfx950.
//
// Measurement only (not part of the attention path): each kernel repeats one
// group of instructions with no memory traffic in the loop, as independent
// chains, so the time it takes is set by how fast the SIMD issues that group.
// The attention loop's phase is one 32-key chunk: 4 v_mfma_f32_32x32x16_bf16 and
// 2 v_mfma_f32_16x16x32_bf16 (in dependent pairs, like the score and P.V chains)
// beside 16 v_exp_f32, 8 v_cvt_pk_bf16_f32 and 9 v_cvt_f32_f16 (the exponentials,
// the P conversions and the bias widenings).  Cycles come from s_memtime (the
// core clock) per wave and from the kernel time; SIMD-cycles per iteration =
// kernel time x clock / (waves per SIMD x iterations).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int ITER = 1024;

enum Mode {
  EXP_F32 = 0,      // 8 x v_exp_f32 per iteration
  EXP_F16 = 1,      // 8 x v_exp_f16
  CVT_PK_BF16 = 2,  // 8 x v_cvt_pk_bf16_f32
  MFMA_32 = 3,      // 4 x v_mfma_f32_32x32x16_bf16, independent
  MFMA_16 = 4,      // 4 x v_mfma_f32_16x16x32_bf16, independent
  PHASE_MFMA = 5,   // a phase's products alone
  PHASE_VALU = 6,   // a phase's VALU work alone
  PHASE_BOTH = 7,   // both, one product between every five or six VALU instructions
  NMODES = 8
};

#define P_EXP(r) "v_exp_f32_e64 " r ", -|" r "|\n"
#define P_CVT(d, a, b) "v_cvt_pk_bf16_f32 " d ", " a ", " b "\n"
#define P_WID(d, s) "v_cvt_f32_f16_e32 " d ", " s "\n"
// the products take their accumulators in AGPRs: the loop then holds no moves
// the compiler would otherwise add around VGPR-form inline products
#define P_M32(c, x, y) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));
#define P_M16(c, x, y) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));

template <int MODE>
__global__ __launch_bounds__(256) void issue_kernel(float* out, long long* cyc) {
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  f32x4 d0 = {}, d1 = {};
  bf16x8 a, b;
  for (int t = 0; t < 8; ++t) {
    a[t] = (__bf16)(threadIdx.x * 1e-3f + t);
    b[t] = (__bf16)(0.5f - t * 1e-2f);
  }
  float e[16];
  for (int i = 0; i < 16; ++i) e[i] = threadIdx.x * 1e-4f + i * 0.01f;
  uint32_t pk[8], hw[9];
  float wf[9];
  for (int i = 0; i < 8; ++i) pk[i] = threadIdx.x + i;
  for (int i = 0; i < 9; ++i) {
    hw[i] = 0x3c003c00u + i;
    wf[i] = 0.f;
  }
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < ITER; ++it) {
    if (MODE == EXP_F32) {
      asm volatile(P_EXP("%0") P_EXP("%1") P_EXP("%2") P_EXP("%3") P_EXP("%4") P_EXP("%5") P_EXP("%6") P_EXP("%7")
                   : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]), "+v"(e[6]), "+v"(e[7]));
    } else if (MODE == EXP_F16) {
      asm volatile(
          "v_exp_f16_e64 %0, -|%0|\n v_exp_f16_e64 %1, -|%1|\n v_exp_f16_e64 %2, -|%2|\n v_exp_f16_e64 %3, -|%3|\n"
          "v_exp_f16_e64 %4, -|%4|\n v_exp_f16_e64 %5, -|%5|\n v_exp_f16_e64 %6, -|%6|\n v_exp_f16_e64 %7, -|%7|\n"
          : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]), "+v"(e[6]), "+v"(e[7]));
    } else if (MODE == CVT_PK_BF16) {
      asm volatile(P_CVT("%0", "%0", "%1") P_CVT("%1", "%1", "%2") P_CVT("%2", "%2", "%3") P_CVT("%3", "%3", "%4")
                   P_CVT("%4", "%4", "%5") P_CVT("%5", "%5", "%6") P_CVT("%6", "%6", "%7") P_CVT("%7", "%7", "%0")
                   : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]), "+v"(e[6]), "+v"(e[7]));
    } else if (MODE == MFMA_32) {
      P_M32(c0, a, b) P_M32(c1, a, b) P_M32(c2, a, b) P_M32(c3, a, b)
    } else if (MODE == MFMA_16) {
      P_M16(d0, a, b) P_M16(d1, a, b) P_M16(c2.lo.lo, a, b) P_M16(c3.lo.lo, a, b)
    } else if (MODE == PHASE_MFMA) {
      P_M32(c0, a, b) P_M32(c1, a, b) P_M16(d0, a, b) P_M32(c0, b, a) P_M32(c1, b, a) P_M16(d0, b, a)
    } else if (MODE == PHASE_VALU) {
      asm volatile(P_EXP("%0") P_EXP("%1") P_EXP("%2") P_EXP("%3") P_EXP("%4") P_EXP("%5") P_EXP("%6") P_EXP("%7")
                   : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]), "+v"(e[6]), "+v"(e[7]));
      asm volatile(P_CVT("%0", "%8", "%9") P_CVT("%1", "%10", "%11") P_CVT("%2", "%12", "%13") P_CVT("%3", "%14", "%15")
                   P_WID("%4", "%16") P_WID("%5", "%17") P_WID("%6", "%18") P_WID("%7", "%19")
                   : "=&v"(pk[0]), "=&v"(pk[1]), "=&v"(pk[2]), "=&v"(pk[3]), "=&v"(wf[0]), "=&v"(wf[1]), "=&v"(wf[2]),
                     "=&v"(wf[3])
                   : "v"(e[0]), "v"(e[1]), "v"(e[2]), "v"(e[3]), "v"(e[4]), "v"(e[5]), "v"(e[6]), "v"(e[7]),
                     "v"(hw[0]), "v"(hw[1]), "v"(hw[2]), "v"(hw[3]));
      asm volatile(P_EXP("%0") P_EXP("%1") P_EXP("%2") P_EXP("%3") P_EXP("%4") P_EXP("%5") P_EXP("%6") P_EXP("%7")
                   : "+v"(e[8]), "+v"(e[9]), "+v"(e[10]), "+v"(e[11]), "+v"(e[12]), "+v"(e[13]), "+v"(e[14]),
                     "+v"(e[15]));
      asm volatile(P_CVT("%0", "%9", "%10") P_CVT("%1", "%11", "%12") P_CVT("%2", "%13", "%14")
                   P_CVT("%3", "%15", "%16") P_WID("%4", "%17") P_WID("%5", "%18") P_WID("%6", "%19")
                   P_WID("%7", "%20") P_WID("%8", "%21")
                   : "=&v"(pk[4]), "=&v"(pk[5]), "=&v"(pk[6]), "=&v"(pk[7]), "=&v"(wf[4]), "=&v"(wf[5]), "=&v"(wf[6]),
                     "=&v"(wf[7]), "=&v"(wf[8])
                   : "v"(e[8]), "v"(e[9]), "v"(e[10]), "v"(e[11]), "v"(e[12]), "v"(e[13]), "v"(e[14]), "v"(e[15]),
                     "v"(hw[4]), "v"(hw[5]), "v"(hw[6]), "v"(hw[7]), "v"(hw[8]));
    } else if (MODE == PHASE_BOTH) {
      P_M32(c0, a, b)
      asm volatile(P_EXP("%0") P_EXP("%1") P_EXP("%2") P_EXP("%3") : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]));
      asm volatile(P_CVT("%0", "%2", "%3") P_WID("%1", "%4") : "=&v"(pk[0]), "=&v"(wf[0]) : "v"(e[0]), "v"(e[1]), "v"(hw[0]));
      P_M32(c1, a, b)
      asm volatile(P_EXP("%0") P_EXP("%1") P_EXP("%2") P_EXP("%3") : "+v"(e[4]), "+v"(e[5]), "+v"(e[6]), "+v"(e[7]));
      asm volatile(P_CVT("%0", "%2", "%3") P_WID("%1", "%4") : "=&v"(pk[1]), "=&v"(wf[1]) : "v"(e[2]), "v"(e[3]), "v"(hw[1]));
      P_M16(d0, a, b)
      asm volatile(P_CVT("%0", "%3", "%4") P_WID("%1", "%5") P_WID("%2", "%6")
                   : "=&v"(pk[2]), "=&v"(wf[2]), "=&v"(wf[3]) : "v"(e[4]), "v"(e[5]), "v"(hw[2]), "v"(hw[3]));
      P_M32(c0, b, a)
      asm volatile(P_EXP("%0") P_EXP("%1") P_EXP("%2") P_EXP("%3") : "+v"(e[8]), "+v"(e[9]), "+v"(e[10]), "+v"(e[11]));
      asm volatile(P_CVT("%0", "%2", "%3") P_WID("%1", "%4") : "=&v"(pk[3]), "=&v"(wf[4]) : "v"(e[6]), "v"(e[7]), "v"(hw[4]));
      P_M32(c1, b, a)
      asm volatile(P_EXP("%0") P_EXP("%1") P_EXP("%2") P_EXP("%3") : "+v"(e[12]), "+v"(e[13]), "+v"(e[14]), "+v"(e[15]));
      asm volatile(P_CVT("%0", "%2", "%3") P_WID("%1", "%4") : "=&v"(pk[4]), "=&v"(wf[5]) : "v"(e[8]), "v"(e[9]), "v"(hw[5]));
      P_M16(d0, b, a)
      asm volatile(P_CVT("%0", "%4", "%5") P_CVT("%1", "%6", "%7") P_CVT("%2", "%8", "%9") P_WID("%3", "%10")
                   : "=&v"(pk[5]), "=&v"(pk[6]), "=&v"(pk[7]), "=&v"(wf[6])
                   : "v"(e[10]), "v"(e[11]), "v"(e[12]), "v"(e[13]), "v"(e[14]), "v"(e[15]), "v"(hw[6]));
      asm volatile(P_WID("%0", "%2") P_WID("%1", "%3") : "=&v"(wf[7]), "=&v"(wf[8]) : "v"(hw[7]), "v"(hw[8]));
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i] + e[i];
  for (int i = 0; i < 4; ++i) s += d0[i] + d1[i];
  for (int i = 0; i < 8; ++i) s += (float)pk[i] + wf[i];
  out[gid] = s + wf[8];
  if ((threadIdx.x & 63) == 0) cyc[gid >> 6] = t1 - t0;
}

typedef void (*kernel_t)(float*, long long*);
const kernel_t KERNELS[NMODES] = {issue_kernel<0>, issue_kernel<1>, issue_kernel<2>, issue_kernel<3>,
                                  issue_kernel<4>, issue_kernel<5>, issue_kernel<6>, issue_kernel<7>};

}  // namespace

extern "C" {

// Number of probe kernels (the modes above).
int issue_probe_modes(void) { return NMODES; }

// Run probe `mode` with `waves_per_simd` (1..4) waves on every SIMD (256 threads
// per workgroup, 256 * waves_per_simd workgroups), once to warm up and once
// timed.  Writes SIMD-cycles per loop iteration and the core clock (GHz, from
// s_memtime over the kernel time).  Allocates its own device buffers and
// synchronises the device.  Returns 0, or a negative value on a bad argument or
// a HIP error.
int issue_probe_run(int mode, int waves_per_simd, double* simd_cycles_per_iter, double* clock_ghz) {
  if (mode < 0 || mode >= NMODES || waves_per_simd < 1 || waves_per_simd > 4 || !simd_cycles_per_iter || !clock_ghz)
    return -1;
  const int blocks = 256 * waves_per_simd, nw = blocks * 4;
  float* out = nullptr;
  long long* cyc = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = -2;
  std::vector<long long> h(nw);
  float ms = 0.f;
  if (hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)) != hipSuccess) goto done;
  if (hipMalloc(&cyc, (size_t)nw * sizeof(long long)) != hipSuccess) goto done;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) goto done;
  hipLaunchKernelGGL(KERNELS[mode], dim3(blocks), dim3(256), 0, 0, out, cyc);
  if (hipEventRecord(e0, 0) != hipSuccess) goto done;
  hipLaunchKernelGGL(KERNELS[mode], dim3(blocks), dim3(256), 0, 0, out, cyc);
  if (hipEventRecord(e1, 0) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) goto done;
  if (hipGetLastError() != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) goto done;
  if (hipMemcpy(h.data(), cyc, (size_t)nw * sizeof(long long), hipMemcpyDeviceToHost) != hipSuccess) goto done;
  {
    const double longest = (double)*std::max_element(h.begin(), h.end());
    const double ghz = longest / (ms * 1e6);
    *clock_ghz = ghz;
    *simd_cycles_per_iter = ms * 1e6 * ghz / ((double)waves_per_simd * ITER);
    rc = 0;
  }
done:
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (out) (void)hipFree(out);
  if (cyc) (void)hipFree(cyc);
  return rc;
}

}  // extern "C"
