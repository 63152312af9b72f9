// Diagnostic entry point (include/sla.h, sla_diag_fp8_mfma): one 32 x 32 x 64 product of
// E4M3 operands on the scaled fp8 matrix instruction that the quantised forward uses for P.V,
// and the same product on the bf16 instruction (every E4M3 value and every product of two is
// exact in bf16 / fp32), so that a test can measure how the fp8 instruction accumulates.
#include "common.h"

namespace sla {
namespace {

// a: 32 x 64 codes (row i, column k), b: 64 x 32 codes (row k, column j), row-major.
// Outputs c_fp8, c_bf16: 32 x 32 fp32, row-major.
__global__ __launch_bounds__(64) void fp8_mfma_probe_kernel(const uint8_t* __restrict__ a,
                                                            const uint8_t* __restrict__ b,
                                                            float* __restrict__ c_fp8,
                                                            float* __restrict__ c_bf16) {
  const int lane = threadIdx.x, h = lane >> 5, l32 = lane & 31;
  // fp8 operands: lane (row or column l32) holds the 32 reduction indices 32 h .. 32 h + 31
  i32x8 af, bf;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t wa = 0, wb = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kk = 32 * h + 4 * w + e;
      wa |= (uint32_t)a[l32 * 64 + kk] << (8 * e);
      wb |= (uint32_t)b[kk * 32 + l32] << (8 * e);
    }
    af[w] = (int)wa;
    bf[w] = (int)wb;
  }
  f32x16 c8 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, f32x16{}, 0, 0, 0, 127, 0,
                                                              127);
  // bf16 operands: four 16-deep steps, lane holds the 8 indices 16 s + 8 h .. + 7
  f32x16 c16 = f32x16{};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 ab, bb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k0 = 16 * s + 8 * h + 2 * e;
      ab[e] = e4m3_to_bf16(a[l32 * 64 + k0]) | (e4m3_to_bf16(a[l32 * 64 + k0 + 1]) << 16);
      bb[e] = e4m3_to_bf16(b[k0 * 32 + l32]) | (e4m3_to_bf16(b[(k0 + 1) * 32 + l32]) << 16);
    }
    c16 = mfma_bf16(ab, bb, c16);
  }
  // C[i][j]: lane j + 32 ((i / 4) % 2), element (i % 4) + 4 (i / 8)
#pragma unroll
  for (int el = 0; el < 16; ++el) {
    const int i = (el & 3) + 4 * h + 8 * (el >> 2);
    c_fp8[i * 32 + l32] = c8[el];
    c_bf16[i * 32 + l32] = c16[el];
  }
}

}  // namespace
}  // namespace sla

extern "C" sla_status sla_diag_fp8_mfma(const uint8_t* a, const uint8_t* b, float* c_fp8,
                                        float* c_bf16, hipStream_t stream) {
  if (!a || !b || !c_fp8 || !c_bf16) return SLA_ERR_NULL;
  hipLaunchKernelGGL(sla::fp8_mfma_probe_kernel, dim3(1), dim3(64), 0, stream, a, b, c_fp8,
                     c_bf16);
  return hipGetLastError() == hipSuccess ? SLA_OK : SLA_ERR_HIP;
}
