// Diagnostic entry points (include/sla.h):
// * sla_diag_fp8_mfma: one 32 x 32 x 64 product of E4M3 operands on the scaled fp8 matrix
//   instruction that the quantised forward uses for P.V, and the same product on the bf16
//   instruction (every E4M3 value and every product of two is exact in bf16 / fp32), so that
//   a test can measure how the fp8 instruction accumulates.
// * sla_diag_mfma_rate: a matrix-instruction throughput loop (the 32x32x16 bf16 product of the
//   exact branch's Q K^T), timed by the caller, which gives the rate the matrix cores reach on
//   this GPU at the clock they run under that load.
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

// Every wave runs four independent accumulator chains of 32x32x16 bf16 products, `iters`
// rounds (4 iters products per wave); each thread writes one sum to `sink` so that nothing is
// optimised away.
__global__ __launch_bounds__(256) void mfma_rate_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  u32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = pack_bf16(1e-3f * (float)(lane + e), 1e-3f * (float)(lane - e));
    b[e] = pack_bf16(2e-3f * (float)(e + 1), -1e-3f * (float)lane);
  }
  // distinct starting values keep the four chains distinct computations
  f32x16 c0, c1, c2, c3;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    c0[e] = (float)e;
    c1[e] = (float)(e + lane);
    c2[e] = (float)(2 * e - lane);
    c3[e] = (float)(3 * e + 1);
  }
  for (int it = 0; it < iters; ++it) {
    c0 = mfma_bf16(a, b, c0);
    c1 = mfma_bf16(a, b, c1);
    c2 = mfma_bf16(a, b, c2);
    c3 = mfma_bf16(a, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace
}  // namespace sla

extern "C" sla_status sla_diag_mfma_rate(float* sink, int blocks, int iters, hipStream_t stream) {
  if (!sink) return SLA_ERR_NULL;
  if (blocks <= 0 || iters <= 0) return SLA_ERR_SHAPE;
  hipLaunchKernelGGL(sla::mfma_rate_kernel, dim3(blocks), dim3(256), 0, stream, sink, iters);
  return hipGetLastError() == hipSuccess ? SLA_OK : SLA_ERR_HIP;
}

extern "C" sla_status sla_diag_fp8_mfma(const uint8_t* a, const uint8_t* b, float* c_fp8,
                                        float* c_bf16, hipStream_t stream) {
  if (!a || !b || !c_fp8 || !c_bf16) return SLA_ERR_NULL;
  hipLaunchKernelGGL(sla::fp8_mfma_probe_kernel, dim3(1), dim3(64), 0, stream, a, b, c_fp8,
                     c_bf16);
  return hipGetLastError() == hipSuccess ? SLA_OK : SLA_ERR_HIP;
}
