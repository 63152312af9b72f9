// Quantisation of Q, K and V to OCP E4M3 for the quantised sparse branch (SLA2 page,
// section 2.C: the sparse branch runs on low-precision operands and the forward uses the
// quantised attention).
//
// Per (batch*head, 64-token block): e = the smallest integer with 448 * 2^e >= absmax of
// the block (valid tokens, all channels; 0 for an all-zero block), x8 = E4M3(x * 2^-e).
// The scaling by 2^-e is exact, so each value is rounded exactly once (hardware
// round-to-nearest-even; |x * 2^-e| <= 448 so nothing saturates). The power-of-two scale is
// an E8M0 block scale that the scaled MFMA applies in hardware.
//
// Layouts written:
//   row-major  [BH][nb*64][D] bf16 (Q8, K8): the E4M3 values stored as bf16, which holds
//              every E4M3 value exactly; rows beyond n are zero. Q K^T is formed on the
//              bf16 MFMA because the fp8 MFMA of gfx950 keeps only about 12-13 significant
//              bits when it accumulates products of very different magnitude, which the
//              softmax then amplifies for large logits;
//   V8 tiles   [BH][nb][D][64] bytes: per key block, channel-major, the 64 keys in the order
//              the P8 operand of the P.V product uses (see sparse.hip): byte 32*hh + slot of
//              channel c holds key 32*(slot/16) + 8*((slot%16)/4) + 4*hh + slot%4.
//   exponents  [BH][nb] int32.
#include "common.h"
#include "kernels.h"

namespace sla {

template <int D, bool VTILE>
__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* __restrict__ x,
                                                    uint8_t* __restrict__ x8,
                                                    int32_t* __restrict__ ex, int n, int nb) {
  constexpr int CH = D / 8;               // 8-element chunks per row
  constexpr int CPT = 64 * CH / 256;      // chunks per thread
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[VTILE ? D * 64 : 16];
  const int j = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int row0 = j * kBlock;
  const uint16_t* xb = x + (size_t)bh * n * D;
  float v[CPT][8];
  float amax = 0.f;
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int id = t + 256 * u, r = id / CH, c = id % CH;
    u32x4 w = {0, 0, 0, 0};
    if (row0 + r < n) w = *reinterpret_cast<const u32x4*>(xb + (size_t)(row0 + r) * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[u][2 * e] = bf16_lo(w[e]);
      v[u][2 * e + 1] = bf16_hi(w[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[u][e]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = e8m0_exponent(amax);
  if (t == 0) ex[(size_t)bh * nb + j] = e;
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int id = t + 256 * u, r = id / CH, c = id % CH;
    uint32_t w0, w1;
    e4m3x8(v[u], e, w0, w1);
    if constexpr (!VTILE) {
      *reinterpret_cast<u32x4*>(x8 + (((size_t)bh * nb * kBlock + row0 + r) * D + c * 8) * 2) =
          e4m3x8_as_bf16(w0, w1);
    } else {
      const int pos = v8_slot_pos(r);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        tile[(c * 8 + b) * 64 + pos] = (uint8_t)(w0 >> (8 * b));
        tile[(c * 8 + 4 + b) * 64 + pos] = (uint8_t)(w1 >> (8 * b));
      }
    }
  }
  if constexpr (VTILE) {
    __syncthreads();
    uint8_t* dst = x8 + ((size_t)bh * nb + j) * D * 64;
    for (int id = t; id < D * 64 / 16; id += 256)
      *reinterpret_cast<u32x4*>(dst + id * 16) = *reinterpret_cast<const u32x4*>(&tile[id * 16]);
  }
}

template <int D>
static hipError_t launch_quant_T(const Plan& s, const void* q, const void* k, const void* v,
                                 char* ws, hipStream_t st) {
  hipLaunchKernelGGL((quant_kernel<D, false>), dim3(s.nbq, s.BH), dim3(256), 0, st,
                     (const uint16_t*)q, reinterpret_cast<uint8_t*>(ws + s.q8),
                     reinterpret_cast<int32_t*>(ws + s.sq8), s.nq, s.nbq);
  if (k == nullptr) return hipGetLastError();   // K and V quantised by the key/value pass
  hipLaunchKernelGGL((quant_kernel<D, false>), dim3(s.nbk, s.BH), dim3(256), 0, st,
                     (const uint16_t*)k, reinterpret_cast<uint8_t*>(ws + s.k8),
                     reinterpret_cast<int32_t*>(ws + s.sk8), s.nkv, s.nbk);
  hipLaunchKernelGGL((quant_kernel<D, true>), dim3(s.nbk, s.BH), dim3(256), 0, st,
                     (const uint16_t*)v, reinterpret_cast<uint8_t*>(ws + s.v8),
                     reinterpret_cast<int32_t*>(ws + s.sv8), s.nkv, s.nbk);
  return hipGetLastError();
}

hipError_t launch_quant(const Plan& s, const void* q, const void* k, const void* v, char* ws,
                        hipStream_t st) {
  if (s.D == 128) return launch_quant_T<128>(s, q, k, v, ws, st);
  return launch_quant_T<64>(s, q, k, v, ws, st);
}

}  // namespace sla
