// Linear branch (SALAD page, section 2: ReLU kernel feature map with linear cost; SPLA
// page, section 2.2: the linear term over the unselected blocks equals the global linear
// term minus the selected blocks' term).
//
// kv_summary:  one pass over K and V. For every key block j: S_j = phi(K_j)^T V_j (d x d,
//              bf16 MFMA, fp32 accumulate, stored bf16 as S_j^T[c][r]), z_j = sum phi(K_j)
//              (fp32), the block mean of K (float64, for the router) and an f16 copy of V
//              for the sparse branch's P.V. Per-chunk fp32 partial totals are written for
//              a fixed-order reduction (no atomics).
// reduce:      S_tot = sum of the partials, z_tot likewise.
// complement:  per query block i, S_c(i) = S_tot - sum_{j in sel(i)} S_j and
//              z_c(i) = z_tot - sum_{j in sel(i)} z_j; all-blocks selections give exactly 0.
#include "common.h"
#include "kernels.h"

namespace sla {

// Fragment of an MFMA operand whose lane owns index x0 + lane%32 and the 8 consecutive
// reduction indices k0 + 8*(lane/32) .. +7, read with two transposing LDS reads from a
// row-major LDS matrix M[k][x] of 16-bit elements with a row stride of `stride` elements.
__device__ __forceinline__ u32x4 frag_tr(const uint16_t* M, int stride, int x0, int k0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, L = lane & 15;
  const int row = k0 + 8 * (g >> 1) + (L >> 2);
  const int col = x0 + 16 * (g & 1) + 4 * (L & 3);
  const u32x2 lo = lds_read_tr16(M + row * stride + col);
  const u32x2 hi = lds_read_tr16(M + (row + 4) * stride + col);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

__device__ __forceinline__ uint32_t f16_sat_pack(float a, float b) {
  const float m = 65504.0f;
  return pack_f16(fminf(fmaxf(a, -m), m), fminf(fmaxf(b, -m), m));
}

template <typename T, int D>
__global__ __launch_bounds__(256) void kv_summary_kernel(
    const T* __restrict__ k, const T* __restrict__ v, double* __restrict__ kbar,
    uint16_t* __restrict__ v16, uint16_t* __restrict__ sblk, float* __restrict__ zblk,
    float* __restrict__ spart, float* __restrict__ zpart, int nkv, int nbk) {
  constexpr int LS = D + 8;                  // padded LDS row (elements)
  constexpr int TPR = D / 8, RPP = 256 / TPR;
  constexpr int CPT = 64 * TPR / 256;        // 16-byte chunks per thread per tensor
  constexpr int NT = D / 32;                 // 32-wide tiles per dimension
  constexpr int TILES_PER_WAVE = NT * NT / 4;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * LS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[64 * LS];
  __shared__ double pool_lds[RPP * D];

  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int j0 = chunk * kSummaryChunk, j1 = min(j0 + kSummaryChunk, nbk);
  const T* kb = k + (size_t)bh * nkv * D;
  const T* vb = v + (size_t)bh * nkv * D;

  f32x16 part[TILES_PER_WAVE];
#pragma unroll
  for (int u = 0; u < TILES_PER_WAVE; ++u) part[u] = f32x16{};
  float zp = 0.f;

  for (int j = j0; j < j1; ++j) {
    const int row0 = j * kBlock;
    const int nrows = min(kBlock, nkv - row0);
    double pacc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pacc[e] = 0.0;
    __syncthreads();   // previous block's LDS readers are done
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int cidx = t + 256 * u;
      const int r = cidx / TPR, c8 = cidx % TPR;
      u32x4 kw = {0, 0, 0, 0}, vw = {0, 0, 0, 0}, v16w = {0, 0, 0, 0};
      if (r < nrows) {
        const size_t off = (size_t)(row0 + r) * D + c8 * 8;
        if constexpr (sizeof(T) == 2) {
          kw = *reinterpret_cast<const u32x4*>(kb + off);
          vw = *reinterpret_cast<const u32x4*>(vb + off);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pacc[2 * e] += (double)bf16_lo(kw[e]);
            pacc[2 * e + 1] += (double)bf16_hi(kw[e]);
            v16w[e] = f16_sat_pack(bf16_lo(vw[e]), bf16_hi(vw[e]));
          }
        } else {
          const f32x4 k0 = *reinterpret_cast<const f32x4*>(kb + off);
          const f32x4 k1 = *reinterpret_cast<const f32x4*>(kb + off + 4);
          const f32x4 v0 = *reinterpret_cast<const f32x4*>(vb + off);
          const f32x4 v1 = *reinterpret_cast<const f32x4*>(vb + off + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pacc[e] += (double)k0[e];
            pacc[4 + e] += (double)k1[e];
          }
          kw = u32x4{pack_bf16(k0[0], k0[1]), pack_bf16(k0[2], k0[3]),
                     pack_bf16(k1[0], k1[1]), pack_bf16(k1[2], k1[3])};
          vw = u32x4{pack_bf16(v0[0], v0[1]), pack_bf16(v0[2], v0[3]),
                     pack_bf16(v1[0], v1[1]), pack_bf16(v1[2], v1[3])};
          v16w = u32x4{f16_sat_pack(v0[0], v0[1]), f16_sat_pack(v0[2], v0[3]),
                       f16_sat_pack(v1[0], v1[1]), f16_sat_pack(v1[2], v1[3])};
        }
      }
      *reinterpret_cast<u32x4*>(&Ks[r * LS + c8 * 8]) = kw;
      *reinterpret_cast<u32x4*>(&Vs[r * LS + c8 * 8]) = vw;
      *reinterpret_cast<u32x4*>(&v16[((size_t)bh * nbk * kBlock + row0 + r) * D + c8 * 8]) = v16w;
    }
    // pooled K mean (float64, valid rows only)
    {
      const int cg = t % TPR, r = t / TPR;
#pragma unroll
      for (int e = 0; e < 8; ++e) pool_lds[r * D + cg * 8 + e] = pacc[e];
    }
    __syncthreads();
    if (t < D) {
      double s = 0.0;
      for (int rr = 0; rr < RPP; ++rr) s += pool_lds[rr * D + t];
      kbar[((size_t)bh * nbk + j) * D + t] = s / (double)nrows;
      float z = 0.f;
      for (int m = 0; m < 64; ++m) z += fmaxf(bf16_bits_to_f32(Ks[m * LS + t]), 0.f);
      zblk[((size_t)bh * nbk + j) * D + t] = z;
      zp += z;
    }
    // S_j[r][c] = sum_m relu(K[m][r]) V[m][c]: M = r, N = c, reduction over the 64 keys.
#pragma unroll
    for (int u = 0; u < TILES_PER_WAVE; ++u) {
      const int mt = (NT == 4) ? w : (w >> 1);
      const int nt = (NT == 4) ? u : (w & 1);
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 a = relu_bf16x8(frag_tr(Ks, LS, 32 * mt, 16 * s));
        const u32x4 b = frag_tr(Vs, LS, 32 * nt, 16 * s);
        acc = mfma_bf16(a, b, acc);
      }
      part[u] += acc;
      // store S_j^T[c][r] (bf16): lane column c = 32 nt + l32, rows r in runs of 4
      const int c = 32 * nt + l32;
      uint16_t* dst = sblk + (((size_t)bh * nbk + j) * D + c) * D;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 32 * mt + 8 * q + 4 * h;
        const u32x2 pk = {pack_bf16(acc[4 * q], acc[4 * q + 1]),
                          pack_bf16(acc[4 * q + 2], acc[4 * q + 3])};
        *reinterpret_cast<u32x2*>(dst + r) = pk;
      }
    }
  }
  // chunk partial totals (fp32, layout [c][r])
#pragma unroll
  for (int u = 0; u < TILES_PER_WAVE; ++u) {
    const int mt = (NT == 4) ? w : (w >> 1);
    const int nt = (NT == 4) ? u : (w & 1);
    const int c = 32 * nt + l32;
    float* dst = spart + (((size_t)bh * gridDim.x + chunk) * D + c) * D;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 32 * mt + 8 * q + 4 * h;
      *reinterpret_cast<f32x4*>(dst + r) =
          f32x4{part[u][4 * q], part[u][4 * q + 1], part[u][4 * q + 2], part[u][4 * q + 3]};
    }
  }
  if (t < D) zpart[((size_t)bh * gridDim.x + chunk) * D + t] = zp;
}

template <int D>
__global__ __launch_bounds__(256) void reduce_totals_kernel(const float* __restrict__ spart,
                                                            const float* __restrict__ zpart,
                                                            float* __restrict__ stot,
                                                            float* __restrict__ ztot, int nchunk) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  float s = 0.f;
  for (int c = 0; c < nchunk; ++c) s += spart[((size_t)bh * nchunk + c) * D * D + e];
  stot[(size_t)bh * D * D + e] = s;
  if (blockIdx.x == 0 && threadIdx.x < D) {
    float z = 0.f;
    for (int c = 0; c < nchunk; ++c) z += zpart[((size_t)bh * nchunk + c) * D + threadIdx.x];
    ztot[(size_t)bh * D + threadIdx.x] = z;
  }
}

template <int D>
__global__ __launch_bounds__(256) void complement_kernel(
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ sblk,
    const float* __restrict__ zblk, const float* __restrict__ stot, const float* __restrict__ ztot,
    uint16_t* __restrict__ sc, float* __restrict__ zc, int nbq, int nbk, int k, int total) {
  constexpr int E = D * D / 256;   // elements per thread
  const int wid = xcd_remap(blockIdx.x, total);
  const int bh = wid / nbq, i = wid % nbq;
  const int t = threadIdx.x;
  const int32_t* sel = idx + ((size_t)bh * nbq + i) * k;
  uint16_t* out = sc + ((size_t)bh * nbq + i) * D * D + t * E;
  float* zout = zc + ((size_t)bh * nbq + i) * D;
  if (k >= nbk) {   // every block is selected: the complement is empty, exactly zero
#pragma unroll
    for (int e = 0; e < E; e += 8) *reinterpret_cast<u32x4*>(out + e) = u32x4{0, 0, 0, 0};
    if (t < D) zout[t] = 0.f;
    return;
  }
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int s = 0; s < k; ++s) {
    const int j = sel[s];
    const uint16_t* src = sblk + ((size_t)bh * nbk + j) * D * D + t * E;
#pragma unroll
    for (int e = 0; e < E; e += 8) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(src + e);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[e + 2 * q] += bf16_lo(w[q]);
        acc[e + 2 * q + 1] += bf16_hi(w[q]);
      }
    }
  }
  const float* tot = stot + (size_t)bh * D * D + t * E;
#pragma unroll
  for (int e = 0; e < E; e += 8) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = pack_bf16(tot[e + 2 * q] - acc[e + 2 * q], tot[e + 2 * q + 1] - acc[e + 2 * q + 1]);
    *reinterpret_cast<u32x4*>(out + e) = o;
  }
  if (t < D) {
    float z = 0.f;
    for (int s = 0; s < k; ++s) z += zblk[((size_t)bh * nbk + sel[s]) * D + t];
    zout[t] = ztot[(size_t)bh * D + t] - z;
  }
}

template <int D>
static hipError_t launch_kv_summary_T(const Plan& s, const void* k, const void* v, char* ws,
                                      hipStream_t st) {
  double* kbar = reinterpret_cast<double*>(ws + s.kbar);
  uint16_t* v16 = reinterpret_cast<uint16_t*>(ws + s.v16);
  uint16_t* sblk = reinterpret_cast<uint16_t*>(ws + s.sblk);
  float* zblk = reinterpret_cast<float*>(ws + s.zblk);
  float* spart = reinterpret_cast<float*>(ws + s.spart);
  float* zpart = reinterpret_cast<float*>(ws + s.zpart);
  const dim3 grid(s.nchunk, s.BH);
  if (s.in_bf16)
    hipLaunchKernelGGL((kv_summary_kernel<uint16_t, D>), grid, dim3(256), 0, st,
                       (const uint16_t*)k, (const uint16_t*)v, kbar, v16, sblk, zblk, spart, zpart,
                       s.nkv, s.nbk);
  else
    hipLaunchKernelGGL((kv_summary_kernel<float, D>), grid, dim3(256), 0, st, (const float*)k,
                       (const float*)v, kbar, v16, sblk, zblk, spart, zpart, s.nkv, s.nbk);
  hipLaunchKernelGGL((reduce_totals_kernel<D>), dim3(D * D / 256, s.BH), dim3(256), 0, st, spart,
                     zpart, reinterpret_cast<float*>(ws + s.stot),
                     reinterpret_cast<float*>(ws + s.ztot), s.nchunk);
  return hipGetLastError();
}

hipError_t launch_kv_summary(const Plan& s, const void* k, const void* v, char* ws, hipStream_t st) {
  if (s.D == 128) return launch_kv_summary_T<128>(s, k, v, ws, st);
  return launch_kv_summary_T<64>(s, k, v, ws, st);
}

hipError_t launch_complement(const Plan& s, const int32_t* idx, char* ws, hipStream_t st) {
  const int total = s.BH * s.nbq;
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(total), dim3(256), 0, st, idx,
                       reinterpret_cast<const uint16_t*>(ws + s.sblk),
                       reinterpret_cast<const float*>(ws + s.zblk),
                       reinterpret_cast<const float*>(ws + s.stot),
                       reinterpret_cast<const float*>(ws + s.ztot),
                       reinterpret_cast<uint16_t*>(ws + s.sc), reinterpret_cast<float*>(ws + s.zc),
                       s.nbq, s.nbk, s.k, total);
  };
  if (s.D == 128) args(complement_kernel<128>);
  else args(complement_kernel<64>);
  return hipGetLastError();
}

}  // namespace sla
