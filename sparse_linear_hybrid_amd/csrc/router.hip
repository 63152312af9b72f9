// Router kernels (SLA2 page, section 2.B "Roteador Aprendível"): block mean-pool of Q and
// K, learnable projection, block scores and per-row top-k.
//
// Precision: pooled sums, projections and scores are float64. Block sums of bf16 inputs
// are exact in float64 (at most 64 terms of 8-bit significands), so pooled means are
// bit-identical to any other exact computation and the selection only depends on the
// rounding of the projection/score dot products (relative 1e-16).
#include "common.h"
#include "kernels.h"

namespace sla {

// ----------------------------------------------------------------------------- pooling
// Sum of one 64-token block into per-thread partials: each thread owns 8 consecutive
// channels of rows r0, r0 + RPP, ... (RPP = rows covered by the 256 threads per pass).
template <typename T, int D>
__device__ __forceinline__ void block_sum_partial(const T* __restrict__ x, int row0, int nrows,
                                                  double (&acc)[8]) {
  constexpr int TPR = D / 8;           // threads per row
  constexpr int RPP = 256 / TPR;       // rows per pass
  const int t = threadIdx.x;
  const int cg = t % TPR, r = t / TPR;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int rr = r; rr < nrows; rr += RPP) {
    const T* p = x + (size_t)(row0 + rr) * D + cg * 8;
    if constexpr (sizeof(T) == 2) {
      u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += (double)bf16_lo(w[e]);
        acc[2 * e + 1] += (double)bf16_hi(w[e]);
      }
    } else {
      f32x4 a = *reinterpret_cast<const f32x4*>(p);
      f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += (double)a[e];
        acc[4 + e] += (double)b[e];
      }
    }
  }
}

// Combine the per-thread partials (fixed order) and write the mean over nrows tokens.
template <int D>
__device__ __forceinline__ void block_mean_finish(double (&acc)[8], int nrows, double* lds,
                                                  double* __restrict__ out) {
  constexpr int TPR = D / 8;
  constexpr int RPP = 256 / TPR;
  const int t = threadIdx.x;
  const int cg = t % TPR, r = t / TPR;
#pragma unroll
  for (int e = 0; e < 8; ++e) lds[r * D + cg * 8 + e] = acc[e];
  __syncthreads();
  if (t < D) {
    double s = 0.0;
    for (int rr = 0; rr < RPP; ++rr) s += lds[rr * D + t];
    out[t] = s / (double)nrows;
  }
  __syncthreads();
}

// Pool + project for PB consecutive blocks of one (batch, head): block means over the
// valid tokens (float64 sums, exact for bf16 data) and x~ = mean @ P in float64. Reading P
// once per PB blocks keeps the projection off the critical path.
constexpr int PB = 8;

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_project_kernel(const T* __restrict__ x,
                                                           const float* __restrict__ P,
                                                           double* __restrict__ out, int n, int nb) {
  constexpr int RPP = 256 / (D / 8);
  __shared__ double part[RPP * D];
  __shared__ double means[PB][D];
  const int j0 = blockIdx.x * PB, bh = blockIdx.y;
  const int nblk = min(PB, nb - j0);
  const T* xb = x + (size_t)bh * n * D;
  const int t = threadIdx.x;
  for (int b = 0; b < nblk; ++b) {
    const int row0 = (j0 + b) * kBlock;
    const int nrows = min(kBlock, n - row0);
    double acc[8];
    block_sum_partial<T, D>(xb, row0, nrows, acc);
    block_mean_finish<D>(acc, nrows, part, &means[b][0]);
  }
  for (int b = t / D; b < nblk; b += 256 / D) {
    const int c = t % D;
    double acc = 0.0;
    for (int r = 0; r < D; ++r) acc = fma(means[b][r], (double)P[r * D + c], acc);
    out[((size_t)bh * nb + j0 + b) * D + c] = acc;
  }
}

// ----------------------------------------------------------------------------- scores
// scores[bh][i][j] = sum_c qt[bh][i][c] * kt[bh][j][c]; float64, 64x64 output tile per
// 256-thread workgroup, 4x4 outputs per thread, channel chunks of 32 staged in LDS.
template <int D>
__global__ __launch_bounds__(256) void score_kernel(const double* __restrict__ qt,
                                                    const double* __restrict__ kt,
                                                    double* __restrict__ scores, int nbq, int nbk) {
  constexpr int T = 64, C = 32;
  __shared__ double As[C][T + 1];
  __shared__ double Bs[C][T + 1];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * T, j0 = blockIdx.x * T;
  const double* qb = qt + (size_t)bh * nbq * D;
  const double* kb = kt + (size_t)bh * nbk * D;
  const int t = threadIdx.x;
  const int ty = t / 16, tx = t % 16;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int c0 = 0; c0 < D; c0 += C) {
    // 64 rows x 32 channels per operand = 2048 values, 8 per thread
    for (int e = t; e < T * C; e += 256) {
      const int r = e / C, cc = e % C;
      const int gi = i0 + r, gj = j0 + r;
      As[cc][r] = gi < nbq ? qb[(size_t)gi * D + c0 + cc] : 0.0;
      Bs[cc][r] = gj < nbk ? kb[(size_t)gj * D + c0 + cc] : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int cc = 0; cc < C; ++cc) {
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = As[cc][ty + 16 * u];
        b[u] = Bs[cc][tx + 16 * u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[u][w] = fma(a[u], b[w], acc[u][w]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int gi = i0 + ty + 16 * u;
    if (gi >= nbq) continue;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int gj = j0 + tx + 16 * w;
      if (gj < nbk) scores[((size_t)bh * nbq + gi) * nbk + gj] = acc[u][w];
    }
  }
}

// ----------------------------------------------------------------------------- top-k
// Order-preserving 64-bit key of a float64 score: larger score -> larger key. -0 is
// folded into +0 (they compare equal), NaN ranks below everything.
__device__ __forceinline__ uint64_t score_key(double s) {
  if (s != s) return 0ull;
  if (s == 0.0) s = 0.0;
  const uint64_t u = (uint64_t)__double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// One wave per (bh, query block) row. Radix-select (8 passes of 8 bits, most significant
// first) finds the k-th largest key T exactly; then one ascending sweep over j keeps every
// key > T and the lowest-index keys == T until k are kept. The output is therefore
// ascending and ties go to the lowest index.
__global__ __launch_bounds__(64) void topk_kernel(const double* __restrict__ scores,
                                                  int32_t* __restrict__ idx, int rows, int nbk,
                                                  int k) {
  extern __shared__ uint64_t smem[];
  uint64_t* keys = smem;                                   // nbk
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + nbk); // 256
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  const double* s = scores + (size_t)row * nbk;
  int32_t* out = idx + (size_t)row * k;
  if (k <= 0) return;
  if (k >= nbk) {
    for (int j = lane; j < nbk; j += 64) out[j] = j;
    return;
  }
  for (int j = lane; j < nbk; j += 64) keys[j] = score_key(s[j]);
  __syncthreads();
  uint64_t prefix = 0, mask = 0;
  int remaining = k;   // rank of the wanted key among keys matching `prefix`
  for (int pass = 7; pass >= 0; --pass) {
    const int shift = pass * 8;
#pragma unroll
    for (int b = 0; b < 4; ++b) hist[lane * 4 + b] = 0;
    __syncthreads();
    for (int j = lane; j < nbk; j += 64) {
      const uint64_t key = keys[j];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // lane l owns digits 4l..4l+3; suffix sums over lanes (high digits first)
    uint32_t h[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) h[b] = hist[lane * 4 + b];
    const uint32_t own = h[0] + h[1] + h[2] + h[3];
    uint32_t suf = own;                       // sum over lanes >= lane
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = __shfl_down(suf, o, 64);
      if (lane + o < 64) suf += v;
    }
    const unsigned long long ge = __ballot(suf >= (uint32_t)remaining);
    const int L = 63 - __clzll(ge);           // highest lane whose suffix reaches `remaining`
    uint32_t above = __shfl(suf - own, L, 64);
    int digit = 0;
    if (lane == L) {
      uint32_t acc = above;
      digit = 4 * L;
      for (int b = 3; b >= 0; --b) {
        if (acc + h[b] >= (uint32_t)remaining) { digit = 4 * L + b; break; }
        acc += h[b];
      }
      above = acc;
    }
    digit = __shfl(digit, L, 64);
    above = __shfl(above, L, 64);
    remaining -= (int)above;
    prefix |= (uint64_t)digit << shift;
    mask |= 255ull << shift;
    __syncthreads();
  }
  // prefix == T, the k-th largest key; `remaining` keys equal to T are to be kept.
  const uint64_t T = prefix;
  int written = 0, eq_seen = 0;
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  for (int base = 0; base < nbk; base += 64) {
    const int j = base + lane;
    const bool valid = j < nbk;
    const uint64_t key = valid ? keys[j] : 0ull;
    const bool gt = valid && key > T;
    const bool eq = valid && key == T;
    const unsigned long long eqb = __ballot(eq);
    const int eq_rank = eq_seen + __popcll(eqb & lt_mask);
    const bool sel = gt || (eq && eq_rank < remaining);
    const unsigned long long sb = __ballot(sel);
    if (sel) out[written + __popcll(sb & lt_mask)] = j;
    written += __popcll(sb);
    eq_seen += __popcll(eqb);
  }
}

// ----------------------------------------------------------------------------- launchers
template <int D>
static hipError_t launch_route_T(const Plan& s, const void* q, const void* k, const float* pq,
                                 const float* pk, int32_t* idx, char* ws, bool pool_k,
                                 hipStream_t st) {
  double* qt = reinterpret_cast<double*>(ws + s.qt);
  double* kt = reinterpret_cast<double*>(ws + s.kt);
  double* sc = reinterpret_cast<double*>(ws + s.scores);
  const dim3 gq((s.nbq + PB - 1) / PB, s.BH), gk((s.nbk + PB - 1) / PB, s.BH);
  if (s.in_bf16) {
    hipLaunchKernelGGL((pool_project_kernel<uint16_t, D>), gq, dim3(256), 0, st,
                       (const uint16_t*)q, pq, qt, s.nq, s.nbq);
    if (pool_k)
      hipLaunchKernelGGL((pool_project_kernel<uint16_t, D>), gk, dim3(256), 0, st,
                         (const uint16_t*)k, pk, kt, s.nkv, s.nbk);
  } else {
    hipLaunchKernelGGL((pool_project_kernel<float, D>), gq, dim3(256), 0, st, (const float*)q,
                       pq, qt, s.nq, s.nbq);
    if (pool_k)
      hipLaunchKernelGGL((pool_project_kernel<float, D>), gk, dim3(256), 0, st, (const float*)k,
                         pk, kt, s.nkv, s.nbk);
  }
  const int rq = s.BH * s.nbq;
  hipLaunchKernelGGL((score_kernel<D>), dim3((s.nbk + 63) / 64, (s.nbq + 63) / 64, s.BH),
                     dim3(256), 0, st, qt, kt, sc, s.nbq, s.nbk);
  if (s.k > 0) {
    const size_t lds = (size_t)s.nbk * 8 + 256 * 4;
    hipLaunchKernelGGL(topk_kernel, dim3(rq), dim3(64), lds, st, sc, idx, rq, s.nbk, s.k);
  }
  return hipGetLastError();
}

hipError_t launch_route(const Plan& s, const void* q, const void* k, const float* pq,
                        const float* pk, int32_t* idx, char* ws, bool pool_k, hipStream_t st) {
  if (s.D == 128) return launch_route_T<128>(s, q, k, pq, pk, idx, ws, pool_k, st);
  return launch_route_T<64>(s, q, k, pq, pk, idx, ws, pool_k, st);
}

}  // namespace sla
