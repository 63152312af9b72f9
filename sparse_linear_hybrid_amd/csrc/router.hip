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
// Pool + project for PB consecutive blocks of one (batch, head): block means over the
// valid tokens (float64 sums, exact for bf16 data, so the summation order does not matter)
// and x~ = mean @ P in float64. The loads of G blocks are issued together; each thread sums
// its rows of 8 channels, the rows of a wave are combined with lane exchanges and the four
// waves through LDS. Each thread then projects one output channel for PB * D / 256 of the
// blocks, reading P once per PB blocks.
constexpr int PB = 8;

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_project_kernel(const T* __restrict__ x,
                                                           const float* __restrict__ P,
                                                           double* __restrict__ out, int n, int nb) {
  constexpr int TPR = D / 8;            // threads per row (8 channels each)
  constexpr int RPP = 256 / TPR;        // rows per pass of the workgroup
  constexpr int LPB = kBlock / RPP;     // rows per thread and block
  constexpr int G = 4;                  // blocks whose loads are in flight together
  __shared__ double part[4][G][D];
  __shared__ double means[PB][D];
  const int j0 = blockIdx.x * PB, bh = blockIdx.y;
  const int nblk = min(PB, nb - j0);
  const T* xb = x + (size_t)bh * n * D;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  const int cg = t % TPR, r = t / TPR;
  for (int b0 = 0; b0 < nblk; b0 += G) {
    double acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = 0.0;
    }
    if constexpr (sizeof(T) == 2) {
      u32x4 raw[G][LPB];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int u = 0; u < LPB; ++u) {
          const int row = (j0 + b0 + g) * kBlock + r + RPP * u;
          raw[g][u] = (b0 + g < nblk && row < n)
                          ? *reinterpret_cast<const u32x4*>(xb + (size_t)row * D + cg * 8)
                          : u32x4{0, 0, 0, 0};
        }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int u = 0; u < LPB; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[g][2 * e] += (double)bf16_lo(raw[g][u][e]);
            acc[g][2 * e + 1] += (double)bf16_hi(raw[g][u][e]);
          }
    } else {
      f32x4 raw[G][LPB][2];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int u = 0; u < LPB; ++u) {
          const int row = (j0 + b0 + g) * kBlock + r + RPP * u;
          const bool ok = b0 + g < nblk && row < n;
          const float* p = xb + (size_t)(ok ? row : 0) * D + cg * 8;
          raw[g][u][0] = ok ? *reinterpret_cast<const f32x4*>(p) : f32x4{0, 0, 0, 0};
          raw[g][u][1] = ok ? *reinterpret_cast<const f32x4*>(p + 4) : f32x4{0, 0, 0, 0};
        }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int u = 0; u < LPB; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[g][e] += (double)raw[g][u][0][e];
            acc[g][4 + e] += (double)raw[g][u][1][e];
          }
    }
    // rows of one wave: lanes with the same channel group differ by multiples of TPR
#pragma unroll
    for (int o = TPR; o < 64; o <<= 1)
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] += __shfl_xor(acc[g][e], o, 64);
    if (lane < TPR) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) part[w][g][cg * 8 + e] = acc[g][e];
    }
    __syncthreads();
    for (int e = t; e < G * D; e += 256) {
      const int g = e / D, c = e % D;
      if (b0 + g < nblk) {
        const int nrows = min(kBlock, n - (j0 + b0 + g) * kBlock);
        means[b0 + g][c] = (part[0][g][c] + part[1][g][c] + part[2][g][c] + part[3][g][c]) /
                           (double)nrows;
      }
    }
    __syncthreads();
  }
  // (means are visible: the last pooling round ended with a barrier)
  constexpr int NBT = PB * D / 256;     // blocks per thread
  const int c = t % D, b0 = t / D;      // blocks b0, b0 + 256/D, ...
  double acc[NBT];
#pragma unroll
  for (int u = 0; u < NBT; ++u) acc[u] = 0.0;
#pragma unroll 8
  for (int rr = 0; rr < D; ++rr) {
    const double pv = (double)P[rr * D + c];
#pragma unroll
    for (int u = 0; u < NBT; ++u) acc[u] = fma(means[b0 + u * (256 / D)][rr], pv, acc[u]);
  }
#pragma unroll
  for (int u = 0; u < NBT; ++u) {
    const int b = b0 + u * (256 / D);
    if (b < nblk) out[((size_t)bh * nb + j0 + b) * D + c] = acc[u];
  }
}

// Block means and (optionally) per-channel population variances of kStatsBlocks<D>
// consecutive blocks of one (batch, head), float64, two passes over the register-held tokens
// (the training-free router's block statistics, SPLA page, section 2.1). Only valid tokens
// count. Two blocks per workgroup keep the tokens of two waves per SIMD in registers.
template <int D>
constexpr int kStatsBlocks = 2;
template <typename T, int D>
__global__ __launch_bounds__(256, 2) void pool_stats_kernel(const T* __restrict__ x,
                                                         double* __restrict__ mean_out,
                                                         double* __restrict__ var_out, int n,
                                                         int nb) {
  constexpr int TPR = D / 8, RPP = 256 / TPR, LPB = kBlock / RPP, G = kStatsBlocks<D>;
  __shared__ double part[4][G][D];
  __shared__ double mean[G][D];
  const int j0 = blockIdx.x * G, bh = blockIdx.y;
  const int nblk = min(G, nb - j0);
  const T* xb = x + (size_t)bh * n * D;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  const int cg = t % TPR, r = t / TPR;
  float xv[G][LPB][8];
  bool ok[G][LPB];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int u = 0; u < LPB; ++u) {
      const int row = (j0 + g) * kBlock + r + RPP * u;
      ok[g][u] = g < nblk && row < n;
      const size_t off = (size_t)(ok[g][u] ? row : 0) * D + cg * 8;
      if constexpr (sizeof(T) == 2) {
        const u32x4 wv = ok[g][u] ? *reinterpret_cast<const u32x4*>(xb + off) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv[g][u][2 * e] = bf16_lo(wv[e]);
          xv[g][u][2 * e + 1] = bf16_hi(wv[e]);
        }
      } else {
        const f32x4 a = ok[g][u] ? *reinterpret_cast<const f32x4*>(xb + off) : f32x4{0, 0, 0, 0};
        const f32x4 b = ok[g][u] ? *reinterpret_cast<const f32x4*>(xb + off + 4) : f32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv[g][u][e] = a[e];
          xv[g][u][4 + e] = b[e];
        }
      }
    }
  auto reduce_rows = [&](double (&acc)[G][8]) {   // sum over all rows of the workgroup -> part
#pragma unroll
    for (int o = TPR; o < 64; o <<= 1)
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] += __shfl_xor(acc[g][e], o, 64);
    if (lane < TPR) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) part[w][g][cg * 8 + e] = acc[g][e];
    }
    __syncthreads();
  };
  double acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double sm = 0.0;
#pragma unroll
      for (int u = 0; u < LPB; ++u) sm += ok[g][u] ? (double)xv[g][u][e] : 0.0;
      acc[g][e] = sm;
    }
  reduce_rows(acc);
  for (int e = t; e < G * D; e += 256) {
    const int g = e / D, c = e % D;
    if (g < nblk) {
      const int nrows = min(kBlock, n - (j0 + g) * kBlock);
      const double m = (part[0][g][c] + part[1][g][c] + part[2][g][c] + part[3][g][c]) /
                       (double)nrows;
      mean[g][c] = m;
      mean_out[((size_t)bh * nb + j0 + g) * D + c] = m;
    }
  }
  if (var_out == nullptr) return;
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double m = g < nblk ? mean[g][cg * 8 + e] : 0.0;
      double sq = 0.0;
#pragma unroll
      for (int u = 0; u < LPB; ++u) {
        const double dv = (double)xv[g][u][e] - m;
        sq += ok[g][u] ? dv * dv : 0.0;
      }
      acc[g][e] = sq;
    }
  reduce_rows(acc);
  for (int e = t; e < G * D; e += 256) {
    const int g = e / D, c = e % D;
    if (g < nblk) {
      const int nrows = min(kBlock, n - (j0 + g) * kBlock);
      var_out[((size_t)bh * nb + j0 + g) * D + c] =
          (part[0][g][c] + part[1][g][c] + part[2][g][c] + part[3][g][c]) / (double)nrows;
    }
  }
}

// ----------------------------------------------------------------------------- scores
// scores[bh][i][j] = sum_c qt[bh][i][c] * kt[bh][j][c]; float64, 64x64 output tile per
// 256-thread workgroup on float64 MFMA (16x16x4), channel chunks of 32 staged in LDS.
// k~ of key block j of (batch, head) bh is at kt + bh * kbh + j * kj.
// TAYLOR (training-free router, SPLA page, section 2.1): qt holds the block means of Q, kt
// those of K and kv the variances of K (same strides); the score is
// tau q.k + log1p(tau^2 (q*q).var / 2) with tau = 1/sqrt(d).
template <int D, bool TAYLOR>
__global__ __launch_bounds__(256) void score_kernel(const double* __restrict__ qt,
                                                    const double* __restrict__ kt,
                                                    const double* __restrict__ kv,
                                                    double* __restrict__ scores, int nbq, int nbk,
                                                    size_t kbh, size_t kj) {
  constexpr int T = 64, C = 32;
  __shared__ double As[C][T + 1];
  __shared__ double Bs[C][T + 1];
  __shared__ double Vs[TAYLOR ? C : 1][TAYLOR ? T + 1 : 1];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * T, j0 = blockIdx.x * T;
  const double* qb = qt + (size_t)bh * nbq * D;
  const double* kb = kt + (size_t)bh * kbh;
  const double* vb = TAYLOR ? kv + (size_t)bh * kbh : nullptr;
  const int t = threadIdx.x;
  // wave w: the 32 x 32 sub-tile (rows 32 (w / 2), columns 32 (w % 2)) as 2 x 2 float64
  // MFMA 16x16x4 tiles. Operand lane l holds row (A) or column (B) l % 16 at reduction
  // index l / 16; result element e of lane l is row l / 16 + 4 e, column l % 16.
  const int w = t >> 6, lane = t & 63, lr = lane & 15, lk = lane >> 4;
  const int wi = (w >> 1) * 32, wj = (w & 1) * 32;
  typedef double f64x4 __attribute__((ext_vector_type(4)));
  f64x4 acc[2][2], acc2[TAYLOR ? 2 : 1][TAYLOR ? 2 : 1];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
  if constexpr (TAYLOR) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc2[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
  }
  // 64 rows x 32 channels per operand and chunk = 2048 values, 8 per thread; the next
  // chunk is fetched into registers while the current one is multiplied
  constexpr int PER = T * C / 256;
  double ra[PER], rb[PER], rv[TAYLOR ? PER : 1];
  auto fetch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = t + 256 * u, r = e / C, cc = e % C;
      const int gi = i0 + r, gj = j0 + r;
      ra[u] = gi < nbq ? qb[(size_t)gi * D + c0 + cc] : 0.0;
      rb[u] = gj < nbk ? kb[(size_t)gj * kj + c0 + cc] : 0.0;
      if constexpr (TAYLOR) rv[u] = gj < nbk ? vb[(size_t)gj * kj + c0 + cc] : 0.0;
    }
  };
  fetch(0);
  for (int c0 = 0; c0 < D; c0 += C) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = t + 256 * u, r = e / C, cc = e % C;
      As[cc][r] = ra[u];
      Bs[cc][r] = rb[u];
      if constexpr (TAYLOR) Vs[cc][r] = rv[u];
    }
    __syncthreads();
    if (c0 + C < D) fetch(c0 + C);
#pragma unroll
    for (int st = 0; st < C / 4; ++st) {
      const int cc = 4 * st + lk;
      double a[2], b[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        a[x] = As[cc][wi + 16 * x + lr];
        b[x] = Bs[cc][wj + 16 * x + lr];
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[x], b[y], acc[x][y], 0, 0, 0);
      if constexpr (TAYLOR) {
        double vv[2];
#pragma unroll
        for (int y = 0; y < 2; ++y) vv[y] = Vs[cc][wj + 16 * y + lr];
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int y = 0; y < 2; ++y)
            acc2[x][y] =
                __builtin_amdgcn_mfma_f64_16x16x4f64(a[x] * a[x], vv[y], acc2[x][y], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  const double tau = 1.0 / sqrt((double)D);
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int gi = i0 + wi + 16 * x + lk + 4 * e;
      if (gi >= nbq) continue;
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        const int gj = j0 + wj + 16 * y + lr;
        double sc = acc[x][y][e];
        if constexpr (TAYLOR) sc = tau * acc[x][y][e] + log1p(0.5 * tau * tau * acc2[x][y][e]);
        if (gj < nbk) scores[((size_t)bh * nbq + gi) * nbk + gj] = sc;
      }
    }
}

// Scores for few query blocks (nbq <= kFewRows): one workgroup per 64 key blocks of a head;
// four threads share a key block (32 channels each, contiguous 256-byte loads), the query
// rows sit in LDS, and the four partial dot products are added with lane exchanges.
constexpr int kFewRows = 8;

template <int D, bool TAYLOR>
__global__ __launch_bounds__(256) void score_few_kernel(const double* __restrict__ qt,
                                                        const double* __restrict__ kt,
                                                        const double* __restrict__ kv,
                                                        double* __restrict__ scores, int nbq,
                                                        int nbk, size_t kbh, size_t kj) {
  constexpr int CPT = D / 4;               // channels per thread
  __shared__ double qs[kFewRows][D];
  const int bh = blockIdx.y;
  const int t = threadIdx.x, c4 = t & 3;
  const int j = blockIdx.x * 64 + (t >> 2);
  for (int e = t; e < nbq * D; e += 256) qs[e / D][e % D] = qt[((size_t)bh * nbq) * D + e];
  double kvals[CPT], vvals[TAYLOR ? CPT : 1];
  const size_t roff = (size_t)bh * kbh + (size_t)(j < nbk ? j : 0) * kj + CPT * c4;
#pragma unroll
  for (int u = 0; u < CPT; u += 2) {
    const double2 w = *reinterpret_cast<const double2*>(kt + roff + u);
    kvals[u] = w.x;
    kvals[u + 1] = w.y;
    if constexpr (TAYLOR) {
      const double2 z = *reinterpret_cast<const double2*>(kv + roff + u);
      vvals[u] = z.x;
      vvals[u + 1] = z.y;
    }
  }
  __syncthreads();
  const double tau = 1.0 / sqrt((double)D);
  for (int i = 0; i < nbq; ++i) {
    double acc = 0.0, acc2 = 0.0;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const double qv = qs[i][CPT * c4 + u];
      acc = fma(qv, kvals[u], acc);
      if constexpr (TAYLOR) acc2 = fma(qv * qv, vvals[u], acc2);
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    if constexpr (TAYLOR) {
      acc2 += __shfl_xor(acc2, 1, 64);
      acc2 += __shfl_xor(acc2, 2, 64);
      acc = tau * acc + log1p(0.5 * tau * tau * acc2);
    }
    if (c4 == 0 && j < nbk) scores[((size_t)bh * nbq + i) * nbk + j] = acc;
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
// ascending and ties go to the lowest index. bits != nullptr: the row of the routed-block
// bitmap (bit j of word j / 32: key block j kept; nwords words) is written as well.
__global__ __launch_bounds__(64) void topk_kernel(const double* __restrict__ scores,
                                                  int32_t* __restrict__ idx,
                                                  uint32_t* __restrict__ bits, int rows, int nbk,
                                                  int k, int nwords) {
  extern __shared__ uint64_t smem[];
  uint64_t* keys = smem;                                   // nbk
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + nbk); // 256
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  const double* s = scores + (size_t)row * nbk;
  int32_t* out = idx + (size_t)row * k;
  uint32_t* brow = bits ? bits + (size_t)row * nwords : nullptr;
  if (k <= 0 || k >= nbk) {
    if (k > 0)
      for (int j = lane; j < nbk; j += 64) out[j] = j;
    if (brow)
      for (int w = lane; w < nwords; w += 64) {
        const int left = nbk - 32 * w;   // valid blocks from bit 0 of this word
        brow[w] = k <= 0 ? 0u : (left >= 32 ? 0xffffffffu : (1u << left) - 1u);
      }
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
    uint32_t cnt = 0;
    if (lane == L) {
      uint32_t acc = above;
      digit = 4 * L;
      for (int b = 3; b >= 0; --b) {
        if (acc + h[b] >= (uint32_t)remaining) { digit = 4 * L + b; cnt = h[b]; break; }
        acc += h[b];
      }
      above = acc;
    }
    digit = __shfl(digit, L, 64);
    above = __shfl(above, L, 64);
    cnt = __shfl(cnt, L, 64);
    remaining -= (int)above;
    prefix |= (uint64_t)digit << shift;
    mask |= 255ull << shift;
    __syncthreads();
    if (cnt == (uint32_t)remaining) break;   // the whole bucket is kept: no further digits
  }
  // Keys whose masked value exceeds `prefix` are kept, and of those equal to it under the
  // mask the first `remaining` in index order (all of them when the loop stopped early;
  // after all 8 digits the mask is complete and these are exact ties, lowest index first).
  int written = 0, eq_seen = 0;
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  for (int base = 0; base < nbk; base += 64) {
    const int j = base + lane;
    const bool valid = j < nbk;
    const uint64_t key = valid ? (keys[j] & mask) : 0ull;
    const bool gt = valid && key > prefix;
    const bool eq = valid && key == prefix;
    const unsigned long long eqb = __ballot(eq);
    const int eq_rank = eq_seen + __popcll(eqb & lt_mask);
    const bool sel = gt || (eq && eq_rank < remaining);
    const unsigned long long sb = __ballot(sel);
    if (sel) out[written + __popcll(sb & lt_mask)] = j;
    if (brow && lane < 2 && base / 32 + lane < nwords)
      brow[base / 32 + lane] = (uint32_t)(sb >> (32 * lane));
    written += __popcll(sb);
    eq_seen += __popcll(eqb);
  }
}

// Rows of at most 64 * KPL key blocks (0 < k < nbk): one wave per row with its keys in
// registers (KPL per lane) and no histogram. The k-th largest key T is found one bit at a
// time, most significant first: a candidate bit is kept when at least k keys are >= the
// candidate, counted with one compare per key whose wave mask is popcounted. Keys above the
// undecided range of T are carried as a count; once at most 64 keys remain inside that range
// they are gathered one per lane (through LDS) and the remaining bits compare only those. The
// search stops as soon as exactly k keys are >= the candidate (then those k are the
// selection); otherwise it ends with T exact, and every key > T is kept plus the lowest-index
// keys == T. Same selection, ascending output and bitmap rows as topk_kernel.
// Four rows (one per wave) per workgroup; the waves never wait for each other.
template <int KPL>
__global__ __launch_bounds__(256) void topk_reg_kernel(const double* __restrict__ scores,
                                                       int32_t* __restrict__ idx,
                                                       uint32_t* __restrict__ bits, int rows,
                                                       int nbk, int k, int nwords) {
  __shared__ uint64_t bucket_all[4][64];
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;   // whole waves only
  uint64_t* bucket = bucket_all[threadIdx.x >> 6];
  const double* s = scores + (size_t)row * nbk;
  int32_t* out = idx + (size_t)row * k;
  uint32_t* brow = bits ? bits + (size_t)row * nwords : nullptr;
  uint64_t key[KPL];   // padding (j >= nbk) is 0: below every candidate, never counted
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const int j = 64 * u + lane;
    key[u] = j < nbk ? score_key(s[j]) : 0ull;
  }
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  uint64_t T = 0;
  bool exact = false;
  // Undecided range of T after deciding bits 63 .. b: [T, T + 2^b). ge: keys >= T (valid
  // keys only), above: keys >= T + 2^b.
  int ge = nbk, above = 0, bit = 63;
  for (; bit >= 0; --bit) {
    const uint64_t c = T | (1ull << bit);
    int n = 0;
#pragma unroll
    for (int u = 0; u < KPL; ++u) n += __popcll(__ballot(key[u] >= c));
    if (n >= k) {
      T = c;
      ge = n;
      if (n == k) {
        exact = true;
        break;
      }
    } else {
      above = n;
    }
    if (ge - above <= 64) break;   // few keys left inside the range: gather them
  }
  if (!exact && bit > 0) {
    // gather the keys in [T, T + 2^bit) (valid ones), then decide bits bit-1 .. 0 on them
    const uint64_t hi = T + (1ull << bit);   // 0 (wrapped): the range reaches the top key
    int base = 0;
#pragma unroll
    for (int u = 0; u < KPL; ++u) {
      const bool in = 64 * u + lane < nbk && key[u] >= T && (hi == 0 || key[u] < hi);
      const unsigned long long m = __ballot(in);
      if (in) bucket[base + __popcll(m & lt_mask)] = key[u];
      base += __popcll(m);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // this wave's writes, then reads
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint64_t bk = lane < base ? bucket[lane] : 0ull;
    for (--bit; bit >= 0; --bit) {
      const uint64_t c = T | (1ull << bit);
      const int n = above + __popcll(__ballot(bk >= c));
      if (n >= k) {
        T = c;
        if (n == k) {
          exact = true;
          break;
        }
      }
    }
  }
  int remaining = 0;   // keys == T to keep, lowest index first
  if (!exact) {
    int n_gt = 0;
#pragma unroll
    for (int u = 0; u < KPL; ++u) n_gt += __popcll(__ballot(key[u] > T));
    remaining = k - n_gt;
  }
  int written = 0, eq_seen = 0;
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const int j = 64 * u + lane;
    if (64 * u >= nbk) break;   // uniform
    const bool valid = j < nbk;
    const bool gt = valid && (exact ? key[u] >= T : key[u] > T);
    const bool eq = !exact && valid && key[u] == T;
    const unsigned long long eqb = __ballot(eq);
    const int eq_rank = eq_seen + __popcll(eqb & lt_mask);
    const bool sel = gt || (eq && eq_rank < remaining);
    const unsigned long long sb = __ballot(sel);
    if (sel) out[written + __popcll(sb & lt_mask)] = j;
    if (brow && lane < 2 && 2 * u + lane < nwords)
      brow[2 * u + lane] = (uint32_t)(sb >> (32 * lane));
    written += __popcll(sb);
    eq_seen += __popcll(eqb);
  }
}

// ----------------------------------------------------------------------------- launchers
template <int D>
static void launch_pool_q(const Plan& s, const void* q, const float* pq, double* qt,
                          hipStream_t st) {
  const dim3 gq((s.nbq + PB - 1) / PB, s.BH);
  if (s.in_bf16)
    launch_pool_stream(s, q, pq, qt, s.nq, s.nbq, st);
  else
    hipLaunchKernelGGL((pool_project_kernel<float, D>), gq, dim3(256), 0, st, (const float*)q,
                       pq, qt, s.nq, s.nbq);
}

// kv != nullptr: training-free (Taylor) scores with the key variances kv
template <int D>
static void launch_select(const Plan& s, const double* qt, const double* kt, const double* kv,
                          size_t kbh, size_t kj, double* sc, int32_t* idx, uint32_t* bits,
                          hipStream_t st) {
  const int rq = s.BH * s.nbq;
  const dim3 gf((s.nbk + 63) / 64, s.BH), gt((s.nbk + 63) / 64, (s.nbq + 63) / 64, s.BH);
  if (s.nbq <= kFewRows) {
    if (kv)
      hipLaunchKernelGGL((score_few_kernel<D, true>), gf, dim3(256), 0, st, qt, kt, kv, sc, s.nbq,
                         s.nbk, kbh, kj);
    else
      hipLaunchKernelGGL((score_few_kernel<D, false>), gf, dim3(256), 0, st, qt, kt, kv, sc, s.nbq,
                         s.nbk, kbh, kj);
  } else {
    if (kv)
      hipLaunchKernelGGL((score_kernel<D, true>), gt, dim3(256), 0, st, qt, kt, kv, sc, s.nbq,
                         s.nbk, kbh, kj);
    else
      hipLaunchKernelGGL((score_kernel<D, false>), gt, dim3(256), 0, st, qt, kt, kv, sc, s.nbq,
                         s.nbk, kbh, kj);
  }
  if (s.k > 0 && s.k < s.nbk && s.nbk <= 64 * 32) {   // keys fit in registers
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3((rq + 3) / 4), dim3(256), 0, st, sc, idx, bits, rq, s.nbk,
                         s.k, s.nwords);
    };
    if (s.nbk <= 64 * 8) go(topk_reg_kernel<8>);
    else if (s.nbk <= 64 * 12) go(topk_reg_kernel<12>);
    else if (s.nbk <= 64 * 16) go(topk_reg_kernel<16>);
    else if (s.nbk <= 64 * 20) go(topk_reg_kernel<20>);
    else if (s.nbk <= 64 * 24) go(topk_reg_kernel<24>);
    else go(topk_reg_kernel<32>);
  } else if (s.k > 0 || bits) {
    const size_t lds = (size_t)s.nbk * 8 + 256 * 4;
    hipLaunchKernelGGL(topk_kernel, dim3(rq), dim3(64), lds, st, sc, idx, bits, rq, s.nbk, s.k,
                       s.nwords);
  }
}

template <int D>
static hipError_t launch_route_T(const Plan& s, const void* q, const void* k, const float* pq,
                                 const float* pk, int32_t* idx, uint32_t* bits, char* ws,
                                 bool pool_k, hipStream_t st) {
  double* qt = reinterpret_cast<double*>(ws + s.qt);
  double* kt = reinterpret_cast<double*>(ws + s.kt);
  double* sc = reinterpret_cast<double*>(ws + s.scores);
  launch_pool_q<D>(s, q, pq, qt, st);
  if (pool_k) {
    const dim3 gk((s.nbk + PB - 1) / PB, s.BH);
    if (s.in_bf16)
      launch_pool_stream(s, k, pk, kt, s.nkv, s.nbk, st);
    else
      hipLaunchKernelGGL((pool_project_kernel<float, D>), gk, dim3(256), 0, st, (const float*)k,
                         pk, kt, s.nkv, s.nbk);
  }
  launch_select<D>(s, qt, kt, nullptr, (size_t)s.nbk * s.D, (size_t)s.D, sc, idx, bits, st);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_route_taylor_T(const Plan& s, const void* q, const void* k,
                                        int32_t* idx, uint32_t* bits, char* ws, hipStream_t st) {
  double* qt = reinterpret_cast<double*>(ws + s.qt);
  double* kt = reinterpret_cast<double*>(ws + s.kt);
  double* kv = reinterpret_cast<double*>(ws + s.kvar);
  double* sc = reinterpret_cast<double*>(ws + s.scores);
  constexpr int G = kStatsBlocks<D>;
  const dim3 gq((s.nbq + G - 1) / G, s.BH), gk((s.nbk + G - 1) / G, s.BH);
  if (s.in_bf16) {
    hipLaunchKernelGGL((pool_stats_kernel<uint16_t, D>), gq, dim3(256), 0, st, (const uint16_t*)q,
                       qt, nullptr, s.nq, s.nbq);
    hipLaunchKernelGGL((pool_stats_kernel<uint16_t, D>), gk, dim3(256), 0, st, (const uint16_t*)k,
                       kt, kv, s.nkv, s.nbk);
  } else {
    hipLaunchKernelGGL((pool_stats_kernel<float, D>), gq, dim3(256), 0, st, (const float*)q, qt,
                       nullptr, s.nq, s.nbq);
    hipLaunchKernelGGL((pool_stats_kernel<float, D>), gk, dim3(256), 0, st, (const float*)k, kt,
                       kv, s.nkv, s.nbk);
  }
  launch_select<D>(s, qt, kt, kv, (size_t)s.nbk * s.D, (size_t)s.D, sc, idx, bits, st);
  return hipGetLastError();
}

hipError_t launch_route_taylor(const Plan& s, const void* q, const void* k, int32_t* idx,
                               uint32_t* bits, char* ws, hipStream_t st) {
  if (s.D == 128) return launch_route_taylor_T<128>(s, q, k, idx, bits, ws, st);
  return launch_route_taylor_T<64>(s, q, k, idx, bits, ws, st);
}

hipError_t launch_route(const Plan& s, const void* q, const void* k, const float* pq,
                        const float* pk, int32_t* idx, uint32_t* bits, char* ws, bool pool_k,
                        hipStream_t st) {
  if (s.D == 128) return launch_route_T<128>(s, q, k, pq, pk, idx, bits, ws, pool_k, st);
  return launch_route_T<64>(s, q, k, pq, pk, idx, bits, ws, pool_k, st);
}

hipError_t launch_route_cached(const Plan& s, const void* q, const float* pq, const double* kt,
                               size_t kbh, size_t kj, int32_t* idx, double* qt, double* sc,
                               hipStream_t st) {
  if (s.D == 128) {
    launch_pool_q<128>(s, q, pq, qt, st);
    launch_select<128>(s, qt, kt, nullptr, kbh, kj, sc, idx, nullptr, st);
  } else {
    launch_pool_q<64>(s, q, pq, qt, st);
    launch_select<64>(s, qt, kt, nullptr, kbh, kj, sc, idx, nullptr, st);
  }
  return hipGetLastError();
}

}  // namespace sla
