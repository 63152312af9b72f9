// Key/value summary cache pass (SPLA page, section 2.2: the linear state kept with the key
// blocks is a running total, from which the unselected blocks' term is the total minus the
// selected ones; SLA2 page, section 2.B: the router needs only the pooled, projected keys).
// One streaming pass over K and V (bf16) computes, per key block j, the projected block
// mean k~_j = mean(K_j) P_k in float64, and per chunk of key blocks the partial totals
// sum phi(K)^T V (fp32) and sum phi(K); reduce_totals_kernel adds the chunks.
//
// Nothing per key block except k~ leaves the kernel, so it is bound by reading K and V. The
// tiles go from HBM straight into an NS-deep LDS ring (loads into LDS, as in the exact
// branch), NS - 1 blocks ahead of the one being reduced. Wave w owns the 32-channel strip
// r = 32 mt .. 32 mt + 31 of phi(K)^T (mt = w at d = 128; at d = 64 two waves share a strip
// and split the value columns):
//   * the strip's A fragments are read transposed from the K tile; before the ReLU the same
//     fragments give the block's per-channel sums, accumulated in float64 (exact for bf16
//     inputs, so the order does not matter) and divided by the valid token count;
//   * S += relu(K)^T V on bf16 MFMA straight into the chunk's running total (fp32);
//   * k~ partial over the strip: sum_{r in strip} mean_r P_k[r][c] for every output channel c,
//     with the strip's rows of P_k held in registers as float64; the four strip partials are
//     added in a fixed order one iteration later (after the next barrier) and stored.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace sla {

namespace {

struct TotalsArgs {
  const uint16_t* k;
  const uint16_t* v;
  const float* pk;     // [D(in)][D(out)]
  double* kt;          // k~ of block j of head bh at kt + bh * kbh + j * kj
  size_t kbh, kj;
  float* spart;        // [BH][nchunk][D(c)][D(r)]
  float* zpart;        // [BH][nchunk][D]
  int nkv, nbk, jbase, t0, nchunk;
  int chunk;           // key blocks per workgroup
};

template <int D, bool POOL>
struct TotalsCfg {
  static constexpr int NS = 4;                         // ring depth (blocks)
  static constexpr int TILE = 64 * D;                  // elements of a K or V tile
  static constexpr int KPW = TILE * 2 / 1024 / 4;      // 1-KB pieces per wave and tensor
  static constexpr int NT = D / 32;                    // 32-column tiles of the value side
  static constexpr int TPW = D == 128 ? NT : 1;        // value tiles per wave
  static constexpr int OCC = (D == 128 && !POOL) ? 1 : 2;   // workgroups per CU
  static constexpr int CPL = D / 64;                   // output channels of k~ per lane
  static constexpr int STRIPS = D / 32;                // 32-channel strips of phi(K)^T
};

// POOL: only the projected block means of one tensor (the router's pooling of Q, or of K
// when it routes on its own): the V tiles, the MFMA product and the partial totals drop out.
template <int D, bool POOL>
__global__ __launch_bounds__(256, (TotalsCfg<D, POOL>::OCC)) void kv_totals_kernel(TotalsArgs a) {
  using C = TotalsCfg<D, POOL>;
  constexpr int NS = C::NS, TILE = C::TILE, KPW = C::KPW, TPW = C::TPW, CPL = C::CPL;
  constexpr int STRIPS = C::STRIPS;
  constexpr int CH = D / 8;
  constexpr int TPS = POOL ? 1 : 2;                     // tiles per ring slot
  constexpr int LPS = TPS * KPW;                         // loads per wave and slot
  __shared__ __attribute__((aligned(16))) uint16_t ring[NS * TPS * TILE];   // [slot][K, V]
  __shared__ double kpart[2][STRIPS][D];   // per strip: partial k~ of the last two blocks

  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int wvs = __builtin_amdgcn_readfirstlane(w);
  const int mt = D == 128 ? w : (w >> 1);             // 32-channel strip of phi(K)^T
  const int nt0 = D == 128 ? 0 : (w & 1);             // first value tile of this wave
  const bool proj_wave = D == 128 || (w & 1) == 0;    // computes the strip's k~ partial
  const int j0 = a.jbase + chunk * a.chunk;
  const int j1 = min(j0 + a.chunk, a.nbk);
  const uint16_t* kb = a.k + (size_t)bh * a.nkv * D;
  const uint16_t* vb = a.v + (size_t)bh * a.nkv * D;

  // rows of P_k for this strip, float64: pk[i][u] = P_k[32 mt + i][lane + 64 u]
  double pk[32][CPL];
  if (proj_wave) {
#pragma unroll
    for (int i = 0; i < 32; ++i)
#pragma unroll
      for (int u = 0; u < CPL; ++u) pk[i][u] = (double)a.pk[(32 * mt + i) * D + lane + 64 * u];
  }
  wait_vmem();   // the loads into LDS below are waited for by count alone

  // loads into LDS: piece u of this wave lands at elements 512 (KPW w + u) + 8 lane of a
  // tile; the lane fetches the chunk that the tile's swizzle puts there
  uint32_t koff[KPW], voff[KPW];
#pragma unroll
  for (int u = 0; u < KPW; ++u) {
    const int e = (wvs * KPW + u) * 512 + lane * 8;
    const int r = e / D, pch = (e % D) / 8;
    koff[u] = (uint32_t)(r * D * 2 + ((pch ^ r) & (CH - 1)) * 16);
    voff[u] = (uint32_t)(r * D * 2 + ((pch ^ swzv_f<D>(r)) & (CH - 1)) * 16);
  }
  // j >= j1: an empty range (no memory access), so every step issues the same number of
  // loads and the vmcnt waits below hold
  auto stage = [&](int j, int slot) __attribute__((always_inline)) {
    const bool live = j < j1;
    const int row0 = live ? j * kBlock : 0;
    const uint32_t bytes = live ? (uint32_t)(min(kBlock, a.nkv - row0) * D * 2) : 0u;
    const i32x4 rk = make_rsrc(kb + (size_t)row0 * D, bytes);
    const i32x4 rv = make_rsrc(vb + (size_t)row0 * D, bytes);
    const uint32_t kd = lds_addr(ring + slot * TPS * TILE) + wvs * KPW * 1024;
#pragma unroll
    for (int u = 0; u < KPW; ++u) load_lds16(rk, kd + u * 1024, koff[u]);
    if constexpr (!POOL) {
      const uint32_t vd = lds_addr(ring + (slot * 2 + 1) * TILE) + wvs * KPW * 1024;
#pragma unroll
      for (int u = 0; u < KPW; ++u) load_lds16(rv, vd + u * 1024, voff[u]);
    }
  };

  // transposing fragment reads (lane: index x0 + lane % 32, 8 tokens k0 + 8 h ..)
  auto frag = [&](const uint16_t* M, int x0, int k0, bool vtile) __attribute__((always_inline)) {
    const int g = lane >> 4, L = lane & 15;
    const int row = k0 + 8 * (g >> 1) + (L >> 2);
    const int col = x0 + 16 * (g & 1) + 4 * (L & 3);
    const int o0 = vtile ? swzv<D>(row, col) : swz<D>(row, col);
    const int o1 = vtile ? swzv<D>(row + 4, col) : swz<D>(row + 4, col);
    const u32x2 lo = lds_read_tr16(M + o0);
    const u32x2 hi = lds_read_tr16(M + o1);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  f32x16 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = f32x16{};
  float zsum = 0.f;

  // k~ of block jj from the four strip partials (fixed order), by threads t < D
  auto finish_kt = [&](int jj) __attribute__((always_inline)) {
    if (t < D) {
      const double* p = &kpart[jj & 1][0][0];
      double s = p[t];
#pragma unroll
      for (int q = 1; q < STRIPS; ++q) s += p[q * D + t];
      a.kt[(size_t)bh * a.kbh + (size_t)jj * a.kj + t] = s;
    }
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s) stage(j0 + s, s);
  for (int j = j0; j < j1; ++j) {
    const int it = j - j0;
    const int slot = it % NS;
    // tile j has landed for every wave (at most the NS - 2 later tiles are in flight), every
    // wave is done with the slot refilled below, and its kpart stores of block j - 1 are
    // complete (ordinary LDS stores: the barrier waits for them explicitly)
    barrier_vmem_lds_n<(NS - 2) * LPS>();
    stage(j + NS - 1, (it + NS - 1) % NS);
    if (j > j0) finish_kt(j - 1);
    const uint16_t* Kt = ring + slot * TPS * TILE;
    const uint16_t* Vt = Kt + TILE;
    const int row0 = j * kBlock;
    const int nrows = min(kBlock, a.nkv - row0);
    const bool clip = __builtin_amdgcn_readfirstlane(row0 < a.t0 ? 1 : 0);
    u32x4 af[4];
    double csum = 0.0;
    float zl = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const u32x4 raw = frag(Kt, 32 * mt, 16 * s4, false);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        csum += (double)bf16_lo(raw[e]) + (double)bf16_hi(raw[e]);
      af[s4] = relu_bf16x8(raw);
      if (clip) {   // tokens before t0 are already in the totals
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tok = row0 + 16 * s4 + 8 * h + 2 * e;
          const uint32_t lo = tok < a.t0 ? 0u : (af[s4][e] & 0xffffu);
          const uint32_t hi = tok + 1 < a.t0 ? 0u : (af[s4][e] & 0xffff0000u);
          af[s4][e] = lo | hi;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) zl += bf16_lo(af[s4][e]) + bf16_hi(af[s4][e]);
    }
    zsum += zl;
    if constexpr (!POOL) {
#pragma unroll
      for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          acc[u] = mfma_bf16(af[s4], frag(Vt, 32 * (nt0 + u), 16 * s4, true), acc[u]);
    }
    if (proj_wave) {
      // column sums over the 64 tokens (lane halves hold 32 each), then the strip's k~ part
      const double mean = (csum + __shfl_xor(csum, 32, 64)) / (double)nrows;
      double kp[CPL];
#pragma unroll
      for (int u = 0; u < CPL; ++u) kp[u] = 0.0;
      const uint64_t mbits = (uint64_t)__double_as_longlong(mean);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)mbits, i);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(mbits >> 32), i);
        const double mi = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
#pragma unroll
        for (int u = 0; u < CPL; ++u) kp[u] = fma(mi, pk[i][u], kp[u]);
      }
#pragma unroll
      for (int u = 0; u < CPL; ++u) kpart[j & 1][mt][lane + 64 * u] = kp[u];
    }
  }
  wait_vmem();          // no load into LDS outlives the workgroup
  __syncthreads();
  if (j1 > j0) finish_kt(j1 - 1);
  if constexpr (POOL) return;

  // chunk partial totals, layout [c][r]; z over the strip (both lane halves hold it)
  const int cidx = chunk;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int c = 32 * (nt0 + u) + l32;
    float* dst = a.spart + (((size_t)bh * a.nchunk + cidx) * D + c) * D;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 32 * mt + 8 * q + 4 * h;
      *reinterpret_cast<f32x4*>(dst + r) =
          f32x4{acc[u][4 * q], acc[u][4 * q + 1], acc[u][4 * q + 2], acc[u][4 * q + 3]};
    }
  }
  zsum += swap_halves(zsum);
  if (proj_wave && h == 0) a.zpart[((size_t)bh * a.nchunk + cidx) * D + 32 * mt + l32] = zsum;
}

}  // namespace

// The cache update from n_done tokens (bf16 inputs): the streaming pass above, then the
// fixed-order reduction of its chunk partials onto (or, from zero tokens, into) the totals.
hipError_t launch_kv_totals(const Plan& s, const void* k, const void* v, const float* pk,
                            int n_done, double* kt, size_t kbh, size_t kj, float* stot,
                            float* ztot, char* ws, hipStream_t st) {
  (void)stot;
  (void)ztot;
  TotalsArgs a;
  a.k = reinterpret_cast<const uint16_t*>(k);
  a.v = reinterpret_cast<const uint16_t*>(v);
  a.pk = pk;
  a.kt = kt;
  a.kbh = kbh;
  a.kj = kj;
  a.spart = reinterpret_cast<float*>(ws);
  a.zpart = reinterpret_cast<float*>(ws + cache_update_zpart_offset(s, n_done));
  a.nkv = s.nkv;
  a.nbk = s.nbk;
  a.jbase = n_done / kBlock;
  a.t0 = n_done;
  a.nchunk = cache_update_chunks(s, n_done);
  a.chunk = kCacheChunk;
  if (a.nchunk == 0) return hipSuccess;
  const dim3 grid(a.nchunk, s.BH);
  if (s.D == 128)
    hipLaunchKernelGGL((kv_totals_kernel<128, false>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((kv_totals_kernel<64, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// Projected block means x~ = mean(x_j) P (float64) of a bf16 tensor x [BH][n][D], written to
// out[bh][j][D], streamed through the same ring.
hipError_t launch_pool_stream(const Plan& s, const void* x, const float* P, double* out, int n,
                              int nb, hipStream_t st) {
  TotalsArgs a{};
  a.k = reinterpret_cast<const uint16_t*>(x);
  a.pk = P;
  a.kt = out;
  a.kbh = (size_t)nb * s.D;
  a.kj = (size_t)s.D;
  a.nkv = n;
  a.nbk = nb;
  // about three workgroups per CU over the whole tensor, at least four blocks each
  const long long total = (long long)s.BH * nb;
  a.chunk = (int)std::max(4LL, (total + 767) / 768);
  a.nchunk = (nb + a.chunk - 1) / a.chunk;
  const dim3 grid(a.nchunk, s.BH);
  if (s.D == 128)
    hipLaunchKernelGGL((kv_totals_kernel<128, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((kv_totals_kernel<64, true>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sla
