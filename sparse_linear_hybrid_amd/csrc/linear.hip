// Linear branch (SALAD page, section 2: ReLU kernel feature map with linear cost; SPLA
// page, section 2.2: the linear term over the unselected blocks equals the global linear
// term minus the selected blocks' term).
//
// kv_summary:  one pass over K and V. For every key block j: S_j = phi(K_j)^T V_j (d x d,
//              bf16 MFMA, fp32 accumulate, stored bf16 as S_j^T[c][r]), z_j = sum phi(K_j)
//              (fp32), the projected block mean of K (float64, for the router) and an f16
//              copy of V for the sparse branch's P.V. The next block's loads are in flight
//              while a block is processed. Per-chunk fp32 partial totals are written for a
//              fixed-order reduction (no atomics).
// reduce:      S_tot = sum of the partials, z_tot likewise.
// complement:  per query block i, S_c(i) = S_tot - sum_{j in sel(i)} S_j (an MFMA product of
//              the 0/1 selection matrix with the stacked S_j) and z_c(i) likewise; an
//              all-blocks selection gives exactly 0.
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
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ Pk,
    double* __restrict__ kt, uint16_t* __restrict__ v16, uint16_t* __restrict__ sblk,
    float* __restrict__ zblk, float* __restrict__ spart, float* __restrict__ zpart, int nkv,
    int nbk) {
  constexpr int LS = D + 8;                  // padded LDS row (elements)
  constexpr int TPR = D / 8, RPP = 256 / TPR;
  constexpr int CPT = 64 * TPR / 256;        // 16-byte chunks per thread per tensor
  constexpr int NT = D / 32;                 // 32-wide tiles per dimension
  constexpr int TILES_PER_WAVE = NT * NT / 4;
  constexpr int EPC = sizeof(T) == 2 ? 1 : 2;   // 16-byte loads per 8-element chunk
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * LS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[64 * LS];
  __shared__ double pool_lds[RPP * D];
  __shared__ double means[kSummaryChunk][D];

  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int j0 = chunk * kSummaryChunk, j1 = min(j0 + kSummaryChunk, nbk);
  const T* kb = k + (size_t)bh * nkv * D;
  const T* vb = v + (size_t)bh * nkv * D;
  const int mt = (NT == 4) ? w : (w >> 1);   // this wave's 32-row tile of S_j (rows r)

  f32x16 part[TILES_PER_WAVE];
#pragma unroll
  for (int u = 0; u < TILES_PER_WAVE; ++u) part[u] = f32x16{};
  float zp = 0.f;

  // raw prefetch registers for one block (rows beyond n_kv read row n_kv-1, zeroed later)
  u32x4 kraw[CPT * EPC], vraw[CPT * EPC];
  auto load_block = [&](int j) {
    const int row0 = j * kBlock;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int cidx = t + 256 * u;
      const int r = cidx / TPR, c8 = cidx % TPR;
      const size_t off = (size_t)min(row0 + r, nkv - 1) * D + c8 * 8;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        kraw[u * EPC + e] = *reinterpret_cast<const u32x4*>(kb + off + 4 * e);
        vraw[u * EPC + e] = *reinterpret_cast<const u32x4*>(vb + off + 4 * e);
      }
    }
  };
  if (j0 < j1) load_block(j0);

  for (int j = j0; j < j1; ++j) {
    const int row0 = j * kBlock;
    const int nrows = min(kBlock, nkv - row0);
    double pacc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pacc[e] = 0.0;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int cidx = t + 256 * u;
      const int r = cidx / TPR, c8 = cidx % TPR;
      const bool ok = r < nrows;
      float kf[8], vf[8];
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[2 * e] = bf16_lo(kraw[u][e]); kf[2 * e + 1] = bf16_hi(kraw[u][e]);
          vf[2 * e] = bf16_lo(vraw[u][e]); vf[2 * e + 1] = bf16_hi(vraw[u][e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[e] = __uint_as_float(kraw[2 * u][e]); kf[4 + e] = __uint_as_float(kraw[2 * u + 1][e]);
          vf[e] = __uint_as_float(vraw[2 * u][e]); vf[4 + e] = __uint_as_float(vraw[2 * u + 1][e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kf[e] = ok ? kf[e] : 0.f;
        vf[e] = ok ? vf[e] : 0.f;
        pacc[e] += (double)kf[e];
      }
      u32x4 kw, vw, v16w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kw[e] = pack_bf16(kf[2 * e], kf[2 * e + 1]);
        vw[e] = pack_bf16(vf[2 * e], vf[2 * e + 1]);
        v16w[e] = f16_sat_pack(vf[2 * e], vf[2 * e + 1]);
      }
      *reinterpret_cast<u32x4*>(&Ks[r * LS + c8 * 8]) = kw;
      *reinterpret_cast<u32x4*>(&Vs[r * LS + c8 * 8]) = vw;
      *reinterpret_cast<u32x4*>(&v16[((size_t)bh * nbk * kBlock + row0 + r) * D + c8 * 8]) = v16w;
    }
    {
      const int cg = t % TPR, r = t / TPR;
#pragma unroll
      for (int e = 0; e < 8; ++e) pool_lds[r * D + cg * 8 + e] = pacc[e];
    }
    if (j + 1 < j1) load_block(j + 1);   // in flight during this block's compute
    __syncthreads();
    if (t < D) {
      double sm = 0.0;
      for (int rr = 0; rr < RPP; ++rr) sm += pool_lds[rr * D + t];
      means[j - j0][t] = sm / (double)nrows;
    }
    // S_j[r][c] = sum_m relu(K[m][r]) V[m][c]: M = r, N = c, reduction over the 64 keys;
    // z_j[r] = sum_m relu(K[m][r]) from the same A fragments.
    u32x4 af[4];
    float zl = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      af[s4] = relu_bf16x8(frag_tr(Ks, LS, 32 * mt, 16 * s4));
#pragma unroll
      for (int e = 0; e < 4; ++e) zl += bf16_lo(af[s4][e]) + bf16_hi(af[s4][e]);
    }
    zl += swap_halves(zl);
    if (((NT == 4) || (w & 1) == 0) && h == 0) {
      zblk[((size_t)bh * nbk + j) * D + 32 * mt + l32] = zl;
    }
    zp += zl;
#pragma unroll
    for (int u = 0; u < TILES_PER_WAVE; ++u) {
      const int nt = (NT == 4) ? u : (w & 1);
      f32x16 acc = {};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) acc = mfma_bf16(af[s4], frag_tr(Vs, LS, 32 * nt, 16 * s4), acc);
      part[u] += acc;
      // store S_j^T[c][r] (bf16): lane column c = 32 nt + l32, rows r in runs of 4
      const int c = 32 * nt + l32;
      uint16_t* dst = sblk + (((size_t)bh * nbk + j) * D + c) * D;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 32 * mt + 8 * q + 4 * h;
        *reinterpret_cast<u32x2*>(dst + r) =
            u32x2{pack_bf16(acc[4 * q], acc[4 * q + 1]), pack_bf16(acc[4 * q + 2], acc[4 * q + 3])};
      }
    }
    __syncthreads();   // LDS tiles and pool_lds are rewritten by the next block
  }
  // projected pooled K for the router: k~ = mean @ P_k (float64)
  for (int b = t / D; b < j1 - j0; b += 256 / D) {
    const int c = t % D;
    double acc = 0.0;
    for (int r = 0; r < D; ++r) acc = fma(means[b][r], (double)Pk[r * D + c], acc);
    kt[((size_t)bh * nbk + j0 + b) * D + c] = acc;
  }
  // chunk partial totals (fp32, layout [c][r])
#pragma unroll
  for (int u = 0; u < TILES_PER_WAVE; ++u) {
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
  if (((NT == 4) || (w & 1) == 0) && h == 0)
    zpart[((size_t)bh * gridDim.x + chunk) * D + 32 * mt + l32] = zp;
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

// Complement, summary part: for a tile of CQ query blocks and CN columns n of the d x d
// summary, C[n][i] = sum_j M[i][j] S_j[n] with M the 0/1 selection matrix, computed as an
// MFMA product over steps of CK key blocks (M is exact in bf16), then S_c = S_tot - C.
// The tile's selections are first scattered into an LDS bitmap (one bit per query block and
// key block of a window of WIN key blocks) together with a per-step occupancy bitmap, so
// steps that no query block of the tile selects are skipped; the summaries of the next
// occupied step are prefetched into registers while the current step runs. Query tiles
// sharing a column slice are consecutive workgroups (same XCD), so each S_j slice comes
// from HBM about once.
constexpr int CQ = 128;    // query blocks per workgroup
constexpr int CN = 128;    // summary columns per workgroup
constexpr int CK = 32;     // key blocks per step (two 16-deep MFMA reductions)
constexpr int WIN = 2048;  // key blocks per bitmap window

template <int D>
__global__ __launch_bounds__(256) void complement_kernel(
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ sblk,
    const float* __restrict__ stot, uint16_t* __restrict__ sc, int nbq, int nbk, int k,
    int nqt, int total) {
  constexpr int NCS = D * D / CN;      // column slices per (batch, head)
  constexpr int SS = CN + 8;           // padded LDS row of staged summaries
  constexpr int WW = WIN / 32 + 1;     // bitmap words per query block (+1: no bank conflicts)
  constexpr int NSTEP = WIN / CK;      // steps per window
  __shared__ uint32_t bits[CQ * WW];
  __shared__ uint32_t occ[NSTEP / 32];
  __shared__ __attribute__((aligned(16))) uint16_t Ss[2][CK * SS];

  const int wid = xcd_remap(blockIdx.x, total);
  const int qt = wid % nqt;
  const int cs = (wid / nqt) % NCS;
  const int bh = wid / (nqt * NCS);
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const size_t col0 = (size_t)cs * CN;

  if (k >= nbk) {   // every block selected: the complement is empty, exactly zero
    for (int e = t; e < CQ * CN / 8; e += 256) {
      const int il = e / (CN / 8), c8 = e % (CN / 8);
      const int i = qt * CQ + il;
      if (i < nbq)
        *reinterpret_cast<u32x4*>(sc + ((size_t)bh * nbq + i) * D * D + col0 + c8 * 8) =
            u32x4{0, 0, 0, 0};
    }
    return;
  }
  const int nq_tile = min(CQ, nbq - qt * CQ);
  const int32_t* sel0 = idx + ((size_t)bh * nbq + qt * CQ) * k;
  // staging: thread t loads summary rows t/16 and 16 + t/16 of a step, 8 columns at (t%16)*8
  const int sr = t >> 4, sc8 = t & 15;
  const uint16_t* sbase = sblk + (size_t)bh * nbk * D * D + col0 + sc8 * 8;

  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  for (int win0 = 0; win0 < nbk; win0 += WIN) {
    for (int e = t; e < CQ * WW; e += 256) bits[e] = 0u;
    if (t < NSTEP / 32) occ[t] = 0u;
    __syncthreads();
    for (int e = t; e < nq_tile * k; e += 256) {
      const int j = sel0[e] - win0;
      if (j >= 0 && j < WIN) {
        const int il = e / k;
        atomicOr(&bits[il * WW + (j >> 5)], 1u << (j & 31));
        atomicOr(&occ[(j / CK) >> 5], 1u << ((j / CK) & 31));
      }
    }
    __syncthreads();
    // occupied steps of this window, in order
    auto next_step = [&](int from) {
      for (int st = from; st < NSTEP; ++st)
        if ((occ[st >> 5] >> (st & 31)) & 1u) return st;
      return NSTEP;
    };
    auto load_step = [&](int st, u32x4& r0, u32x4& r1) {
      const int ja = win0 + st * CK + sr, jb = ja + 16;
      r0 = ja < nbk ? *reinterpret_cast<const u32x4*>(sbase + (size_t)ja * D * D) : u32x4{0, 0, 0, 0};
      r1 = jb < nbk ? *reinterpret_cast<const u32x4*>(sbase + (size_t)jb * D * D) : u32x4{0, 0, 0, 0};
    };
    int st = next_step(0);
    u32x4 r0, r1;
    if (st < NSTEP) load_step(st, r0, r1);
    int buf = 0;
    while (st < NSTEP) {
      *reinterpret_cast<u32x4*>(&Ss[buf][sr * SS + sc8 * 8]) = r0;
      *reinterpret_cast<u32x4*>(&Ss[buf][(sr + 16) * SS + sc8 * 8]) = r1;
      __syncthreads();
      const int nst = next_step(st + 1);
      if (nst < NSTEP) load_step(nst, r0, r1);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x4 a = frag_tr(Ss[buf], SS, 32 * w, 16 * kk);
        const int bit0 = st * CK + 16 * kk + 8 * h;          // first key block of the slot
#pragma unroll
        for (int tq = 0; tq < 4; ++tq) {
          const uint32_t word = bits[(32 * tq + l32) * WW + (bit0 >> 5)];
          const uint32_t m8 = (word >> (bit0 & 31)) & 0xffu;
          u32x4 b;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            b[e] = ((m8 >> (2 * e)) & 1u ? 0x3F80u : 0u) | ((m8 >> (2 * e + 1)) & 1u ? 0x3F800000u : 0u);
          acc[tq] = mfma_bf16(a, b, acc[tq]);
        }
      }
      buf ^= 1;
      st = nst;
    }
    __syncthreads();   // bitmap reuse in the next window
  }
  // S_c = S_tot - C; lane column = query block, rows = 4-column runs
#pragma unroll
  for (int tq = 0; tq < 4; ++tq) {
    const int i = qt * CQ + 32 * tq + l32;
    if (i >= nbq) continue;
    uint16_t* dst = sc + ((size_t)bh * nbq + i) * D * D + col0;
    const float* tot = stot + (size_t)bh * D * D + col0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = 32 * w + 8 * g + 4 * h;
      const f32x4 tv = *reinterpret_cast<const f32x4*>(tot + n);
      *reinterpret_cast<u32x2*>(dst + n) =
          u32x2{pack_bf16(tv[0] - acc[tq][4 * g], tv[1] - acc[tq][4 * g + 1]),
                pack_bf16(tv[2] - acc[tq][4 * g + 2], tv[3] - acc[tq][4 * g + 3])};
    }
  }
}

// Complement, normaliser part: z_c(i) = z_tot - sum_{j in sel(i)} z_j (fp32, fixed order).
template <int D>
__global__ __launch_bounds__(D) void complement_z_kernel(const int32_t* __restrict__ idx,
                                                         const float* __restrict__ zblk,
                                                         const float* __restrict__ ztot,
                                                         float* __restrict__ zc, int nbq, int nbk,
                                                         int k) {
  const int i = blockIdx.x, bh = blockIdx.y, r = threadIdx.x;
  float* out = zc + ((size_t)bh * nbq + i) * D;
  if (k >= nbk) {
    out[r] = 0.f;
    return;
  }
  const int32_t* sel = idx + ((size_t)bh * nbq + i) * k;
  float z = 0.f;
  for (int s = 0; s < k; ++s) z += zblk[((size_t)bh * nbk + sel[s]) * D + r];
  out[r] = ztot[(size_t)bh * D + r] - z;
}

template <int D>
static hipError_t launch_kv_summary_T(const Plan& s, const void* k, const void* v, const float* pk,
                                      char* ws, hipStream_t st) {
  double* kt = reinterpret_cast<double*>(ws + s.kt);
  uint16_t* v16 = reinterpret_cast<uint16_t*>(ws + s.v16);
  uint16_t* sblk = reinterpret_cast<uint16_t*>(ws + s.sblk);
  float* zblk = reinterpret_cast<float*>(ws + s.zblk);
  float* spart = reinterpret_cast<float*>(ws + s.spart);
  float* zpart = reinterpret_cast<float*>(ws + s.zpart);
  const dim3 grid(s.nchunk, s.BH);
  if (s.in_bf16)
    hipLaunchKernelGGL((kv_summary_kernel<uint16_t, D>), grid, dim3(256), 0, st,
                       (const uint16_t*)k, (const uint16_t*)v, pk, kt, v16, sblk, zblk, spart,
                       zpart, s.nkv, s.nbk);
  else
    hipLaunchKernelGGL((kv_summary_kernel<float, D>), grid, dim3(256), 0, st, (const float*)k,
                       (const float*)v, pk, kt, v16, sblk, zblk, spart, zpart, s.nkv, s.nbk);
  hipLaunchKernelGGL((reduce_totals_kernel<D>), dim3(D * D / 256, s.BH), dim3(256), 0, st, spart,
                     zpart, reinterpret_cast<float*>(ws + s.stot),
                     reinterpret_cast<float*>(ws + s.ztot), s.nchunk);
  return hipGetLastError();
}

hipError_t launch_kv_summary(const Plan& s, const void* k, const void* v, const float* pk,
                             char* ws, hipStream_t st) {
  if (s.D == 128) return launch_kv_summary_T<128>(s, k, v, pk, ws, st);
  return launch_kv_summary_T<64>(s, k, v, pk, ws, st);
}

hipError_t launch_complement(const Plan& s, const int32_t* idx, char* ws, hipStream_t st) {
  const int nqt = (s.nbq + CQ - 1) / CQ;
  const int ncs = s.D * s.D / CN;
  const int total = s.BH * ncs * nqt;
  auto go = [&](auto kern, auto zkern) {
    hipLaunchKernelGGL(kern, dim3(total), dim3(256), 0, st, idx,
                       reinterpret_cast<const uint16_t*>(ws + s.sblk),
                       reinterpret_cast<const float*>(ws + s.stot),
                       reinterpret_cast<uint16_t*>(ws + s.sc), s.nbq, s.nbk, s.k, nqt, total);
    hipLaunchKernelGGL(zkern, dim3(s.nbq, s.BH), dim3(s.D), 0, st, idx,
                       reinterpret_cast<const float*>(ws + s.zblk),
                       reinterpret_cast<const float*>(ws + s.ztot),
                       reinterpret_cast<float*>(ws + s.zc), s.nbq, s.nbk, s.k);
  };
  if (s.D == 128) go(complement_kernel<128>, complement_z_kernel<128>);
  else go(complement_kernel<64>, complement_z_kernel<64>);
  return hipGetLastError();
}

}  // namespace sla
