// Piecewise attention tail (PISA page, "Piecewise Sparse Attention", core algorithm): for
// every query row, the zero-order Taylor terms of the key blocks that were NOT routed to its
// query block, expressed in the row's own softmax frame:
//   y_j = log2(e) tau q . k_bar_j                (base-2 logits, tau = 1/sqrt(d))
//   m_U = running max of y_j over the unrouted blocks j
//   D_U = sum_j n_j 2^(y_j - m_U),  A_U = sum_j 2^(y_j - m_U),  N_U = sum_j 2^(y_j - m_U) Vsum_j
// The exact branch adds its routed blocks and the global first-order term tau (q H_bar) A_U
// and normalises the sum once (sparse.hip, piecewise epilogue).
//
// A workgroup of 8 waves covers 4 query blocks (wave w: rows 32 (w % 2) .. +31 of query
// block w / 2). The centroid tiles (64 centroids each) are walked in order through LDS rings
// filled by loads straight into LDS, pipelined like the exact branch: step s multiplies tile
// s while the value sums of tile s + 1 and the centroids of tile s + 2 load, and one barrier
// per step releases the slots (centroid ring: 3 slots of hi + lo tiles; value-sum ring: 2).
// Each tile is computed transposed, in two 32-centroid halves whose MFMA chains interleave
// with the other half's softmax:
//   S^T (32 centroids x 32 queries) = K_bar Q^T    bf16 MFMA 32x32x16, K_bar as hi + lo
//   O^T (D x 32 queries)          += Vsum^T P^T    f16 MFMA 32x32x16
// The running max may lag the true one while the weights stay below 2^8 (f16). D_U and A_U
// are register sums of the f16-rounded weights that enter the product (n_j = 64 except for a
// partial last block). A wave skips a tile whose every centroid is routed to its query block.
#include "common.h"
#include "kernels.h"

namespace sla {

namespace {


struct TailArgs {
  const void* q;                 // [BH][nq][D] (bf16 or fp32)
  const int32_t* idx;            // [BH][nbq][topk], ascending
  const uint16_t* cent_hi;       // bf16 [BH][npad][D]
  const uint16_t* cent_lo;
  const uint16_t* vsum;          // f16 [BH][npad][D]
  float* tail_m;                 // [BH][nbq * 64]
  float* tail_d;
  float* tail_a;
  float* tail_n;                 // [BH][nbq * 64][D]
  int nq, nbq, nbk, npad, topk, ngroups, nlast;   // nlast: valid tokens of the last key block
};

template <typename T>
__device__ __forceinline__ void load_q8(const T* p, u32x4& hi, u32x4& lo) {
  if constexpr (sizeof(T) == 2) {
    hi = *reinterpret_cast<const u32x4*>(p);
    lo = u32x4{0, 0, 0, 0};
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t hv = pack_bf16(x[2 * e], x[2 * e + 1]);
      hi[e] = hv;
      lo[e] = pack_bf16(x[2 * e] - bf16_lo(hv), x[2 * e + 1] - bf16_hi(hv));
    }
  }
}

constexpr int kTailGroup = 4;                  // query blocks per workgroup

template <typename T, int D>
__global__ __launch_bounds__(128 * kTailGroup, 2) void pisa_tail_kernel(TailArgs a) {
  constexpr bool SPLIT = sizeof(T) == 4;   // fp32 queries: hi + lo bf16 parts
  constexpr int QG = kTailGroup;
  constexpr int NW = 2 * QG;               // waves
  constexpr int KS = D / 16;
  constexpr int CT = D / 32;
  constexpr int CH = D / 8;
  constexpr int TILE = 64 * D;             // elements of one 64-row tile
  constexpr int TP = TILE * 2 / 1024;      // 1-KB pieces of a tile
  constexpr int KPW = TP / NW;             // pieces of each tile array per wave
  static_assert(KPW * NW == TP, "tile pieces split evenly over the waves");
  // centroid ring: slot s holds hi at 2 s TILE and lo at (2 s + 1) TILE; value sums after it
  __shared__ __attribute__((aligned(16))) uint16_t smem[(3 * 2 + 2) * TILE];
  __shared__ uint32_t bits[QG][kMaxKeyBlocks / 32];

  const int bh = blockIdx.x / a.ngroups, grp = blockIdx.x % a.ngroups;
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int wvs = __builtin_amdgcn_readfirstlane(wv);
  const int qb = wv >> 1;
  const int iq = grp * QG + qb;
  const bool active = iq < a.nbq;
  const int qrow0 = iq * kBlock + 32 * (wv & 1);
  const int nwords = a.npad / 32;

  // routed-block bitmap of each query block; centroid slots past nbk are marked as well
  for (int i = t; i < QG * nwords; i += NW * 64) bits[i / nwords][i % nwords] = 0u;
  __syncthreads();
  for (int b = 0; b < QG; ++b) {
    const int ib = grp * QG + b;
    if (ib >= a.nbq) continue;
    const int32_t* sel = a.idx + ((size_t)bh * a.nbq + ib) * a.topk;
    for (int i = t; i < a.topk; i += NW * 64) {
      const int j = sel[i];
      atomicOr(&bits[b][j >> 5], 1u << (j & 31));
    }
    for (int j = a.nbk + t; j < a.npad; j += NW * 64) atomicOr(&bits[b][j >> 5], 1u << (j & 31));
  }
  __syncthreads();   // the bitmap is complete (its LDS atomics have finished)

  // Q^T fragments (B operand): lane column q = qrow0 + l32, channels 16 s + 8 h .. +7
  u32x4 qf[KS], ql[SPLIT ? KS : 1];
  {
    const int q = qrow0 + l32;
    const bool ok = active && q < a.nq;
    const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t)bh * a.nq + (ok ? q : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 hi, lo;
      load_q8<T>(qp + 16 * s + 8 * h, hi, lo);
      qf[s] = ok ? hi : u32x4{0, 0, 0, 0};
      if constexpr (SPLIT) ql[s] = ok ? lo : u32x4{0, 0, 0, 0};
    }
  }

  // Loads into LDS: piece p (1 KB, elements 512 p ..) of a tile; wave w moves pieces
  // KPW w .. KPW w + KPW - 1 of each array. Lane l lands at row 512 p / D + l / CH, physical
  // chunk l % CH, and fetches the logical chunk the swizzle puts there; the offset is p KB
  // plus a lane part (value sums), or p KB plus a lane part XORed with a constant of the
  // piece (centroids at d = 128, whose chunk swizzle sees the low bits of the first row).
  // Rows past nbk read as zero (the buffer bound); j < 0: an empty range, so that every step
  // issues the same number of loads.
  uint32_t klane, vlane;
  {
    const int lr = lane / CH, pc = lane % CH;
    klane = (uint32_t)(lr * D * 2 + ((pc ^ lr) & (CH - 1)) * 16);
    vlane = (uint32_t)(lr * D * 2 + ((pc ^ swzv_f<D>(lr)) & (CH - 1)) * 16);
  }
  const uint16_t* chb = a.cent_hi + (size_t)bh * a.npad * D;
  const uint16_t* clb = a.cent_lo + (size_t)bh * a.npad * D;
  const uint16_t* vxb = a.vsum + (size_t)bh * a.npad * D;
  auto tile_bytes = [&](int j) -> uint32_t {
    return j < 0 ? 0u : (uint32_t)(min(kBlock, a.nbk - j * kBlock) * D * 2);
  };
  auto stage_k = [&](int j, int slot) __attribute__((always_inline)) {
    const size_t row0 = (size_t)(j < 0 ? 0 : j) * kBlock * D;
    const auto rh = make_rsrc(chb + row0, tile_bytes(j));
    const auto rl = make_rsrc(clb + row0, tile_bytes(j));
    const uint32_t dh = lds_addr(smem + 2 * slot * TILE), dl = lds_addr(smem + (2 * slot + 1) * TILE);
#pragma unroll
    for (int u = 0; u < KPW; ++u) {
      const int pp = wvs * KPW + u;
      const uint32_t off = (uint32_t)(pp * 1024) + (klane ^ (D == 128 ? (uint32_t)((pp & 3) << 6) : 0u));
      load_lds16(rh, dh + pp * 1024, off);
      load_lds16(rl, dl + pp * 1024, off);
    }
  };
  auto stage_v = [&](int j, int slot) __attribute__((always_inline)) {
    const auto rv = make_rsrc(vxb + (size_t)(j < 0 ? 0 : j) * kBlock * D, tile_bytes(j));
    const uint32_t dv = lds_addr(smem + (6 + slot) * TILE);
#pragma unroll
    for (int u = 0; u < KPW; ++u) {
      const int pp = wvs * KPW + u;
      load_lds16(rv, dv + pp * 1024, (uint32_t)(pp * 1024) + vlane);
    }
  };

  f32x16 o[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) o[c] = f32x16{};
  float m = kNegBig, dsum = 0.f, asum = 0.f;
  const float qk_scale = kLog2e / sqrtf((float)D);
  const int ntiles = a.npad / kBlock;
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  const f16x2 ones2 = {(_Float16)1.0f, (_Float16)1.0f};

  // One tile for this wave in two 32-centroid halves: Q K_bar^T of half 0, its mask and
  // rescale check; Q K_bar^T of half 1 alongside the weights of half 0; the check of half 1;
  // the value-sum product of half 0 alongside the weights of half 1; then that of half 1.
  u32x4 pf[4];
  auto qk_half = [&](const uint16_t* Kh, const uint16_t* Kl, int mt, f32x16& sh)
                     __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = swz<D>(32 * mt + l32, 16 * ks + 8 * h);
      const u32x4 ah = *reinterpret_cast<const u32x4*>(&Kh[off]);
      const u32x4 al = *reinterpret_cast<const u32x4*>(&Kl[off]);
      sh = mfma_bf16(ah, qf[ks], sh);
      sh = mfma_bf16(al, qf[ks], sh);
      if constexpr (SPLIT) sh = mfma_bf16(ah, ql[ks], sh);
    }
  };
  // routed centroids and padding -> -inf; rescale when the half's max passes m + slack
  auto check_half = [&](f32x16& sh, int mt, uint64_t mask) __attribute__((always_inline)) {
    float r = kNegBig;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int jl = 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
      sh[e] = ((mask >> jl) & 1u) ? -INFINITY : sh[e];
      r = fmaxf(r, sh[e]);
    }
    r = fmaxf(r, swap_halves(r)) * qk_scale;
    if (__ballot(r > m + kRescaleSlack)) {
      const float mn = fmaxf(m, r);
      const float corr = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
      for (int c = 0; c < CT; ++c) o[c] *= corr;
      dsum *= corr;
      asum *= corr;
      if (mt == 1) {   // the weights of half 0 are formed but not yet multiplied
        const _Float16 ch = (_Float16)corr;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          pf[kk] = __builtin_bit_cast(u32x4, __builtin_bit_cast(f16x8, pf[kk]) * ch);
      }
      m = mn;
    }
  };
  // weights of one half (P^T fragments pf[2 mt], pf[2 mt + 1]) and their sums: fragment hh
  // holds centroids 32 mt + 16 hh + 8 (i / 4) + 4 h + i % 4
  auto exp_half = [&](const f32x16& sh, int mt, int tt) __attribute__((always_inline)) {
    float ps = 0.f, pl = 0.f;   // plain sum, and the part that belongs to the last block
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int e = 8 * hh + 2 * e2;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sh[e], qk_scale, -m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sh[e + 1], qk_scale, -m));
        const uint32_t pk = pack_f16(p0, p1);
        pf[2 * mt + hh][e2] = pk;
        ps = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), ones2, ps, false);
        const int j = tt * kBlock + 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
        const f16x2 pv = __builtin_bit_cast(f16x2, pk);
        pl += (j == a.nbk - 1 ? (float)pv[0] : 0.f) + (j + 1 == a.nbk - 1 ? (float)pv[1] : 0.f);
      }
    asum += ps;
    dsum += (float)kBlock * ps - (float)(kBlock - a.nlast) * pl;
  };
  // O^T += Vsum^T P^T over the 32 centroids of one half
  auto pv_half = [&](const uint16_t* Vt, int mt) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 2 * mt; kk < 2 * mt + 2; ++kk) {
#pragma unroll
      for (int c = 0; c < CT; ++c) o[c] = mfma_f16(vt_frag<D>(Vt, 32 * c, 16 * kk), pf[kk], o[c]);
    }
  };
  auto compute_tile = [&](int kslot, int vslot, int tt, uint64_t mask)
                          __attribute__((always_inline)) {
    const uint16_t* Kh = smem + 2 * kslot * TILE;
    const uint16_t* Kl = Kh + TILE;
    const uint16_t* Vt = smem + (6 + vslot) * TILE;
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    qk_half(Kh, Kl, 0, s0);
    check_half(s0, 0, mask);
    qk_half(Kh, Kl, 1, s1);
    exp_half(s0, 0, tt);
    check_half(s1, 1, mask);
    pv_half(Vt, 0);
    exp_half(s1, 1, tt);
    pv_half(Vt, 1);
  };

  stage_k(0, 0);
  stage_k(ntiles > 1 ? 1 : -1, 1);
  stage_v(0, 0);
  barrier_vmem_n<0>();
  int ks = 0, vs = 0;
  for (int tt = 0; tt < ntiles; ++tt) {
    stage_v(tt + 1 < ntiles ? tt + 1 : -1, vs ^ 1);
    stage_k(tt + 2 < ntiles ? tt + 2 : -1, ks == 0 ? 2 : ks - 1);
    const uint64_t mask = ((uint64_t)bits[qb][2 * tt + 1] << 32) | bits[qb][2 * tt];
    if (active && mask != ~0ull) compute_tile(ks, vs, tt, mask);
    barrier_vmem_n<2 * KPW>();   // V(tt + 1) and K(tt + 1) landed; this step's slots are free
    ks = ks == 2 ? 0 : ks + 1;
    vs ^= 1;
  }
  wait_vmem();   // no load into LDS outlives the workgroup
  if (!active) return;

  // O^T layout: lane column q, rows 32 c + 8 g + 4 h + e in element 4 g + e
  const int q = qrow0 + l32;
  if (q >= a.nq) return;
  const size_t row = (size_t)bh * a.nbq * kBlock + q;
  float* dst = a.tail_n + row * D;
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<f32x4*>(dst + 32 * c + 8 * g + 4 * h) =
          f32x4{o[c][4 * g], o[c][4 * g + 1], o[c][4 * g + 2], o[c][4 * g + 3]};
  dsum += swap_halves(dsum);    // each lane half summed 16 of every 32 centroids
  asum += swap_halves(asum);
  if (h == 0) {
    a.tail_m[row] = m;
    a.tail_d[row] = dsum;
    a.tail_a[row] = asum;
  }
}

template <typename T, int D>
hipError_t launch_tail_T(const Plan& s, const void* q, const int32_t* idx, char* ws,
                         hipStream_t st) {
  TailArgs a;
  a.q = q;
  a.idx = idx;
  a.cent_hi = reinterpret_cast<const uint16_t*>(ws + s.cent_hi);
  a.cent_lo = reinterpret_cast<const uint16_t*>(ws + s.cent_lo);
  a.vsum = reinterpret_cast<const uint16_t*>(ws + s.vsum);
  a.tail_m = reinterpret_cast<float*>(ws + s.tail_m);
  a.tail_d = reinterpret_cast<float*>(ws + s.tail_d);
  a.tail_a = reinterpret_cast<float*>(ws + s.tail_a);
  a.tail_n = reinterpret_cast<float*>(ws + s.tail_n);
  a.nq = s.nq; a.nbq = s.nbq; a.nbk = s.nbk; a.npad = s.npad; a.topk = s.k;
  a.nlast = s.nkv - (s.nbk - 1) * kBlock;
  a.ngroups = (s.nbq + kTailGroup - 1) / kTailGroup;
  hipLaunchKernelGGL((pisa_tail_kernel<T, D>), dim3(s.BH * a.ngroups), dim3(128 * kTailGroup), 0,
                     st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pisa_tail(const Plan& s, const void* q, const int32_t* idx, char* ws,
                            hipStream_t st) {
  if (s.in_bf16) {
    if (s.D == 128) return launch_tail_T<uint16_t, 128>(s, q, idx, ws, st);
    return launch_tail_T<uint16_t, 64>(s, q, idx, ws, st);
  }
  if (s.D == 128) return launch_tail_T<float, 128>(s, q, idx, ws, st);
  return launch_tail_T<float, 64>(s, q, idx, ws, st);
}

}  // namespace sla
