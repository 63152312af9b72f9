// Piecewise attention tail (PISA page, "Piecewise Sparse Attention", core algorithm): for
// every query row, the zero-order Taylor terms of the key blocks that were NOT routed to its
// query block, expressed in the row's own softmax frame:
//   y_j = log2(e) tau q . k_bar_j                (base-2 logits, tau = 1/sqrt(d))
//   m_U = running max of y_j over the unrouted blocks j
//   D_U = sum_j n_j 2^(y_j - m_U),  A_U = sum_j 2^(y_j - m_U),  N_U = sum_j 2^(y_j - m_U) Vsum_j
// The exact branch adds its routed blocks and the global first-order term tau (q H_bar) A_U
// and normalises the sum once (sparse.hip, piecewise epilogue).
//
// A workgroup of 4 waves covers 2 query blocks (wave w: rows 32 (w % 2) .. +31 of query
// block w / 2). The centroids are walked in tiles of 64 staged through LDS, computed
// transposed like the exact branch, one 32-centroid half at a time (the running max is
// updated per half):
//   S^T (32 centroids x 32 queries) = K_bar Q^T    bf16 MFMA 32x32x16, K_bar as hi + lo
//   O^T (D x 32 queries)          += Vsum^T P^T    f16 MFMA 32x32x16
// D_U and A_U are register sums of the f16-rounded weights that enter the product (n_j = 64
// except for a partial last block).
#include "common.h"
#include "kernels.h"

namespace sla {

namespace {

constexpr float kLog2eT = 1.4426950408889634f;
constexpr float kNegBigT = -1.0e30f;   // finite "minus infinity" for the running max

struct TailArgs {
  const void* q;                 // [BH][nq][D] (bf16 or fp32)
  const int32_t* idx;            // [BH][nbq][topk], ascending
  const uint16_t* cent_hi;       // bf16 [BH][npad][D]
  const uint16_t* cent_lo;
  const uint16_t* vsum;          // f16 [BH][D][npad]
  float* tail_m;                 // [BH][nbq * 64]
  float* tail_d;
  float* tail_a;
  float* tail_n;                 // [BH][nbq * 64][D]
  int nq, nbq, nbk, npad, topk, ngroups, nlast;   // nlast: valid tokens of the last key block
};

// Swizzled offset of (row, col) in a 64 x D bf16 centroid tile: 16-byte chunk index XOR row.
template <int D>
__device__ __forceinline__ int cswz(int row, int col) {
  constexpr int CH = D / 8;
  return row * D + ((((col >> 3) ^ row) & (CH - 1)) << 3) + (col & 7);
}

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

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void pisa_tail_kernel(TailArgs a) {
  constexpr bool SPLIT = sizeof(T) == 4;   // fp32 queries: hi + lo bf16 parts
  constexpr int KS = D / 16;
  constexpr int CT = D / 32;
  constexpr int CH = D / 8;
  constexpr int VR = 64 + 4;               // Vsum^T LDS row: 136 bytes (8-byte reads spread)
  constexpr int KCPT = 64 * CH / 256;      // 16-byte centroid chunks per thread per array
  constexpr int VCPT = D * 8 / 256;        // 16-byte value-sum chunks per thread
  static_assert(64 * CH % 256 == 0 && D * 8 % 256 == 0, "tile staging split");
  __shared__ __attribute__((aligned(16))) uint16_t khi[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t klo[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vx[D * VR];
  __shared__ uint32_t bits[2][kMaxKeyBlocks / 32];

  const int bh = blockIdx.x / a.ngroups, grp = blockIdx.x % a.ngroups;
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int qb = wv >> 1;
  const int iq = grp * 2 + qb;
  const bool active = iq < a.nbq;
  const int qrow0 = iq * kBlock + 32 * (wv & 1);
  const int nwords = a.npad / 32;

  // routed-block bitmap of each query block; centroid slots past nbk are marked as well
  for (int i = t; i < 2 * nwords; i += 256) bits[i / nwords][i % nwords] = 0u;
  __syncthreads();
  for (int b = 0; b < 2; ++b) {
    const int ib = grp * 2 + b;
    if (ib >= a.nbq) continue;
    const int32_t* sel = a.idx + ((size_t)bh * a.nbq + ib) * a.topk;
    for (int i = t; i < a.topk; i += 256) {
      const int j = sel[i];
      atomicOr(&bits[b][j >> 5], 1u << (j & 31));
    }
    for (int j = a.nbk + t; j < a.npad; j += 256) atomicOr(&bits[b][j >> 5], 1u << (j & 31));
  }

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

  // tile staging: global -> registers -> LDS; centroid rows and value columns past nbk are
  // zeroed (their memory is allocated but never written)
  const uint16_t* chb = a.cent_hi + (size_t)bh * a.npad * D;
  const uint16_t* clb = a.cent_lo + (size_t)bh * a.npad * D;
  const uint16_t* vxb = a.vsum + (size_t)bh * D * a.npad;
  u32x4 rh[KCPT], rl[KCPT], rv[VCPT];
  auto load_tile = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < KCPT; ++u) {
      const int id = t + 256 * u;
      const int r = id / CH, c = id % CH;
      const bool ok = j0 + r < a.nbk;
      const size_t off = (size_t)(ok ? j0 + r : 0) * D + c * 8;
      rh[u] = ok ? *reinterpret_cast<const u32x4*>(chb + off) : u32x4{0, 0, 0, 0};
      rl[u] = ok ? *reinterpret_cast<const u32x4*>(clb + off) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < VCPT; ++u) {
      const int id = t + 256 * u;
      const int r = id / 8, g = id % 8;
      const int j = j0 + 8 * g;
      u32x4 w = j < a.nbk ? *reinterpret_cast<const u32x4*>(vxb + (size_t)r * a.npad + j)
                          : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t keep_lo = j + 2 * e < a.nbk ? 0xffffu : 0u;
        const uint32_t keep_hi = j + 2 * e + 1 < a.nbk ? 0xffff0000u : 0u;
        w[e] &= keep_lo | keep_hi;
      }
      rv[u] = w;
    }
  };
  auto store_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < KCPT; ++u) {
      const int id = t + 256 * u;
      const int r = id / CH, c = id % CH;
      *reinterpret_cast<u32x4*>(&khi[cswz<D>(r, c * 8)]) = rh[u];
      *reinterpret_cast<u32x4*>(&klo[cswz<D>(r, c * 8)]) = rl[u];
    }
#pragma unroll
    for (int u = 0; u < VCPT; ++u) {
      const int id = t + 256 * u;
      const int r = id / 8, g = id % 8;
      uint16_t* dst = &vx[r * VR + 8 * g];     // 8-byte aligned rows
      *reinterpret_cast<u32x2*>(dst) = u32x2{rv[u][0], rv[u][1]};
      *reinterpret_cast<u32x2*>(dst + 4) = u32x2{rv[u][2], rv[u][3]};
    }
  };

  f32x16 o[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) o[c] = f32x16{};
  float m = kNegBigT, dsum = 0.f, asum = 0.f;
  const float qk_scale = kLog2eT / sqrtf((float)D);
  const int ntiles = a.npad / kBlock;
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 ones2 = {(_Float16)1.0f, (_Float16)1.0f};

  load_tile(0);
  store_tile();
  __syncthreads();   // bitmap and tile 0 visible
  for (int tt = 0; tt < ntiles; ++tt) {
    if (tt + 1 < ntiles) load_tile((tt + 1) * kBlock);
    if (active) {
      const uint64_t mask = ((uint64_t)bits[qb][2 * tt + 1] << 32) | bits[qb][2 * tt];
#pragma unroll 1
      for (int mt = 0; mt < 2; ++mt) {
        f32x16 sh = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int off = cswz<D>(32 * mt + l32, 16 * ks + 8 * h);
          const u32x4 ah = *reinterpret_cast<const u32x4*>(&khi[off]);
          const u32x4 al = *reinterpret_cast<const u32x4*>(&klo[off]);
          sh = mfma_bf16(ah, qf[ks], sh);
          sh = mfma_bf16(al, qf[ks], sh);
          if constexpr (SPLIT) sh = mfma_bf16(ah, ql[ks], sh);
        }
        // routed blocks and padding -> -inf; max of this lane's query over the half
        float r = kNegBigT;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int jl = 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
          sh[e] = ((mask >> jl) & 1u) ? -INFINITY : sh[e];
          r = fmaxf(r, sh[e]);
        }
        r = fmaxf(r, swap_halves(r)) * qk_scale;
        if (__ballot(r > m)) {
          const float mn = fmaxf(m, r);
          const float corr = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
          for (int c = 0; c < CT; ++c) o[c] *= corr;
          dsum *= corr;
          asum *= corr;
          m = mn;
        }
        // P^T fragments: fragment hh holds centroids 32 mt + 16 hh + 8 (i / 4) + 4 h + i % 4;
        // the row sums add the f16-rounded weights
        u32x4 pf[2];
        float ps = 0.f, pl = 0.f;   // plain sum, and the part that belongs to the last block
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const int e = 8 * hh + 2 * e2;
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sh[e], qk_scale, -m));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sh[e + 1], qk_scale, -m));
            const uint32_t pk = pack_f16(p0, p1);
            pf[hh][e2] = pk;
            ps = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), ones2, ps, false);
            const int j = tt * kBlock + 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
            const f16x2 pv = __builtin_bit_cast(f16x2, pk);
            pl += (j == a.nbk - 1 ? (float)pv[0] : 0.f) + (j + 1 == a.nbk - 1 ? (float)pv[1] : 0.f);
          }
        asum += ps;
        dsum += (float)kBlock * ps - (float)(kBlock - a.nlast) * pl;
        // O^T += Vsum^T P^T; the A operand row c, reduction slot 8 h + i takes centroid
        // 16 kk + 8 (i / 4) + 4 h + i % 4, matching the P^T fragment
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int kk = 2 * mt + hh;
#pragma unroll
          for (int c = 0; c < CT; ++c) {
            const uint16_t* row = &vx[(32 * c + l32) * VR + 16 * kk + 4 * h];
            const u32x2 v0 = *reinterpret_cast<const u32x2*>(row);
            const u32x2 v1 = *reinterpret_cast<const u32x2*>(row + 8);
            o[c] = mfma_f16(u32x4{v0[0], v0[1], v1[0], v1[1]}, pf[hh], o[c]);
          }
        }
      }
    }
    if (tt + 1 < ntiles) {
      __syncthreads();   // every wave is done with tile tt
      store_tile();
      __syncthreads();   // tile tt + 1 visible
    }
  }
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
  a.ngroups = (s.nbq + 1) / 2;
  hipLaunchKernelGGL((pisa_tail_kernel<T, D>), dim3(s.BH * a.ngroups), dim3(256), 0, st, a);
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
