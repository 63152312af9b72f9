// Sparse branch (SLA2 page, sections 1 and 2.B: exact softmax attention on the routed key
// blocks) with the linear-branch apply and the alpha mix (section 2.A) fused into the
// epilogue.
//
// One workgroup of two waves per (batch*head, query block). Both waves hold all 64 query
// rows; wave w takes keys 32w .. 32w+31 of every routed 64-key tile, so each K/V element
// staged in LDS is read by exactly one wave. Each wave keeps its own running max, row sum
// and output partial (an online softmax over its half of the keys); the two partials are
// merged once at the end.
//
// Everything is computed transposed so that no register shuffles are needed:
//   S^T (keys x queries) = K Q^T            bf16 MFMA 32x32x16, fp32 accumulate
//   O^T (channels x queries) += V^T P^T     f16 MFMA 32x32x16 (P in [0, 2^8], f16 keeps
//                                            11 significant bits), fp32 accumulate
// The S^T accumulator layout (lane = query column, 16 key rows per lane) is exactly the
// B-operand layout P^T needs, up to a fixed permutation of the keys inside each 16-key
// step; the V^T operand is read from the row-major V tile with transposing LDS reads in the
// same permuted key order.
//
// Epilogue: O_s = O / l; O_l^T = S_c^T phi(Q)^T / (phi(Q) . z_c + eps) on bf16 MFMA (the
// phi(Q)^T operand is the register-resident Q fragment with ReLU applied);
// O = alpha O_s + (1 - alpha) O_l.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace sla {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;      // finite "minus infinity" for running maxima
constexpr float kRescaleSlack = 8.0f;    // keep a stale max while p <= 2^8

// P^T-matched V^T fragment: lane row x0 + lane%32; reduction slot e holds key
// k0 + 4h + e (e < 4) or k0 + 8 + 4h + (e - 4) (e >= 4), h = lane / 32.
__device__ __forceinline__ u32x4 frag_tr_perm(const uint16_t* M, int stride, int x0, int k0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, L = lane & 15;
  const int row = k0 + 4 * (g >> 1) + (L >> 2);
  const int col = x0 + 16 * (g & 1) + 4 * (L & 3);
  const u32x2 lo = lds_read_tr16(M + row * stride + col);
  const u32x2 hi = lds_read_tr16(M + (row + 8) * stride + col);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

struct SparseArgs {
  const void* q;
  const void* k;
  const uint16_t* v16;     // f16 [BH][nbk*64][D], rows beyond n_kv are zero
  const int32_t* idx;      // [BH][nbq][top_k]
  const uint16_t* sc;      // bf16 S_c^T [BH][nbq][D(c)][D(r)]
  const float* zc;         // [BH][nbq][D]
  const float* alpha;      // [H][D]
  void* out;
  int nq, nkv, nbq, nbk, topk, H, total;
};

template <typename T>
__device__ __forceinline__ u32x4 load_bf16x8(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const u32x4*>(p);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    return u32x4{pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(b[0], b[1]),
                 pack_bf16(b[2], b[3])};
  }
}

// fp32 inputs: x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), so that Q K^T can be
// formed as Qhi Khi^T + Qhi Klo^T + Qlo Khi^T with near-fp32 accuracy on bf16 MFMA.
__device__ __forceinline__ void load_split_bf16x8(const float* p, u32x4& hi, u32x4& lo) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t h = pack_bf16(x[2 * e], x[2 * e + 1]);
    hi[e] = h;
    lo[e] = pack_bf16(x[2 * e] - bf16_lo(h), x[2 * e + 1] - bf16_hi(h));
  }
}

template <typename T, int D, bool OUT_BF16>
__global__ __launch_bounds__(128) void sparse_attn_kernel(SparseArgs a) {
  constexpr bool SPLIT = sizeof(T) == 4;   // fp32 inputs: three-term bf16 product
  constexpr int LS = D + 8;             // padded LDS row, elements
  constexpr int KS = D / 16;            // 16-channel reduction steps for Q K^T
  constexpr int CT = D / 32;            // 32-channel tiles of the output
  constexpr int TPR = D / 8;            // 16-byte chunks per row
  constexpr int CPT = 64 * TPR / 128;   // chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][64 * LS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][64 * LS];
  __shared__ __attribute__((aligned(16))) uint16_t Kl[SPLIT ? 2 : 1][SPLIT ? 64 * LS : 8];

  const int wid = xcd_remap(blockIdx.x, a.total);
  const int bh = wid / a.nbq, i = wid % a.nbq;
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int q0 = i * kBlock;
  const T* qb = reinterpret_cast<const T*>(a.q) + (size_t)bh * a.nq * D;
  const T* kb = reinterpret_cast<const T*>(a.k) + (size_t)bh * a.nkv * D;
  const uint16_t* vb = a.v16 + (size_t)bh * a.nbk * kBlock * D;
  const int32_t* sel = a.idx + ((size_t)bh * a.nbq + i) * a.topk;

  // Q^T fragments (B operand): lane column q = 32 t + l32, channels 16 s + 8 h .. +7
  u32x4 qf[2][KS];
  u32x4 ql[2][SPLIT ? KS : 1];
#pragma unroll
  for (int tq = 0; tq < 2; ++tq) {
    const int q = q0 + 32 * tq + l32;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[tq][s] = u32x4{0, 0, 0, 0};
      if constexpr (SPLIT) {
        ql[tq][s] = u32x4{0, 0, 0, 0};
        if (q < a.nq)
          load_split_bf16x8(reinterpret_cast<const float*>(qb) + (size_t)q * D + 16 * s + 8 * h,
                            qf[tq][s], ql[tq][s]);
      } else {
        if (q < a.nq) qf[tq][s] = load_bf16x8(qb + (size_t)q * D + 16 * s + 8 * h);
      }
    }
  }

  f32x16 o[CT][2];
#pragma unroll
  for (int c = 0; c < CT; ++c) o[c][0] = o[c][1] = f32x16{};
  float m[2] = {kNegBig, kNegBig};
  float l[2] = {0.f, 0.f};
  const float qk_scale = kLog2e / sqrtf((float)D);

  // tile staging: registers -> LDS
  u32x4 kreg[CPT], vreg[CPT], klreg[SPLIT ? CPT : 1];
  auto load_tile = [&](int j) {
    const int row0 = j * kBlock;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int cidx = t + 128 * u;
      const int r = cidx / TPR, c8 = cidx % TPR;
      kreg[u] = u32x4{0, 0, 0, 0};
      if constexpr (SPLIT) {
        klreg[u] = u32x4{0, 0, 0, 0};
        if (row0 + r < a.nkv)
          load_split_bf16x8(reinterpret_cast<const float*>(kb) + (size_t)(row0 + r) * D + c8 * 8,
                            kreg[u], klreg[u]);
      } else {
        if (row0 + r < a.nkv) kreg[u] = load_bf16x8(kb + (size_t)(row0 + r) * D + c8 * 8);
      }
      vreg[u] = *reinterpret_cast<const u32x4*>(vb + (size_t)(row0 + r) * D + c8 * 8);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int cidx = t + 128 * u;
      const int r = cidx / TPR, c8 = cidx % TPR;
      *reinterpret_cast<u32x4*>(&Ks[buf][r * LS + c8 * 8]) = kreg[u];
      *reinterpret_cast<u32x4*>(&Vs[buf][r * LS + c8 * 8]) = vreg[u];
      if constexpr (SPLIT) *reinterpret_cast<u32x4*>(&Kl[buf][r * LS + c8 * 8]) = klreg[u];
    }
  };

  const int ntiles = a.topk;
  if (ntiles > 0) {
    load_tile(sel[0]);
    store_tile(0);
    __syncthreads();
  }
  for (int tt = 0; tt < ntiles; ++tt) {
    const int buf = tt & 1;
    const int j = sel[tt];
    if (tt + 1 < ntiles) load_tile(sel[tt + 1]);
    const uint16_t* Kt = Ks[buf];
    const uint16_t* Vt = Vs[buf];

    // S^T tile: rows = keys 32 wv + (0..31), columns = queries
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = (32 * wv + l32) * LS + 16 * ks + 8 * h;
      const u32x4 af = *reinterpret_cast<const u32x4*>(&Kt[off]);
      s[0] = mfma_bf16(af, qf[0][ks], s[0]);
      s[1] = mfma_bf16(af, qf[1][ks], s[1]);
      if constexpr (SPLIT) {
        const u32x4 al = *reinterpret_cast<const u32x4*>(&Kl[buf][off]);
        s[0] = mfma_bf16(af, ql[0][ks], s[0]);
        s[1] = mfma_bf16(af, ql[1][ks], s[1]);
        s[0] = mfma_bf16(al, qf[0][ks], s[0]);
        s[1] = mfma_bf16(al, qf[1][ks], s[1]);
      }
    }
    // key validity (only the last key block can be partial)
    const int key_base = j * kBlock + 32 * wv;
    const bool partial = key_base + 32 > a.nkv;
    float mx[2];
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      float r = kNegBig;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float z = s[tq][e] * qk_scale;
        if (partial) {
          const int key = key_base + 8 * (e >> 2) + 4 * h + (e & 3);
          if (key >= a.nkv) z = -INFINITY;
        }
        s[tq][e] = z;
        r = fmaxf(r, z);
      }
      mx[tq] = fmaxf(r, swap_halves(r));
    }
    const bool grow = (mx[0] > m[0] + kRescaleSlack) || (mx[1] > m[1] + kRescaleSlack);
    if (__ballot(grow)) {
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        const float mn = fmaxf(m[tq], mx[tq]);
        const float corr = exp2f(m[tq] - mn);
        l[tq] *= corr;
#pragma unroll
        for (int c = 0; c < CT; ++c) o[c][tq] *= corr;
        m[tq] = mn;
      }
    }
    u32x4 pf[2][2];
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      float p[16];
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = __builtin_amdgcn_exp2f(s[tq][e] - m[tq]);
        rs += p[e];
      }
      l[tq] += rs;
#pragma unroll
      for (int ss = 0; ss < 2; ++ss)
        pf[tq][ss] = u32x4{pack_f16(p[8 * ss + 0], p[8 * ss + 1]), pack_f16(p[8 * ss + 2], p[8 * ss + 3]),
                           pack_f16(p[8 * ss + 4], p[8 * ss + 5]), pack_f16(p[8 * ss + 6], p[8 * ss + 7])};
    }
    // O^T += V^T P^T over this wave's 32 keys (two 16-key steps)
#pragma unroll
    for (int c = 0; c < CT; ++c) {
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const u32x4 vf = frag_tr_perm(Vt, LS, 32 * c, 32 * wv + 16 * ss);
        o[c][0] = mfma_f16(vf, pf[0][ss], o[c][0]);
        o[c][1] = mfma_f16(vf, pf[1][ss], o[c][1]);
      }
    }
    if (tt + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- merge the two waves
  float* xl = reinterpret_cast<float*>(&Ks[0][0]);   // LDS reuse after the loop
  // [wave][tq][32] maxima and sums
  l[0] += swap_halves(l[0]);
  l[1] += swap_halves(l[1]);
  if (h == 0) {
    xl[(wv * 2 + 0) * 32 + l32] = m[0];
    xl[(wv * 2 + 1) * 32 + l32] = m[1];
    xl[128 + (wv * 2 + 0) * 32 + l32] = l[0];
    xl[128 + (wv * 2 + 1) * 32 + l32] = l[1];
  }
  // Exchange the output channel half this wave does not keep: wave w keeps tiles
  // [w*HALF, (w+1)*HALF). Tile indices are compile-time constants in each branch so the
  // accumulators stay in registers.
  constexpr int HALF = CT / 2;
  float* xo = xl + 256;   // [wave][HALF][2][16][64]
  const int other = 1 - wv;
  auto give = [&](auto keep_tag) {
    constexpr int GIVE0 = HALF - decltype(keep_tag)::value;
#pragma unroll
    for (int c = 0; c < HALF; ++c)
#pragma unroll
      for (int tq = 0; tq < 2; ++tq)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          xo[(((wv * HALF + c) * 2 + tq) * 16 + e) * 64 + lane] = o[GIVE0 + c][tq][e];
  };
  if (wv == 0) give(std::integral_constant<int, 0>{});
  else give(std::integral_constant<int, HALF>{});
  __syncthreads();
  auto finish = [&](auto keep_tag) {
    constexpr int KEEP0 = decltype(keep_tag)::value;
    float fs[2], fo[2], inv_l[2];
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      const float mo = xl[(other * 2 + tq) * 32 + l32];
      const float lo_ = xl[128 + (other * 2 + tq) * 32 + l32];
      const float M = fmaxf(m[tq], mo);
      fs[tq] = exp2f(m[tq] - M);
      fo[tq] = exp2f(mo - M);
      const float L = l[tq] * fs[tq] + lo_ * fo[tq];
      inv_l[tq] = L > 0.f ? 1.f / L : 0.f;
    }

    // ------------------------------------------------------------ linear apply + mix
    const uint16_t* scb = a.sc + ((size_t)bh * a.nbq + i) * D * D;
    const float* zcb = a.zc + ((size_t)bh * a.nbq + i) * D;
    // phi(Q) . z_c per query column: this lane holds channels 16 s + 8 h .. +7
    float den[2];
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      float d = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const f32x4 z0 = *reinterpret_cast<const f32x4*>(zcb + 16 * s + 8 * h);
        const f32x4 z1 = *reinterpret_cast<const f32x4*>(zcb + 16 * s + 8 * h + 4);
        const u32x4 w = qf[tq][s];
        d += fmaxf(bf16_lo(w[0]), 0.f) * z0[0] + fmaxf(bf16_hi(w[0]), 0.f) * z0[1] +
             fmaxf(bf16_lo(w[1]), 0.f) * z0[2] + fmaxf(bf16_hi(w[1]), 0.f) * z0[3] +
             fmaxf(bf16_lo(w[2]), 0.f) * z1[0] + fmaxf(bf16_hi(w[2]), 0.f) * z1[1] +
             fmaxf(bf16_lo(w[3]), 0.f) * z1[2] + fmaxf(bf16_hi(w[3]), 0.f) * z1[3];
      }
      d += swap_halves(d);
      den[tq] = 1.f / (d + kEps);
    }
    const float* al = a.alpha + (size_t)(bh % a.H) * D;
#pragma unroll
    for (int cc = 0; cc < HALF; ++cc) {
      const int c = KEEP0 + cc;
      f32x16 lin[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const u32x4 af =
            *reinterpret_cast<const u32x4*>(scb + (size_t)(32 * c + l32) * D + 16 * s + 8 * h);
        lin[0] = mfma_bf16(af, relu_bf16x8(qf[0][s]), lin[0]);
        lin[1] = mfma_bf16(af, relu_bf16x8(qf[1][s]), lin[1]);
      }
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        const int q = q0 + 32 * tq + l32;
        if (q >= a.nq) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ch = 32 * c + 8 * g + 4 * h;
          const f32x4 alv = *reinterpret_cast<const f32x4*>(al + ch);
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ix = 4 * g + e;
            const float other_o = xo[(((other * HALF + cc) * 2 + tq) * 16 + ix) * 64 + lane];
            const float os = (o[KEEP0 + cc][tq][ix] * fs[tq] + other_o * fo[tq]) * inv_l[tq];
            const float ol = lin[tq][ix] * den[tq];
            r[e] = alv[e] * os + (1.f - alv[e]) * ol;
          }
          if constexpr (OUT_BF16) {
            uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + ((size_t)bh * a.nq + q) * D + ch;
            *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3])};
          } else {
            float* dst = reinterpret_cast<float*>(a.out) + ((size_t)bh * a.nq + q) * D + ch;
            *reinterpret_cast<f32x4*>(dst) = f32x4{r[0], r[1], r[2], r[3]};
          }
        }
      }
    }
  };
  if (wv == 0) finish(std::integral_constant<int, 0>{});
  else finish(std::integral_constant<int, HALF>{});
}

template <typename T, int D>
hipError_t launch_sparse_T(const Plan& s, const void* q, const void* k, const int32_t* idx,
                           const float* alpha, void* o, char* ws, hipStream_t st) {
  SparseArgs a;
  a.q = q;
  a.k = k;
  a.v16 = reinterpret_cast<const uint16_t*>(ws + s.v16);
  a.idx = idx;
  a.sc = reinterpret_cast<const uint16_t*>(ws + s.sc);
  a.zc = reinterpret_cast<const float*>(ws + s.zc);
  a.alpha = alpha;
  a.out = o;
  a.nq = s.nq; a.nkv = s.nkv; a.nbq = s.nbq; a.nbk = s.nbk; a.topk = s.k; a.H = s.H;
  a.total = s.BH * s.nbq;
  if (s.out_bf16)
    hipLaunchKernelGGL((sparse_attn_kernel<T, D, true>), dim3(a.total), dim3(128), 0, st, a);
  else
    hipLaunchKernelGGL((sparse_attn_kernel<T, D, false>), dim3(a.total), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse(const Plan& s, const void* q, const void* k, const int32_t* idx,
                         const float* alpha, void* o, char* ws, hipStream_t st) {
  if (s.in_bf16) {
    if (s.D == 128) return launch_sparse_T<uint16_t, 128>(s, q, k, idx, alpha, o, ws, st);
    return launch_sparse_T<uint16_t, 64>(s, q, k, idx, alpha, o, ws, st);
  }
  if (s.D == 128) return launch_sparse_T<float, 128>(s, q, k, idx, alpha, o, ws, st);
  return launch_sparse_T<float, 64>(s, q, k, idx, alpha, o, ws, st);
}

}  // namespace sla
