// Backward of the SLA2 forward at a given block selection (SLA2 page, section 2.B: the hard
// top-k selection is held fixed, so proj_q and proj_k receive no gradient through it; section
// 2.C: the backward runs in higher precision than a quantised forward — here bf16 / f16 MFMA
// with fp32 accumulation on the unquantised branches). Given dO, per (batch, head):
//   mix:     dalpha = sum_n dO (.) (O_s - O_l), dO_s = alpha dO, dO_l = (1 - alpha) dO;
//   sparse:  FlashAttention-style, P recomputed from the row log-sum-exp:
//            dV += P^T dO_s, dS = P (.) (dO_s V^T - D_n), dQ += tau dS K, dK += tau dS^T Q,
//            D_n = dO_s[n] . O_s[n];
//   linear:  g_n = dO_l[n] / den_n, h_n = -(dO_l[n] . O_l[n]) / den_n,
//            dQ += (g S_c^T + h z_c) (.) 1[q > 0], dS_c(i) = phi(Q_i)^T g, dz_c(i) = phi(Q_i)^T h,
//            and per key block j with G_j = sum_{i: j not in sel(i)} dS_c(i) (the transposed
//            complement, computed by the complement kernel with the roles of query and key
//            blocks swapped) and gz_j likewise: dV += phi(K_j) G_j,
//            dK += (V_j G_j^T + gz_j) (.) 1[k > 0].
// Kernels, in launch order:
//   bwd_bits_kernel     routed-block bitmaps of both orientations and the per-key-block
//                       counts from the index lists (into rows bwd_clear_kernel cleared);
//   (key/value pass)    S_j as bf16 high and low parts, z_j, z_tot and the f16 copy of V;
//   (complement, fp32)  S_c(i) = sum of the unselected S_j, high and low parts summed in fp32
//                       (with at most kFewBwdRows query blocks per head selecting at most half
//                       the key blocks: a key/value pass that keeps S_tot instead of every
//                       S_j, and S_c(i) = S_tot - the selected S_j in fp32);
//                       z_c(i);
//   (sparse kernel)     the exact branch of the forward again, saving O_s (fp32) and each
//                       row's log-sum-exp instead of mixing;
//   bwd_query_kernel    per query block: O_l, D, dO_s (f16), dalpha partials, the linear
//                       part of dQ, dS_c(i) (bf16 high and low parts, summary layout), dz_c(i);
//   (complement, fp32)  G_j from the dS_c(i), roles of query and key blocks swapped (with at
//                       most kFewBwdRows query blocks per head the key kernel sums each G_j
//                       from the dS_c(i) itself instead);
//   bwd_gz_kernel       gz_j;
//   bwd_order_kernel    key-block tasks by number of routing query blocks, most first (with
//                       few query blocks, bwd_routed_kernel lists the routed ones instead);
//   bwd_key_kernel      per key block: dK, dV over the query blocks that selected it, plus
//                       the linear parts (with few query blocks: only the routed key blocks;
//                       bwd_key_linear_kernel does the others);
//   bwd_dq_kernel       per query block: the exact branch's dQ, added to the linear part;
//   bwd_dalpha_kernel   dalpha from the per-query-block partials (fixed order).
// The linear gradients are differences of nearly equal terms (g S_c^T against h z_c, and
// V G^T against gz: both are covariances of the value with the feature map over the
// complement), so S_c, g, dS_c and G are carried as bf16 high + low parts into the MFMAs.
// Layout conventions follow the forward (transposed products so that an accumulator feeds
// the next MFMA as an operand; transposing LDS reads supply the other operand in the same
// permuted order). Every result is deterministic: no atomics on values, fixed reduction
// orders (the key kernel's task order comes from LDS atomics but changes no output bit).
#include "common.h"
#include "kernels.h"

namespace sla {

namespace {

struct BwdArgs {
  const uint16_t* q;        // bf16 [BH][nq][D]
  const uint16_t* k;        // bf16 [BH][nkv][D]
  const uint16_t* v;        // bf16 [BH][nkv][D]
  const uint16_t* v16;      // f16 copy of V [BH][nbk*64][D], padded rows zero
  const void* dout;         // [BH][nq][D], f32 or bf16
  int dout_bf16;
  const float* alpha;       // [H][D]
  const int32_t* idx;       // [BH][nbq][topk], ascending
  const uint32_t* bitsT;    // [BH][nbk][nwq]: bit i of key block j's row: j in sel(i)
  const float* sc;          // S_c^T [BH][nbq][D(c)][D(r)] fp32
  const float* zc;          // [BH][nbq][D]
  const float* os;          // O_s fp32 [BH][nq][D] (the forward's exact branch, saved)
  const float* lse;         // [BH][nbq*64] (base-2 units; kNoRowLse where a row has no exact part)
  float* dr;                // [BH][nbq*64]: D_n
  uint16_t* dos;            // f16 [BH][nbq*64][D]: dO_s
  uint16_t* dsc;            // bf16 [BH][D*D/128][nbq][128]: dS_c(i)^T flattened [c][r]
  uint16_t* dsclo;          // dS_c(i)^T - bf16(dS_c(i)^T) rounded to bf16, same layout
  float* dzc;               // [BH][nbq][D]
  const float* gt;          // G_j^T [BH][nbk][D(c)][D(r)] fp32
  float* gz;                // [BH][nbk][D]
  float* dapart;            // [BH][nbq][D]
  const int32_t* order;     // [BH*nbk]: key-block tasks, most routed query blocks first
  const int32_t* counts;    // [BH*nbk]: query blocks that routed each key block
  float* dq;                // [BH][nq][D]
  float* dk;                // [BH][nkv][D]
  float* dv;                // [BH][nkv][D]
  int nq, nkv, nbq, nbk, topk, H, nwq;
};


// Transposing fragment read in natural order from a swz-swizzled [row][col] tile of 16-bit
// elements: lane owns column x0 + lane % 32 and the 8 rows k0 + 8 (lane / 32) .. + 7.
template <int D>
__device__ __forceinline__ u32x4 tr_nat(const uint16_t* M, int x0, int k0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, L = lane & 15;
  const int row = k0 + 8 * (g >> 1) + (L >> 2);
  const int col = x0 + 16 * (g & 1) + 4 * (L & 3);
  const u32x2 lo = lds_read_tr16(M + swz<D>(row, col));
  const u32x2 hi = lds_read_tr16(M + swz<D>(row + 4, col));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// 64-row tile of 16-bit elements, global rows src[0 .. nvalid) -> swizzled LDS tile, as loads
// straight into LDS shared by the NW waves of the workgroup (1-KB pieces: lane l of a piece
// lands at element 8 l of it and fetches the logical chunk that the swizzle puts there);
// rows >= nvalid read as zero. The caller waits (wait_vmem / barrier_vmem*) before reading.
template <int D, bool SWZV, int NW>
__device__ __forceinline__ void dma_tile(uint16_t* dst, const uint16_t* src, int nvalid) {
  constexpr int CH = D / 8, RPP = 512 / D, PPW = (D / 8) / NW;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the descriptor and the LDS address live in scalar registers: every argument is uniform
  // over the workgroup, made explicit for the compiler
  const uint64_t b = reinterpret_cast<uint64_t>(src);
  // (readfirstlane returns int: each half goes through uint32_t, so that a low word with bit
  // 31 set is not sign-extended into the high word)
  const uint32_t bhi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t blo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t bu = ((uint64_t)bhi << 32) | (uint64_t)blo;
  const int nv = __builtin_amdgcn_readfirstlane(nvalid > 0 ? nvalid : 0);
  const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(dst));
  const i32x4 r = make_rsrc(reinterpret_cast<const void*>(bu), (uint32_t)nv * D * 2);
#pragma unroll
  for (int u = 0; u < PPW; ++u) {
    const int pp = w * PPW + u;
    const int row = pp * RPP + lane / CH, pc = lane % CH;
    const int lc = (pc ^ (SWZV ? swzv_f<D>(row) : row)) & (CH - 1);
    load_lds16(r, l0 + pp * 1024, (uint32_t)(row * D * 2 + lc * 16));
  }
}

// 8 consecutive fp32 values as two bf16 fragments: the rounded values and the remainders
__device__ __forceinline__ void split8(const float* p, u32x4& hi, u32x4& lo) {
  const f32x4 x = *reinterpret_cast<const f32x4*>(p);
  const f32x4 y = *reinterpret_cast<const f32x4*>(p + 4);
  const float v[8] = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = pack_bf16(v[2 * e], v[2 * e + 1]);
    lo[e] = pack_bf16(v[2 * e] - bf16_lo(hi[e]), v[2 * e + 1] - bf16_hi(hi[e]));
  }
}

// 8 consecutive elements of row `row` at column col (a multiple of 8) of a swizzled tile
template <int D, bool SWZV>
__device__ __forceinline__ u32x4 row_frag(const uint16_t* M, int row, int col) {
  return *reinterpret_cast<const u32x4*>(M + (SWZV ? swzv<D>(row, col) : swz<D>(row, col)));
}

// Wait for every memory operation of this wave (loads into LDS included), then a workgroup
// barrier. Unlike a wait written in asm, the compiler sees this one: no load is pending for
// it afterwards, so it places no wait for the loop's register operands inside the loop,
// where its count would also cover the next block's tile loads issued on each pass.
__device__ __forceinline__ void drain_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// ----------------------------------------------------------------------------- bitmaps
// Row i of selbits: bit j set iff key block j is routed to query block i; row j of bitsT:
// bit i set iff j is routed to i; counts[j]: how many query blocks routed j. bitsT and counts
// start cleared (bwd_clear_kernel); one workgroup per (batch*head, query block) builds its
// selbits row in LDS, then ORs its bit into the bitsT row of each key block it routed and
// adds one to that block's count (integer OR and sum: the same whatever the order).
__global__ __launch_bounds__(256) void bwd_clear_kernel(uint32_t* __restrict__ bitsT,
                                                        size_t nwords,
                                                        int32_t* __restrict__ counts,
                                                        size_t ncounts) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < nwords; e += stride) bitsT[e] = 0u;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < ncounts; e += stride) counts[e] = 0;
}

__global__ __launch_bounds__(256) void bwd_bits_kernel(const int32_t* __restrict__ idx,
                                                       uint32_t* __restrict__ selbits,
                                                       uint32_t* __restrict__ bitsT,
                                                       int32_t* __restrict__ counts, int nbq,
                                                       int nbk, int topk, int nwk, int nwq) {
  extern __shared__ uint32_t wbits[];
  const int bh = blockIdx.y, row = blockIdx.x, t = threadIdx.x;
  for (int w = t; w < nwk; w += 256) wbits[w] = 0u;
  __syncthreads();
  const int32_t* sel = idx + ((size_t)bh * nbq + row) * topk;
  for (int e = t; e < topk; e += 256) {
    const int j = sel[e];
    atomicOr(&wbits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  for (int w = t; w < nwk; w += 256) {
    uint32_t word = wbits[w];
    selbits[((size_t)bh * nbq + row) * nwk + w] = word;
    while (word) {
      const int j = 32 * w + __builtin_ctz(word);
      word &= word - 1u;
      atomicOr(&bitsT[((size_t)bh * nbk + j) * nwq + (row >> 5)], 1u << (row & 31));
      atomicAdd(&counts[(size_t)bh * nbk + j], 1);
    }
  }
}

// ----------------------------------------------------------------------------- per query block
// Two waves, wave w owns query rows 32 w .. 32 w + 31 of query block iq; the O^T accumulator
// layout (lane: query row, elements: channels 32 c + 8 g + 4 h + e) is kept throughout.
// LDS is used in three phases: S_c^T as bf16 high and low parts (O_l and the linear dQ),
// then the dalpha terms (fp32 [64][D]), then g as bf16 high and low parts and the Q tile
// (dS_c and dz_c): 64 KB at D = 128, so two workgroups share a CU.
template <int D>
__global__ __launch_bounds__(128) void bwd_query_kernel(BwdArgs a) {
  constexpr int KS = D / 16, CT = D / 32, CH = D / 8, TILE = 64 * D;
  constexpr int NCS = D * D / 128;
  constexpr int SMEM = 2 * D * D > 3 * TILE ? 2 * D * D : 3 * TILE;
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM];
  __shared__ float hh_s[64];
  const int bh = blockIdx.x / a.nbq, iq = blockIdx.x % a.nbq;
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int row = 32 * wv + l32;              // row within the query block
  const int n = iq * kBlock + row;            // query token
  const bool valid = n < a.nq;
  const int hd = bh % a.H;
  const uint16_t* qrow = a.q + ((size_t)bh * a.nq + (valid ? n : 0)) * D;

  // phase 1: S_c^T [D][D] as bf16 high and low parts, V swizzle (row reads and vt_frag)
  uint16_t* Sct = smem;
  uint16_t* Scl = smem + D * D;
  const float* scb = a.sc + ((size_t)bh * a.nbq + iq) * D * D;
  for (int id = t; id < D * CH; id += 128) {
    const int rr = id / CH, cc = id % CH;
    u32x4 hi, lo;
    split8(scb + (size_t)rr * D + cc * 8, hi, lo);
    *reinterpret_cast<u32x4*>(Sct + swzv<D>(rr, cc * 8)) = hi;
    *reinterpret_cast<u32x4*>(Scl + swzv<D>(rr, cc * 8)) = lo;
  }

  u32x4 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = valid ? *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};

  // the exact branch's output, saved by the forward's sparse kernel in this backward
  const float* osr = a.os + ((size_t)bh * a.nq + (valid ? n : 0)) * D;
  const float* dof = reinterpret_cast<const float*>(a.dout) + ((size_t)bh * a.nq + n) * D;
  const uint16_t* dob = reinterpret_cast<const uint16_t*>(a.dout) + ((size_t)bh * a.nq + n) * D;
  auto load_dout = [&](int ch, float (&dov)[4]) __attribute__((always_inline)) {
    dov[0] = dov[1] = dov[2] = dov[3] = 0.f;
    if (!valid) return;
    if (a.dout_bf16) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(dob + ch);
      dov[0] = bf16_lo(w[0]); dov[1] = bf16_hi(w[0]); dov[2] = bf16_lo(w[1]); dov[3] = bf16_hi(w[1]);
    } else {
      const f32x4 w = *reinterpret_cast<const f32x4*>(dof + ch);
      dov[0] = w[0]; dov[1] = w[1]; dov[2] = w[2]; dov[3] = w[3];
    }
  };

  // ---------------------------------------------------------------- linear branch again
  const bool empty_c = a.topk >= a.nbk;
  const float* zcb = a.zc + ((size_t)bh * a.nbq + iq) * D;
  f32x16 lin[CT];
  float den = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const u32x4 rq = relu_bf16x8(qf[s]);
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2)
      den += bf16_lo(rq[e2]) * zcb[16 * s + 8 * h + 2 * e2] +
             bf16_hi(rq[e2]) * zcb[16 * s + 8 * h + 2 * e2 + 1];
  }
  den += swap_halves(den);
  den += kEps;
  __syncthreads();   // S_c^T is in place
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    lin[c] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 qb = relu_bf16x8(qf[s]);
      lin[c] = mfma_bf16(row_frag<D, true>(Sct, 32 * c + l32, 16 * s + 8 * h), qb, lin[c]);
      lin[c] = mfma_bf16(row_frag<D, true>(Scl, 32 * c + l32, 16 * s + 8 * h), qb, lin[c]);
    }
  }
  const float inv_den = empty_c ? 0.f : 1.f / den;

  // ---------------------------------------------------------------- upstream gradient
  const float* al = a.alpha + (size_t)hd * D;
  float dsum = 0.f, hsum = 0.f;
  f32x16 gv[CT];                                  // g = dO_l / den, O^T layout
  uint16_t* dosr = a.dos + ((size_t)bh * a.nbq * kBlock + iq * kBlock + row) * D;
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int ch = 32 * c + 8 * g4 + 4 * h;
      float dov[4];
      load_dout(ch, dov);
      const f32x4 alv = *reinterpret_cast<const f32x4*>(al + ch);
      const f32x4 osv = valid ? *reinterpret_cast<const f32x4*>(osr + ch) : f32x4{0.f, 0.f, 0.f, 0.f};
      float dsv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ix = 4 * g4 + e;
        const float ol = lin[c][ix] * inv_den;
        dsv[e] = alv[e] * dov[e];
        const float dl = (1.f - alv[e]) * dov[e];
        dsum += dsv[e] * osv[e];
        hsum += dl * ol;
        gv[c][ix] = dl * inv_den;
      }
      *reinterpret_cast<u32x2*>(dosr + ch) = u32x2{pack_f16(dsv[0], dsv[1]), pack_f16(dsv[2], dsv[3])};
    }
  dsum += swap_halves(dsum);
  hsum += swap_halves(hsum);
  const float hn = empty_c ? 0.f : -hsum * inv_den;
  if (h == 0) {
    a.dr[(size_t)bh * a.nbq * kBlock + iq * kBlock + row] = valid ? dsum : 0.f;
    hh_s[row] = valid ? hn : 0.f;
  }

  // ---------------------------------------------------------------- linear part of dQ
  // da^T = S_c g^T: M = r, N = this wave's rows, K = c (g's elements in vt_frag's order).
  // S_c and g enter as bf16 high and low parts (the low x low product is below fp32's
  // rounding): g S_c^T and h z_c nearly cancel (their difference is the covariance of phi(k)
  // and v over the complement), so one bf16 rounding of either would show in dQ.
  f32x16 da[CT];
#pragma unroll
  for (int rt = 0; rt < CT; ++rt) da[rt] = f32x16{};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int c = s >> 1, e0 = 8 * (s & 1);
    u32x4 gb, gl;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const float x0 = gv[c][e0 + 2 * e2], x1 = gv[c][e0 + 2 * e2 + 1];
      gb[e2] = pack_bf16(x0, x1);
      gl[e2] = pack_bf16(x0 - bf16_lo(gb[e2]), x1 - bf16_hi(gb[e2]));
    }
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) {
      const u32x4 sa = vt_frag<D>(Sct, 32 * rt, 16 * s);
      da[rt] = mfma_bf16(sa, gb, da[rt]);
      da[rt] = mfma_bf16(sa, gl, da[rt]);
      da[rt] = mfma_bf16(vt_frag<D>(Scl, 32 * rt, 16 * s), gb, da[rt]);
    }
  }
  if (valid) {
    float* dqr = a.dq + ((size_t)bh * a.nq + n) * D;
#pragma unroll
    for (int rt = 0; rt < CT; ++rt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int r0 = 32 * rt + 8 * g4 + 4 * h;
        const f32x4 z = *reinterpret_cast<const f32x4*>(zcb + r0);
        const u32x2 qw = *reinterpret_cast<const u32x2*>(qrow + r0);
        const float qv[4] = {bf16_lo(qw[0]), bf16_hi(qw[0]), bf16_lo(qw[1]), bf16_hi(qw[1])};
        f32x4 outv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float dav = da[rt][4 * g4 + e] + hn * z[e];
          outv[e] = qv[e] > 0.f ? dav : 0.f;
        }
        *reinterpret_cast<f32x4*>(dqr + r0) = outv;
      }
  }

  // ---------------------------------------------------------------- dalpha partial
  // phase 2: the terms dO (.) (O_s - O_l) as fp32 [64][D], summed over the block's rows in order
  __syncthreads();   // S_c^T is no longer read
  float* xs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int ch = 32 * c + 8 * g4 + 4 * h;
      float dov[4];
      load_dout(ch, dov);
      const f32x4 osv = valid ? *reinterpret_cast<const f32x4*>(osr + ch) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        xs[row * D + ch + e] = dov[e] * (osv[e] - lin[c][4 * g4 + e] * inv_den);
    }
  __syncthreads();
  for (int c = t; c < D; c += 128) {
    float sacc = 0.f;
    for (int r2 = 0; r2 < kBlock; ++r2) sacc += xs[r2 * D + c];
    a.dapart[((size_t)bh * a.nbq + iq) * D + c] = sacc;
  }
  __syncthreads();

  // ---------------------------------------------------------------- dS_c and dz_c
  // phase 3: g as bf16 high and low parts and the Q tile (row swizzle, read with tr_nat)
  uint16_t* Gt = smem;          // g rounded to bf16
  uint16_t* Gl = smem + TILE;   // and its remainder, also bf16
  uint16_t* Qt = smem + 2 * TILE;
  dma_tile<D, false, 2>(Qt, a.q + ((size_t)bh * a.nq + (size_t)iq * kBlock) * D,
                        min(kBlock, a.nq - iq * kBlock));
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int ch = 32 * c + 8 * g4 + 4 * h;
      const uint32_t h0 = pack_bf16(gv[c][4 * g4], gv[c][4 * g4 + 1]);
      const uint32_t h1 = pack_bf16(gv[c][4 * g4 + 2], gv[c][4 * g4 + 3]);
      *reinterpret_cast<u32x2*>(Gt + swz<D>(row, ch)) = u32x2{h0, h1};
      *reinterpret_cast<u32x2*>(Gl + swz<D>(row, ch)) =
          u32x2{pack_bf16(gv[c][4 * g4] - bf16_lo(h0), gv[c][4 * g4 + 1] - bf16_hi(h0)),
                pack_bf16(gv[c][4 * g4 + 2] - bf16_lo(h1), gv[c][4 * g4 + 3] - bf16_hi(h1))};
    }
  barrier_vmem_lds_n<0>();   // the g tiles (stores) and the Q tile (loads into LDS) are in place
  // dS_c(i)^T[c][r] = sum_n g[n][c] relu(q[n][r]): M = c, N = r, K = the block's 64 rows.
  // Wave w takes the c tiles w, w + 2, ...
  for (int ct = wv; ct < CT; ct += 2) {
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4 qb = relu_bf16x8(tr_nat<D>(Qt, 32 * rt, 16 * kk));
        acc = mfma_bf16(tr_nat<D>(Gt, 32 * ct, 16 * kk), qb, acc);
        acc = mfma_bf16(tr_nat<D>(Gl, 32 * ct, 16 * kk), qb, acc);
      }
      // element el: c = 32 ct + 8 (el / 4) + 4 h + el % 4, r = 32 rt + l32
      const int r = 32 * rt + l32;
#pragma unroll
      for (int el = 0; el < 16; ++el) {
        const int c = 32 * ct + 8 * (el >> 2) + 4 * h + (el & 3);
        const int f = c * D + r;
        const size_t o = (((size_t)bh * NCS + f / 128) * a.nbq + iq) * 128 + f % 128;
        const uint32_t hi = pack_bf16(acc[el], 0.f);
        a.dsc[o] = (uint16_t)(hi & 0xffffu);
        a.dsclo[o] = (uint16_t)(pack_bf16(acc[el] - bf16_lo(hi), 0.f) & 0xffffu);
      }
    }
  }
  // dz_c(i)[r] = sum_n relu(q[n][r]) h_n
  for (int r = t; r < D; r += 128) {
    float s = 0.f;
    for (int r2 = 0; r2 < kBlock; ++r2)
      s += fmaxf(bf16_bits_to_f32(Qt[swz<D>(r2, r)]), 0.f) * hh_s[r2];
    a.dzc[((size_t)bh * a.nbq + iq) * D + r] = s;
  }
}

// gz_j = sum over the query blocks i that did not select j of dz_c(i), in order of i.
// One thread per channel; a workgroup takes kGzBlocks key blocks, so that each dz_c row is
// read once for all of them.
constexpr int kGzBlocks = 16;
template <int D>
__global__ __launch_bounds__(D) void bwd_gz_kernel(BwdArgs a) {
  const int ngrp = (a.nbk + kGzBlocks - 1) / kGzBlocks;
  const int bh = blockIdx.x / ngrp, j0 = (blockIdx.x % ngrp) * kGzBlocks, c = threadIdx.x;
  const int nj = min(kGzBlocks, a.nbk - j0);
  float acc[kGzBlocks];
#pragma unroll
  for (int u = 0; u < kGzBlocks; ++u) acc[u] = 0.f;
  const uint32_t* rows = a.bitsT + ((size_t)bh * a.nbk + j0) * a.nwq;
  const float* dz = a.dzc + (size_t)bh * a.nbq * D + c;
  for (int w = 0; w < a.nwq; ++w) {
    uint32_t word[kGzBlocks];
#pragma unroll
    for (int u = 0; u < kGzBlocks; ++u) word[u] = u < nj ? rows[(size_t)u * a.nwq + w] : ~0u;
    const int nb = min(32, a.nbq - 32 * w);
    float v[32];   // the word's 32 rows of dz_c in flight together
#pragma unroll
    for (int b = 0; b < 32; ++b) v[b] = b < nb ? dz[(size_t)(32 * w + b) * D] : 0.f;
#pragma unroll
    for (int b = 0; b < 32; ++b)
#pragma unroll
      for (int u = 0; u < kGzBlocks; ++u)
        if (b < nb && !((word[u] >> b) & 1u)) acc[u] += v[b];
  }
#pragma unroll
  for (int u = 0; u < kGzBlocks; ++u)
    if (u < nj) a.gz[((size_t)bh * a.nbk + j0 + u) * D + c] = acc[u];
}

// Key-block tasks ordered by the number of query blocks that routed them, most first (a
// counting sort in one workgroup), so that the longest tasks of the key kernel start first
// and its tail stays short. Tasks with the same count land in any order: each task's
// results depend only on its own key block, so the order changes no output bit.
constexpr int kOrderBins = 4096;
__global__ __launch_bounds__(1024) void bwd_order_kernel(const int32_t* __restrict__ counts,
                                                         int ntask, int nbq,
                                                         int32_t* __restrict__ order) {
  __shared__ int bins[kOrderBins];
  const int nbin = min(nbq + 1, kOrderBins);
  for (int b = threadIdx.x; b < nbin; b += 1024) bins[b] = 0;
  __syncthreads();
  for (int task = threadIdx.x; task < ntask; task += 1024)
    atomicAdd(&bins[min(counts[task], nbin - 1)], 1);
  __syncthreads();
  if (threadIdx.x == 0) {   // exclusive offsets, largest count first
    int off = 0;
    for (int b = nbin - 1; b >= 0; --b) {
      const int n = bins[b];
      bins[b] = off;
      off += n;
    }
  }
  __syncthreads();
  for (int task = threadIdx.x; task < ntask; task += 1024)
    order[atomicAdd(&bins[min(counts[task], nbin - 1)], 1)] = task;
}

// Few query blocks per head: the key kernel's tasks are the routed key blocks only, at most
// cap = min(nbk, nbq k) per head (each query block routes at most k). One workgroup per head
// lists them in index order at order[bh cap ..] and fills the rest of its cap slots with -1.
__global__ __launch_bounds__(256) void bwd_routed_kernel(const int32_t* __restrict__ counts,
                                                         int nbk, int cap,
                                                         int32_t* __restrict__ order) {
  __shared__ int wsum[4];
  const int bh = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int32_t* cnt = counts + (size_t)bh * nbk;
  int32_t* out = order + (size_t)bh * cap;
  int base = 0;
  for (int j0 = 0; j0 < nbk; j0 += 256) {
    const int j = j0 + t;
    const bool routed = j < nbk && cnt[j] > 0;
    const unsigned long long m = __ballot(routed);
    if (lane == 0) wsum[w] = __popcll(m);
    __syncthreads();
    int off = base + __popcll(m & ((1ull << lane) - 1ull)), tot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      off += q < w ? wsum[q] : 0;
      tot += wsum[q];
    }
    if (routed && off < cap) out[off] = bh * nbk + j;
    base += tot;
    __syncthreads();   // wsum is rewritten next round
  }
  for (int p = base + t; p < cap; p += 256) out[p] = -1;
}

// ----------------------------------------------------------------------------- per key block
// Few query blocks (no G_j region): G_j^T is the sum of dS_c(i)^T over the query blocks i that
// did not route j (brow: j's row of the transposed bitmap; nullptr: every query block), each
// as its high plus low part in fp32, in ascending i; then split into bf16 high and low parts,
// staged into Gs / Gl (row swizzle) by the workgroup's NT threads.
template <int D, int NT>
__device__ __forceinline__ void stage_g_sum(const BwdArgs& a, int bh, const uint32_t* brow,
                                            uint16_t* Gs, uint16_t* Gl) {
  static_assert(D * (D / 8) % NT == 0, "whole rounds of ids");
#pragma unroll 4
  for (int u = 0; u < D * (D / 8) / NT; ++u) {
    const int id = threadIdx.x + u * NT;
    const int rr = id / (D / 8), cc = id % (D / 8);
    const int f = rr * D + cc * 8;   // flattened [c][r] index, summary layout of 128-slices
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < a.nbq; ++i) {
      if (brow && ((brow[i >> 5] >> (i & 31)) & 1u)) continue;   // i routed j
      const size_t o = (((size_t)bh * (D * D / 128) + (f >> 7)) * a.nbq + i) * 128 + (f & 127);
      const u32x4 hv = *reinterpret_cast<const u32x4*>(a.dsc + o);
      const u32x4 lv = *reinterpret_cast<const u32x4*>(a.dsclo + o);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] += bf16_lo(hv[e]) + bf16_lo(lv[e]);
        x[2 * e + 1] += bf16_hi(hv[e]) + bf16_hi(lv[e]);
      }
    }
    u32x4 hi, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hi[e] = pack_bf16(x[2 * e], x[2 * e + 1]);
      lo[e] = pack_bf16(x[2 * e] - bf16_lo(hi[e]), x[2 * e + 1] - bf16_hi(hi[e]));
    }
    *reinterpret_cast<u32x4*>(Gs + swz<D>(rr, cc * 8)) = hi;
    *reinterpret_cast<u32x4*>(Gl + swz<D>(rr, cc * 8)) = lo;
  }
}

// Two waves, wave w owns keys 32 w .. 32 w + 31 of key block j. Products are oriented so that
// the score accumulator (rows: queries, lane: key) feeds the dV^T and dK^T products directly.
template <int D>
__global__ __launch_bounds__(128) void bwd_key_kernel(BwdArgs a) {
  constexpr int KS = D / 16, CT = D / 32, TILE = 64 * D;
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE > 2 * D * D ? 4 * TILE : 2 * D * D];
  __shared__ __attribute__((aligned(16))) float lse_s[2][64], dr_s[2][64];
  const int task = a.order[blockIdx.x];
  // few query blocks: the routed key blocks only, -1 past a head's last one (the key blocks
  // no query block routed are bwd_key_linear_kernel's)
  if (task < 0) return;
  const int bh = task / a.nbk, j = task % a.nbk;
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int key = j * kBlock + 32 * wv + l32;
  const bool kvalid = key < a.nkv;
  const float qk_scale = kLog2e / sqrtf((float)D);
  const float tau = 1.f / sqrtf((float)D);
  const uint16_t* krow = a.k + ((size_t)bh * a.nkv + (kvalid ? key : 0)) * D;
  const uint16_t* v16row = a.v16 + ((size_t)bh * a.nbk * kBlock + (size_t)j * kBlock + 32 * wv + l32) * D;
  u32x4 kf[KS], vf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    kf[s] = kvalid ? *reinterpret_cast<const u32x4*>(krow + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};
    vf[s] = *reinterpret_cast<const u32x4*>(v16row + 16 * s + 8 * h);
  }
  f32x16 dvt[CT], dkt[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) dvt[c] = dkt[c] = f32x16{};
  // Two slots of (Q tile, dO_s tile), both V-swizzled (row reads and vt_frag reads): the
  // next routed query block's tiles load straight into LDS while this one is multiplied.
  // j's row of the transposed bitmap, staged in LDS (nwq words of dynamic shared memory) so
  // that finding the next routed query block is no memory round trip inside the loop
  const uint32_t* brow = a.bitsT + ((size_t)bh * a.nbk + j) * a.nwq;
  extern __shared__ uint32_t brow_s[];
  for (int w = t; w < a.nwq; w += 128) brow_s[w] = brow[w];
  __syncthreads();
  auto next_routed = [&](int from) -> int {   // first query block >= from that routed j, or -1
    for (int w = from >> 5; w < a.nwq; ++w) {
      uint32_t word = brow_s[w];
      if (w == (from >> 5)) word &= ~0u << (from & 31);
      if (word) return 32 * w + __builtin_ctz(word);
    }
    return -1;
  };
  auto stage = [&](int i, int slot) __attribute__((always_inline)) {
    dma_tile<D, true, 2>(smem + 2 * slot * TILE, a.q + ((size_t)bh * a.nq + (size_t)i * kBlock) * D,
                         min(kBlock, a.nq - i * kBlock));
    dma_tile<D, true, 2>(smem + (2 * slot + 1) * TILE,
                         a.dos + ((size_t)bh * a.nbq * kBlock + (size_t)i * kBlock) * D, kBlock);
  };
  const size_t rbase = (size_t)bh * a.nbq * kBlock;
  int i = next_routed(0);
  if (i >= 0) {
    stage(i, 0);
    if (t < 64) {
      lse_s[0][t] = a.lse[rbase + i * kBlock + t];
      dr_s[0][t] = a.dr[rbase + i * kBlock + t];
    }
  }
  drain_barrier();
  int slot = 0;
  while (i >= 0) {
    const int inext = next_routed(i + 1);
    float lnext = 0.f, dnext = 0.f;
    if (inext >= 0) {
      stage(inext, slot ^ 1);
      if (t < 64) {
        lnext = a.lse[rbase + inext * kBlock + t];
        dnext = a.dr[rbase + inext * kBlock + t];
      }
    }
    {
      const uint16_t* Qs = smem + 2 * slot * TILE;
      const uint16_t* Os = smem + (2 * slot + 1) * TILE;
      const float* lsv = lse_s[slot];
      const float* drv = dr_s[slot];
      // S = Q K^T and dP = dO_s V^T: rows n (two 32-row tiles), lane: key
      f32x16 sv[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          sv[mt] = mfma_bf16(row_frag<D, true>(Qs, 32 * mt + l32, 16 * s + 8 * h), kf[s], sv[mt]);
          dp[mt] = mfma_f16(row_frag<D, true>(Os, 32 * mt + l32, 16 * s + 8 * h), vf[s], dp[mt]);
        }
      u32x4 pf[4], df[4], dl[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int nb0 = 32 * mt + 16 * hh + 4 * h;   // rows of elements 8 hh .. 8 hh + 3
          const f32x4 l0 = *reinterpret_cast<const f32x4*>(&lsv[nb0]);
          const f32x4 l1 = *reinterpret_cast<const f32x4*>(&lsv[nb0 + 8]);
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(&drv[nb0]);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(&drv[nb0 + 8]);
          float pv[8], dsv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int el = 8 * hh + e;
            const float lv = e < 4 ? l0[e] : l1[e - 4];
            const float dv_ = e < 4 ? d0[e] : d1[e - 4];
            // (no mask for a key past n_kv: every product below keeps a key's terms in that
            // key's own column, and the lane's results are not stored)
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[mt][el], qk_scale, -lv));
            pv[e] = p;
            dsv[e] = p * (dp[mt][el] - dv_);   // tau is applied to the sum
          }
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            pf[2 * mt + hh][e2] = pack_f16(pv[2 * e2], pv[2 * e2 + 1]);
            const uint32_t hi = pack_bf16(dsv[2 * e2], dsv[2 * e2 + 1]);
            df[2 * mt + hh][e2] = hi;
            dl[2 * mt + hh][e2] = pack_bf16(dsv[2 * e2] - bf16_lo(hi), dsv[2 * e2 + 1] - bf16_hi(hi));
          }
        }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          dvt[c] = mfma_f16(vt_frag<D>(Os, 32 * c, 16 * kk), pf[kk], dvt[c]);
          const u32x4 qa = vt_frag<D>(Qs, 32 * c, 16 * kk);
          dkt[c] = mfma_bf16(qa, df[kk], dkt[c]);
          dkt[c] = mfma_bf16(qa, dl[kk], dkt[c]);
        }
    }
    if (inext >= 0 && t < 64) {
      lse_s[slot ^ 1][t] = lnext;
      dr_s[slot ^ 1][t] = dnext;
    }
    drain_barrier();   // the next tiles and their rows' lse / D are in place
    slot ^= 1;
    i = inext;
  }
  // linear parts: dV^T += G_j^T relu(K)^T (M = c, K = r), dK_lin^T = G_j V^T (M = r, K = c),
  // with G_j as bf16 high and low parts (V G^T + gz nearly cancels, like the query side)
  __syncthreads();
  uint16_t* Gs = smem;           // G_j^T [c][r], row swizzle (tr_nat gives G[r][c] fragments)
  uint16_t* Gl = smem + D * D;   // its low parts
  if (a.gt) {
    const float* gtb = a.gt + ((size_t)bh * a.nbk + j) * D * D;
    for (int id = t; id < D * (D / 8); id += 128) {
      const int rr = id / (D / 8), cc = id % (D / 8);
      u32x4 hi, lo;
      split8(gtb + (size_t)rr * D + cc * 8, hi, lo);
      *reinterpret_cast<u32x4*>(Gs + swz<D>(rr, cc * 8)) = hi;
      *reinterpret_cast<u32x4*>(Gl + swz<D>(rr, cc * 8)) = lo;
    }
  } else {
    stage_g_sum<D, 128>(a, bh, brow_s, Gs, Gl);
  }
  __syncthreads();
  const uint16_t* vrow = a.v + ((size_t)bh * a.nkv + (kvalid ? key : 0)) * D;
  f32x16 lk[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    lk[c] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      // G^T rows 32 c + l32, columns 16 s + 8 h .. +7, from the staged high and low parts
      const u32x4 gh = *reinterpret_cast<const u32x4*>(Gs + swz<D>(32 * c + l32, 16 * s + 8 * h));
      const u32x4 glo = *reinterpret_cast<const u32x4*>(Gl + swz<D>(32 * c + l32, 16 * s + 8 * h));
      const u32x4 kb = relu_bf16x8(kf[s]);
      dvt[c] = mfma_bf16(gh, kb, dvt[c]);
      dvt[c] = mfma_bf16(glo, kb, dvt[c]);
      const u32x4 vb = kvalid ? *reinterpret_cast<const u32x4*>(vrow + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};
      lk[c] = mfma_bf16(tr_nat<D>(Gs, 32 * c, 16 * s), vb, lk[c]);
      lk[c] = mfma_bf16(tr_nat<D>(Gl, 32 * c, 16 * s), vb, lk[c]);
    }
  }
  if (!kvalid) return;
  const float* gzb = a.gz + ((size_t)bh * a.nbk + j) * D;
  float* dkr = a.dk + ((size_t)bh * a.nkv + key) * D;
  float* dvr = a.dv + ((size_t)bh * a.nkv + key) * D;
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int r0 = 32 * c + 8 * g4 + 4 * h;
      const f32x4 z = *reinterpret_cast<const f32x4*>(gzb + r0);
      const u32x2 kw = *reinterpret_cast<const u32x2*>(krow + r0);
      const float kv[4] = {bf16_lo(kw[0]), bf16_hi(kw[0]), bf16_lo(kw[1]), bf16_hi(kw[1])};
      f32x4 ko, vo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ix = 4 * g4 + e;
        ko[e] = tau * dkt[c][ix] + (kv[e] > 0.f ? lk[c][ix] + z[e] : 0.f);
        vo[e] = dvt[c][ix];
      }
      *reinterpret_cast<f32x4*>(dkr + r0) = ko;
      *reinterpret_cast<f32x4*>(dvr + r0) = vo;
    }
}

// Few query blocks per head: the key blocks that no query block routed only have the linear
// gradients, all with the same G (the sum of every dS_c(i)) within a head. A workgroup takes
// kLinBlocks consecutive key blocks of one head, stages that G once and computes dV = phi(K)
// G and dK = (V G^T + gz) (.) 1[k > 0] for its unrouted blocks, as bwd_key_kernel's linear
// part does (the routed ones are bwd_key_kernel's). Four waves (two per SIMD with two
// workgroups per CU) take the 32-key halves of those blocks in turn. The epilogue reads gz
// from LDS and k > 0 from the K fragments in registers: its only memory accesses are the
// stores, so no wait on them stalls the next item.
constexpr int kLinBlocks = 16;
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_key_linear_kernel(BwdArgs a) {
  constexpr int KS = D / 16, CT = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Gs[D * D];
  __shared__ __attribute__((aligned(16))) uint16_t Gl[D * D];
  __shared__ __attribute__((aligned(16))) float zs[kLinBlocks * D];   // gz of the blocks here
  __shared__ int items[2 * kLinBlocks];
  __shared__ int nitems;
  static_assert(kLinBlocks <= 64, "one ballot lists the blocks");
  const int chunks = (a.nbk + kLinBlocks - 1) / kLinBlocks;
  const int bh = blockIdx.x / chunks, j0 = (blockIdx.x % chunks) * kLinBlocks;
  const int j1 = min(j0 + kLinBlocks, a.nbk);
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  if (wv == 0) {   // the halves of the unrouted blocks, in order
    const int j = j0 + lane;
    const bool un = j < j1 && a.counts[(size_t)bh * a.nbk + j] == 0;
    const unsigned long long m = __ballot(un);
    if (un) {
      const int pos = __popcll(m & ((1ull << lane) - 1ull));
      items[2 * pos] = 2 * j;
      items[2 * pos + 1] = 2 * j + 1;
    }
    if (lane == 0) nitems = 2 * __popcll(m);
  }
  for (int e = t; e < (j1 - j0) * D; e += 256)
    zs[e] = a.gz[((size_t)bh * a.nbk + j0) * D + e];
  __syncthreads();
  const int n = __builtin_amdgcn_readfirstlane(nitems);
  if (n == 0) return;   // uniform: every block here was routed
  stage_g_sum<D, 256>(a, bh, nullptr, Gs, Gl);
  __syncthreads();
  // Item it covers keys 32 items[it] .. + 31 (block items[it] / 2, half items[it] % 2), of
  // which nrows(it) exist. Its loads and stores go through buffer resources that end at the
  // last existing key: rows past it read as zero and are not written, with no branch (a
  // branch around a load or store leaves the compiler's wait counts at their most cautious).
  // (item, wave and count are wave-uniform: read as such, the resources stay scalar)
  auto first = [&](int it) { return min(32 * __builtin_amdgcn_readfirstlane(items[it]), a.nkv); };
  auto nrows = [&](int it) { return min(a.nkv - first(it), 32); };
  const uint16_t* kbase = a.k + (size_t)bh * a.nkv * D;
  const uint16_t* vbase = a.v + (size_t)bh * a.nkv * D;
  // this lane's 8-channel pieces 16 s + 8 h .. of its key's row of K or V
  auto load = [&](const uint16_t* base, int it, u32x4* f) {
    const auto rs = buf_rsrc(base + (size_t)first(it) * D, nrows(it) * D * 2);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      f[s] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (l32 * D + 16 * s + 8 * h) * 2, 0, 0));
  };
  // LDS element offsets of this lane's G fragments. Row reads (G^T row 32 c + l32, columns
  // 16 s + 8 h ..): the swizzle XORs the chunk with row % (D / 8), the same for every c, so
  // c is a constant offset and s picks one of KS bases. Transposing reads (tr_nat at x0 =
  // 32 c, k0 = 16 s): rows 16 s + 8 (g / 2) + L / 4 (+ 4) keep row % 16 for every s, so s is a
  // constant offset and (c, upper four rows) picks one of 2 CT bases.
  static_assert(D / 8 <= 16, "row % chunks is independent of the 16-row step");
  static_assert(CT % 2 == 0, "slices go in pairs");
  int rb[KS], tb[CT][2];
#pragma unroll
  for (int s = 0; s < KS; ++s) rb[s] = swz<D>(l32, 16 * s + 8 * h);
  {
    const int g = lane >> 4, L = lane & 15;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        tb[c][u] = swz<D>(8 * (g >> 1) + (L >> 2) + 4 * u, 32 * c + 16 * (g & 1) + 4 * (L & 3));
  }
  auto tr_frag = [&](const uint16_t* M, int c, int s) {
    const u32x2 lo = lds_read_tr16(M + tb[c][0] + 16 * s * D);
    const u32x2 hi = lds_read_tr16(M + tb[c][1] + 16 * s * D);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  // Per item: dV^T = G^T relu(K)^T first (K only), then dK^T = G V^T (V only), so that V's
  // load is in flight during the dV half; the next item's K loads during this one.
  // k > 0 of this lane's key at channels 16 s + 8 h + e (bit 8 s + e); the partner lane
  // (lane ^ 32) holds the channels 16 s + 8 (1 - h) + e
  auto kmask = [&](const u32x4* f) {
    uint64_t m = 0;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m |= (uint64_t)(bf16_lo(f[s][e]) > 0.f) << (8 * s + 2 * e);
        m |= (uint64_t)(bf16_hi(f[s][e]) > 0.f) << (8 * s + 2 * e + 1);
      }
    return m;
  };
  // K of an item and its mask are both ready at the loop head on every path into it (the
  // mask consumes the load), so the compiler's wait there does not hold for the stores
  // issued after the next item's K load.
  const int w0 = __builtin_amdgcn_readfirstlane(wv);
  u32x4 kf[KS];
  uint64_t own = 0;
  if (w0 < n) {
    load(kbase, w0, kf);
    own = kmask(kf);
  }
  for (int it = w0; it < n; it += 4) {
    // keeps the G fragment reads inside the loop (hoisted, they would not fit in registers)
    asm volatile("" ::: "memory");
    const uint64_t other = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(own >> 32), 32, 64) << 32) |
                           (uint32_t)__shfl_xor((int)(uint32_t)own, 32, 64);
    // bit 16 c + 4 g4 + e: k > 0 at output row 32 c + 8 g4 + 4 h + e of the epilogue (16-channel
    // group 2 c + g4 / 2, half g4 & 1, element 4 h + e within it)
    uint64_t need = 0;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const uint64_t pm = ((g4 & 1) == h) ? own : other;
        need |= ((pm >> (8 * (2 * c + (g4 >> 1)) + 4 * h)) & 15u) << (16 * c + 4 * g4);
      }
    u32x4 kb[KS], vf[KS], kn[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) kb[s] = relu_bf16x8(kf[s]);
    load(vbase, it, vf);
    load(kbase, min(it + 4, n - 1), kn);   // the last item's K again after the last item
    const int jl = (__builtin_amdgcn_readfirstlane(items[it]) >> 1) - j0;
    const size_t o = (size_t)bh * a.nkv + first(it);
    const auto rdk = buf_rsrc(a.dk + o * D, nrows(it) * D * 4);
    const auto rdv = buf_rsrc(a.dv + o * D, nrows(it) * D * 4);
    // dV^T rows 32 c .. 32 c + 31, two slices at a time
#pragma unroll
    for (int c0 = 0; c0 < CT; c0 += 2) {
      f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s % 2 == 0) asm volatile("" ::: "memory");   // two 16-channel groups in flight
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int c = c0 + u;
          const u32x4 gh = *reinterpret_cast<const u32x4*>(Gs + rb[s] + 32 * c * D);
          const u32x4 glo = *reinterpret_cast<const u32x4*>(Gl + rb[s] + 32 * c * D);
          acc[u] = mfma_bf16(gh, kb[s], acc[u]);
          acc[u] = mfma_bf16(glo, kb[s], acc[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int r0 = 32 * (c0 + u) + 8 * g4 + 4 * h;
          const f32x4 vo{acc[u][4 * g4], acc[u][4 * g4 + 1], acc[u][4 * g4 + 2], acc[u][4 * g4 + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, vo), rdv,
                                                 (l32 * D + r0) * 4, 0, 0);
        }
    }
    own = kmask(kn);   // the next item's
    // dK^T rows (V G^T + gz) (.) 1[k > 0], two slices at a time
#pragma unroll
    for (int c0 = 0; c0 < CT; c0 += 2) {
      f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s % 2 == 0) asm volatile("" ::: "memory");
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          acc[u] = mfma_bf16(tr_frag(Gs, c0 + u, s), vf[s], acc[u]);
          acc[u] = mfma_bf16(tr_frag(Gl, c0 + u, s), vf[s], acc[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int c = c0 + u, r0 = 32 * c + 8 * g4 + 4 * h;
          const f32x4 z = *reinterpret_cast<const f32x4*>(zs + jl * D + r0);
          const uint32_t bits = (uint32_t)(need >> (16 * c + 4 * g4)) & 15u;
          f32x4 ko;
#pragma unroll
          for (int e = 0; e < 4; ++e) ko[e] = (bits >> e) & 1u ? acc[u][4 * g4 + e] + z[e] : 0.f;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ko), rdk,
                                                 (l32 * D + r0) * 4, 0, 0);
        }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = kn[s];
  }
}

// ----------------------------------------------------------------------------- dQ of the exact branch
template <int D>
__global__ __launch_bounds__(128) void bwd_dq_kernel(BwdArgs a) {
  constexpr int KS = D / 16, CT = D / 32, TILE = 64 * D;
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE];
  const int bh = blockIdx.x / a.nbq, iq = blockIdx.x % a.nbq;
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int row = 32 * wv + l32;
  const int n = iq * kBlock + row;
  const bool valid = n < a.nq;
  const float qk_scale = kLog2e / sqrtf((float)D);
  const float tau = 1.f / sqrtf((float)D);
  const uint16_t* qrow = a.q + ((size_t)bh * a.nq + (valid ? n : 0)) * D;
  const uint16_t* drow = a.dos + ((size_t)bh * a.nbq * kBlock + iq * kBlock + row) * D;
  u32x4 qf[KS], of[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = valid ? *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};
    of[s] = *reinterpret_cast<const u32x4*>(drow + 16 * s + 8 * h);
  }
  const float lse = a.lse[(size_t)bh * a.nbq * kBlock + iq * kBlock + row];
  const float dn = a.dr[(size_t)bh * a.nbq * kBlock + iq * kBlock + row];
  f32x16 dqt[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) dqt[c] = f32x16{};
  // Two slots of (K tile, V-swizzled: row reads and vt_frag reads; f16 V tile, row swizzle):
  // the next selected block's tiles load straight into LDS while this one is multiplied.
  // the selection, staged in LDS (topk words of dynamic shared memory) so that the next
  // block's address is no memory round trip inside the loop
  const int32_t* selg = a.idx + ((size_t)bh * a.nbq + iq) * a.topk;
  extern __shared__ int32_t sel[];
  for (int e = t; e < a.topk; e += 128) sel[e] = selg[e];
  __syncthreads();
  auto stage = [&](int e, int slot) __attribute__((always_inline)) {
    const int j = sel[e];
    dma_tile<D, true, 2>(smem + 2 * slot * TILE, a.k + ((size_t)bh * a.nkv + (size_t)j * kBlock) * D,
                         min(kBlock, a.nkv - j * kBlock));
    dma_tile<D, false, 2>(smem + (2 * slot + 1) * TILE,
                          a.v16 + ((size_t)bh * a.nbk * kBlock + (size_t)j * kBlock) * D, kBlock);
  };
  if (a.topk > 0) stage(0, 0);
  drain_barrier();
  int slot = 0;
  for (int e = 0; e < a.topk; ++e) {
    if (e + 1 < a.topk) stage(e + 1, slot ^ 1);
    const int j = sel[e];
    const int nval = min(kBlock, a.nkv - j * kBlock);
    const uint16_t* Ks = smem + 2 * slot * TILE;
    const uint16_t* Vs = smem + (2 * slot + 1) * TILE;
    f32x16 st[2] = {f32x16{}, f32x16{}}, dpt[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        st[mt] = mfma_bf16(row_frag<D, true>(Ks, 32 * mt + l32, 16 * s + 8 * h), qf[s], st[mt]);
        dpt[mt] = mfma_f16(row_frag<D, false>(Vs, 32 * mt + l32, 16 * s + 8 * h), of[s], dpt[mt]);
      }
    u32x4 df[4], dl[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float dsv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int el = 8 * hh + 2 * e2 + u;
            const int kk = 32 * mt + 8 * (el >> 2) + 4 * h + (el & 3);
            const float p = kk < nval ? __builtin_amdgcn_exp2f(__builtin_fmaf(st[mt][el], qk_scale, -lse)) : 0.f;
            dsv[u] = p * (dpt[mt][el] - dn);   // tau is applied to the sum
          }
          const uint32_t hi = pack_bf16(dsv[0], dsv[1]);
          df[2 * mt + hh][e2] = hi;
          dl[2 * mt + hh][e2] = pack_bf16(dsv[0] - bf16_lo(hi), dsv[1] - bf16_hi(hi));
        }
    // dS enters as bf16 high and low parts: its rows sum to zero, so dQ is a small difference
    // of large terms and one bf16 rounding of dS would show in it
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const u32x4 ka = vt_frag<D>(Ks, 32 * c, 16 * kk);
        dqt[c] = mfma_bf16(ka, df[kk], dqt[c]);
        dqt[c] = mfma_bf16(ka, dl[kk], dqt[c]);
      }
    drain_barrier();   // the next tiles have landed; this slot is free
    slot ^= 1;
  }
  if (!valid) return;
  float* dqr = a.dq + ((size_t)bh * a.nq + n) * D;
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int r0 = 32 * c + 8 * g4 + 4 * h;
      f32x4 cur = *reinterpret_cast<const f32x4*>(dqr + r0);
#pragma unroll
      for (int e = 0; e < 4; ++e) cur[e] += tau * dqt[c][4 * g4 + e];
      *reinterpret_cast<f32x4*>(dqr + r0) = cur;
    }
}

// dalpha[h][c] = sum over batches and query blocks of the partials: eight interleaved
// partial sums per channel (rows r = p, p + 8, ... in order), then the eight in order.
template <int D>
__global__ __launch_bounds__(256) void bwd_dalpha_kernel(const float* __restrict__ part,
                                                         float* __restrict__ dalpha, int B, int H,
                                                         int nbq) {
  __shared__ float red[8][32];
  const int hd = blockIdx.x, c = blockIdx.y * 32 + (threadIdx.x & 31), p = threadIdx.x >> 5;
  const int rows = B * nbq;
  float s = 0.f;
  for (int r = p; r < rows; r += 8) {
    const int b = r / nbq, i = r % nbq;
    s += part[(((size_t)b * H + hd) * nbq + i) * D + c];
  }
  red[p][threadIdx.x & 31] = s;
  __syncthreads();
  if (threadIdx.x < 32) {
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) tot += red[q][threadIdx.x];
    dalpha[(size_t)hd * D + c] = tot;
  }
}

template <int D>
hipError_t launch_backward_T(const Plan& s, const BwdPlan& bp, BwdArgs a, char* ws,
                             hipStream_t st) {
  const int nwk = s.nwords;
  hipLaunchKernelGGL(bwd_clear_kernel, dim3(512), dim3(256), 0, st,
                     reinterpret_cast<uint32_t*>(ws + bp.bitsT), (size_t)s.BH * s.nbk * a.nwq,
                     reinterpret_cast<int32_t*>(ws + bp.counts), (size_t)s.BH * s.nbk);
  hipLaunchKernelGGL(bwd_bits_kernel, dim3(s.nbq, s.BH), dim3(256),
                     (size_t)(nwk > 1 ? nwk : 1) * 4, st, a.idx,
                     reinterpret_cast<uint32_t*>(ws + s.selbits),
                     reinterpret_cast<uint32_t*>(ws + bp.bitsT),
                     reinterpret_cast<int32_t*>(ws + bp.counts), s.nbq, s.nbk, s.k, nwk, a.nwq);
  hipError_t e;
  if (bwd_few_sc(s)) {   // S_c(i) = S_tot - the selected blocks' summaries
    e = launch_kv_totals_blocks(s, a.k, a.v, ws, st);
    if (e != hipSuccess) return e;
    e = launch_sc_subtract(s, a.k, a.v, a.idx, reinterpret_cast<const float*>(ws + s.stot),
                           const_cast<float*>(a.sc), ws, st);
    if (e != hipSuccess) return e;
  } else {
    uint16_t* sblo = reinterpret_cast<uint16_t*>(ws + bp.sblo);
    e = launch_kv_summary(s, a.k, a.v, nullptr, ws, st, false, sblo);
    if (e != hipSuccess) return e;
    e = launch_complement_f32(s, reinterpret_cast<const uint32_t*>(ws + s.selbits), nwk, s.nbq,
                              s.nbk, s.k, reinterpret_cast<const uint16_t*>(ws + s.sblk), sblo,
                              const_cast<float*>(a.sc), st);
    if (e != hipSuccess) return e;
  }
  e = launch_complement_z(s, a.idx, ws, st);
  if (e != hipSuccess) return e;
  e = launch_sparse_save(s, a.q, a.k, a.idx, const_cast<float*>(a.os), const_cast<float*>(a.lse),
                         ws, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_query_kernel<D>, dim3(s.BH * s.nbq), dim3(128), 0, st, a);
  if (a.gt) {   // else the key kernel sums each G_j from the few dS_c(i) itself
    e = launch_complement_f32(s, reinterpret_cast<const uint32_t*>(ws + bp.bitsT), a.nwq, s.nbk,
                              s.nbq, 0, a.dsc, a.dsclo, const_cast<float*>(a.gt), st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_gz_kernel<D>, dim3(s.BH * ((s.nbk + kGzBlocks - 1) / kGzBlocks)),
                     dim3(D), 0, st, a);
  if (a.gt) {
    hipLaunchKernelGGL(bwd_order_kernel, dim3(1), dim3(1024), 0, st,
                       reinterpret_cast<const int32_t*>(ws + bp.counts), s.BH * s.nbk, s.nbq,
                       const_cast<int32_t*>(a.order));
    hipLaunchKernelGGL(bwd_key_kernel<D>, dim3(s.BH * s.nbk), dim3(128), (size_t)a.nwq * 4, st,
                       a);
  } else {   // few query blocks: routed key blocks in bwd_key_kernel, the others linear only
    const int cap = s.nbk < s.nbq * s.k ? s.nbk : s.nbq * s.k;
    if (cap > 0) {
      hipLaunchKernelGGL(bwd_routed_kernel, dim3(s.BH), dim3(256), 0, st,
                         reinterpret_cast<const int32_t*>(ws + bp.counts), s.nbk, cap,
                         const_cast<int32_t*>(a.order));
      hipLaunchKernelGGL(bwd_key_kernel<D>, dim3(s.BH * cap), dim3(128), (size_t)a.nwq * 4, st,
                         a);
    }
    hipLaunchKernelGGL(bwd_key_linear_kernel<D>,
                       dim3((s.nbk + kLinBlocks - 1) / kLinBlocks * s.BH), dim3(256), 0, st, a);
  }
  hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(s.BH * s.nbq), dim3(128), (size_t)s.k * 4, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const Plan& s, const void* q, const void* k, const void* v,
                           const float* alpha, const void* dout, const int32_t* idx, float* dq,
                           float* dk, float* dv, float* dalpha, char* ws, hipStream_t st) {
  const BwdPlan bp = make_bwd_plan(s);
  BwdArgs a;
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.k = reinterpret_cast<const uint16_t*>(k);
  a.v = reinterpret_cast<const uint16_t*>(v);
  a.v16 = reinterpret_cast<const uint16_t*>(ws + s.v16);
  a.dout = dout;
  a.dout_bf16 = s.out_bf16 ? 1 : 0;
  a.alpha = alpha;
  a.idx = idx;
  a.bitsT = reinterpret_cast<const uint32_t*>(ws + bp.bitsT);
  a.sc = reinterpret_cast<const float*>(ws + bp.scf);
  a.zc = reinterpret_cast<const float*>(ws + s.zc);
  a.os = reinterpret_cast<const float*>(ws + bp.os);
  a.lse = reinterpret_cast<const float*>(ws + bp.lse);
  a.dr = reinterpret_cast<float*>(ws + bp.dr);
  a.dos = reinterpret_cast<uint16_t*>(ws + bp.dos);
  a.dsc = reinterpret_cast<uint16_t*>(ws + bp.dsc);
  a.dsclo = reinterpret_cast<uint16_t*>(ws + bp.dsclo);
  a.dzc = reinterpret_cast<float*>(ws + bp.dzc);
  a.gt = bwd_few_g(s) ? nullptr : reinterpret_cast<const float*>(ws + bp.gt);
  a.gz = reinterpret_cast<float*>(ws + bp.gz);
  a.dapart = reinterpret_cast<float*>(ws + bp.dapart);
  a.order = reinterpret_cast<const int32_t*>(ws + bp.order);
  a.counts = reinterpret_cast<const int32_t*>(ws + bp.counts);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.nq = s.nq; a.nkv = s.nkv; a.nbq = s.nbq; a.nbk = s.nbk; a.topk = s.k; a.H = s.H;
  a.nwq = bp.nwq;
  hipError_t e = s.D == 128 ? launch_backward_T<128>(s, bp, a, ws, st)
                            : launch_backward_T<64>(s, bp, a, ws, st);
  if (e != hipSuccess) return e;
  if (s.D == 128)
    hipLaunchKernelGGL(bwd_dalpha_kernel<128>, dim3(s.H, 128 / 32), dim3(256), 0, st, a.dapart,
                       dalpha, s.B, s.H, s.nbq);
  else
    hipLaunchKernelGGL(bwd_dalpha_kernel<64>, dim3(s.H, 64 / 32), dim3(256), 0, st, a.dapart,
                       dalpha, s.B, s.H, s.nbq);
  return hipGetLastError();
}

}  // namespace sla
