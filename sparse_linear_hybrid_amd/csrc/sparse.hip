// Sparse branch (SLA2 page, sections 1 and 2.B: exact softmax attention on the routed key
// blocks) with the linear-branch apply and the alpha mix (section 2.A) fused into the
// epilogue.
//
// A workgroup handles QB consecutive query blocks of one (batch, head) with 2*QB waves;
// wave w owns the 32 query rows 32*(w%2) .. +31 of query block w/2 and all 64 keys of each
// key tile, so every softmax row lives in one wave. The workgroup walks the ascending union
// of its query blocks' selections: neighbouring query blocks mostly select the same key
// blocks, so each shared K/V tile is staged in LDS once for all of them; a wave skips the
// tiles its own query block did not select.
//
// Per tile and wave, everything is computed transposed so that no register shuffles are
// needed:
//   S^T (64 keys x 32 queries) = K Q^T        bf16 MFMA 32x32x16, fp32 accumulate
//   O^T (d x 32 queries)     += V^T P^T       f16 MFMA 32x32x16 (P in [0, 2^8]), fp32
// Softmax runs in base 2 with the 1/sqrt(d) scale folded into the exponent's FMA; the row
// sum adds the f16-rounded P actually used by the P.V product.
// The S^T accumulator layout (lane = query column, 16 key rows per lane per 32-key half) is
// the B-operand layout P^T needs, up to a fixed permutation of the keys inside each 16-key
// step; the V^T operand is read from the row-major V tile with transposing LDS reads in the
// same permuted key order. LDS rows are XOR-swizzled in 16-byte chunks so that both the K
// fragment reads and the transposing V reads are free of bank conflicts.
//
// Epilogue per wave: O_s = O / l; O_l^T = S_c^T phi(Q)^T / (phi(Q) . z_c + eps) on bf16 MFMA
// (phi(Q)^T is the register-resident Q fragment with ReLU applied);
// O = alpha O_s + (1 - alpha) O_l.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace sla {

namespace {


// Ascending walk over the union of QB ascending selection lists. Each list is held 64
// entries at a time in a VGPR (lane l: entry base + l) and read with readlane, so the walk
// costs no memory round trip per step.
template <int QB>
struct UnionWalk {
  const int32_t* selp[QB];
  int nsel[QB], ptr[QB], base[QB], head[QB];
  int selv[QB];

  __device__ __forceinline__ void reload(int b) {
    const int lane = threadIdx.x & 63;
    selv[b] = base[b] + lane < nsel[b] ? selp[b][base[b] + lane] : 0;
  }
  __device__ __forceinline__ int read(int b) {
    if (ptr[b] - base[b] >= 64) {
      base[b] += 64;
      reload(b);
    }
    return __builtin_amdgcn_readlane(selv[b], ptr[b] - base[b]);
  }
  __device__ __forceinline__ void init(const int32_t* idx, int bh, int nbq, int grp, int k) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int ib = grp * QB + b;
      selp[b] = idx + ((size_t)bh * nbq + (ib < nbq ? ib : 0)) * k;
      nsel[b] = ib < nbq ? k : 0;
      ptr[b] = 0;
      base[b] = 0;
      reload(b);
      head[b] = nsel[b] > 0 ? __builtin_amdgcn_readlane(selv[b], 0) : 0x7fffffff;
    }
  }
  // next key block of the union and the mask of lists that contain it
  __device__ __forceinline__ bool next_direct(int& j, int& flags) {
    j = 0x7fffffff;
#pragma unroll
    for (int b = 0; b < QB; ++b) j = min(j, head[b]);
    flags = 0;
#pragma unroll
    for (int b = 0; b < QB; ++b)
      if (head[b] == j && j != 0x7fffffff) {
        flags |= 1 << b;
        ++ptr[b];
        head[b] = ptr[b] < nsel[b] ? read(b) : 0x7fffffff;
      }
    return flags != 0;
  }

  // The walk is buffered 64 union entries at a time (lane i: entry i, key block | flags<<24,
  // -1 past the end), so the per-step read is a readlane and any list reload, with its wait
  // on all outstanding loads, happens once per 64 steps.
  int uvec = -1, upos = 64;
  // Quantised branch: each buffered entry's key-block exponents (e_K low 16 bits, e_V high,
  // both signed) are gathered with the entries, so no step waits on a load of its own.
  const int32_t* ekp = nullptr;
  const int32_t* evp = nullptr;
  int evec = 0, ex = 0;
  __device__ __forceinline__ int exps(int j) const {
    return (ekp[j] & 0xffff) | (evp[j] << 16);
  }
  __device__ __forceinline__ void fill() {
    uvec = -1;
#pragma unroll 1
    for (int i = 0; i < 64; ++i) {
      int j, f;
      if (!next_direct(j, f)) break;     // lanes past the end of the walk stay -1
      uvec = (int)(threadIdx.x & 63) == i ? (j | (f << 24)) : uvec;
    }
    if (ekp != nullptr) evec = uvec >= 0 ? exps(uvec & 0xffffff) : 0;
    upos = 0;
  }
  __device__ __forceinline__ bool next(int& j, int& flags) {
    if (upos == 64) fill();
    const int e = __builtin_amdgcn_readlane(uvec, upos);
    if (ekp != nullptr) ex = __builtin_amdgcn_readlane(evec, upos);
    ++upos;
    j = e & 0xffffff;
    flags = e < 0 ? 0 : e >> 24;
    return e >= 0;
  }
};

struct SparseArgs {
  const void* q;
  const void* k;
  const uint16_t* v16;     // f16 [BH][nbk*64][D], rows beyond n_kv are zero
  const int32_t* idx;      // [BH][nbq][top_k], ascending
  const uint16_t* sc;      // bf16 S_c^T [BH][nbq][D(c)][D(r)]
  const float* zc;         // [BH][nbq][D]
  const float* alpha;      // [H][D]
  void* out;
  int nq, nkv, nbq, nbk, topk, H, ngroups, total;
  // quantised branch only
  uint16_t* q8;            // E4M3 values of Q as bf16 [BH][nbq*64][D] (written here)
  const uint16_t* k8;      // E4M3 values as bf16 [BH][nbk*64][D]
  const uint8_t* v8;       // E4M3 [BH][nbk][D][64], keys in P8 slot order
  int32_t* eq;             // Q's block exponents [BH][nbq] (written here)
  const int32_t* ek;       // [BH][nbk]
  const int32_t* ev;       // [BH][nbk]
  // piecewise epilogue only
  const uint16_t* hbar;    // bf16 H_bar^T [BH][D(c)][D(r)]
  const float* tail_m;     // [BH][nbq * 64]: the tail's running max (base-2 scaled units)
  const float* tail_d;     // its token-count-weighted row sum
  const float* tail_a;     // its plain row sum
  const float* tail_n;     // [BH][nbq * 64][D]: its numerator
  // saved exact-branch state for the backward only
  float* lse;              // [BH][nbq * 64]: m + log2(l) in base-2 scaled units (kNoRowLse
                           // for a row with no exact part or past n_q)
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
    const uint32_t hv = pack_bf16(x[2 * e], x[2 * e + 1]);
    hi[e] = hv;
    lo[e] = pack_bf16(x[2 * e] - bf16_lo(hv), x[2 * e + 1] - bf16_hi(hv));
  }
}

// SAVE (bf16 inputs, for the backward): instead of the linear apply and the mix, the
// epilogue writes the exact branch's normalised output O_s (fp32, `out` [BH][n_q][D]) and each
// row's log-sum-exp (`lse`).
// The exact branch's body, shared by the bf16/fp32 kernel and the quantised one (FP8).
template <typename T, int D, int QB, bool OUT_BF16, bool PISA, bool SAVE, bool FP8>
__device__ __forceinline__ void sparse_attn_body(const SparseArgs& a) {
  constexpr bool SPLIT = sizeof(T) == 4;   // fp32 inputs: three-term bf16 product
  constexpr bool DMA = !SPLIT;             // bf16 inputs: K/V tiles go global -> LDS directly
  static_assert(!FP8 || (DMA && !PISA && !SAVE), "quantised branch: bf16-input SLA2 forward");
  constexpr int NT = 128 * QB;             // threads
  constexpr int NW = 2 * QB;               // waves
  constexpr int KS = D / 16;               // 16-channel reduction steps for Q K^T
  constexpr int CT = D / 32;               // 32-channel tiles of the output
  constexpr int CH = D / 8;                // 16-byte chunks per row
  constexpr int CPT = SPLIT ? 64 * CH / NT : 1;   // chunks per thread per tile (register path)
  constexpr int KPW = 64 * D * 2 / 1024 / NW;     // 1-KB pieces per wave per tile (LDS DMA)
  constexpr int TILE = 64 * D;             // elements of one K or V tile
  constexpr int VT = FP8 ? TILE / 2 : TILE;   // 16-bit elements of one V slot (V8: 1 byte each)
  constexpr int VPW = FP8 ? D * 64 / 1024 / NW : KPW;   // 1-KB pieces per wave of a V tile
  // LDS DMA path: K ring of 3 tiles, then V ring of 2. Register path: K[2], V[2], Klo[2].
  __shared__ __attribute__((aligned(16))) uint16_t smem[(DMA ? 5 : 6) * TILE];

  const int wid = xcd_remap(blockIdx.x, a.total);
  const int bh = wid / a.ngroups, grp = wid % a.ngroups;
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int qb = wv >> 1;                       // this wave's query block within the group
  const int iq = grp * QB + qb;                 // its query block index
  const bool active = iq < a.nbq;
  const int qrow0 = iq * kBlock + 32 * (wv & 1);
  const T* qb_ptr = reinterpret_cast<const T*>(a.q) + (size_t)bh * a.nq * D;
  // quantised branch: K8 (E4M3 values held as bf16) and V8 tiles of 64 padded key rows
  const T* kb = FP8 ? reinterpret_cast<const T*>(a.k8) + (size_t)bh * a.nbk * kBlock * D
                    : reinterpret_cast<const T*>(a.k) + (size_t)bh * a.nkv * D;
  const uint16_t* vb = a.v16 + (size_t)bh * a.nbk * kBlock * D;
  const uint8_t* v8b = a.v8 + (size_t)bh * a.nbk * kBlock * D;

  // Q^T fragments (B operand): lane column q = qrow0 + l32, channels 16 s + 8 h .. +7
  // (the quantised branch turns them into Q8 below and reloads Q for the epilogue)
  u32x4 qf[KS];
  u32x4 ql[SPLIT ? KS : 1];
  {
    const int q = qrow0 + l32;
    const bool ok = active && q < a.nq;
    const int qc = ok ? q : 0;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if constexpr (SPLIT) {
        load_split_bf16x8(reinterpret_cast<const float*>(qb_ptr) + (size_t)qc * D + 16 * s + 8 * h,
                          qf[s], ql[s]);
        if (!ok) ql[s] = u32x4{0, 0, 0, 0};
      } else {
        qf[s] = load_bf16x8(qb_ptr + (size_t)qc * D + 16 * s + 8 * h);
      }
      if (!ok) qf[s] = u32x4{0, 0, 0, 0};
    }
  }

  // the selection lists load after Q, so that both round trips overlap
  UnionWalk<QB> walk;
  walk.init(a.idx, bh, a.nbq, grp, a.topk);
  if constexpr (FP8) {
    walk.ekp = a.ek + (size_t)bh * a.nbk;
    walk.evp = a.ev + (size_t)bh * a.nbk;
  }
  // Quantised branch: Q's E4M3 block quantisation (SLA2 page, section 2.C) from the
  // register-held fragments. e_Q is the smallest integer with 448 2^e_Q >= the query block's
  // absmax over its valid tokens (0 for an all-zero block); Q8 = E4M3(Q 2^-e_Q), one
  // round-to-nearest-even of an exactly scaled value, held as bf16 (exact). The two waves of
  // a query block meet through LDS for the absmax. Q8 (rows past n_q zero) and e_Q are also
  // written to the workspace.
  int eq = 0;
  if constexpr (FP8) {
    // the last 128 bytes of the LDS array, which neither the tile rings nor the epilogue's
    // staging reach (a separate array would take the footprint past two workgroups per CU)
    float* const qmax_lds = reinterpret_cast<float*>(smem + 5 * TILE - 64);
    static_assert(4 * TILE + 1024 <= 5 * TILE - 64, "ring and epilogue staging stay below");
    float amax = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(qf[s][e])), fabsf(bf16_hi(qf[s][e]))));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    if (lane == 0) qmax_lds[wv] = amax;
    __syncthreads();
    eq = e8m0_exponent(fmaxf(qmax_lds[2 * qb], qmax_lds[2 * qb + 1]));
    uint16_t* q8row = a.q8 + ((size_t)bh * a.nbq * kBlock + (active ? qrow0 + l32 : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = bf16_lo(qf[s][e]);
        v[2 * e + 1] = bf16_hi(qf[s][e]);
      }
      uint32_t w0, w1;
      e4m3x8(v, eq, w0, w1);
      qf[s] = e4m3x8_as_bf16(w0, w1);
      if (active) *reinterpret_cast<u32x4*>(q8row + 16 * s + 8 * h) = qf[s];
    }
    if (active && (wv & 1) == 0 && lane == 0)
      a.eq[(size_t)bh * a.nbq + iq] = eq;
  }

  f32x16 o[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) o[c] = f32x16{};
  // quantised branch: the running maximum is an integer, far below any logit at the start
  float m = FP8 ? -16384.f : kNegBig, l = 0.f;
  const float qk_scale = kLog2e / sqrtf((float)D);

  // LDS DMA: wave w moves the 1-KB pieces p = KPW w .. KPW w + KPW - 1 of the swizzled tile
  // (elements 512 p ..), each lane the logical chunk that the swizzle puts where it lands.
  // Lane l lands at element 512 p + 8 l of piece p: row 512 p / D + l / CH, physical chunk
  // l % CH. Its source offset is p KB plus a lane part (V), or p KB plus a lane part XORed
  // with a constant of the piece (K at d = 128, whose chunk swizzle sees the low bits of the
  // piece's first row), so two lane registers serve every piece.
  uint32_t klane = 0, vlane = 0;
  const int wvs = __builtin_amdgcn_readfirstlane(wv);
  if constexpr (DMA) {
    const int lr = lane / CH, pc = lane % CH;
    klane = (uint32_t)(lr * D * 2 + ((pc ^ lr) & (CH - 1)) * 16);
    vlane = (uint32_t)(lr * D * 2 + ((pc ^ swzv_f<D>(lr)) & (CH - 1)) * 16);
    if constexpr (FP8) {
      // V8 tile: D rows (channels) of 64 key bytes; 16-byte chunk c of row r sits at chunk
      // c ^ ((r / 4) % 4), so that the 16 lanes of a fragment read (16 consecutive rows, one
      // logical chunk) hit 16 distinct 16-byte bank groups. Lane l lands at row 16 p + l / 4,
      // physical chunk l % 4 of piece p.
      vlane = (uint32_t)((lane >> 2) * 64 + (((lane & 3) ^ ((lane >> 4) & 3)) * 16));
    }
  }
  // j < 0: an absent tile; the loads then cover an empty range (no memory access) so that
  // every step issues the same number of loads, which the vmcnt waits below rely on.
  // (pieces u0 .. u1 - 1 of this wave's share)
  auto stage_k = [&](int j, uint16_t* slot, int u0, int u1)
                     __attribute__((always_inline)) {
    const int row0 = j < 0 ? 0 : j * kBlock;
    const uint32_t bytes = j < 0 ? 0u : (uint32_t)(min(kBlock, a.nkv - row0) * D * 2);
    const auto r = make_rsrc(kb + (size_t)row0 * D, bytes);
#pragma unroll
    for (int u = u0; u < u1; ++u) {
      const int pp = wvs * KPW + u;
      const uint32_t xo = D == 128 ? (uint32_t)((pp & 3) << 6) : 0u;
      load_lds16(r, lds_addr(slot) + pp * 1024, (uint32_t)(pp * 1024) + (klane ^ xo));
    }
  };
  auto stage_v = [&](int j, uint16_t* slot, int u0, int u1)
                     __attribute__((always_inline)) {
    const int row0 = j < 0 ? 0 : j * kBlock;
    const auto r = FP8 ? make_rsrc(v8b + (size_t)row0 * D, j < 0 ? 0u : (uint32_t)(kBlock * D))
                       : make_rsrc(vb + (size_t)row0 * D, j < 0 ? 0u : (uint32_t)(kBlock * D * 2));
#pragma unroll
    for (int u = u0; u < u1; ++u) {
      const int pp = wvs * VPW + u;
      load_lds16(r, lds_addr(slot) + pp * 1024, (uint32_t)(pp * 1024) + vlane);
    }
  };

  // Register path (fp32 inputs): rows beyond n_kv read row n_kv-1; their logits are masked
  // to -inf, so the values never contribute.
  u32x4 kreg[CPT], vreg[CPT], klreg[SPLIT ? CPT : 1];
  auto load_tile = [&](int j) __attribute__((always_inline)) {
    const int row0 = j * kBlock;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int id = t + NT * u;
      const int r = id / CH, c = id % CH;
      const size_t goff = (size_t)min(row0 + r, a.nkv - 1) * D + c * 8;
      load_split_bf16x8(reinterpret_cast<const float*>(kb) + goff, kreg[u], klreg[u]);
      vreg[u] = *reinterpret_cast<const u32x4*>(vb + (size_t)(row0 + r) * D + c * 8);
    }
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int id = t + NT * u;
      const int r = id / CH, c = id % CH;
      const int off = swz<D>(r, c * 8);
      *reinterpret_cast<u32x4*>(&smem[buf * TILE + off]) = kreg[u];
      *reinterpret_cast<u32x4*>(&smem[(2 + buf) * TILE + swzv<D>(r, c * 8)]) = vreg[u];
      *reinterpret_cast<u32x4*>(&smem[(4 + buf) * TILE + off]) = klreg[u];
    }
  };

  // One routed tile for this wave, in two 32-key halves so that the MFMAs of one half run
  // while the VALU works on the other:
  //   S0 = K[0:32] Q^T; rescale check of half 0;
  //   S1 = K[32:64] Q^T            alongside  P0 = exp2(S0 - m) (f16), row sums;
  //   rescale check of half 1;
  //   O^T += V[0:32]^T P0^T        alongside  P1 = exp2(S1 - m), row sums;
  //   O^T += V[32:64]^T P1^T.
  // The online softmax runs in base 2 with the running max m in scaled units; the rescale of
  // O and l happens only when a half's max exceeds m by more than the slack (a uniform
  // branch, so each straight-line stretch between the checks can be interleaved). P0 is
  // formed before half 1 is checked and added to O after it, so a rescale at half 1 scales
  // P0 as well.
  u32x4 pf[4];
  auto qk_half = [&](const uint16_t* Kt, const uint16_t* Klo, int mt, f32x16& sh)
                     __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = swz<D>(32 * mt + l32, 16 * ks + 8 * h);
      const u32x4 af = *reinterpret_cast<const u32x4*>(&Kt[off]);
      sh = mfma_bf16(af, qf[ks], sh);
      if constexpr (SPLIT) {
        const u32x4 alo = *reinterpret_cast<const u32x4*>(&Klo[off]);
        sh = mfma_bf16(af, ql[ks], sh);
        sh = mfma_bf16(alo, qf[ks], sh);
      }
    }
  };
  // tail mask and rescale check of one half (its row max over 32 keys, both lane halves)
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 ones2 = {(_Float16)1.0f, (_Float16)1.0f};
  auto check_half = [&](f32x16& sh, int mt, int j) __attribute__((always_inline)) {
    if (__builtin_amdgcn_readfirstlane((j + 1) * kBlock > a.nkv ? 1 : 0)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = j * kBlock + 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
        sh[e] = key < a.nkv ? sh[e] : -INFINITY;
      }
    }
    float r = kNegBig;
#pragma unroll
    for (int e = 0; e < 16; ++e) r = fmaxf(r, sh[e]);
    r = fmaxf(r, swap_halves(r)) * qk_scale;
    if (__ballot(r > m + kRescaleSlack)) {
      const float mn = fmaxf(m, r);
      const float corr = __builtin_amdgcn_exp2f(m - mn);
      l *= corr;
#pragma unroll
      for (int c = 0; c < CT; ++c) o[c] *= corr;
      if (mt == 1) {
        const _Float16 ch = (_Float16)corr;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          pf[kk] = __builtin_bit_cast(u32x4, __builtin_bit_cast(f16x8, pf[kk]) * ch);
      }
      m = mn;
    }
  };
  // P^T fragments pf[2 mt], pf[2 mt + 1] of one half and its row-sum contribution
  auto exp_half = [&](const f32x16& sh, int mt) __attribute__((always_inline)) {
    float rs = 0.f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int e = 8 * hh + 2 * e2;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sh[e], qk_scale, -m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sh[e + 1], qk_scale, -m));
        const uint32_t pk = pack_f16(p0, p1);
        pf[2 * mt + hh][e2] = pk;
        rs = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), ones2, rs, false);
      }
    }
    l += rs;
  };
  // O^T += V^T P^T over the 32 keys of one half (two 16-key steps)
  auto pv_half = [&](const uint16_t* Vt, int mt) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 2 * mt; kk < 2 * mt + 2; ++kk) {
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const u32x4 vf = vt_frag<D>(Vt, 32 * c, 16 * kk);
        o[c] = mfma_f16(vf, pf[kk], o[c]);
      }
    }
  };
  // ld(p), p = 0 .. 3: a quarter of this step's tile loads into LDS, issued between the
  // phases so that the loads leave while the MFMAs of the phase before them run
  auto compute_tile = [&](const uint16_t* Kt, const uint16_t* Klo, const uint16_t* Vt, int j,
                          auto&& ld) __attribute__((always_inline)) {
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    if constexpr (SPLIT) {
      ld(0);
      qk_half(Kt, Klo, 0, s0);
      ld(1);
      check_half(s0, 0, j);
      qk_half(Kt, Klo, 1, s1);
      ld(2);
      exp_half(s0, 0);
      check_half(s1, 1, j);
      ld(3);
      pv_half(Vt, 0);
      exp_half(s1, 1);
      pv_half(Vt, 1);
    } else {
      // every K fragment of the tile is read from LDS before the first product, and the
      // V fragments of a half before its softmax, so that the reads are in flight while
      // the matrix cores and the softmax work
      u32x4 ka[KS], kb[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[ks] = *reinterpret_cast<const u32x4*>(&Kt[swz<D>(l32, 16 * ks + 8 * h)]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kb[ks] = *reinterpret_cast<const u32x4*>(&Kt[swz<D>(32 + l32, 16 * ks + 8 * h)]);
      ld(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s0 = mfma_bf16(ka[ks], qf[ks], s0);
      ld(1);
      check_half(s0, 0, j);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s1 = mfma_bf16(kb[ks], qf[ks], s1);
      u32x4 va[2 * CT];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int c = 0; c < CT; ++c) va[kk * CT + c] = vt_frag<D>(Vt, 32 * c, 16 * kk);
      ld(2);
      exp_half(s0, 0);
      check_half(s1, 1, j);
      ld(3);
      u32x4 vb[2 * CT];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int c = 0; c < CT; ++c) vb[kk * CT + c] = vt_frag<D>(Vt, 32 * c, 16 * (kk + 2));
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int c = 0; c < CT; ++c) o[c] = mfma_f16(va[kk * CT + c], pf[kk], o[c]);
      exp_half(s1, 1);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int c = 0; c < CT; ++c) o[c] = mfma_f16(vb[kk * CT + c], pf[2 + kk], o[c]);
    }
  };
  // Quantised branch (SLA2 page, section 2.C), one routed tile of this wave:
  //   S^T = K8 Q8^T on the bf16 MFMA over the E4M3 values (exact products, fp32 sums),
  //   y = S 2^(eQ + eK) log2(e) / sqrt(d);
  //   per (row, tile): T = floor(max y), P8 = E4M3(2^(y - T + 7)) in (0, 256);
  //   O^T += 2^(T - 7 - m + eV) V8^T P8^T on the scaled fp8 MFMA 32x32x64, the power-of-two
  //   weight applied through its E8M0 scale on P8.
  // The logits stay off the fp8 MFMA: on gfx950 it keeps only about 12-13 significant bits
  // when products of very different magnitude are summed, which the exponential turns into
  // errors of several percent for logits of a few hundred; for P.V the same relative error
  // stays about 1e-4 of sum p |v|. m is the row's running maximum kept on integers, so every
  // rescale is an exact power of two; the row sum adds the unquantised probabilities. In the
  // 32x32x64 MFMA each lane half holds 32 of the 64 reduction elements (the V8 rows are
  // stored in that key order); the two 32-element scale blocks take their E8M0 scale from
  // lanes x and x + 32, which always carry the same value here.
  auto compute_tile_fp8 = [&](const uint16_t* Kt, const uint8_t* Vt, int j, int exw,
                              auto&& ld) __attribute__((always_inline)) {
    u32x4 ka[KS], kb2[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      ka[ks] = *reinterpret_cast<const u32x4*>(&Kt[swz<D>(l32, 16 * ks + 8 * h)]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kb2[ks] = *reinterpret_cast<const u32x4*>(&Kt[swz<D>(32 + l32, 16 * ks + 8 * h)]);
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    ld(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sacc[0] = mfma_bf16(ka[ks], qf[ks], sacc[0]);
    ld(1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sacc[1] = mfma_bf16(kb2[ks], qf[ks], sacc[1]);
    // V8^T fragments: row 32 c + l32, key bytes 32 h .. 32 h + 31 (logical chunks 2h, 2h+1)
    i32x8 vf[CT];
    {
      const int x = (l32 >> 2) & 3;
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const uint8_t* row = Vt + (32 * c + l32) * 64;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(row + (((2 * h) ^ x) << 4));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(row + (((2 * h + 1) ^ x) << 4));
        vf[c] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
    }
    ld(2);
    const int ekj = (exw << 16) >> 16, evj = exw >> 16;
    const float cj = ldexpf(qk_scale, eq + ekj);
    if (__builtin_amdgcn_readfirstlane((j + 1) * kBlock > a.nkv ? 1 : 0)) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = j * kBlock + 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
          sacc[mt][e] = key < a.nkv ? sacc[mt][e] : -INFINITY;
        }
    }
    float r = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) r = fmaxf(r, sacc[mt][e]);
    r = fmaxf(r, swap_halves(r)) * cj;          // row max of y over the tile
    const float tmax = floorf(r);
    if (__ballot(r > m + kRescaleSlack)) {
      const float mn = fmaxf(m, ceilf(r));
      const float corr = ldexpf(1.f, (int)fmaxf(m - mn, -200.f));
      l *= corr;
#pragma unroll
      for (int c = 0; c < CT; ++c) o[c] *= corr;
      m = mn;
    }
    // P8 = E4M3(2^(y - T + 7)); slot 16 mt + e of this lane half holds accumulator element e
    // of key tile half mt
    const int wexp = (int)(tmax - 7.f - m) + evj;
    const bool live = wexp >= -127;   // weights below 2^-127 contribute nothing in fp32
    i32x8 pf8;
    float rs = 0.f;
    const float off = 7.f - tmax;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int mt = w >> 2, e0 = 4 * (w & 3);
      float p4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p4[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][e0 + i], cj, off));
        rs += p4[i];
      }
      int pk = 0;
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(p4[0], p4[1], pk, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(p4[2], p4[3], pk, true);
      pf8[w] = live ? pk : 0;
    }
    l += ldexpf(rs, (int)(tmax - 7.f - m));
    const int sb = min(max(127 + wexp, 0), 254);
    ld(3);
#pragma unroll
    for (int c = 0; c < CT; ++c)
      o[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[c], pf8, o[c], 0, 0, 0, 127, 0, sb);
  };
  auto no_loads = [](int) __attribute__((always_inline)) {};

  if constexpr (DMA) {
    // Ring pipeline. Step s computes tile s while V(s+1) and K(s+2) load (issued in that
    // order), then waits until at most the K(s+2) loads are in flight and meets the others
    // at one barrier: V(s+1) and K(s+1) have then landed. A K slot is rewritten two steps
    // after its Q K^T and a V slot one step after its P.V, both behind that barrier, so K
    // loads get two steps to land and V loads one.
    uint16_t* const kring = smem;
    uint16_t* const vring = smem + 3 * TILE;
    // The first two union entries come straight from the lists, so that their tiles are in
    // flight while the rest of the walk is buffered.
    int j0, f0, j1, f1;
    bool have0 = walk.next_direct(j0, f0);
    bool have1 = walk.next_direct(j1, f1);
    int ex0 = 0, ex1 = 0;   // quantised branch: the key blocks' exponents
    if constexpr (FP8) {
      ex0 = have0 ? walk.exps(j0) : 0;
      ex1 = have1 ? walk.exps(j1) : 0;
    }
    stage_k(have0 ? j0 : -1, kring, 0, KPW);
    stage_k(have1 ? j1 : -1, kring + TILE, 0, KPW);
    stage_v(have0 ? j0 : -1, vring, 0, VPW);
    walk.fill();
    barrier_vmem_n<0>();
    int ks = 0, vs = 0;
    while (have0) {
      int j2, f2;
      const bool have2 = walk.next(j2, f2);
      const int ex2 = walk.ex;
      const int ks2 = ks == 0 ? 2 : ks - 1;          // (ks + 2) % 3
      // V(s + 1) pieces first, then K(s + 2): the wait below counts on that order
      const int jv = have1 ? j1 : -1, jk = have2 ? j2 : -1;
      uint16_t* const vdst = vring + (vs ^ 1) * VT;
      uint16_t* const kdst = kring + ks2 * TILE;
      auto ld = [&](int p) __attribute__((always_inline)) {
        if (p < 2) stage_v(jv, vdst, p * VPW / 2, (p + 1) * VPW / 2);
        else stage_k(jk, kdst, (p - 2) * KPW / 2, (p - 1) * KPW / 2);
      };
      if ((f0 >> qb) & 1) {
        if constexpr (FP8)
          compute_tile_fp8(kring + ks * TILE, reinterpret_cast<const uint8_t*>(vring + vs * VT),
                           j0, ex0, ld);
        else
          compute_tile(kring + ks * TILE, nullptr, vring + vs * VT, j0, ld);
      } else {
        stage_v(jv, vdst, 0, VPW);
        stage_k(jk, kdst, 0, KPW);
      }
      barrier_vmem_n<KPW>();
      j0 = j1; f0 = f1; have0 = have1; ex0 = ex1;
      j1 = j2; f1 = f2; have1 = have2; ex1 = ex2;
      ks = ks == 2 ? 0 : ks + 1;
      vs ^= 1;
    }
    wait_vmem();   // no load into LDS outlives the workgroup
  } else {
    int j_cur, f_cur;
    bool have = walk.next(j_cur, f_cur);
    if (have) {
      load_tile(j_cur);
      store_tile(0);
    }
    __syncthreads();
    // Loop unrolled by two so that the LDS buffer of each half is a compile-time constant.
    auto step = [&](auto bufc) __attribute__((always_inline)) {
      constexpr int B = decltype(bufc)::value;
      int j_nxt, f_nxt;
      const bool have_nxt = walk.next(j_nxt, f_nxt);
      if (have_nxt) load_tile(j_nxt);
      if ((f_cur >> qb) & 1)
        compute_tile(smem + B * TILE, smem + (4 + B) * TILE, smem + (2 + B) * TILE, j_cur,
                     no_loads);
      if (have_nxt) store_tile(B ^ 1);
      __syncthreads();
      j_cur = j_nxt;
      f_cur = f_nxt;
      have = have_nxt;
    };
    while (have) {
      step(std::integral_constant<int, 0>{});
      if (!have) break;
      step(std::integral_constant<int, 1>{});
    }
  }
  // Linear-branch inputs of the epilogue (bf16 path, SLA2 mix): S_c^T of both query blocks,
  // their z_c and this head's alpha are staged into the idle tile ring with one round of
  // loads into LDS, so that no wave waits on several dependent global round trips. S_c^T of
  // query block qb takes two swizzled 64-row tiles at 2 qb TILE; z_c takes the 1 KB at 4 TILE
  // (each load into LDS writes 1 KB, lanes past the data write zeros), alpha the next 1 KB.
  constexpr bool STAGE_EPI = DMA && !PISA && !SAVE;
  if constexpr (STAGE_EPI) {
    __syncthreads();   // every wave has drained its ring loads (wait_vmem above)
    constexpr int SCP = D * D * 2 / 1024;           // 1-KB pieces of one S_c^T
    const int iqs = grp * QB + (wvs >> 1);            // iq, wave-uniform for the descriptor
    const int iqc = iqs < a.nbq ? iqs : a.nbq - 1;
    const auto rs = make_rsrc(a.sc + ((size_t)bh * a.nbq + iqc) * D * D, (uint32_t)(D * D * 2));
    const uint32_t sbase = lds_addr(smem + (wvs >> 1) * 2 * TILE);
#pragma unroll
    for (int u = 0; u < SCP / 2; ++u) {
      const int pc = (wvs & 1) * (SCP / 2) + u;        // piece of this wave
      const int e = pc * 512 + lane * 8;
      const int r = e / D, pch = (e % D) / 8;
      load_lds16(rs, sbase + pc * 1024, (uint32_t)(r * D * 2 + ((pch ^ r) & (CH - 1)) * 16));
    }
    if (wvs == 0) {
      const int iq0 = grp * QB;
      const auto rz = make_rsrc(a.zc + ((size_t)bh * a.nbq + iq0) * D,
                                (uint32_t)(min(QB, a.nbq - iq0) * D * 4));
      load_lds16(rz, lds_addr(smem + 4 * TILE), (uint32_t)(lane * 16));
    } else if (wvs == 1) {
      const auto ra = make_rsrc(a.alpha + (size_t)(bh % a.H) * D, (uint32_t)(D * 4));
      load_lds16(ra, lds_addr(smem + 4 * TILE + 512), (uint32_t)(lane * 16));
    }
    wait_vmem();
    __syncthreads();
  }
  if (!active) return;   // no barrier follows
  if constexpr (FP8) {
    // the epilogue's phi(Q) takes the unquantised Q
    const int q = qrow0 + l32;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = q < a.nq ? load_bf16x8(qb_ptr + (size_t)q * D + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};
  }

  // ---------------------------------------------------------------- epilogue
  l += swap_halves(l);
  if constexpr (SAVE) {
    const int q = qrow0 + l32;
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
    if (h == 0)
      a.lse[(size_t)bh * a.nbq * kBlock + (size_t)iq * kBlock + 32 * (wv & 1) + l32] =
          (l > 0.f && q < a.nq) ? m + log2f(l) : kNoRowLse;
    if (q < a.nq) {
      float* dst = reinterpret_cast<float*>(a.out) + ((size_t)bh * a.nq + q) * D;
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ch = 32 * c + 8 * g + 4 * h;
          *reinterpret_cast<f32x4*>(dst + ch) =
              f32x4{o[c][4 * g] * inv_l, o[c][4 * g + 1] * inv_l, o[c][4 * g + 2] * inv_l,
                    o[c][4 * g + 3] * inv_l};
        }
    }
    return;
  }
  if constexpr (PISA) {
    // Piecewise merge (PISA page, core algorithm): the exact part (o, l in the frame 2^m) and
    // the tail (N_U, D_U, A_U in the frame 2^m_U) share one normalisation; the first-order
    // term tau (q H_bar) A_U joins the tail's numerator.
    const int q = qrow0 + l32;
    const size_t row = (size_t)bh * a.nbq * kBlock + (q < a.nq ? q : qrow0);
    const float tm = a.tail_m[row], td = a.tail_d[row], ta = a.tail_a[row];
    const float mm = fmaxf(m, tm);
    const float cs = __builtin_amdgcn_exp2f(m - mm), cu = __builtin_amdgcn_exp2f(tm - mm);
    const float den = l * cs + td * cu;
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const float first = ta * cu * (1.f / sqrtf((float)D));
    const uint16_t* hb = a.hbar + (size_t)bh * D * D;
    const float* tn = a.tail_n + row * D;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      f32x16 lin = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const u32x4 af =
            *reinterpret_cast<const u32x4*>(hb + (size_t)(32 * c + l32) * D + 16 * s + 8 * h);
        lin = mfma_bf16(af, qf[s], lin);
      }
      if (q < a.nq) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ch = 32 * c + 8 * g + 4 * h;
          const f32x4 nu = *reinterpret_cast<const f32x4*>(tn + ch);
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ix = 4 * g + e;
            r[e] = (o[c][ix] * cs + nu[e] * cu + lin[ix] * first) * inv;
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
    return;
  }
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  const uint16_t* scb = a.sc + ((size_t)bh * a.nbq + iq) * D * D;
  const float* zcb = STAGE_EPI ? reinterpret_cast<const float*>(smem + 4 * TILE) + qb * D
                               : a.zc + ((size_t)bh * a.nbq + iq) * D;
  // A fragment of S_c^T (rows 32 c + lane % 32, columns 16 s + 8 h .. +7)
  auto sc_frag = [&](int c, int s_) __attribute__((always_inline)) {
    if constexpr (STAGE_EPI)
      return *reinterpret_cast<const u32x4*>(&smem[qb * 2 * TILE + swz<D>(32 * c + l32, 16 * s_ + 8 * h)]);
    else
      return *reinterpret_cast<const u32x4*>(scb + (size_t)(32 * c + l32) * D + 16 * s_ + 8 * h);
  };
  // phi(Q) . z_c for this lane's query: this lane holds channels 16 s + 8 h .. +7
  float d = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const f32x4 z0 = *reinterpret_cast<const f32x4*>(zcb + 16 * s + 8 * h);
    const f32x4 z1 = *reinterpret_cast<const f32x4*>(zcb + 16 * s + 8 * h + 4);
    const u32x4 w = qf[s];
    d += fmaxf(bf16_lo(w[0]), 0.f) * z0[0] + fmaxf(bf16_hi(w[0]), 0.f) * z0[1] +
         fmaxf(bf16_lo(w[1]), 0.f) * z0[2] + fmaxf(bf16_hi(w[1]), 0.f) * z0[3] +
         fmaxf(bf16_lo(w[2]), 0.f) * z1[0] + fmaxf(bf16_hi(w[2]), 0.f) * z1[1] +
         fmaxf(bf16_lo(w[3]), 0.f) * z1[2] + fmaxf(bf16_hi(w[3]), 0.f) * z1[3];
  }
  d += swap_halves(d);
  const float inv_den = 1.f / (d + kEps);
  const float* al = STAGE_EPI ? reinterpret_cast<const float*>(smem + 4 * TILE + 512)
                              : a.alpha + (size_t)(bh % a.H) * D;
  const int q = qrow0 + l32;
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    f32x16 lin = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) lin = mfma_bf16(sc_frag(c, s), relu_bf16x8(qf[s]), lin);
    if (q < a.nq) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = 32 * c + 8 * g + 4 * h;
        const f32x4 alv = *reinterpret_cast<const f32x4*>(al + ch);
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ix = 4 * g + e;
          r[e] = alv[e] * (o[c][ix] * inv_l) + (1.f - alv[e]) * (lin[ix] * inv_den);
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
}

template <typename T, int D, int QB, bool OUT_BF16, bool PISA = false, bool SAVE = false>
__global__ __launch_bounds__(128 * QB, 2) void sparse_attn_kernel(SparseArgs a) {
  sparse_attn_body<T, D, QB, OUT_BF16, PISA, SAVE, false>(a);
}

template <int D, int QB, bool OUT_BF16>
__global__ __launch_bounds__(128 * QB, 2) void sparse_attn_fp8_kernel(SparseArgs a) {
  sparse_attn_body<uint16_t, D, QB, OUT_BF16, false, false, true>(a);
}

template <typename T, int D, int QB, bool FP8, bool PISA = false>
hipError_t launch_sparse_T(const Plan& s, const void* q, const void* k, const int32_t* idx,
                           const float* alpha, void* o, char* ws, hipStream_t st) {
  SparseArgs a{};
  a.q = q;
  a.k = k;
  a.v16 = reinterpret_cast<const uint16_t*>(ws + s.v16);
  a.idx = idx;
  a.sc = reinterpret_cast<const uint16_t*>(ws + s.sc);
  a.zc = reinterpret_cast<const float*>(ws + s.zc);
  a.alpha = alpha;
  a.out = o;
  a.nq = s.nq; a.nkv = s.nkv; a.nbq = s.nbq; a.nbk = s.nbk; a.topk = s.k; a.H = s.H;
  a.ngroups = (s.nbq + QB - 1) / QB;
  a.total = s.BH * a.ngroups;
  a.q8 = reinterpret_cast<uint16_t*>(ws + s.q8);
  a.k8 = reinterpret_cast<const uint16_t*>(ws + s.k8);
  a.v8 = reinterpret_cast<const uint8_t*>(ws + s.v8);
  a.eq = reinterpret_cast<int32_t*>(ws + s.sq8);
  a.ek = reinterpret_cast<const int32_t*>(ws + s.sk8);
  a.ev = reinterpret_cast<const int32_t*>(ws + s.sv8);
  a.hbar = reinterpret_cast<const uint16_t*>(ws + s.hbar);
  a.tail_m = reinterpret_cast<const float*>(ws + s.tail_m);
  a.tail_d = reinterpret_cast<const float*>(ws + s.tail_d);
  a.tail_a = reinterpret_cast<const float*>(ws + s.tail_a);
  a.tail_n = reinterpret_cast<const float*>(ws + s.tail_n);
  if constexpr (PISA) {
    if (s.out_bf16)
      hipLaunchKernelGGL((sparse_attn_kernel<T, D, QB, true, true>), dim3(a.total), dim3(128 * QB), 0, st, a);
    else
      hipLaunchKernelGGL((sparse_attn_kernel<T, D, QB, false, true>), dim3(a.total), dim3(128 * QB), 0, st, a);
  } else if constexpr (FP8) {
    if (s.out_bf16)
      hipLaunchKernelGGL((sparse_attn_fp8_kernel<D, QB, true>), dim3(a.total), dim3(128 * QB), 0, st, a);
    else
      hipLaunchKernelGGL((sparse_attn_fp8_kernel<D, QB, false>), dim3(a.total), dim3(128 * QB), 0, st, a);
  } else {
    if (s.out_bf16)
      hipLaunchKernelGGL((sparse_attn_kernel<T, D, QB, true>), dim3(a.total), dim3(128 * QB), 0, st, a);
    else
      hipLaunchKernelGGL((sparse_attn_kernel<T, D, QB, false>), dim3(a.total), dim3(128 * QB), 0, st, a);
  }
  return hipGetLastError();
}

template <typename T, int D, bool FP8 = false, bool PISA = false>
hipError_t launch_sparse_D(const Plan& s, const void* q, const void* k, const int32_t* idx,
                           const float* alpha, void* o, char* ws, hipStream_t st) {
  // Pair neighbouring query blocks when there are enough of them to fill the GPU.
  if (s.nbq >= 2 && (long long)s.BH * s.nbq >= 1024)
    return launch_sparse_T<T, D, 2, FP8, PISA>(s, q, k, idx, alpha, o, ws, st);
  return launch_sparse_T<T, D, 1, FP8, PISA>(s, q, k, idx, alpha, o, ws, st);
}

}  // namespace

hipError_t launch_sparse(const Plan& s, const void* q, const void* k, const int32_t* idx,
                         const float* alpha, void* o, char* ws, hipStream_t st) {
  if (s.in_bf16) {
    if (s.D == 128) return launch_sparse_D<uint16_t, 128>(s, q, k, idx, alpha, o, ws, st);
    return launch_sparse_D<uint16_t, 64>(s, q, k, idx, alpha, o, ws, st);
  }
  if (s.D == 128) return launch_sparse_D<float, 128>(s, q, k, idx, alpha, o, ws, st);
  return launch_sparse_D<float, 64>(s, q, k, idx, alpha, o, ws, st);
}

hipError_t launch_sparse_pisa(const Plan& s, const void* q, const void* k, const int32_t* idx,
                              void* o, char* ws, hipStream_t st) {
  if (s.in_bf16) {
    if (s.D == 128) return launch_sparse_D<uint16_t, 128, false, true>(s, q, k, idx, nullptr, o, ws, st);
    return launch_sparse_D<uint16_t, 64, false, true>(s, q, k, idx, nullptr, o, ws, st);
  }
  if (s.D == 128) return launch_sparse_D<float, 128, false, true>(s, q, k, idx, nullptr, o, ws, st);
  return launch_sparse_D<float, 64, false, true>(s, q, k, idx, nullptr, o, ws, st);
}

hipError_t launch_sparse_save(const Plan& s, const void* q, const void* k, const int32_t* idx,
                              float* os, float* lse, char* ws, hipStream_t st) {
  if (!s.in_bf16) return hipErrorInvalidValue;
  SparseArgs a{};
  a.q = q;
  a.k = k;
  a.v16 = reinterpret_cast<const uint16_t*>(ws + s.v16);
  a.idx = idx;
  a.out = os;
  a.lse = lse;
  a.nq = s.nq; a.nkv = s.nkv; a.nbq = s.nbq; a.nbk = s.nbk; a.topk = s.k; a.H = s.H;
  auto go = [&](auto kern, int qb) {
    a.ngroups = (s.nbq + qb - 1) / qb;
    a.total = s.BH * a.ngroups;
    hipLaunchKernelGGL(kern, dim3(a.total), dim3(128 * qb), 0, st, a);
  };
  const bool pair = s.nbq >= 2 && (long long)s.BH * s.nbq >= 1024;
  if (s.D == 128) {
    if (pair) go(sparse_attn_kernel<uint16_t, 128, 2, false, false, true>, 2);
    else go(sparse_attn_kernel<uint16_t, 128, 1, false, false, true>, 1);
  } else {
    if (pair) go(sparse_attn_kernel<uint16_t, 64, 2, false, false, true>, 2);
    else go(sparse_attn_kernel<uint16_t, 64, 1, false, false, true>, 1);
  }
  return hipGetLastError();
}

hipError_t launch_sparse_fp8(const Plan& s, const void* q, const int32_t* idx,
                             const float* alpha, void* o, char* ws, hipStream_t st) {
  if (s.D == 128) return launch_sparse_D<uint16_t, 128, true>(s, q, nullptr, idx, alpha, o, ws, st);
  return launch_sparse_D<uint16_t, 64, true>(s, q, nullptr, idx, alpha, o, ws, st);
}

}  // namespace sla
