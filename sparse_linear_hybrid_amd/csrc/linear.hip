// Linear branch (SALAD page, section 2: ReLU kernel feature map with linear cost; SPLA
// page, section 2.2: the linear term over the unselected blocks equals the global linear
// term minus the selected blocks' term).
//
// kv_summary:  one pass over K and V. For every key block j: S_j = phi(K_j)^T V_j (d x d,
//              bf16 MFMA, fp32 accumulate, stored bf16 as S_j^T[c][r]), z_j = sum phi(K_j)
//              (fp32), the projected block mean of K (float64, for the router) and an f16
//              copy of V for the bf16 exact branch's P.V (the fp8 forward writes K8 and V8
//              instead). The next block's loads are in flight
//              while a block is processed. Per-chunk fp32 partial totals are written for a
//              fixed-order reduction (no atomics).
// reduce:      z_tot = sum of the chunk partials (fixed order); S_tot only where a pass keeps
//              d x d chunk totals (the summary cache, the piecewise statistics).
// complement:  per query block i, S_c(i) = sum of the S_j that i did not select: an MFMA
//              product of the 0/1 complement bitmap with the stacked S_j, slice by slice.
//              It equals S_tot - sum_{j in sel(i)} S_j exactly in real arithmetic, without that
//              difference's cancellation when the selected blocks hold most of the mass; an
//              all-blocks selection gives exactly 0. z_c(i) (fp32, d values per block) is
//              z_tot - sum_{j in sel(i)} z_j while at most half the blocks are selected, else
//              the direct sum of the unselected z_j.
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

// One pass over the key blocks jbase, jbase+1, ... (CHUNK per workgroup): the
// projected pooled K of each block (all its valid tokens) goes to kt + bh*kbh + j*kj, and
// phi(K)^T V, sum phi(K) over the tokens t0 <= t < nkv go into the chunk's partial totals.
// BLOCKS: also store each block's S_j^T, z_j and its f16 copy of V (the full forward; then
// jbase = t0 = 0). Without BLOCKS this is the key/value summary cache update. Pk = nullptr
// (the training-free router) skips k~.
// PISA (piecewise forward, PISA page, core algorithm; needs BLOCKS): the MFMA product uses
// the keys centred on their block mean instead of phi(K), so the partial totals add up
// H_j = sum_n (k_n - k_bar_j)^T v_n; no S_j or z_j is stored; instead each block's centroid
// (bf16 hi + lo, [BH][npad][D]) and its row of the value-sum table ([BH][npad][D] f16) are
// written.
// The per-block summaries S_j^T are stored slice-major: the flattened d x d matrix (row c,
// column r at c d + r) is cut into slices of kSlice consecutive elements, and slice s of
// every key block of a (batch, head) is contiguous: [BH][d d / kSlice][nbk][kSlice]. The
// complement reads one slice of consecutive key blocks per step.
constexpr int kSlice = 128;

// FP8 (fp8 forward, bf16 inputs; needs BLOCKS): the pass also quantises each block of K and V
// to E4M3 (SLA2 page, section 2.C) by the rule the quantised sparse kernel applies to Q: e =
// the smallest integer with 448 2^e >= the block's absmax over its valid tokens (0 for an
// all-zero block), x8 = E4M3(x 2^-e), one round-to-nearest-even of an exactly scaled value.
// It works from the tiles it has staged in LDS and writes K8 ([BH][nbk*64][D], the E4M3 values
// held as bf16, padded rows zero), the V8 tiles ([BH][nbk][D][64] bytes, channel-major, byte
// 32 hh + slot of a channel holding key 32 (slot / 16) + 8 ((slot % 16) / 4) + 4 hh + slot % 4:
// the order of the P8 operand of the P.V product) and the block exponents (Fp8Out). The f16
// copy of V, which only the bf16 exact branch reads, is not written on this path.
// NOSJ (the few-query-block backward, bf16 inputs): no S_j and no f16 copy of V are stored
// (sc_subtract_kernel writes that of the selected blocks); the pass keeps the d x d chunk
// totals instead (z_j and the z partials as usual).
template <typename T, int D, bool BLOCKS, int CHUNK, bool PISA = false, bool FP8 = false,
          bool LO = false, bool NOSJ = false>
__global__ __launch_bounds__(256, FP8 && D == 128 ? 3 : 2) void kv_summary_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ Pk,
    double* __restrict__ kt, size_t kbh, size_t kj, uint16_t* __restrict__ v16,
    uint16_t* __restrict__ sblk, uint16_t* __restrict__ sblk_lo, float* __restrict__ zblk, float* __restrict__ spart,
    float* __restrict__ zpart, int nkv, int nbk, int jbase, int t0,
    uint16_t* __restrict__ cent_hi, uint16_t* __restrict__ cent_lo, uint16_t* __restrict__ vsum,
    int npad, Fp8Out f8) {
  static_assert(!PISA || BLOCKS, "the piecewise pass is a full-forward pass");
  static_assert(!FP8 || (BLOCKS && !PISA && sizeof(T) == 2), "fused E4M3: bf16 full forward");
  static_assert(!LO || (BLOCKS && !PISA && !FP8), "low parts of S_j: plain full pass");
  static_assert(!NOSJ || (BLOCKS && !PISA && !FP8 && !LO), "totals instead of S_j: plain pass");
  // The SLA2 forward's complement sums the unselected S_j itself, so its pass keeps no d x d
  // chunk totals (only the z partials); the cache update, the piecewise pass and the
  // few-query-block backward do.
  constexpr bool TOTALS = !BLOCKS || PISA || NOSJ;
  constexpr int LS = D + 8;                  // padded LDS row (elements)
  constexpr int TPR = D / 8, RPP = 256 / TPR;
  constexpr int CPT = 64 * TPR / 256;        // 16-byte chunks per thread per tensor
  constexpr int NT = D / 32;                 // 32-wide tiles per dimension
  constexpr int TILES_PER_WAVE = NT * NT / 4;
  constexpr int EPC = sizeof(T) == 2 ? 1 : 2;   // 16-byte loads per 8-element chunk
  // K and V tiles, one array: the full forward stages each block's S_j^T over both
  __shared__ __attribute__((aligned(16))) uint16_t KVs[2 * 64 * LS];
  uint16_t* const Ks = KVs;
  uint16_t* const Vs = KVs + 64 * LS;
  static_assert(D * LS <= 2 * 64 * LS, "S_j^T staging fits the K and V tiles");
  __shared__ double pool_lds[4 * D];          // per-wave block sums (rows folded by shuffles)
  __shared__ double means[kSummaryChunk][D];   // pooled means of the current group of blocks
  __shared__ double vpool_lds[PISA ? 4 * D : 1];
  __shared__ float amax_lds[8];                                             // per wave: K, V

  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int j0 = jbase + chunk * CHUNK, j1 = min(j0 + CHUNK, nbk);
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
    double pacc[8], vacc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pacc[e] = vacc[e] = 0.0;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int cidx = t + 256 * u;
      const int r = cidx / TPR, c8 = cidx % TPR;
      const bool ok = r < nrows;                 // valid token: pooled
      const bool ok_sum = ok && row0 + r >= t0;  // and counted in the summaries
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
        pacc[e] += ok ? (double)kf[e] : 0.0;
        kf[e] = ok_sum ? kf[e] : 0.f;
        vf[e] = ok_sum ? vf[e] : 0.f;
        if constexpr (PISA) vacc[e] += (double)vf[e];
      }
      u32x4 kw, vw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kw[e] = pack_bf16(kf[2 * e], kf[2 * e + 1]);
        vw[e] = pack_bf16(vf[2 * e], vf[2 * e + 1]);
      }
      *reinterpret_cast<u32x4*>(&Ks[r * LS + c8 * 8]) = kw;
      *reinterpret_cast<u32x4*>(&Vs[r * LS + c8 * 8]) = vw;
      if constexpr (BLOCKS && !NOSJ && !FP8) {   // the quantised branch reads V8 instead
        u32x4 v16w;
#pragma unroll
        for (int e = 0; e < 4; ++e) v16w[e] = f16_sat_pack(vf[2 * e], vf[2 * e + 1]);
        *reinterpret_cast<u32x4*>(&v16[((size_t)bh * nbk * kBlock + row0 + r) * D + c8 * 8]) = v16w;
      }
    }
    {
      // lanes lane ^ TPR, lane ^ 2 TPR, ... of a wave hold the same channels: fold them, then
      // one partial per wave goes to LDS
      const int cg = t % TPR;
#pragma unroll
      for (int o = TPR; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pacc[e] += __shfl_xor(pacc[e], o, 64);
          if constexpr (PISA) vacc[e] += __shfl_xor(vacc[e], o, 64);
        }
      if (lane < TPR) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pool_lds[w * D + cg * 8 + e] = pacc[e];
        if constexpr (PISA) {
#pragma unroll
          for (int e = 0; e < 8; ++e) vpool_lds[w * D + cg * 8 + e] = vacc[e];
        }
      }
    }
    if (j + 1 < j1) load_block(j + 1);   // in flight during this block's compute
    __syncthreads();
    if (t < D) {
      double sm = 0.0;
      for (int ww_ = 0; ww_ < 4; ++ww_) sm += pool_lds[ww_ * D + t];
      means[(j - j0) % kSummaryChunk][t] = sm / (double)nrows;
      if constexpr (PISA) {
        const double mean = sm / (double)nrows;
        const float hi = bf16_lo(pack_bf16((float)mean, 0.f));
        const size_t ci = ((size_t)bh * npad + j) * D + t;
        cent_hi[ci] = (uint16_t)(pack_bf16(hi, 0.f) & 0xffffu);
        cent_lo[ci] = (uint16_t)(pack_bf16((float)(mean - (double)hi), 0.f) & 0xffffu);
        double vs = 0.0;
        for (int ww_ = 0; ww_ < 4; ++ww_) vs += vpool_lds[ww_ * D + t];
        vsum[((size_t)bh * npad + j) * D + t] = (uint16_t)(f16_sat_pack((float)vs, 0.f) & 0xffffu);
      }
    }
    if constexpr (FP8) {
      // E4M3 of the staged (masked) tiles: K8 in this thread's row chunks, the V8 tile in
      // 16-byte chunks of one channel's key slots, so that it goes out in whole chunks.
      // The block absmax comes from the same reads in a first pass (not from the staging
      // loop, whose registers it would add to).
      float kmx = 0.f, vmx = 0.f;
#pragma unroll 1
      for (int u = 0; u < CPT; ++u) {
        const int cidx = t + 256 * u;
        const u32x4 kw = *reinterpret_cast<const u32x4*>(&Ks[(cidx / TPR) * LS + (cidx % TPR) * 8]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          kmx = fmaxf(kmx, fmaxf(fabsf(bf16_lo(kw[e])), fabsf(bf16_hi(kw[e]))));
      }
#pragma unroll 1
      for (int u = 0; u < D * 4 / 256; ++u) {
        const int id = t + 256 * u, c = id >> 2, pq = id & 3;
        const int mt = pq & 1, hh = pq >> 1;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vmx = fmaxf(vmx, fabsf(__uint_as_float(
                                 (uint32_t)Vs[(32 * mt + 8 * g + 4 * hh + i) * LS + c] << 16)));
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        kmx = fmaxf(kmx, __shfl_xor(kmx, o, 64));
        vmx = fmaxf(vmx, __shfl_xor(vmx, o, 64));
      }
      if (lane == 0) {
        amax_lds[2 * w] = kmx;
        amax_lds[2 * w + 1] = vmx;
      }
      __syncthreads();
      const int ek = e8m0_exponent(fmaxf(fmaxf(amax_lds[0], amax_lds[2]),
                                         fmaxf(amax_lds[4], amax_lds[6])));
      const int ev = e8m0_exponent(fmaxf(fmaxf(amax_lds[1], amax_lds[3]),
                                         fmaxf(amax_lds[5], amax_lds[7])));
      if (t == 0) {
        f8.ek[(size_t)bh * nbk + j] = ek;
        f8.ev[(size_t)bh * nbk + j] = ev;
      }
#pragma unroll 1
      for (int u = 0; u < CPT; ++u) {
        const int cidx = t + 256 * u;
        const int r = cidx / TPR, c8 = cidx % TPR;
        const u32x4 kw = *reinterpret_cast<const u32x4*>(&Ks[r * LS + c8 * 8]);
        float kf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[2 * e] = bf16_lo(kw[e]); kf[2 * e + 1] = bf16_hi(kw[e]);
        }
        uint32_t w0, w1;
        e4m3x8(kf, ek, w0, w1);
        *reinterpret_cast<u32x4*>(f8.k8 + (((size_t)bh * nbk * kBlock + row0 + r) * D + c8 * 8) * 2) =
            e4m3x8_as_bf16(w0, w1);
      }
      // chunk (channel c, slot quarter pq = 2 hh + mt): slot 16 pq + 4 g + i holds key
      // 32 mt + 8 g + 4 hh + i
      uint8_t* v8t = f8.v8 + ((size_t)bh * nbk + j) * D * 64;
#pragma unroll 1
      for (int u = 0; u < D * 4 / 256; ++u) {
        const int id = t + 256 * u, c = id >> 2, pq = id & 3;
        const int mt = pq & 1, hh = pq >> 1;
#pragma unroll 1
        for (int g2 = 0; g2 < 4; g2 += 2) {   // slots 4 g2 .. 4 g2 + 7
          float va[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            va[e] = __uint_as_float(
                (uint32_t)Vs[(32 * mt + 8 * (g2 + (e >> 2)) + 4 * hh + (e & 3)) * LS + c] << 16);
          uint32_t w0, w1;
          e4m3x8(va, ev, w0, w1);
          *reinterpret_cast<u32x2*>(v8t + c * 64 + 16 * pq + 4 * g2) = u32x2{w0, w1};
        }
      }
    }
    if constexpr (PISA) __syncthreads();   // block means are read by every wave below
    // S_j[r][c] = sum_m relu(K[m][r]) V[m][c]: M = r, N = c, reduction over the 64 keys;
    // z_j[r] = sum_m relu(K[m][r]) from the same A fragments. (PISA: K[m][r] - mean_r
    // instead of relu(K[m][r]); padded keys have V = 0 and contribute nothing.)
    u32x4 af[4];
    float zl = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      if constexpr (PISA) {
        const float mr = (float)means[(j - j0) % kSummaryChunk][32 * mt + l32];
        const u32x4 raw = frag_tr(Ks, LS, 32 * mt, 16 * s4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          af[s4][e] = pack_bf16(bf16_lo(raw[e]) - mr, bf16_hi(raw[e]) - mr);
      } else {
        af[s4] = relu_bf16x8(frag_tr(Ks, LS, 32 * mt, 16 * s4));
#pragma unroll
        for (int e = 0; e < 4; ++e) zl += bf16_lo(af[s4][e]) + bf16_hi(af[s4][e]);
      }
    }
    zl += swap_halves(zl);
    if (BLOCKS && !PISA && ((NT == 4) || (w & 1) == 0) && h == 0) {
      zblk[((size_t)bh * nbk + j) * D + 32 * mt + l32] = zl;
    }
    zp += zl;
    // Plain forward at d = 128: S_j^T in two halves of 64 value columns, so that only two
    // accumulator tiles are live at a time (fewer registers: three workgroups per CU instead
    // of two, more loads in flight). Half 0 is staged over the K tile once every wave holds its
    // A fragments, half 1 over the V tile after every wave's last product.
    constexpr bool HALVES = BLOCKS && !PISA && !LO && !NOSJ && NT == 4;
    if constexpr (HALVES) {
      f32x16 acc2[2];
      auto product = [&](int half) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          acc2[u] = f32x16{};
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4)
            acc2[u] = mfma_bf16(af[s4], frag_tr(Vs, LS, 32 * (2 * half + u), 16 * s4), acc2[u]);
        }
      };
      auto stage_half = [&](int half) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int c = 32 * (2 * half + u) + l32;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 32 * mt + 8 * q + 4 * h;
            *reinterpret_cast<u32x2*>(&KVs[c * LS + r]) =
                u32x2{pack_bf16(acc2[u][4 * q], acc2[u][4 * q + 1]),
                      pack_bf16(acc2[u][4 * q + 2], acc2[u][4 * q + 3])};
          }
        }
      };
      auto store_half = [&](int half) __attribute__((always_inline)) {
#pragma unroll
        for (int e = t; e < D * D / 16; e += 256) {
          const int c = 64 * half + e / (D / 8), ch = e % (D / 8);
          const int f = c * D + ch * 8;
          uint16_t* dst = sblk + (((size_t)bh * (D * D / kSlice) + f / kSlice) * nbk + j) * kSlice +
                          f % kSlice;
          *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(&KVs[c * LS + ch * 8]);
        }
      };
      product(0);
      __syncthreads();   // every wave has its A fragments: the K tile is free
      stage_half(0);
      product(1);
      __syncthreads();   // half 0 is staged and every wave is done with the V tile
      store_half(0);
      stage_half(1);
      __syncthreads();
      store_half(1);
    } else {
      f32x16 accs[TILES_PER_WAVE];
  #pragma unroll
      for (int u = 0; u < TILES_PER_WAVE; ++u) {
        const int nt = (NT == 4) ? u : (w & 1);
        accs[u] = f32x16{};
  #pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          accs[u] = mfma_bf16(af[s4], frag_tr(Vs, LS, 32 * nt, 16 * s4), accs[u]);
        if constexpr (TOTALS) part[u] += accs[u];
      }
      if constexpr (BLOCKS && !PISA && !NOSJ) {
        // S_j^T[c][r] (bf16) goes out in whole 2D-byte rows: staged over the K and V tiles
        // (row c at LS elements) once every wave has read them, then 16-byte chunks per thread.
        // Lane column c = 32 nt + l32 holds rows r in runs of 4.
        __syncthreads();
  #pragma unroll
        for (int u = 0; u < TILES_PER_WAVE; ++u) {
          const int c = 32 * ((NT == 4) ? u : (w & 1)) + l32;
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 32 * mt + 8 * q + 4 * h;
            *reinterpret_cast<u32x2*>(&KVs[c * LS + r]) =
                u32x2{pack_bf16(accs[u][4 * q], accs[u][4 * q + 1]),
                      pack_bf16(accs[u][4 * q + 2], accs[u][4 * q + 3])};
          }
        }
        __syncthreads();
  #pragma unroll
        for (int e = t; e < D * D / 8; e += 256) {
          const int c = e / (D / 8), ch = e % (D / 8);
          const int f = c * D + ch * 8;             // flattened index of the chunk
          uint16_t* dst = sblk + (((size_t)bh * (D * D / kSlice) + f / kSlice) * nbk + j) * kSlice +
                          f % kSlice;
          *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(&KVs[c * LS + ch * 8]);
        }
        if constexpr (LO) {   // S_j - bf16(S_j), rounded to bf16, in the same layout
          __syncthreads();
  #pragma unroll
          for (int u = 0; u < TILES_PER_WAVE; ++u) {
            const int c = 32 * ((NT == 4) ? u : (w & 1)) + l32;
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int r = 32 * mt + 8 * q + 4 * h;
              float lo[4];
  #pragma unroll
              for (int e = 0; e < 4; ++e)
                lo[e] = accs[u][4 * q + e] - bf16_lo(pack_bf16(accs[u][4 * q + e], 0.f));
              *reinterpret_cast<u32x2*>(&KVs[c * LS + r]) =
                  u32x2{pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3])};
            }
          }
          __syncthreads();
  #pragma unroll
          for (int e = t; e < D * D / 8; e += 256) {
            const int c = e / (D / 8), ch = e % (D / 8);
            const int f = c * D + ch * 8;
            uint16_t* dst = sblk_lo +
                            (((size_t)bh * (D * D / kSlice) + f / kSlice) * nbk + j) * kSlice +
                            f % kSlice;
            *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(&KVs[c * LS + ch * 8]);
          }
        }
      }
    }
    __syncthreads();   // LDS tiles and pool_lds are rewritten by the next block
    // projected pooled K of each finished group of kSummaryChunk blocks: k~ = mean @ P_k
    // (float64; means are visible after the barrier above)
    if (Pk != nullptr && ((j - j0) % kSummaryChunk == kSummaryChunk - 1 || j + 1 == j1)) {
      // thread (c, b0) projects blocks b0, b0 + 256 / D, ... of the group for output channel
      // c, reading each P_k entry once for all of them (rows of a partial group are computed
      // and not stored)
      constexpr int NBT = kSummaryChunk * D / 256;
      const int g0 = j - (j - j0) % kSummaryChunk;
      const int c = t % D, b0 = t / D;
      double acc[NBT];
#pragma unroll
      for (int u = 0; u < NBT; ++u) acc[u] = 0.0;
#pragma unroll 4
      for (int r = 0; r < D; ++r) {
        const double pv = (double)Pk[r * D + c];
#pragma unroll
        for (int u = 0; u < NBT; ++u) acc[u] = fma(means[b0 + u * (256 / D)][r], pv, acc[u]);
      }
#pragma unroll
      for (int u = 0; u < NBT; ++u) {
        const int b = b0 + u * (256 / D);
        if (b <= j - g0) kt[(size_t)bh * kbh + (size_t)(g0 + b) * kj + c] = acc[u];
      }
      __syncthreads();   // means are rewritten by the next group
    }
  }
  // chunk partial totals (fp32, layout [c][r])
#pragma unroll
  for (int u = 0; u < (TOTALS ? TILES_PER_WAVE : 0); ++u) {
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
                                                            float* __restrict__ ztot, int nchunk,
                                                            int accumulate,
                                                            uint16_t* __restrict__ scaled_bf16,
                                                            float scale, int z_only) {
  // A workgroup owns 32 consecutive entries e of the d x d total (and, for the first D / 32
  // workgroups, 32 entries of z). Thread group g (8 of 32 threads) adds the chunk partials
  // c = g, g + 8, ... with all its loads in flight at once; the 8 group sums are then added
  // in group order, onto the previous totals when accumulating (summary cache update), so
  // the result does not depend on timing. scaled_bf16 (optional): also store
  // bf16(scale * total) (the piecewise forward's H_bar^T = H_sum^T / nbk). z_only: only the
  // z partials exist (grid of D / 32 workgroups per head).
  constexpr int G = 8;
  __shared__ float part[2][G][32];
  const int bh = blockIdx.y;
  const int t = threadIdx.x, lane = t & 31, g = t >> 5;
  const int e = blockIdx.x * 32 + lane;
  const bool do_z = blockIdx.x * 32 < D;
  auto group_sum = [&](const float* src, size_t stride) {
    float acc = 0.f;
    int c = g;
    for (; c + 3 * G < nchunk; c += 4 * G) {
      const float v0 = src[(size_t)c * stride], v1 = src[(size_t)(c + G) * stride];
      const float v2 = src[(size_t)(c + 2 * G) * stride], v3 = src[(size_t)(c + 3 * G) * stride];
      acc += v0; acc += v1; acc += v2; acc += v3;
    }
    for (; c < nchunk; c += G) acc += src[(size_t)c * stride];
    return acc;
  };
  if (!z_only) part[0][g][lane] = group_sum(spart + (size_t)bh * nchunk * D * D + e, (size_t)D * D);
  if (do_z) part[1][g][lane] = group_sum(zpart + (size_t)bh * nchunk * D + e, (size_t)D);
  __syncthreads();
  if (g == 0 && !z_only) {
    float s = accumulate ? stot[(size_t)bh * D * D + e] : 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) s += part[0][i][lane];
    stot[(size_t)bh * D * D + e] = s;
    if (scaled_bf16 != nullptr)
      scaled_bf16[(size_t)bh * D * D + e] = (uint16_t)(pack_bf16(s * scale, 0.f) & 0xffffu);
  } else if (g == 1 && do_z) {
    float z = accumulate ? ztot[(size_t)bh * D + e] : 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) z += part[1][i][lane];
    ztot[(size_t)bh * D + e] = z;
  }
}

// Complement, summary part: for a tile of CQ query blocks and CN columns n of the d x d
// summary, S_c[n][i] = sum_j (1 - M[i][j]) S_j[n] with M the 0/1 selection matrix (SPLA
// page, section 2.2: the linear term covers the blocks the sparse part did not select),
// computed as an MFMA product over steps of CK key blocks (the 0/1 matrix is exact in bf16).
// Each thread first copies one query block's row of the routed-block bitmap (written by the
// router's top-k pass; one 32-bit word per step of a window of up to 32 * MAXW key blocks)
// into LDS, inverted over the valid key blocks, and steps in which every query block of the
// tile selected every block are skipped. The summary slices of a step (CK rows of CN bf16)
// are loaded straight into a CBUF-deep LDS ring, two pairs of steps ahead of their use.
// Wave w owns query blocks 64 w .. 64 w + 63 of the tile and all CN columns: per step it
// reads 8 A fragments (summaries, transposing LDS reads, shared by the four waves) and
// builds 4 B fragments (its bitmap bits -> bf16 0/1) for 16 MFMAs. Query tiles sharing a
// column slice are consecutive workgroups (same XCD), so each S_j slice comes from HBM
// about once and from L2 ceil(n_blocks / CQ) times.
constexpr int CQ = 256;    // query blocks per workgroup (64 per wave)
constexpr int CN = kSlice; // summary columns per workgroup: one slice
constexpr int CK = 32;     // key blocks per step = bits per bitmap word
constexpr int CBUF = 6;    // steps in the LDS ring (three pairs)
constexpr int MAXW = 30;   // bitmap words per query block and window (window <= 960 blocks)
constexpr int RING_BYTES = CBUF * CK * CN * 2;

// Dynamic LDS of complement_kernel for a window of `ww` words: ring, bitmap (ww + 1 words
// per query block: the odd row length keeps the per-lane word accesses on distinct banks)
// and four 64-bit step-occupancy masks.
// (at least 32 KB: the epilogue stages its stores there)
inline size_t complement_lds_bytes(int ww) {
  const size_t b = (size_t)RING_BYTES + (size_t)CQ * (ww + 1) * 4 + 4 * 8;
  return b > 32768 ? b : 32768;
}

// Swizzle of a ring row (CN bf16 = 16 chunks of 16 bytes): chunk c of row r sits at
// c ^ f(r % 4), which keeps the transposing fragment reads (4 rows x 2 or 4 adjacent chunks
// per 16 or 32 lanes) on distinct banks.
__device__ __forceinline__ int ring_f(int r) {
  const int q = r & 3;
  return ((q & 1) ? 6 : 0) ^ ((q & 2) ? 10 : 0);
}
// A fragment from a ring step buffer M[j][n]: lane owns n = x0 + lane%32 and the 8 key
// blocks k0 + 8*(lane/32) .. +7.
__device__ __forceinline__ u32x4 ring_frag(const uint16_t* M, int x0, int k0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, L = lane & 15;
  const int row = k0 + 8 * (g >> 1) + (L >> 2);
  const int col = x0 + 16 * (g & 1) + 4 * (L & 3);
  const int off = ((((col >> 3) ^ ring_f(row)) & 15) << 3) + (col & 7);
  const u32x2 lo = lds_read_tr16(M + row * CN + off);
  const u32x2 hi = lds_read_tr16(M + (row + 4) * CN + off);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}
// bf16 0/1 B fragment from 8 selection bits (bit e -> element e)
__device__ __forceinline__ u32x4 bits_to_bf16x8(uint32_t m8) {
  u32x4 b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t x = (m8 >> (2 * e)) & 3u;
    b[e] = ((x * 0x8001u) & 0x10001u) * 0x3F80u;   // bit 0 -> low half, bit 1 -> high half
  }
  return b;
}

// F32 (the backward): the stacked summaries come as bf16 high parts (sblk) and low parts
// (sblk_lo); both are summed into the same accumulators (high parts first) and the sums go
// out once, as fp32.
template <int D, bool F32 = false>
__global__ __launch_bounds__(256, 2) void complement_kernel(
    const uint32_t* __restrict__ selbits, int nwords, const uint16_t* __restrict__ sblk,
    const uint16_t* __restrict__ sblk_lo, void* __restrict__ out, int nbq, int nbk, int k,
    int nqt, int total, int ww) {
  uint16_t* sc = reinterpret_cast<uint16_t*>(out);
  float* scf = reinterpret_cast<float*>(out);
  constexpr int NCS = D * D / CN;      // column slices per (batch, head)
  constexpr int LPW = CK * CN * 2 / 1024 / 4;   // 1-KB ring loads per wave per step
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  uint16_t* ring = reinterpret_cast<uint16_t*>(dyn);
  const int WW = ww + 1;
  uint32_t* bits = reinterpret_cast<uint32_t*>(dyn + RING_BYTES);
  uint64_t* occw = reinterpret_cast<uint64_t*>(bits + CQ * WW);

  const int wid = xcd_remap(blockIdx.x, total);
  const int qt = wid % nqt;
  const int cs = (wid / nqt) % NCS;
  const int bh = wid / (nqt * NCS);
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const size_t col0 = (size_t)cs * CN;

  if (k >= nbk) {   // every block selected: the complement is empty, exactly zero
    if constexpr (F32) {
      for (int e = t; e < CQ * CN / 4; e += 256) {
        const int il = e / (CN / 4), c4 = e % (CN / 4);
        const int i = qt * CQ + il;
        if (i < nbq)
          *reinterpret_cast<f32x4*>(scf + ((size_t)bh * nbq + i) * D * D + col0 + c4 * 4) =
              f32x4{0.f, 0.f, 0.f, 0.f};
      }
      return;
    }
    for (int e = t; e < CQ * CN / 8; e += 256) {
      const int il = e / (CN / 8), c8 = e % (CN / 8);
      const int i = qt * CQ + il;
      if (i < nbq)
        *reinterpret_cast<u32x4*>(sc + ((size_t)bh * nbq + i) * D * D + col0 + c8 * 8) =
            u32x4{0, 0, 0, 0};
    }
    return;
  }
  // this thread's query block and its row of the routed-block bitmap
  const int qi = qt * CQ + t;
  const uint32_t* my_bits = selbits + ((size_t)bh * nbq + min(qi, nbq - 1)) * nwords;

  // ring loads: wave w moves pieces LPW w .. LPW w + LPW - 1 (1 KB = 4 rows of 256 bytes);
  // lane l lands at row 4 piece + l / 16, physical chunk l % 16, and fetches the logical
  // chunk that the swizzle puts there
  uint32_t roff[LPW];
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int r = 4 * (LPW * w + u) + (lane >> 4), pch = lane & 15;
    roff[u] = (uint32_t)(r * CN * 2 + ((pch ^ ring_f(r)) & 15) * 16);
  }
  const int ws = __builtin_amdgcn_readfirstlane(w);
  const uint16_t* sbase = sblk + ((size_t)bh * NCS + cs) * nbk * CN;   // this slice, block 0
  auto stage = [&](int j0, int slot) __attribute__((always_inline)) {   // j0 < 0: nothing
    const uint32_t bytes = j0 < 0 ? 0u : (uint32_t)min(CK, nbk - j0) * CN * 2;
    const i32x4 r = make_rsrc(sbase + (size_t)(j0 < 0 ? 0 : j0) * CN, bytes);
    const uint32_t dst = lds_addr(ring + slot * CK * CN) + ws * LPW * 1024;
#pragma unroll
    for (int u = 0; u < LPW; ++u) load_lds16(r, dst + u * 1024, roff[u]);
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int tq = 0; tq < 2; ++tq)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[tq][nt] = f32x16{};

  const int win = ww * CK;
  for (int pass = 0; pass < (F32 ? 2 : 1); ++pass) {
  if (pass == 1) sbase = sblk_lo + ((size_t)bh * NCS + cs) * nbk * CN;
  for (int win0 = 0; win0 < nbk; win0 += win) {
    const int nstep = min(ww, (nbk - win0 + CK - 1) / CK);
    barrier_vmem_n<0>();   // the previous window's ring and bitmap are no longer in use
    // this window's words of the thread's bitmap row (loads in flight together)
    uint64_t my_occ = 0;
    {
      const int w0 = win0 / CK;
      const int nw = qi < nbq ? min(ww, nwords - w0) : 0;
      uint32_t wv_[MAXW];
#pragma unroll
      for (int wi = 0; wi < MAXW; ++wi) {
        // unselected valid key blocks of this word (bits past nbk stay clear)
        const int jb = (w0 + wi) * CK;
        const uint32_t valid =
            nbk - jb >= CK ? 0xffffffffu : (nbk > jb ? (1u << (nbk - jb)) - 1u : 0u);
        wv_[wi] = wi < nw ? ~my_bits[w0 + wi] & valid : 0u;
      }
#pragma unroll
      for (int wi = 0; wi < MAXW; ++wi) {
        if (wi < ww) bits[t * WW + wi] = wv_[wi];
        my_occ |= (uint64_t)(wv_[wi] != 0) << wi;
      }
    }
    // union of the occupancy masks over the workgroup
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)my_occ, o, 64);
      const uint32_t hi = __shfl_xor((uint32_t)(my_occ >> 32), o, 64);
      my_occ |= ((uint64_t)hi << 32) | lo;
    }
    if (lane == 0) occw[w] = my_occ;
    __syncthreads();
    const uint64_t occ = (occw[0] | occw[1] | occw[2] | occw[3]) &
                         (nstep >= 64 ? ~0ull : ((1ull << nstep) - 1ull));
    auto next_after = [&](int st) -> int {   // first occupied step > st, or -1
      const uint64_t rest = st >= 63 ? 0ull : occ & ~((2ull << st) - 1ull);
      return rest ? __builtin_ctzll(rest) : -1;
    };
    // Occupied steps are taken in pairs, one barrier per pair: while a pair is multiplied, the
    // pair two ahead loads into the slots of the pair before it (6-slot ring), so every load
    // has two pairs' time to land.
    auto compute_step = [&](int sl, int st) __attribute__((always_inline)) {
      const uint16_t* M = ring + sl * CK * CN;
      uint32_t word[2];
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) word[tq] = bits[(64 * w + 32 * tq + l32) * WW + st];
      // all eight A fragments of the step are read before its first product
      u32x4 a[2][4];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) a[kk][nt] = ring_frag(M, 32 * nt, 16 * kk);
      u32x4 b[2][2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int tq = 0; tq < 2; ++tq)
          b[kk][tq] = bits_to_bf16x8((word[tq] >> (16 * kk + 8 * h)) & 0xffu);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int tq = 0; tq < 2; ++tq)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) acc[tq][nt] = mfma_bf16(a[kk][nt], b[kk][tq], acc[tq][nt]);
    };
    // the next six occupied steps (-1: none); st[0], st[1] is the pair being multiplied
    int st[6];
    st[0] = occ ? __builtin_ctzll(occ) : -1;
#pragma unroll
    for (int u = 1; u < 6; ++u) st[u] = st[u - 1] < 0 ? -1 : next_after(st[u - 1]);
#pragma unroll
    for (int u = 0; u < 4; ++u) stage(st[u] < 0 ? -1 : win0 + st[u] * CK, u);
    barrier_vmem_n<2 * LPW>();   // the first pair has landed (the second may be in flight)
    int slot = 0;
    while (st[0] >= 0) {
      const int ls = slot == 0 ? 4 : slot - 2;   // the slots of the previous pair
      stage(st[4] < 0 ? -1 : win0 + st[4] * CK, ls);
      stage(st[5] < 0 ? -1 : win0 + st[5] * CK, ls + 1);
      compute_step(slot, st[0]);
      if (st[1] >= 0) compute_step(slot + 1, st[1]);
      barrier_vmem_n<2 * LPW>();   // the next pair has landed; this pair's slots are free
#pragma unroll
      for (int u = 0; u < 4; ++u) st[u] = st[u + 2];
      st[4] = st[3] < 0 ? -1 : next_after(st[3]);
      st[5] = st[4] < 0 ? -1 : next_after(st[4]);
      slot = slot == 4 ? 0 : slot + 2;
    }
  }
  }   // pass
  wait_vmem();   // no load into LDS outlives the workgroup
  if constexpr (F32) {
    // lane: query block 64 w + 32 tq + l32 of the group; elements 4 g .. 4 g + 3: the four
    // consecutive columns 32 nt + 8 g + 4 h ..
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      const int i = qt * CQ + 64 * w + 32 * tq + l32;
      if (i >= nbq) continue;
      float* row = scf + ((size_t)bh * nbq + i) * D * D + col0;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          *reinterpret_cast<f32x4*>(row + 32 * nt + 8 * g + 4 * h) =
              f32x4{acc[tq][nt][4 * g], acc[tq][nt][4 * g + 1], acc[tq][nt][4 * g + 2],
                    acc[tq][nt][4 * g + 3]};
        }
    }
    return;
  }
  // S_c, staged through LDS (the ring and bitmap are free now) so that every
  // query block's CN columns go out as contiguous 16-byte stores. Per half tq, wave w
  // stages its 32 query blocks x CN columns; 16-byte chunk c of staged row q sits at
  // c ^ (q % 16).
  __syncthreads();
  uint16_t* stg = reinterpret_cast<uint16_t*>(dyn) + w * 32 * CN;
#pragma unroll
  for (int tq = 0; tq < 2; ++tq) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = 32 * nt + 8 * g + 4 * h;
        const int off = l32 * CN + ((((n >> 3) ^ l32) & 15) << 3) + (n & 7);
        *reinterpret_cast<u32x2*>(stg + off) =
            u32x2{pack_bf16(acc[tq][nt][4 * g], acc[tq][nt][4 * g + 1]),
                  pack_bf16(acc[tq][nt][4 * g + 2], acc[tq][nt][4 * g + 3])};
      }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int u = 0; u < 8; ++u) {           // 4 rows of 16 chunks per pass
      const int q = 4 * u + (lane >> 4), c = lane & 15;
      const int i = qt * CQ + 64 * w + 32 * tq + q;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stg + q * CN + (((c ^ q) & 15) << 3));
      if (i < nbq)
        *reinterpret_cast<u32x4*>(sc + ((size_t)bh * nbq + i) * D * D + col0 + c * 8) = v;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Complement, normaliser part (fp32, fixed order). With at most half the key blocks selected,
// z_c(i) = z_tot - sum_{j in sel(i)} z_j (at most k + 1 terms, and the unselected blocks are
// at least half of them); with more than half selected, the unselected z_j are added directly
// in ascending block order from the routed-block bitmap, so that z_c never comes out of a
// difference of nearly equal sums (a selection of all but one block leaves one block's z).
template <int D>
__global__ __launch_bounds__(D) void complement_z_kernel(const int32_t* __restrict__ idx,
                                                         const uint32_t* __restrict__ selbits,
                                                         int nwords,
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
  const float* zb = zblk + (size_t)bh * nbk * D + r;
  if (2 * k > nbk) {
    const uint32_t* brow = selbits + ((size_t)bh * nbq + i) * nwords;
    float z = 0.f;
    for (int wi = 0; wi < nwords; ++wi) {
      const int jb = 32 * wi;
      uint32_t m = ~brow[wi];
      if (nbk - jb < 32) m &= (1u << (nbk - jb)) - 1u;   // bits past the last block
      while (m) {
        z += zb[(size_t)(jb + __builtin_ctz(m)) * D];
        m &= m - 1u;
      }
    }
    out[r] = z;
    return;
  }
  const int32_t* sel = idx + ((size_t)bh * nbq + i) * k;
  // selected blocks are added in list order (deterministic); loads go out 32 at a time, so a
  // row of k selections waits for about k / 32 round trips
  float z = 0.f;
  int s = 0;
  for (; s + 32 <= k; s += 32) {
    float v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) v[u] = zb[(size_t)sel[s + u] * D];
#pragma unroll
    for (int u = 0; u < 32; ++u) z += v[u];
  }
  if (s < k) {   // the last (partial) batch, also in one round trip: absent slots add 0
    float v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int jj = sel[min(s + u, k - 1)];   // in bounds whichever slot is read
      v[u] = s + u < k ? zb[(size_t)jj * D] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 32; ++u) z += v[u];
  }
  out[r] = ztot[(size_t)bh * D + r] - z;
}

template <int D>
static hipError_t launch_kv_summary_T(const Plan& s, const void* k, const void* v, const float* pk,
                                      char* ws, hipStream_t st, bool fp8, uint16_t* sblk_lo) {
  double* kt = reinterpret_cast<double*>(ws + s.kt);
  uint16_t* v16 = reinterpret_cast<uint16_t*>(ws + s.v16);
  uint16_t* sblk = reinterpret_cast<uint16_t*>(ws + s.sblk);
  float* zblk = reinterpret_cast<float*>(ws + s.zblk);
  float* spart = reinterpret_cast<float*>(ws + s.spart);
  float* zpart = reinterpret_cast<float*>(ws + s.zpart);
  const dim3 grid(s.nchunk, s.BH);
  const size_t kbh = (size_t)s.nbk * D, kj = D;
  if (s.in_bf16 && fp8)
    hipLaunchKernelGGL((kv_summary_kernel<uint16_t, D, true, kSummaryChunk, false, true>), grid,
                       dim3(256), 0, st, (const uint16_t*)k, (const uint16_t*)v, pk, kt, kbh, kj,
                       v16, sblk, nullptr, zblk, spart, zpart, s.nkv, s.nbk, 0, 0, nullptr,
                       nullptr, nullptr, 0,
                       Fp8Out{reinterpret_cast<uint8_t*>(ws + s.k8),
                              reinterpret_cast<uint8_t*>(ws + s.v8),
                              reinterpret_cast<int32_t*>(ws + s.sk8),
                              reinterpret_cast<int32_t*>(ws + s.sv8)});
  else if (s.in_bf16 && sblk_lo)
    hipLaunchKernelGGL((kv_summary_kernel<uint16_t, D, true, kSummaryChunk, false, false, true>),
                       grid, dim3(256), 0, st, (const uint16_t*)k, (const uint16_t*)v, pk, kt, kbh,
                       kj, v16, sblk, sblk_lo, zblk, spart, zpart, s.nkv, s.nbk, 0, 0, nullptr,
                       nullptr, nullptr, 0, Fp8Out{});
  else if (s.in_bf16)
    hipLaunchKernelGGL((kv_summary_kernel<uint16_t, D, true, kSummaryChunk>), grid, dim3(256), 0,
                       st,
                       (const uint16_t*)k, (const uint16_t*)v, pk, kt, kbh, kj, v16, sblk, nullptr,
                       zblk, spart, zpart, s.nkv, s.nbk, 0, 0, nullptr, nullptr, nullptr, 0,
                       Fp8Out{});
  else
    hipLaunchKernelGGL((kv_summary_kernel<float, D, true, kSummaryChunk>), grid, dim3(256), 0, st,
                       (const float*)k, (const float*)v, pk, kt, kbh, kj, v16, sblk, nullptr, zblk,
                       spart, zpart, s.nkv, s.nbk, 0, 0, nullptr, nullptr, nullptr, 0, Fp8Out{});
  // only z_tot: the complement sums the unselected S_j itself
  hipLaunchKernelGGL((reduce_totals_kernel<D>), dim3(D / 32, s.BH), dim3(256), 0, st, spart,
                     zpart, reinterpret_cast<float*>(ws + s.stot),
                     reinterpret_cast<float*>(ws + s.ztot), s.nchunk, 0, nullptr, 0.f, 1);
  return hipGetLastError();
}

// The few-query-block totals pass takes kTotalsChunk key blocks per workgroup: a quarter of
// the usual pass's d x d partial totals to write and reduce (they fit in its partials region).
constexpr int kTotalsChunk = 4 * kSummaryChunk;
template <int D>
static hipError_t launch_kv_totals_blocks_T(const Plan& s, const void* k, const void* v, char* ws,
                                            hipStream_t st) {
  const int nchunk = (s.nbk + kTotalsChunk - 1) / kTotalsChunk;
  const dim3 grid(nchunk, s.BH);
  float* spart = reinterpret_cast<float*>(ws + s.spart);
  float* zpart = reinterpret_cast<float*>(ws + s.zpart);
  hipLaunchKernelGGL((kv_summary_kernel<uint16_t, D, true, kTotalsChunk, false, false, false, true>),
                     grid, dim3(256), 0, st, (const uint16_t*)k, (const uint16_t*)v, nullptr,
                     nullptr, (size_t)0, (size_t)0, nullptr, nullptr, nullptr,
                     reinterpret_cast<float*>(ws + s.zblk), spart, zpart, s.nkv, s.nbk, 0, 0,
                     nullptr, nullptr, nullptr, 0, Fp8Out{});
  hipLaunchKernelGGL((reduce_totals_kernel<D>), dim3(D * D / 32, s.BH), dim3(256), 0, st, spart,
                     zpart, reinterpret_cast<float*>(ws + s.stot),
                     reinterpret_cast<float*>(ws + s.ztot), nchunk, 0, nullptr, 0.f, 0);
  return hipGetLastError();
}

// S_c(i)^T = S_tot^T - sum_{j in sel(i)} S_j^T in fp32 (SPLA page, section 2.2: the linear state
// of the unselected blocks is the total minus that of the selected ones), one workgroup per
// query block; S_j = relu(K_j)^T V_j on bf16 MFMA with fp32 accumulation (the products of the
// key/value pass), summed over the selected blocks in the same accumulators. The next selected
// block's K and V rows load into registers while the current one is multiplied. Each selected
// block's f16 copy of V (padded rows zero) goes to v16 [BH][nbk*64][D] on the way; a block
// that several query blocks select is written with the same values by each.
template <int D>
__global__ __launch_bounds__(256) void sc_subtract_kernel(const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const int32_t* __restrict__ idx,
                                                          const float* __restrict__ stot,
                                                          float* __restrict__ sc,
                                                          uint16_t* __restrict__ v16, int nkv,
                                                          int nbk, int nbq, int topk) {
  constexpr int LS = D + 8, TPR = D / 8, CPT = 64 * TPR / 256, NT = D / 32;
  constexpr int TPW = NT * NT / 4;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * LS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[64 * LS];
  const int bh = blockIdx.x / nbq, i = blockIdx.x % nbq;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int mt = NT == 4 ? w : (w >> 1);   // this wave's 32-row strip r of S_j
  const uint16_t* kb = k + (size_t)bh * nkv * D;
  const uint16_t* vb = v + (size_t)bh * nkv * D;
  const int32_t* sel = idx + ((size_t)bh * nbq + i) * topk;
  u32x4 kraw[CPT], vraw[CPT];
  auto load = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int cidx = t + 256 * u, r = cidx / TPR, c8 = cidx % TPR;
      const int row = j * kBlock + r;
      const bool ok = row < nkv;               // padded keys: zero K and V
      const size_t off = (size_t)(ok ? row : 0) * D + c8 * 8;
      kraw[u] = ok ? *reinterpret_cast<const u32x4*>(kb + off) : u32x4{0, 0, 0, 0};
      vraw[u] = ok ? *reinterpret_cast<const u32x4*>(vb + off) : u32x4{0, 0, 0, 0};
    }
  };
  f32x16 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = f32x16{};
  if (topk > 0) load(sel[0]);
  for (int e = 0; e < topk; ++e) {
    uint16_t* v16b = v16 + ((size_t)bh * nbk + sel[e]) * kBlock * D;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int cidx = t + 256 * u, r = cidx / TPR, c8 = cidx % TPR;
      *reinterpret_cast<u32x4*>(&Ks[r * LS + c8 * 8]) = kraw[u];
      *reinterpret_cast<u32x4*>(&Vs[r * LS + c8 * 8]) = vraw[u];
      u32x4 hw;
#pragma unroll
      for (int q = 0; q < 4; ++q) hw[q] = f16_sat_pack(bf16_lo(vraw[u][q]), bf16_hi(vraw[u][q]));
      *reinterpret_cast<u32x4*>(v16b + (size_t)r * D + c8 * 8) = hw;
    }
    __syncthreads();
    if (e + 1 < topk) load(sel[e + 1]);
    u32x4 af[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) af[s4] = relu_bf16x8(frag_tr(Ks, LS, 32 * mt, 16 * s4));
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int nt = NT == 4 ? u : (w & 1);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        acc[u] = mfma_bf16(af[s4], frag_tr(Vs, LS, 32 * nt, 16 * s4), acc[u]);
    }
    __syncthreads();   // the tiles are rewritten next
  }
  // element 4 q + e of tile u: r = 32 mt + 8 q + 4 h + e, c = 32 nt + l32 ([c][r] layouts)
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int c = 32 * (NT == 4 ? u : (w & 1)) + l32;
    const float* tot = stot + ((size_t)bh * D + c) * D;
    float* dst = sc + (((size_t)bh * nbq + i) * D + c) * D;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 32 * mt + 8 * q + 4 * h;
      const f32x4 tv = *reinterpret_cast<const f32x4*>(tot + r);
      *reinterpret_cast<f32x4*>(dst + r) =
          f32x4{tv[0] - acc[u][4 * q], tv[1] - acc[u][4 * q + 1], tv[2] - acc[u][4 * q + 2],
                tv[3] - acc[u][4 * q + 3]};
    }
  }
}

template <int D>
static hipError_t launch_pisa_stats_T(const Plan& s, const void* k, const void* v, const float* pk,
                                      char* ws, hipStream_t st) {
  double* kt = reinterpret_cast<double*>(ws + s.kt);
  uint16_t* v16 = reinterpret_cast<uint16_t*>(ws + s.v16);
  float* spart = reinterpret_cast<float*>(ws + s.p_spart);
  float* zpart = reinterpret_cast<float*>(ws + s.p_zpart);
  uint16_t* chi = reinterpret_cast<uint16_t*>(ws + s.cent_hi);
  uint16_t* clo = reinterpret_cast<uint16_t*>(ws + s.cent_lo);
  uint16_t* vsum = reinterpret_cast<uint16_t*>(ws + s.vsum);
  const dim3 grid(s.nchunk, s.BH);
  const size_t kbh = (size_t)s.nbk * D, kj = D;
  if (s.in_bf16)
    hipLaunchKernelGGL((kv_summary_kernel<uint16_t, D, true, kSummaryChunk, true>), grid, dim3(256),
                       0, st, (const uint16_t*)k, (const uint16_t*)v, pk, kt, kbh, kj, v16,
                       nullptr, nullptr, nullptr, spart, zpart, s.nkv, s.nbk, 0, 0, chi, clo, vsum,
                       s.npad, Fp8Out{});
  else
    hipLaunchKernelGGL((kv_summary_kernel<float, D, true, kSummaryChunk, true>), grid, dim3(256), 0,
                       st, (const float*)k, (const float*)v, pk, kt, kbh, kj, v16, nullptr,
                       nullptr, nullptr, spart, zpart, s.nkv, s.nbk, 0, 0, chi, clo, vsum, s.npad,
                       Fp8Out{});
  hipLaunchKernelGGL((reduce_totals_kernel<D>), dim3(D * D / 32, s.BH), dim3(256), 0, st, spart,
                     zpart, reinterpret_cast<float*>(ws + s.p_stot),
                     reinterpret_cast<float*>(ws + s.p_ztot), s.nchunk, 0,
                     reinterpret_cast<uint16_t*>(ws + s.hbar), 1.f / (float)s.nbk, 0);
  return hipGetLastError();
}

hipError_t launch_kv_cache_update(const Plan& s, const void* k, const void* v, const float* pk,
                                  int n_done, char* cache, char* ws, hipStream_t st) {
  const CachePlan c = make_cache_plan(s);
  if (cache_update_chunks(s, n_done) == 0) return hipSuccess;
  // the streaming totals pass (bf16 inputs, the only ones the cache takes), then the fixed-
  // order reduction of its chunk partials onto the totals
  hipError_t e = launch_kv_totals(s, k, v, pk, n_done, reinterpret_cast<double*>(cache + c.kt),
                                  (size_t)s.D, (size_t)s.BH * s.D,
                                  reinterpret_cast<float*>(cache + c.stot),
                                  reinterpret_cast<float*>(cache + c.ztot), ws, st);
  if (e != hipSuccess) return e;
  float* spart = reinterpret_cast<float*>(ws);
  float* zpart = reinterpret_cast<float*>(ws + cache_update_zpart_offset(s, n_done));
  const int nchunk = cache_update_chunks(s, n_done);
  if (s.D == 128)
    hipLaunchKernelGGL((reduce_totals_kernel<128>), dim3(128 * 128 / 32, s.BH), dim3(256), 0, st,
                       spart, zpart, reinterpret_cast<float*>(cache + c.stot),
                       reinterpret_cast<float*>(cache + c.ztot), nchunk, n_done > 0 ? 1 : 0,
                       nullptr, 0.f, 0);
  else
    hipLaunchKernelGGL((reduce_totals_kernel<64>), dim3(64 * 64 / 32, s.BH), dim3(256), 0, st,
                       spart, zpart, reinterpret_cast<float*>(cache + c.stot),
                       reinterpret_cast<float*>(cache + c.ztot), nchunk, n_done > 0 ? 1 : 0,
                       nullptr, 0.f, 0);
  return hipGetLastError();
}

hipError_t launch_kv_summary(const Plan& s, const void* k, const void* v, const float* pk,
                             char* ws, hipStream_t st, bool fp8, uint16_t* sblk_lo) {
  if (sblk_lo && (fp8 || !s.in_bf16)) return hipErrorInvalidValue;
  if (s.D == 128) return launch_kv_summary_T<128>(s, k, v, pk, ws, st, fp8, sblk_lo);
  return launch_kv_summary_T<64>(s, k, v, pk, ws, st, fp8, sblk_lo);
}

hipError_t launch_kv_totals_blocks(const Plan& s, const void* k, const void* v, char* ws,
                                   hipStream_t st) {
  if (!s.in_bf16) return hipErrorInvalidValue;
  if (s.D == 128) return launch_kv_totals_blocks_T<128>(s, k, v, ws, st);
  return launch_kv_totals_blocks_T<64>(s, k, v, ws, st);
}

hipError_t launch_sc_subtract(const Plan& s, const void* k, const void* v, const int32_t* idx,
                              const float* stot, float* sc, char* ws, hipStream_t st) {
  if (!s.in_bf16) return hipErrorInvalidValue;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(s.BH * s.nbq), dim3(256), 0, st,
                       reinterpret_cast<const uint16_t*>(k), reinterpret_cast<const uint16_t*>(v),
                       idx, stot, sc, reinterpret_cast<uint16_t*>(ws + s.v16), s.nkv, s.nbk,
                       s.nbq, s.k);
  };
  if (s.D == 128) go(sc_subtract_kernel<128>);
  else go(sc_subtract_kernel<64>);
  return hipGetLastError();
}

hipError_t launch_pisa_stats(const Plan& s, const void* k, const void* v, const float* pk,
                             char* ws, hipStream_t st) {
  if (s.D == 128) return launch_pisa_stats_T<128>(s, k, v, pk, ws, st);
  return launch_pisa_stats_T<64>(s, k, v, pk, ws, st);
}

hipError_t launch_complement_f32(const Plan& s, const uint32_t* bits, int nwords, int rows,
                                 int cols, int k, const uint16_t* hi, const uint16_t* lo,
                                 float* out, hipStream_t st) {
  // out[row] = sum over the columns whose bit is clear of (hi + lo)[col], in fp32: one
  // complement pass over the high parts and then the low parts into the same sums
  const int nqt = (rows + CQ - 1) / CQ;
  const int ncs = s.D * s.D / CN;
  const int total = s.BH * ncs * nqt;
  const int ww = min(MAXW, (cols + CK - 1) / CK);
  const size_t lds = complement_lds_bytes(ww);
  hipError_t err = hipSuccess;
  auto go = [&](auto kern) {
    if (lds > 65536) {
      err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (err != hipSuccess) return;
    }
    hipLaunchKernelGGL(kern, dim3(total), dim3(256), lds, st, bits, nwords, hi, lo, (void*)out,
                       rows, cols, k, nqt, total, ww);
  };
  if (s.D == 128) go(complement_kernel<128, true>);
  else go(complement_kernel<64, true>);
  return err != hipSuccess ? err : hipGetLastError();
}

hipError_t launch_complement_z(const Plan& s, const int32_t* idx, char* ws, hipStream_t st) {
  auto go = [&](auto zkern) {
    hipLaunchKernelGGL(zkern, dim3(s.nbq, s.BH), dim3(s.D), 0, st, idx,
                       reinterpret_cast<const uint32_t*>(ws + s.selbits), s.nwords,
                       reinterpret_cast<const float*>(ws + s.zblk),
                       reinterpret_cast<const float*>(ws + s.ztot),
                       reinterpret_cast<float*>(ws + s.zc), s.nbq, s.nbk, s.k);
  };
  if (s.D == 128) go(complement_z_kernel<128>);
  else go(complement_z_kernel<64>);
  return hipGetLastError();
}

hipError_t launch_complement(const Plan& s, const int32_t* idx, char* ws, hipStream_t st) {
  const int nqt = (s.nbq + CQ - 1) / CQ;
  const int ncs = s.D * s.D / CN;
  const int total = s.BH * ncs * nqt;
  const int ww = min(MAXW, (s.nbk + CK - 1) / CK);
  const size_t lds = complement_lds_bytes(ww);
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(ws + s.selbits);   // from top-k
  hipError_t err = hipSuccess;
  auto go = [&](auto kern, auto zkern) {
    // more than 64 KB of dynamic LDS (wide windows) has to be allowed per kernel
    if (lds > 65536) {
      err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (err != hipSuccess) return;
    }
    hipLaunchKernelGGL(kern, dim3(total), dim3(256), lds, st, bits, s.nwords,
                       reinterpret_cast<const uint16_t*>(ws + s.sblk), nullptr,
                       (void*)(ws + s.sc), s.nbq, s.nbk, s.k, nqt, total, ww);
    hipLaunchKernelGGL(zkern, dim3(s.nbq, s.BH), dim3(s.D), 0, st, idx,
                       reinterpret_cast<const uint32_t*>(ws + s.selbits), s.nwords,
                       reinterpret_cast<const float*>(ws + s.zblk),
                       reinterpret_cast<const float*>(ws + s.ztot),
                       reinterpret_cast<float*>(ws + s.zc), s.nbq, s.nbk, s.k);
  };
  if (s.D == 128) go(complement_kernel<128>, complement_z_kernel<128>);
  else go(complement_kernel<64>, complement_z_kernel<64>);
  return err != hipSuccess ? err : hipGetLastError();
}

}  // namespace sla
