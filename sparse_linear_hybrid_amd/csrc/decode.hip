// Forward against the key/value summary cache (SLA2 page, sections 2.A and 2.B; SPLA page,
// section 2.2: the linear term of the unselected key blocks is the total minus that of the
// selected ones) for shapes with few query blocks per head, such as a decode chunk over a
// long KV cache. The selected blocks' own linear summaries are formed here from the K/V
// tiles that the exact branch loads anyway, so nothing per key block is stored or re-read.
//
// decode_attn_kernel: one workgroup per (batch*head, query block, part of its selection
// list); four waves share the part's K/V tiles, loaded straight into a double-buffered LDS
// ring:
//   waves 0, 1: exact softmax attention of rows 32w .. 32w+31 of the query block over the
//               part's key blocks (the transposed layout of the sparse kernel: S^T = K Q^T,
//               O^T += V^T P^T); out: the part's row max m (base-2 units), row sum l and
//               unnormalised O;
//   waves 2, 3: the part's S_sel^T = sum_j (phi(K_j)^T V_j)^T for half of the rows r each,
//               and z_sel = sum_j sum_t phi(K_j[t]).
// V stays bf16 here, so P is split into a bf16 high part and a bf16 remainder and P.V takes
// two MFMAs (P rounded to bf16 alone costs about 1% of the output RMS).
//
// decode_combine_kernel: merges the parts into O_s, forms S_c = S_tot - S_sel and
// z_c = z_tot - z_sel (zero when every key block is selected), then
// O_l = phi(Q) S_c / (phi(Q) . z_c + eps) and O = alpha O_s + (1 - alpha) O_l; one workgroup
// per 32 output channels.
#include "common.h"
#include "kernels.h"

namespace sla {

namespace {

// Transposing fragment read from a [key][channel] tile: lane owns channel x0 + lane%32 and
// the 8 keys k0 + 8*(lane/32) .. +7 (A or B operand with the keys as reduction index).
template <int D, bool VTILE>
__device__ __forceinline__ u32x4 tr_frag(const uint16_t* M, int x0, int k0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, L = lane & 15;
  const int row = k0 + 8 * (g >> 1) + (L >> 2);
  const int col = x0 + 16 * (g & 1) + 4 * (L & 3);
  const int o0 = VTILE ? swzv<D>(row, col) : swz<D>(row, col);
  const int o1 = VTILE ? swzv<D>(row + 4, col) : swz<D>(row + 4, col);
  const u32x2 lo = lds_read_tr16(M + o0);
  const u32x2 hi = lds_read_tr16(M + o1);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;   // [BH][nbq][topk], ascending
  float* pml;           // [parts][64][2]: m, l
  float* po;            // [parts][64][D]
  float* ps;            // [parts][D(c)][D(r)]
  float* pz;            // [parts][D]
  int nq, nkv, nbq, nbk, topk, nsplit, total;
};

template <int D>
__global__ __launch_bounds__(256, 2) void decode_attn_kernel(DecodeArgs a) {
  constexpr int KS = D / 16;               // 16-channel steps of Q K^T
  constexpr int CT = D / 32;               // 32-channel tiles
  constexpr int CH = D / 8;                // 16-byte chunks per row
  constexpr int TILE = 64 * D;
  constexpr int KPW = 64 * D * 2 / 1024 / 4;   // 1-KB pieces per wave and tensor
  constexpr int MT = D / 64;               // 32-row tiles of S per summary wave
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE];   // K[2], V[2]

  const int wid = xcd_remap(blockIdx.x, a.total);
  const int part = wid % a.nsplit;
  const int iq = (wid / a.nsplit) % a.nbq;
  const int bh = wid / (a.nsplit * a.nbq);
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const size_t pidx = ((size_t)bh * a.nbq + iq) * a.nsplit + part;
  const int e0 = (int)((long long)a.topk * part / a.nsplit);
  const int e1 = (int)((long long)a.topk * (part + 1) / a.nsplit);
  const int32_t* sel = a.idx + ((size_t)bh * a.nbq + iq) * a.topk;
  const uint16_t* kb = a.k + (size_t)bh * a.nkv * D;
  const uint16_t* vb = a.v + (size_t)bh * a.nkv * D;

  // list entries e0.. held 64 at a time in a VGPR (lane = entry - base)
  int lbase = e0;
  int lvec = lbase + lane < e1 ? sel[lbase + lane] : 0;
  auto entry = [&](int e) -> int {
    if (e - lbase >= 64) {
      lbase += 64;
      lvec = lbase + lane < e1 ? sel[lbase + lane] : 0;
    }
    return __builtin_amdgcn_readlane(lvec, e - lbase);
  };

  // LDS DMA offsets: piece u of wave w lands at elements 512 (KPW w + u) + 8 lane
  uint32_t koff[KPW], voff[KPW];
#pragma unroll
  for (int u = 0; u < KPW; ++u) {
    const int e = (wv * KPW + u) * 512 + lane * 8;
    const int r = e / D, pch = (e % D) / 8;
    koff[u] = (uint32_t)(r * D * 2 + ((pch ^ r) & (CH - 1)) * 16);
    voff[u] = (uint32_t)(r * D * 2 + ((pch ^ swzv_f<D>(r)) & (CH - 1)) * 16);
  }
  const int wvs = __builtin_amdgcn_readfirstlane(wv);
  auto stage = [&](int j, int buf) __attribute__((always_inline)) {   // j < 0: nothing
    const int row0 = j < 0 ? 0 : j * kBlock;
    const uint32_t bytes = j < 0 ? 0u : (uint32_t)(min(kBlock, a.nkv - row0) * D * 2);
    const i32x4 rk = make_rsrc(kb + (size_t)row0 * D, bytes);
    const i32x4 rv = make_rsrc(vb + (size_t)row0 * D, bytes);
    const uint32_t kd = lds_addr(smem + buf * TILE) + wvs * KPW * 1024;
    const uint32_t vd = lds_addr(smem + (2 + buf) * TILE) + wvs * KPW * 1024;
#pragma unroll
    for (int u = 0; u < KPW; ++u) load_lds16(rk, kd + u * 1024, koff[u]);
#pragma unroll
    for (int u = 0; u < KPW; ++u) load_lds16(rv, vd + u * 1024, voff[u]);
  };

  const bool attn = wv < 2;
  // ---------------------------------------------------------------- attention state
  const int qrow0 = iq * kBlock + 32 * (wv & 1);
  u32x4 qf[KS];
  f32x16 o[CT];
  float m = kNegBig, l = 0.f;
  const float qk_scale = kLog2e / sqrtf((float)D);
  // ---------------------------------------------------------------- summary state
  f32x16 sacc[MT][CT];
  float zs[MT];
  const int rbase = (D / 2) * (wv & 1);
#pragma unroll
  for (int c = 0; c < CT; ++c) o[c] = f32x16{};
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    zs[mt] = 0.f;
#pragma unroll
    for (int c = 0; c < CT; ++c) sacc[mt][c] = f32x16{};
  }
  if (attn) {
    const int q = qrow0 + l32;
    const uint16_t* qsrc = a.q + ((size_t)bh * a.nq + (q < a.nq ? q : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = q < a.nq ? *reinterpret_cast<const u32x4*>(qsrc + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};
  }

  auto attend = [&](const uint16_t* Kt, const uint16_t* Vt, int j) __attribute__((always_inline)) {
    f32x16 s2[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const u32x4 af = *reinterpret_cast<const u32x4*>(&Kt[swz<D>(32 * mt + l32, 16 * ks + 8 * h)]);
        s2[mt] = mfma_bf16(af, qf[ks], s2[mt]);
      }
    if (__builtin_amdgcn_readfirstlane((j + 1) * kBlock > a.nkv ? 1 : 0)) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = j * kBlock + 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
          s2[mt][e] = key < a.nkv ? s2[mt][e] : -INFINITY;
        }
    }
    float r = kNegBig;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) r = fmaxf(r, s2[mt][e]);
    r = fmaxf(r, swap_halves(r)) * qk_scale;
    if (__ballot(r > m + kRescaleSlack)) {
      const float mn = fmaxf(m, r);
      const float corr = __builtin_amdgcn_exp2f(m - mn);
      l *= corr;
#pragma unroll
      for (int c = 0; c < CT; ++c) o[c] *= corr;
      m = mn;
    }
    u32x4 phi[4], plo[4];
    float rs = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int e = 8 * hh + 2 * e2;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[mt][e], qk_scale, -m));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[mt][e + 1], qk_scale, -m));
          rs += p0 + p1;
          const uint32_t hi = pack_bf16(p0, p1);
          phi[2 * mt + hh][e2] = hi;
          plo[2 * mt + hh][e2] = pack_bf16(p0 - bf16_lo(hi), p1 - bf16_hi(hi));
        }
    l += rs;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const u32x4 vf = vt_frag<D>(Vt, 32 * c, 16 * kk);
        o[c] = mfma_bf16(vf, phi[kk], o[c]);
        o[c] = mfma_bf16(vf, plo[kk], o[c]);
      }
  };

  auto summarise = [&](const uint16_t* Kt, const uint16_t* Vt) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      u32x4 af[4];
      float zl = 0.f;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        af[s4] = relu_bf16x8(tr_frag<D, false>(Kt, rbase + 32 * mt, 16 * s4));
#pragma unroll
        for (int e = 0; e < 4; ++e) zl += bf16_lo(af[s4][e]) + bf16_hi(af[s4][e]);
      }
      zs[mt] += zl;
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          sacc[mt][c] = mfma_bf16(af[s4], tr_frag<D, true>(Vt, 32 * c, 16 * s4), sacc[mt][c]);
    }
  };

  // ---------------------------------------------------------------- tile loop
  // Both wave groups run the same steps and barriers; the loops are separate so that the
  // attention state and the summary accumulators never have to be live together.
  const int ntile = e1 - e0;
  if (ntile > 0) stage(entry(e0), 0);
  barrier_vmem_n<0>();
  if (attn) {
    for (int it = 0; it < ntile; ++it) {
      const int buf = it & 1;
      const int j = entry(e0 + it);
      stage(it + 1 < ntile ? entry(e0 + it + 1) : -1, buf ^ 1);
      attend(smem + buf * TILE, smem + (2 + buf) * TILE, j);
      barrier_vmem_n<0>();
    }
  } else {
    for (int it = 0; it < ntile; ++it) {
      const int buf = it & 1;
      stage(it + 1 < ntile ? entry(e0 + it + 1) : -1, buf ^ 1);
      summarise(smem + buf * TILE, smem + (2 + buf) * TILE);
      barrier_vmem_n<0>();
    }
  }

  // ---------------------------------------------------------------- partial results out
  if (attn) {
    l += swap_halves(l);
    const int qr = 32 * (wv & 1) + l32;          // row within the query block
    if (h == 0) {
      a.pml[(pidx * kBlock + qr) * 2 + 0] = m;
      a.pml[(pidx * kBlock + qr) * 2 + 1] = l;
    }
    float* dst = a.po + (pidx * kBlock + qr) * D;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(dst + 32 * c + 8 * g + 4 * h) =
            f32x4{o[c][4 * g], o[c][4 * g + 1], o[c][4 * g + 2], o[c][4 * g + 3]};
  } else {
    float* dst = a.ps + pidx * D * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float zt = zs[mt] + swap_halves(zs[mt]);
      if (h == 0) a.pz[pidx * D + rbase + 32 * mt + l32] = zt;
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int col = 32 * c + l32;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r = rbase + 32 * mt + 8 * g + 4 * h;
          *reinterpret_cast<f32x4*>(dst + (size_t)col * D + r) =
              f32x4{sacc[mt][c][4 * g], sacc[mt][c][4 * g + 1], sacc[mt][c][4 * g + 2],
                    sacc[mt][c][4 * g + 3]};
        }
      }
    }
  }
}

struct CombineArgs {
  const uint16_t* q;
  const float* alpha;   // [H][D]
  const float* stot;    // [BH][D(c)][D(r)]
  const float* ztot;    // [BH][D]
  const float* pml;
  const float* po;
  const float* ps;
  const float* pz;
  void* out;
  int nq, nbq, nbk, topk, nsplit, H;
};


// One workgroup per (batch*head, query block, 32-channel tile ct of the output): S_c^T rows
// c in the tile (all d columns r), z_c, the merge weights of the parts, then for the two
// 32-row query tiles (waves 0 and 1) O_l^T = S_c^T phi(Q)^T and the mix.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void decode_combine_kernel(CombineArgs a) {
  constexpr int KS = D / 16;
  constexpr int SR = D + 8;                        // padded LDS row of S_c^T (elements)
  __shared__ __attribute__((aligned(16))) uint16_t Sc[32 * SR];
  __shared__ float zc[D];
  __shared__ float wgt[kMaxDecodeParts][kBlock];   // per part and row: exp2(m_p - M) / L
  const int bq = blockIdx.x;                       // bh * nbq + iq
  const int ct = blockIdx.y;
  const int bh = bq / a.nbq, iq = bq % a.nbq;
  const int t = threadIdx.x, wv = t >> 6, h = (t & 63) >> 5, l32 = t & 31;
  const size_t p0 = (size_t)bq * a.nsplit;
  const bool empty_c = a.topk >= a.nbk;            // every block selected: no complement

  // rows c = 32 ct .. 32 ct + 31 of S_c^T = S_tot^T - sum_p S_sel,p^T (bf16); z_c
  for (int e4 = t; e4 < 32 * D / 4; e4 += 256) {
    const size_t off = (size_t)32 * ct * D + 4 * e4;
    f32x4 sv = *reinterpret_cast<const f32x4*>(a.stot + (size_t)bh * D * D + off);
    for (int p = 0; p < a.nsplit; ++p) {
      const f32x4 pv = *reinterpret_cast<const f32x4*>(a.ps + (p0 + p) * D * D + off);
      sv -= pv;
    }
    if (empty_c) sv = f32x4{0.f, 0.f, 0.f, 0.f};
    const int c = (4 * e4) / D, r = (4 * e4) % D;
    *reinterpret_cast<u32x2*>(&Sc[c * SR + r]) = u32x2{pack_bf16(sv[0], sv[1]), pack_bf16(sv[2], sv[3])};
  }
  if (t < D) {
    float z = a.ztot[(size_t)bh * D + t];
    for (int p = 0; p < a.nsplit; ++p) z -= a.pz[(p0 + p) * D + t];
    zc[t] = empty_c ? 0.f : z;
  }
  if (t < kBlock) {
    float M = kNegBig;
    for (int p = 0; p < a.nsplit; ++p) M = fmaxf(M, a.pml[((p0 + p) * kBlock + t) * 2]);
    float L = 0.f;
    for (int p = 0; p < a.nsplit; ++p) {
      const float mp = a.pml[((p0 + p) * kBlock + t) * 2];
      L += __builtin_amdgcn_exp2f(mp - M) * a.pml[((p0 + p) * kBlock + t) * 2 + 1];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    for (int p = 0; p < a.nsplit; ++p)
      wgt[p][t] = __builtin_amdgcn_exp2f(a.pml[((p0 + p) * kBlock + t) * 2] - M) * inv;
  }
  __syncthreads();
  if (wv >= 2) return;

  const float* al = a.alpha + (size_t)(bh % a.H) * D;
  const int qr = 32 * wv + l32;                    // row within the query block
  const int q = iq * kBlock + qr;
  const uint16_t* qsrc = a.q + ((size_t)bh * a.nq + (q < a.nq ? q : 0)) * D;
  f32x16 lin = f32x16{};
  float d = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const u32x4 qw = q < a.nq ? *reinterpret_cast<const u32x4*>(qsrc + 16 * s + 8 * h)
                              : u32x4{0, 0, 0, 0};
    const u32x4 qr8 = relu_bf16x8(qw);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      d += bf16_lo(qr8[e]) * zc[16 * s + 8 * h + 2 * e] + bf16_hi(qr8[e]) * zc[16 * s + 8 * h + 2 * e + 1];
    const u32x4 af = *reinterpret_cast<const u32x4*>(&Sc[l32 * SR + 16 * s + 8 * h]);
    lin = mfma_bf16(af, qr8, lin);
  }
  d += swap_halves(d);
  const float inv_den = 1.f / (d + kEps);
  if (q < a.nq) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int ch = 32 * ct + 8 * g + 4 * h;
      f32x4 os = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int p = 0; p < a.nsplit; ++p) {
        const f32x4 pv = *reinterpret_cast<const f32x4*>(a.po + ((p0 + p) * kBlock + qr) * D + ch);
        os += pv * wgt[p][qr];
      }
      const f32x4 alv = *reinterpret_cast<const f32x4*>(al + ch);
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        r[e] = alv[e] * os[e] + (1.f - alv[e]) * (lin[4 * g + e] * inv_den);
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

template <int D>
hipError_t launch_decode_T(const Plan& s, const DecodePlan& d, const void* q, const void* k,
                           const void* v, const int32_t* idx, const float* alpha,
                           const char* cache, const CachePlan& c, void* o, char* ws,
                           hipStream_t st) {
  DecodeArgs a;
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.k = reinterpret_cast<const uint16_t*>(k);
  a.v = reinterpret_cast<const uint16_t*>(v);
  a.idx = idx;
  a.pml = reinterpret_cast<float*>(ws + d.pml);
  a.po = reinterpret_cast<float*>(ws + d.po);
  a.ps = reinterpret_cast<float*>(ws + d.ps);
  a.pz = reinterpret_cast<float*>(ws + d.pz);
  a.nq = s.nq; a.nkv = s.nkv; a.nbq = s.nbq; a.nbk = s.nbk; a.topk = s.k;
  a.nsplit = d.nsplit;
  a.total = s.BH * s.nbq * d.nsplit;
  hipLaunchKernelGGL((decode_attn_kernel<D>), dim3(a.total), dim3(256), 0, st, a);
  CombineArgs b;
  b.q = a.q;
  b.alpha = alpha;
  b.stot = reinterpret_cast<const float*>(cache + c.stot);
  b.ztot = reinterpret_cast<const float*>(cache + c.ztot);
  b.pml = a.pml; b.po = a.po; b.ps = a.ps; b.pz = a.pz;
  b.out = o;
  b.nq = s.nq; b.nbq = s.nbq; b.nbk = s.nbk; b.topk = s.k; b.nsplit = d.nsplit; b.H = s.H;
  const dim3 grid(s.BH * s.nbq, D / 32);
  if (s.out_bf16)
    hipLaunchKernelGGL((decode_combine_kernel<D, true>), grid, dim3(256), 0, st, b);
  else
    hipLaunchKernelGGL((decode_combine_kernel<D, false>), grid, dim3(256), 0, st, b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const Plan& s, const void* q, const void* k, const void* v,
                         const int32_t* idx, const float* alpha, const char* cache, void* o,
                         char* ws, hipStream_t st) {
  const DecodePlan d = make_decode_plan(s);
  const CachePlan c = make_cache_plan(s);
  if (s.D == 128) return launch_decode_T<128>(s, d, q, k, v, idx, alpha, cache, c, o, ws, st);
  return launch_decode_T<64>(s, d, q, k, v, idx, alpha, cache, c, o, ws, st);
}

}  // namespace sla
