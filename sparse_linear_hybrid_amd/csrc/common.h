// Shared device helpers for the gfx950 (CDNA4) SLA kernels: vector types, MFMA wrappers,
// dtype conversions and the workspace plan shared by the host launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>
#include <stddef.h>

#include "../../include/sla.h"

namespace sla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 64;          // query block = key block = 64 tokens
constexpr float kEps = 1e-6f;       // linear-branch denominator epsilon
constexpr int kMaxKeyBlocks = 8064;   // top-k keeps a row of 64-bit keys in 64 KB of LDS
// Online softmax in base 2: logits are scaled by log2(e)/sqrt(d); running maxima start at a
// finite "minus infinity"; a max may lag the true one while the weights stay below 2^8,
// which f16 weights hold exactly enough and which saves most rescales.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;
constexpr float kRescaleSlack = 8.0f;
// Saved log-sum-exp of a row with no exact part (or past n_q): exp2(x - kNoRowLse) = 0.
constexpr float kNoRowLse = 1.0e30f;

// ----------------------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// low / high bf16 of a packed 32-bit word
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (hardware round-to-nearest-even).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// Two floats -> packed f16 pair (hardware round-to-nearest-even).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// ReLU on 8 packed bf16 values held in 4 dwords: a lane is zeroed when its sign bit is set
// (this also maps -0 to +0, which does not change any product).
__device__ __forceinline__ u32x4 relu_bf16x8(u32x4 w) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t x = w[i];
    uint32_t lo = (x & 0x8000u) ? 0u : (x & 0xffffu);
    uint32_t hi = (x & 0x80000000u) ? 0u : (x & 0xffff0000u);
    r[i] = lo | hi;
  }
  return r;
}

// ----------------------------------------------------------------------------- MFMA
// 32x32x16 bf16 / f16, fp32 accumulate. Operand layout (64 lanes, 8 elements per lane):
//   A[i][k]: lane i + 32*(k/8), element k%8;  B[k][j]: lane j + 32*(k/8), element k%8;
//   C[i][j]: lane j + 32*((i/4)%2), element (i%4) + 4*(i/8).
__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// LDS transposing read of 4 x 16-bit values. Within each group of 16 lanes, lane L
// supplies the address of 4 consecutive 16-bit elements of row r0 + L/4 starting at
// column c0 + 4*(L%4); lane i of the group receives column c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds_ptr) {
  s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(lds_ptr));
  return __builtin_bit_cast(u32x2, t);
}

// Raw buffer descriptor over `bytes` bytes from `base` (stride 0): loads at offsets >= bytes
// return 0 without touching memory.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)b, (int)((b >> 32) & 0xffffu), (int)bytes, 0x00020000};
}
// The same as a compiler buffer resource, for its buffer load and store builtins: loads at
// offsets >= bytes return 0 and stores there are dropped, without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Buffer load of 16 bytes per lane straight into LDS: lane l's bytes from offset voff land at
// LDS byte address lds + 16*l (lds is wave-uniform). Written as asm so that the compiler's
// own wait insertion does not drain these loads before every LDS read; every consumer waits
// explicitly (wait_vmem*, barrier_vmem_n). The instruction writes no VGPR, so nothing of the
// compiler's register allocation is left in flight. M0 is set here and used by nothing else
// in the kernels that call this; an SALU write of M0 needs one wait state before a load
// into LDS reads it.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}
// Wait until every vector-memory load of this wave, including loads into LDS, has landed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector-memory loads of this wave are still in flight (they complete
// in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier for loops whose only LDS writes are loads into LDS: first wait until at
// most N vector-memory loads of this wave are in flight, then s_barrier. Unlike
// __syncthreads() it does not drain every outstanding load; the LDS reads before it have all
// been consumed by then. One asm block, so no memory access moves across it.
template <int N>
__device__ __forceinline__ void barrier_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
// The same for loops that also write LDS with ordinary stores that other waves read after
// the barrier: those stores must have completed (lgkmcnt(0)) before the barrier, which
// s_barrier alone does not ensure.
template <int N>
__device__ __forceinline__ void barrier_vmem_lds_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// ----------------------------------------------------------------------------- tile layout
// 64-row tiles of D 16-bit columns in LDS (attention K and V tiles, centroid and value-sum
// tiles), shared by the exact branch and the piecewise tail.
// Element offset of (row, col) in a swizzled LDS tile with D 16-bit columns per row: the
// 16-byte chunk index is XORed with the row (mod chunks per row).
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  constexpr int CH = D / 8;
  return row * D + ((((col >> 3) ^ row) & (CH - 1)) << 3) + (col & 7);
}

// Swizzle of the V tile. A transposing V^T read has each group of 16 lanes touch 4
// consecutive key rows x 2 adjacent chunks (and each 32 lanes 4 rows x 4 chunks); XORing
// the chunk index with f(row % 4) spreads those accesses over distinct banks whether the LDS
// serves 128 or 256 bytes per clock. Rows are bijective, so the row-wise tile writes stay
// conflict-free as well.
template <int D>
__device__ __forceinline__ int swzv_f(int row) {
  const int r = row & 3;
  return D == 128 ? (((r & 1) ? 6 : 0) ^ ((r & 2) ? 10 : 0)) : 2 * r;
}
template <int D>
__device__ __forceinline__ int swzv(int row, int col) {
  constexpr int CH = D / 8;
  return row * D + ((((col >> 3) ^ swzv_f<D>(row)) & (CH - 1)) << 3) + (col & 7);
}

// P^T-matched V^T fragment from a swizzled row-major [key][channel] tile: lane row (channel)
// x0 + lane%32; reduction slot e holds key k0 + 4h + e (e < 4) or k0 + 8 + 4h + (e - 4)
// (e >= 4), h = lane / 32.
template <int D>
__device__ __forceinline__ u32x4 vt_frag(const uint16_t* M, int x0, int k0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, L = lane & 15;
  const int row = k0 + 4 * (g >> 1) + (L >> 2);
  const int col = x0 + 16 * (g & 1) + 4 * (L & 3);
  const u32x2 lo = lds_read_tr16(M + swzv<D>(row, col));
  const u32x2 hi = lds_read_tr16(M + swzv<D>(row + 8, col));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Exchange with lane l ^ 32: returns the value held by the other half of the wave.
__device__ __forceinline__ float swap_halves(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // r[0]: lanes < 32 keep their own value, lanes >= 32 get lane l-32's;
  // r[1]: lanes < 32 get lane l+32's, lanes >= 32 keep their own.
  const int lane = threadIdx.x & 63;
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

// Workgroup index remap so that consecutive logical indices run on the same XCD (the
// dispatcher assigns workgroup w to XCD w % 8). Bijective for any n.
__device__ __forceinline__ int xcd_remap(int w, int n) {
  const int nx = 8;
  const int per = n / nx, rem = n % nx;
  const int x = w % nx, slot = w / nx;
  // XCD x owns logical range [start_x, start_x + cnt_x)
  const int start = x * per + (x < rem ? x : rem);
  const int cnt = per + (x < rem ? 1 : 0);
  return slot < cnt ? start + slot : w;
}

// ----------------------------------------------------------------------------- E4M3 blocks
// Block exponent for E4M3 (SLA2 page, section 2.C, quantised sparse branch): the smallest
// integer e with 448 * 2^e >= absmax (0 for an all-zero block).
__device__ __forceinline__ int e8m0_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int ex;
  (void)frexpf(amax / 448.f, &ex);
  int e = ex;
  while (448.f * ldexpf(1.f, e - 1) >= amax) --e;    // exact: products with powers of two
  while (448.f * ldexpf(1.f, e) < amax) ++e;
  return e;
}
// position (0..63) of key k inside a V8 tile row (the P8 operand order of P.V)
__device__ __forceinline__ int v8_slot_pos(int k) {
  const int mt = k >> 5, rem = k & 31;
  const int g = rem >> 3, hh = (rem >> 2) & 1, i = rem & 3;
  return 32 * hh + 16 * mt + 4 * g + i;
}
// E4M3 byte -> the same value as bf16 (exact: E4M3 has at most 4 significant bits and its
// exponent range lies inside bf16's).
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t c) {
  const uint32_t sgn = (c & 0x80u) << 8;
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  // subnormal: m * 2^-9, exact in fp32 and in its top 16 bits
  if (e == 0) return sgn | (__float_as_uint((float)m * 0x1p-9f) >> 16);
  return sgn | ((e - 7 + 127) << 7) | (m << 4);
}
// 8 values scaled by 2^-e (exact) and rounded once to E4M3 (hardware round-to-nearest-even):
// bytes 0..3 in w0, 4..7 in w1
__device__ __forceinline__ void e4m3x8(const float (&v)[8], int e, uint32_t& w0, uint32_t& w1) {
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[0], -e), ldexpf(v[1], -e), 0u, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[2], -e), ldexpf(v[3], -e), w0, true);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4], -e), ldexpf(v[5], -e), 0u, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[6], -e), ldexpf(v[7], -e), w1, true);
}
// 8 E4M3 bytes (w0, w1) as 8 bf16 values: the hardware conversion to fp32 is exact, and the
// top 16 bits of the result are the same value in bf16 (E4M3 has at most 4 significant bits
// and its exponent range lies inside bf16's).
__device__ __forceinline__ u32x4 e4m3x8_as_bf16(uint32_t w0, uint32_t w1) {
  // bytes 0, 1 (false) or 2, 3 (true) of w as two bf16 in one word
  auto two = [](uint32_t w, auto hi) __attribute__((always_inline)) {
    const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, decltype(hi)::value);
    return __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
  };
  const std::false_type lo{};
  const std::true_type hi{};
  return u32x4{two(w0, lo), two(w0, hi), two(w1, lo), two(w1, hi)};
}
// Outputs of the E4M3 quantisation of K and V when the key/value pass does it (fp8 forward):
// K8 [BH][nb*64][D] bf16-held, V8 tiles [BH][nb][D][64] bytes, block exponents [BH][nb].
struct Fp8Out {
  uint8_t* k8;
  uint8_t* v8;
  int32_t* ek;
  int32_t* ev;
};

// ----------------------------------------------------------------------------- workspace
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Plan {
  int B, H, BH, nq, nkv, D, nbq, nbk, k, nchunk;
  bool in_bf16, out_bf16;
  // byte offsets into the workspace
  size_t qt, kt, scores, idx, kvar;              // router (kvar: training-free router)
  size_t v16, sblk, zblk, spart, zpart, stot, ztot, sc, zc;   // linear branch
  int nwords;                                   // 32-bit words of a key-block bitmap row
  size_t selbits;                               // routed-block bitmap [BH][nbq][nwords]
  size_t q8, k8, v8, sq8, sk8, sv8;             // fp8 sparse branch
  size_t total_route, total_fwd, total_fp8;
  // piecewise (exact-or-approximate) forward: its own layout after the router's buffers
  int npad;                                     // key blocks rounded up to whole 64-tiles
  size_t p_spart, p_zpart, p_stot, p_ztot;      // chunk partials and totals of H
  size_t cent_hi, cent_lo;                      // centroids, bf16 hi + lo [BH][npad][D]
  size_t vsum;                                  // value sums, f16 [BH][npad][D]
  size_t hbar;                                  // bf16 H_bar^T [BH][D(c)][D(r)]
  size_t tail_m, tail_d, tail_a, tail_n;        // tail state per query row
  size_t total_pisa;
  // Few query blocks over many key blocks (a decode chunk against a long key sequence): the
  // learnable-router forward then builds the key/value summary cache in its workspace and
  // runs the cached forward, instead of storing and re-reading every key block's summary.
  bool few;
  size_t few_cache, few_cws, few_dec;           // cache, its update workspace, decode workspace
  size_t total_few;
};


constexpr int kSummaryChunk = 8;  // key blocks per partial-total chunk

inline Plan make_plan(const sla_problem& p) {
  Plan s{};
  s.B = p.batch; s.H = p.heads; s.BH = p.batch * p.heads;
  s.nq = p.n_q; s.nkv = p.n_kv; s.D = p.head_dim;
  s.nbq = (p.n_q + kBlock - 1) / kBlock;
  s.nbk = (p.n_kv + kBlock - 1) / kBlock;
  s.k = p.top_k;
  s.nchunk = (s.nbk + kSummaryChunk - 1) / kSummaryChunk;
  s.in_bf16 = p.in_dtype == SLA_BF16;
  s.out_bf16 = p.out_dtype == SLA_BF16;
  const size_t BH = s.BH, D = s.D, nbq = s.nbq, nbk = s.nbk;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  s.qt = take(BH * nbq * D * 8);
  s.kt = take(BH * nbk * D * 8);
  s.scores = take(BH * nbq * nbk * 8);
  s.idx = take(BH * nbq * (size_t)(s.k > 0 ? s.k : 1) * 4);
  s.kvar = take(BH * nbk * D * 8);
  s.total_route = off;
  s.v16 = take(BH * nbk * kBlock * D * 2);
  s.sblk = take(BH * nbk * D * D * 2);
  s.zblk = take(BH * nbk * D * 4);
  s.spart = take(BH * (size_t)s.nchunk * D * D * 4);
  s.zpart = take(BH * (size_t)s.nchunk * D * 4);
  s.stot = take(BH * D * D * 4);
  s.ztot = take(BH * D * 4);
  s.sc = take(BH * nbq * D * D * 2);
  s.zc = take(BH * nbq * D * 4);
  s.nwords = (s.nbk + 31) / 32;
  s.selbits = take(BH * nbq * (size_t)s.nwords * 4);
  s.total_fwd = off;
  s.q8 = take(BH * nbq * kBlock * D * 2);   // E4M3 values held as bf16
  s.k8 = take(BH * nbk * kBlock * D * 2);
  s.v8 = take(BH * nbk * kBlock * D);
  s.sq8 = take(BH * nbq * 4);
  s.sk8 = take(BH * nbk * 4);
  s.sv8 = take(BH * nbk * 4);
  s.total_fp8 = off;
  // piecewise forward: router buffers, f16 V, then its own regions
  s.npad = (s.nbk + kBlock - 1) / kBlock * kBlock;
  const size_t npad = s.npad, nqpad = nbq * kBlock;
  off = s.v16;
  take(BH * nbk * kBlock * D * 2);               // v16, same offset as the forward's
  s.p_spart = take(BH * (size_t)s.nchunk * D * D * 4);
  s.p_zpart = take(BH * (size_t)s.nchunk * D * 4);
  s.p_stot = take(BH * D * D * 4);
  s.p_ztot = take(BH * D * 4);
  s.cent_hi = take(BH * npad * D * 2);
  s.cent_lo = take(BH * npad * D * 2);
  s.vsum = take(BH * D * npad * 2);
  s.hbar = take(BH * D * D * 2);
  s.tail_m = take(BH * nqpad * 4);
  s.tail_d = take(BH * nqpad * 4);
  s.tail_a = take(BH * nqpad * 4);
  s.tail_n = take(BH * nqpad * D * 4);
  s.total_pisa = off;
  return s;
}

// Workspace of the backward (sla_backward): the forward's per-block layout (key/value pass,
// complement, bitmap), then the backward's own regions.
// The backward for at most this many query blocks per head forms each key block's G_j in the
// key kernel from the few dS_c(i) instead of materialising every G_j (no G_j region); when
// those query blocks also select at most half the key blocks, S_c(i) is S_tot minus the
// selected blocks' summaries (no per-block S_j and no low parts).
constexpr int kFewBwdRows = 8;
inline bool bwd_few_g(const Plan& s) { return s.nbq <= kFewBwdRows; }
inline bool bwd_few_sc(const Plan& s) { return s.nbq <= kFewBwdRows && 2 * s.k <= s.nbk; }
struct BwdPlan {
  int nwq;                                      // 32-bit words of a query-block bitmap row
  size_t bitsT, counts, sblo, scf, os, lse, dr, dos, dsc, dsclo, dzc, gt, gz, dapart, order,
      bytes;
};
inline BwdPlan make_bwd_plan(const Plan& s) {
  BwdPlan b{};
  const size_t BH = s.BH, D = s.D, nbq = s.nbq, nbk = s.nbk, nq64 = nbq * kBlock;
  b.nwq = (s.nbq + 31) / 32;
  size_t off = s.total_fwd;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  b.bitsT = take(BH * nbk * (size_t)b.nwq * 4);
  b.counts = take(BH * nbk * 4);                // query blocks that routed each key block
  b.sblo = take(bwd_few_sc(s) ? 0 : BH * nbk * D * D * 2);   // S_j - bf16(S_j), bf16
  b.scf = take(BH * nbq * D * D * 4);           // S_c^T fp32
  b.os = take(BH * (size_t)s.nq * D * 4);        // O_s fp32, saved by the sparse kernel
  b.lse = take(BH * nq64 * 4);
  b.dr = take(BH * nq64 * 4);
  b.dos = take(BH * nq64 * D * 2);
  b.dsc = take(BH * nbq * D * D * 2);           // dS_c(i)^T, bf16 high part, summary layout
  b.dsclo = take(BH * nbq * D * D * 2);         // and its low part
  b.dzc = take(BH * nbq * D * 4);
  b.gt = take(bwd_few_g(s) ? 0 : BH * nbk * D * D * 4);   // G_j^T fp32
  b.gz = take(BH * nbk * D * 4);
  b.dapart = take(BH * nbq * D * 4);
  b.order = take(BH * nbk * 4);                 // key-block task order of the key kernel
  b.bytes = off;
  return b;
}

// When the forward takes the cache path (Plan::few): at most kFewQueryBlocks query blocks per
// head and at least kFewMinKeyBlocks key blocks, bf16 inputs.
constexpr int kFewQueryBlocks = 8;
constexpr int kFewMinKeyBlocks = 256;

// ----------------------------------------------------------------------------- summary cache
// Key/value summary cache (caller-owned, see sla_kv_cache_update): S_tot^T [BH][D(c)][D(r)]
// fp32, z_tot [BH][D] fp32, then k~ [nbk][BH][D] fp64. k~ is block-major so that the layout
// only grows at its end as tokens are appended.
struct CachePlan {
  size_t stot, ztot, kt, bytes;
};
inline CachePlan make_cache_plan(const Plan& s) {
  CachePlan c{};
  const size_t BH = s.BH, D = s.D;
  c.stot = 0;
  c.ztot = align_up(BH * D * D * 4, 256);
  c.kt = align_up(c.ztot + BH * D * 4, 256);
  c.bytes = c.kt + (size_t)s.nbk * BH * D * 8;
  return c;
}
// Key blocks per workgroup of a cache update, and the chunks an update from n_done tokens
// to s.nkv touches (larger chunks than the forward's: fewer partial totals to add up).
constexpr int kCacheChunk = 64;
inline int cache_update_chunks(const Plan& s, int n_done) {
  const int nblocks = s.nbk - n_done / kBlock;
  return nblocks > 0 ? (nblocks + kCacheChunk - 1) / kCacheChunk : 0;
}
inline size_t cache_update_zpart_offset(const Plan& s, int n_done) {
  return align_up((size_t)s.BH * cache_update_chunks(s, n_done) * s.D * s.D * 4, 256);
}
inline size_t cache_update_ws_bytes(const Plan& s, int n_done) {
  return cache_update_zpart_offset(s, n_done) +
         (size_t)s.BH * cache_update_chunks(s, n_done) * s.D * 4;
}

// Workspace of the cached forward: router buffers, then the per-part partial results of
// the decode kernel.
constexpr int kMaxDecodeParts = 32;
struct DecodePlan {
  int nsplit;
  size_t qt, scores, idx, pml, po, ps, pz, bytes;
};
inline DecodePlan make_decode_plan(const Plan& s) {
  DecodePlan d{};
  const size_t BH = s.BH, D = s.D, nbq = s.nbq, nbk = s.nbk;
  // enough parts to give the GPU about 1024 workgroups, each with at least 4 key blocks
  int ns = (int)((1024 + BH * nbq - 1) / (BH * nbq));
  ns = ns < s.k / 4 ? ns : s.k / 4;
  ns = ns < kMaxDecodeParts ? ns : kMaxDecodeParts;
  d.nsplit = ns < 1 ? 1 : ns;
  const size_t parts = BH * nbq * d.nsplit;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  d.qt = take(BH * nbq * D * 8);
  d.scores = take(BH * nbq * nbk * 8);
  d.idx = take(BH * nbq * (size_t)(s.k > 0 ? s.k : 1) * 4);
  d.pml = take(parts * kBlock * 2 * 4);
  d.po = take(parts * kBlock * D * 4);
  d.ps = take(parts * D * D * 4);
  d.pz = take(parts * D * 4);
  d.bytes = off;
  return d;
}

// Layout of the forward's workspace on the cache path: the key/value summary cache, the
// update's partial totals, then the cached forward's workspace. Sets s.few and, when the
// path is taken, its size s.total_few.
inline void plan_few_path(Plan& s) {
  s.few = s.in_bf16 && s.nbq <= kFewQueryBlocks && s.nbk >= kFewMinKeyBlocks;
  if (!s.few) return;
  s.few_cache = 0;
  s.few_cws = align_up(make_cache_plan(s).bytes, 256);
  s.few_dec = align_up(s.few_cws + cache_update_ws_bytes(s, 0), 256);
  s.total_few = s.few_dec + make_decode_plan(s).bytes;
}

}  // namespace sla
