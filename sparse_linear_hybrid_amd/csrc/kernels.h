// Host-side launchers of the SLA kernels (one translation unit per kernel family).
#pragma once
#include "common.h"

namespace sla {

// Router: pool + project Q (and K if pool_k), score, top-k -> idx; bits != nullptr: also the
// routed-block bitmap [BH][nbq][nwords] that the complement reads.
hipError_t launch_route(const Plan& s, const void* q, const void* k, const float* pq,
                        const float* pk, int32_t* idx, uint32_t* bits, char* ws, bool pool_k,
                        hipStream_t st);

// Linear branch, part 1 (independent of routing): per key block phi(K)^T V, sum phi(K),
// the projected pooled K (for the router), an f16 copy of V, and the per-head totals.
// sblk_lo (bf16 inputs, not fp8): also S_j - bf16(S_j), rounded to bf16, in the layout of S_j.
hipError_t launch_kv_summary(const Plan& s, const void* k, const void* v, const float* pk, char* ws,
                             hipStream_t st, bool fp8 = false, uint16_t* sblk_lo = nullptr);

// Few-query-block backward (bf16): the key/value pass with S_tot and z_tot instead of the
// per-block S_j and the f16 V copy (z_j as usual), and S_c(i)^T = S_tot^T - sum of the selected
// S_j^T in fp32 from the selected K and V tiles, which also writes the selected blocks' f16 V.
hipError_t launch_kv_totals_blocks(const Plan& s, const void* k, const void* v, char* ws,
                                   hipStream_t st);
hipError_t launch_sc_subtract(const Plan& s, const void* k, const void* v, const int32_t* idx,
                              const float* stot, float* sc, char* ws, hipStream_t st);

// Linear branch, part 2: complement = total - selected, per query block.
hipError_t launch_complement(const Plan& s, const int32_t* idx, char* ws, hipStream_t st);

// Sparse branch (bf16 MFMA for Q K^T, f16 MFMA for P V) with the linear apply and the
// alpha mix fused into its epilogue.
hipError_t launch_sparse(const Plan& s, const void* q, const void* k, const int32_t* idx,
                         const float* alpha, void* o, char* ws, hipStream_t st);

// The sparse branch alone for the backward (bf16 inputs): O_s (fp32 [BH][n_q][D]) and each
// row's log-sum-exp (base 2, scaled units; [BH][nbq*64]).
hipError_t launch_sparse_save(const Plan& s, const void* q, const void* k, const int32_t* idx,
                              float* os, float* lse, char* ws, hipStream_t st);

// Quantised sparse branch (fp8 MFMA) with the same epilogue as launch_sparse.
hipError_t launch_sparse_fp8(const Plan& s, const void* q, const int32_t* idx,
                             const float* alpha, void* o, char* ws, hipStream_t st);

// Training-free router (SPLA page, section 2.1): block means of Q and K, variances of K,
// second-order Taylor scores, top-k -> idx.
hipError_t launch_route_taylor(const Plan& s, const void* q, const void* k, int32_t* idx,
                               uint32_t* bits, char* ws, hipStream_t st);

// Summary cache: bring k~, S_tot, z_tot from the first n_done tokens to s.nkv tokens.
hipError_t launch_kv_cache_update(const Plan& s, const void* k, const void* v, const float* pk,
                                  int n_done, char* cache, char* ws, hipStream_t st);

// Streaming cache pass (bf16): k~ of every key block from n_done / 64 on, and the chunk
// partial totals of phi(K)^T V and phi(K) over the tokens from n_done on (into ws, laid out
// as cache_update_ws_bytes describes).
hipError_t launch_kv_totals(const Plan& s, const void* k, const void* v, const float* pk,
                            int n_done, double* kt, size_t kbh, size_t kj, float* stot,
                            float* ztot, char* ws, hipStream_t st);

// Projected block means (float64) of a bf16 tensor [BH][n][D] through a streaming ring:
// out[bh][j][:] = mean of block j's valid tokens @ P.
hipError_t launch_pool_stream(const Plan& s, const void* x, const float* P, double* out, int n,
                              int nb, hipStream_t st);

// Router against cached k~ (k~ of block j of head bh at kt + bh * kbh + j * kj).
hipError_t launch_route_cached(const Plan& s, const void* q, const float* pq, const double* kt,
                               size_t kbh, size_t kj, int32_t* idx, double* qt, double* sc,
                               hipStream_t st);

// Cached forward: exact branch and selected-block summaries per part, then the combine.
hipError_t launch_decode(const Plan& s, const void* q, const void* k, const void* v,
                         const int32_t* idx, const float* alpha, const char* cache, void* o,
                         char* ws, hipStream_t st);

// Piecewise forward (PISA page, core algorithm), part 1: the learnable router's k~, the f16
// copy of V, per key block its centroid (bf16 hi + lo) and value-sum column, and
// H_bar^T = (1/nbk) sum_j H_j^T in bf16.
hipError_t launch_pisa_stats(const Plan& s, const void* k, const void* v, const float* pk,
                             char* ws, hipStream_t st);

// Piecewise forward, part 2: per query row the zero-order tail over the unrouted blocks'
// centroids (running max, weighted and plain row sums, numerator).
hipError_t launch_pisa_tail(const Plan& s, const void* q, const int32_t* idx, char* ws,
                            hipStream_t st);

// Piecewise forward, part 3: the exact branch, merged with the tail and the first-order
// correction inside one normalisation.
hipError_t launch_sparse_pisa(const Plan& s, const void* q, const void* k, const int32_t* idx,
                              void* o, char* ws, hipStream_t st);

// Complement sums in fp32 for the backward: per row r (rows of [BH][rows][D*D] out),
// out[r] = sum over the columns c < cols whose bit is clear in row r of bits ([BH][rows]
// [nwords]) of hi[c] + lo[c] (hi, lo: bf16 in the per-block summary layout over cols). k >= cols
// gives exactly zero. Forward orientation: rows = query blocks, cols = key blocks, bits the
// selection; transposed: rows = key blocks, cols = query blocks, bits the routed query blocks.
hipError_t launch_complement_f32(const Plan& s, const uint32_t* bits, int nwords, int rows,
                                 int cols, int k, const uint16_t* hi, const uint16_t* lo,
                                 float* out, hipStream_t st);

// z_c(i) = z_tot - sum_{j in sel(i)} z_j alone (fp32), into the workspace's zc.
hipError_t launch_complement_z(const Plan& s, const int32_t* idx, char* ws, hipStream_t st);

// Backward at the given selection (bf16 inputs): dq, dk, dv (fp32, like Q, K, V) and dalpha
// [H][D] (fp32) from dout (out dtype); workspace as make_bwd_plan.
hipError_t launch_backward(const Plan& s, const void* q, const void* k, const void* v,
                           const float* alpha, const void* dout, const int32_t* idx, float* dq,
                           float* dk, float* dv, float* dalpha, char* ws, hipStream_t st);

}  // namespace sla
