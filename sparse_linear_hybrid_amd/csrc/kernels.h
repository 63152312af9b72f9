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
hipError_t launch_kv_summary(const Plan& s, const void* k, const void* v, const float* pk, char* ws,
                             hipStream_t st, bool fp8 = false);

// Linear branch, part 2: complement = total - selected, per query block.
hipError_t launch_complement(const Plan& s, const int32_t* idx, char* ws, hipStream_t st);

// Sparse branch (bf16 MFMA for Q K^T, f16 MFMA for P V) with the linear apply and the
// alpha mix fused into its epilogue.
hipError_t launch_sparse(const Plan& s, const void* q, const void* k, const int32_t* idx,
                         const float* alpha, void* o, char* ws, hipStream_t st);

// Quantised branch: E4M3 copies of Q, K, V with power-of-two block exponents.
hipError_t launch_quant(const Plan& s, const void* q, const void* k, const void* v, char* ws,
                        hipStream_t st);

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

}  // namespace sla
