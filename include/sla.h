/*
 * sla.h - C ABI of the MI355X (gfx950) SLA2 sparse-linear attention forward library.
 *
 * Method (SLA2: Sparse-Linear Attention with Learnable Routing and QAT):
 *   - router, section 2.B: Q and K are mean-pooled over blocks of adjacent tokens, the
 *     pooled vectors are multiplied by the learnable projections proj_q / proj_k, each
 *     query block scores every key block with a dot product, and the top_k key blocks
 *     are kept (ties go to the lower key-block index);
 *   - sparse branch, sections 1 and 2.B: exact softmax attention (scale 1/sqrt(d)) of
 *     each query block over the tokens of its routed key blocks;
 *   - linear branch (SALAD page, section 2; SPLA page, section 2.2): ReLU-kernel linear
 *     attention over the key blocks that were NOT routed: S_c is the sum of the unrouted
 *     blocks' phi(K_j)^T V_j (formed directly on the per-block path; as the total minus the
 *     routed blocks' term on the cache path), z_c the total of phi(K) minus the routed
 *     blocks'; O_l = phi(q) S_c / (phi(q) . z_c + 1e-6);
 *   - mix, section 2.A: O = alpha (.) O_s + (1 - alpha) (.) O_l with a per-head,
 *     per-channel ratio alpha;
 *   - quantised sparse branch, section 2.C: sla_forward_fp8 runs the sparse branch on
 *     OCP E4M3 operands (per 64-token-block absmax scales for Q, K, V; P per key tile and
 *     query row); router, linear branch and mix are the same as in sla_forward.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers to contiguous row-major arrays.
 *     Q is [batch, heads, n_q, head_dim]; K and V are [batch, heads, n_kv, head_dim];
 *     O is [batch, heads, n_q, head_dim]; the channel index is the fastest.
 *   - Q, K, V have element type in_dtype (bf16 or f32); O has out_dtype. With f32 inputs
 *     the logits Q K^T come from three bf16 products (hi hi, hi lo, lo hi: near-fp32), but
 *     P.V still multiplies f16 P by an f16 copy of V and the per-block summaries S_j, S_c are
 *     bf16, so f32 inputs give no more accuracy than bf16 ones beyond the logits.
 *   - Range: the exact (sparse) branch multiplies the softmax weights, held in f16 in
 *     [0, 256], with an f16 copy of V, so entries of V beyond +-65504 saturate there; the
 *     piecewise forward's per-block value sums (64 tokens each) are f16 as well.
 *   - proj_q, proj_k: f32 [head_dim (in), head_dim (out)], shared by all batches and heads;
 *     the pooled row vector x is mapped to x @ proj.
 *   - alpha: f32 [heads, head_dim], values expected in [0, 1].
 *   - block_idx: int32 [batch, heads, ceil(n_q/block), top_k], ascending within a row.
 *   - Every pointer must be 16-byte aligned. The caller owns all memory; the library never
 *     allocates, frees, copies between host and device, or synchronises.
 *   - Work is enqueued on `stream`; calls return as soon as it is enqueued. A non-OK status
 *     other than SLA_ERR_HIP means nothing was enqueued; after SLA_ERR_HIP (a launch was
 *     refused) the outputs are undefined.
 *   - Apart from the allocation-free entry point at the end of this header, which works in
 *     one fixed device array per GPU, the library keeps no mutable global state: concurrent
 *     calls on different streams with separate workspaces are safe. Results are
 *     bit-reproducible for identical inputs (no floating-point atomics).
 */
#ifndef SLA_H
#define SLA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SLA_OK = 0,
  SLA_ERR_NULL = 1,        /* a required pointer is NULL                             */
  SLA_ERR_SHAPE = 2,       /* a size is out of range (see sla_problem)               */
  SLA_ERR_DTYPE = 3,       /* unknown dtype, or a dtype the entry point refuses      */
  SLA_ERR_TOPK = 4,        /* top_k < 0 or top_k > ceil(n_kv / block)                */
  SLA_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                       */
  SLA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than sla_workspace_size()    */
  SLA_ERR_UNSUPPORTED = 7, /* head_dim not in {64, 128}, block != 64, too many blocks */
  SLA_ERR_HIP = 8,         /* a kernel launch failed                                 */
  SLA_ERR_SCRATCH = 9      /* the problem needs more than the fixed scratch array of
                              sla_forward_cached_noalloc (SLA_NOALLOC_SCRATCH_BYTES)      */
} sla_status;

typedef enum { SLA_F32 = 0, SLA_BF16 = 1 } sla_dtype;

typedef struct {
  int32_t batch;      /* >= 1                                                        */
  int32_t heads;      /* >= 1                                                        */
  int32_t n_q;        /* query tokens, >= 1                                          */
  int32_t n_kv;       /* key/value tokens, >= 1; ceil(n_kv/block) <= 8064            */
  int32_t head_dim;   /* 64 or 128                                                   */
  int32_t block;      /* 64: size of both query blocks and key blocks                */
  int32_t top_k;      /* key blocks kept per query block, 0 .. ceil(n_kv/block)      */
  int32_t in_dtype;   /* sla_dtype of Q, K, V                                        */
  int32_t out_dtype;  /* sla_dtype of O                                              */
} sla_problem;

/* Workspace layouts (the `variant` of sla_workspace_size and sla_workspace_region). */
enum {
  SLA_VARIANT_FORWARD = 0,  /* sla_forward, sla_route, sla_route_taylor                    */
  SLA_VARIANT_FP8 = 1,      /* sla_forward_fp8                                            */
  SLA_VARIANT_PISA = 2,     /* sla_forward_pisa                                           */
  SLA_VARIANT_TAYLOR = 3    /* sla_forward_taylor                                         */
};

/* Bytes of device workspace a call of that variant needs. Returns 0 if the problem is
 * invalid or the variant unknown. */
size_t sla_workspace_size(const sla_problem* p, int variant);

/* Router only (SLA2 page, section 2.B): pool -> project -> score -> top-k.
 * Writes block_idx (required). Pooling, projection and scores are computed in float64
 * so that the selection is reproducible; ties go to the lower key-block index. */
sla_status sla_route(const sla_problem* p, const void* q, const void* k,
                     const float* proj_q, const float* proj_k, int32_t* block_idx,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Full forward with the bf16 sparse branch (SLA2 page, sections 2.A and 2.B).
 * block_idx is optional (NULL: the selection stays in the workspace).
 * With bf16 inputs, at most 8 query blocks per head and at least 256 key blocks (a chunk of
 * queries against a long key sequence) the call takes the cache path: one pass over K and V
 * builds the key/value summary cache of sla_kv_cache_update in the workspace, and the rest
 * is sla_forward_cached (same selection, same arithmetic), so no per-key-block summary is
 * stored (SPLA page, section 2.2: the unselected blocks' linear term is the total minus the
 * selected blocks' term). sla_workspace_size(p, SLA_VARIANT_FORWARD) accounts for it; the
 * SCORES, SC and ZC workspace regions do not exist on that path. */
sla_status sla_forward(const sla_problem* p, const void* q, const void* k, const void* v,
                       const float* proj_q, const float* proj_k, const float* alpha,
                       void* o, int32_t* block_idx,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Full forward with the quantised (E4M3) sparse branch (SLA2 page, section 2.C).
 * Same arguments as sla_forward; in_dtype must be SLA_BF16. The router and the linear
 * branch are identical to sla_forward, so block_idx is too. */
sla_status sla_forward_fp8(const sla_problem* p, const void* q, const void* k, const void* v,
                           const float* proj_q, const float* proj_k, const float* alpha,
                           void* o, int32_t* block_idx,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Training-free router (SPLA page, section 2.1: block selection from a second-order Taylor
 * expansion of the attention objective around the block mean, covariance taken diagonal).
 * Query block i and key block j score
 *     tau * (qbar_i . kbar_j) + log1p(tau^2 / 2 * sum_c qbar_ic^2 var_jc),   tau = 1/sqrt(d),
 * the logarithm of exp(tau qbar.kbar)(1 + tau^2 qbar^T diag(var) qbar / 2), with qbar, kbar
 * the block means over valid tokens and var the per-channel population variance of the key
 * block (all float64); no projections. Top-k, tie rule and output order as sla_route.
 * Same workspace as sla_route. */
sla_status sla_route_taylor(const sla_problem* p, const void* q, const void* k,
                            int32_t* block_idx, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* sla_forward with the training-free router instead of the learnable one (no proj_q, proj_k).
 * Workspace: SLA_VARIANT_TAYLOR (the per-key-block layout of sla_forward; the same size as
 * SLA_VARIANT_FORWARD unless sla_forward takes its cache path). */
sla_status sla_forward_taylor(const sla_problem* p, const void* q, const void* k, const void* v,
                              const float* alpha, void* o, int32_t* block_idx, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Piecewise exact-or-approximate forward (PISA page, "Piecewise Sparse Attention", core
 * algorithm), routed by the learnable router of sla_forward (same proj_q, proj_k, same
 * block_idx). Every key block enters one softmax normalisation: the routed blocks exactly,
 * every other block j through its centroid kbar_j (block mean of the valid keys), value sum
 * Vsum_j and token count n_j, plus one global first-order matrix
 * H_bar = mean over all key blocks of H_j = sum_n (k_n - kbar_j)^T v_n. For query row q of
 * query block i, with a_j = exp(tau q . kbar_j), tau = 1/sqrt(d), and U the blocks not routed
 * to i:
 *     N = sum_{routed tokens} e^{tau q.k} v + sum_{j in U} a_j Vsum_j + tau (q H_bar) sum_U a_j
 *     D = sum_{routed tokens} e^{tau q.k}   + sum_{j in U} a_j n_j,          O = N / D.
 * There is no alpha and no separate linear branch. Workspace: SLA_VARIANT_PISA. */
sla_status sla_forward_pisa(const sla_problem* p, const void* q, const void* k, const void* v,
                            const float* proj_q, const float* proj_k, void* o,
                            int32_t* block_idx, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Stages of a forward call, in launch order, for sla_forward_profiled. For the piecewise
 * forward KV_SUMMARY is its per-block statistics pass and COMPLEMENT its tail kernel. */
enum {
  SLA_STAGE_KV_SUMMARY = 0,  /* per-block phi(K)^T V, sum phi(K), pooled K, totals      */
  SLA_STAGE_ROUTE = 1,       /* pooled Q, projections, block scores, top-k              */
  SLA_STAGE_COMPLEMENT = 2,  /* per query block: the unselected blocks' S_c and z_c     */
  SLA_STAGE_QUANT = 3,       /* empty: K and V are quantised in KV_SUMMARY, Q in SPARSE  */
  SLA_STAGE_SPARSE = 4,      /* sparse attention + linear apply + alpha mix            */
  SLA_NUM_STAGES = 5
};

/* Forward variants that sla_forward_profiled can run. */
enum {
  SLA_PROFILE_FP8 = 1,     /* the sla_forward_fp8 path                                   */
  SLA_PROFILE_TAYLOR = 2,  /* the sla_forward_taylor path (proj_q, proj_k ignored)       */
  SLA_PROFILE_PISA = 4     /* the sla_forward_pisa path (alpha ignored)                  */
};

/* Same as sla_forward (flags = 0), sla_forward_fp8 (flags = SLA_PROFILE_FP8),
 * sla_forward_taylor (flags = SLA_PROFILE_TAYLOR) or sla_forward_pisa
 * (flags = SLA_PROFILE_PISA), and additionally records events[2*s]
 * before and events[2*s+1] after stage s on `stream` (caller-created events,
 * 2*SLA_NUM_STAGES of them), so the caller can time each stage with hipEventElapsedTime
 * after synchronising. NULL events: identical to the plain call. Any other flags value
 * (including two bits together) returns SLA_ERR_UNSUPPORTED. */
sla_status sla_forward_profiled(const sla_problem* p, const void* q, const void* k,
                                const void* v, const float* proj_q, const float* proj_k,
                                const float* alpha, void* o, int32_t* block_idx,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                int flags, hipEvent_t* events);

/* Workspace regions that tests and diagnostics may read back after a call. */
typedef enum {
  SLA_WS_Q8 = 0,        /* bf16 holding the E4M3 values of Q [B*H][ceil(n_q/64)*64][d] */
  SLA_WS_K8 = 1,        /* bf16 holding the E4M3 values of K [B*H][ceil(n_kv/64)*64][d]*/
  SLA_WS_V8 = 2,        /* uint8  E4M3 V   [B*H][ceil(n_kv/64)][head_dim][64], keys in
                           the P8 operand order (see sparse.hip)                    */
  SLA_WS_EQ = 3,        /* int32 block exponents of Q  [B*H][ceil(n_q/64)]           */
  SLA_WS_EK = 4,        /* int32 block exponents of K  [B*H][ceil(n_kv/64)]          */
  SLA_WS_EV = 5,        /* int32 block exponents of V  [B*H][ceil(n_kv/64)]          */
  SLA_WS_SCORES = 6,    /* float64 block scores [B*H][ceil(n_q/64)][ceil(n_kv/64)]   */
  SLA_WS_SC = 7,        /* bf16 S_c^T per query block [B*H][ceil(n_q/64)][d][d]      */
  SLA_WS_ZC = 8,        /* fp32 z_c per query block [B*H][ceil(n_q/64)][d]           */
  /* piecewise forward (SLA_VARIANT_PISA); npad = ceil(n_kv/64) rounded up to a multiple of
     64; entries past ceil(n_kv/64) are not written                                   */
  SLA_WS_HBAR = 9,      /* bf16 H_bar^T [B*H][d(value channel)][d(key channel)]      */
  SLA_WS_CENT_HI = 10,  /* bf16 centroids, rounded  [B*H][npad][d]                   */
  SLA_WS_CENT_LO = 11,  /* bf16 centroid minus its rounded value [B*H][npad][d]      */
  SLA_WS_VSUM = 12      /* f16 value sums of the key blocks, [B*H][npad][d]         */
} sla_ws_region;

/* Byte offset and size of a workspace region for problem p in the layout of `variant`
 * (fp8 regions need SLA_VARIANT_FP8, piecewise ones SLA_VARIANT_PISA; SC and ZC do not exist
 * in the piecewise layout). Returns SLA_ERR_SHAPE / SLA_ERR_NULL on invalid arguments. Host
 * only. */
sla_status sla_workspace_region(const sla_problem* p, int variant, int region, size_t* offset,
                                size_t* bytes);

/* ---------------------------------------------------------------- key/value summary cache
 * Decode path (SPLA page, section 2.2: the linear term of the unselected key blocks is the
 * total over all blocks minus that of the selected ones; SLA2 page, section 2.B: the router
 * only needs the pooled, projected keys). The cache keeps, per (batch, head), the totals
 * S_tot = sum_t phi(k_t)^T v_t (fp32, stored transposed [d(c)][d(r)]), z_tot = sum_t phi(k_t)
 * (fp32) and the projected block means k~_j (fp64) of every key block:
 *   bytes [0, B*H*d*d*4)                S_tot^T [B*H][d][d]
 *   then (256-byte aligned)             z_tot   [B*H][d]
 *   then (256-byte aligned)             k~      [ceil(n_kv/64)][B*H][d]  (block-major)
 * The layout only grows at its end with n_kv, so a cache allocated for the final length
 * serves every shorter one. Only bf16 inputs are supported on this path. */

/* Bytes of the cache for p->n_kv tokens. 0 if the problem is invalid. */
size_t sla_kv_cache_size(const sla_problem* p);

/* Workspace bytes sla_kv_cache_update needs for an update from n_done tokens (>= 256). */
size_t sla_kv_cache_workspace_size(const sla_problem* p, int32_t n_done);

/* Bring the cache from the first n_done tokens of K and V to all p->n_kv tokens: adds the
 * new tokens' phi(k)^T v and phi(k) to the totals (n_done = 0 initialises them) and
 * recomputes k~ of every key block holding a new token from all its valid tokens (proj_k:
 * as in sla_forward). K, V: [batch, heads, n_kv, head_dim] bf16, the first n_done tokens
 * unchanged since the last update. Device pointers, 16-byte aligned. Calls on one cache
 * must be ordered (same stream). Returns SLA_ERR_DTYPE for fp32 inputs, SLA_ERR_SHAPE if
 * n_done is outside [0, n_kv]. */
sla_status sla_kv_cache_update(const sla_problem* p, const void* k, const void* v,
                               const float* proj_k, int32_t n_done, void* cache,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of sla_forward_cached. 0 if the problem is invalid. */
size_t sla_cached_workspace_size(const sla_problem* p);

/* The forward of sla_forward computed against a summary cache that covers all p->n_kv tokens
 * (routing against the cached k~; the linear branch from the cached totals minus the
 * selected blocks' summaries, which are formed from the K/V tiles the exact branch reads).
 * Same outputs and conventions as sla_forward; no proj_k argument (it is in the cache). The
 * work per call scales with the selected blocks, not with n_kv: meant for few query blocks
 * per head (decode chunks). bf16 inputs only. */
sla_status sla_forward_cached(const sla_problem* p, const void* q, const void* k, const void* v,
                              const float* proj_q, const float* alpha, const void* cache,
                              void* o, int32_t* block_idx, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- backward
 * Gradients of sla_forward at a given selection (SLA2 page, section 2.B: training replaces
 * the hard top-k by a SoftTop-k the page does not define, so the selection is held fixed here
 * and proj_q, proj_k receive no gradient through it; section 2.C: the backward runs at
 * higher precision than a quantised forward). For the forward output O and the upstream
 * gradient dO of the same shape:
 *   dalpha = sum over batch and rows of dO (.) (O_s - O_l);
 *   the exact branch: softmax-attention gradients over each query block's routed tokens with
 *     dO_s = alpha (.) dO;
 *   the linear branch: gradients of O_l = phi(q) S_c / (phi(q) . z_c + 1e-6) with
 *     dO_l = (1 - alpha) (.) dO, flowing into every key token of the blocks a query block did
 *     not route (phi = ReLU, derivative 0 at 0).
 * Inputs as sla_forward (in_dtype must be SLA_BF16); dout has out_dtype and O's shape;
 * block_idx (required unless top_k is 0) is the forward's selection [B, H, ceil(n_q/64),
 * top_k], ascending.
 * Outputs, fp32: dq like Q, dk and dv like K and V, dalpha [heads, head_dim]; every element
 * is written. Products run on bf16 / f16 MFMA with fp32 accumulation; the quantities whose
 * gradients are small differences of large terms (dS of the exact branch; S_j, S_c, g, dS_c
 * and G of the linear branch) enter as bf16 high + low parts. Results are bit-reproducible.
 * Errors, with nothing enqueued: an invalid problem (as sla_forward), SLA_ERR_DTYPE for fp32
 * inputs, SLA_ERR_NULL for a missing pointer (block_idx may be NULL only when top_k is 0),
 * SLA_ERR_WORKSPACE when workspace_bytes < sla_backward_workspace_size(p), SLA_ERR_ALIGN for
 * an unaligned workspace. The workspace (caller-owned, device) holds the forward's per-block
 * summaries and the backward's intermediates: about 2.3 GB at B = 1, H = 12, n = 32768,
 * d = 128. With at most 8 query blocks per head no per-key-block G_j is kept (and, when they
 * also select at most half the key blocks, no per-block summaries either): 15.9 GB at B = 4,
 * H = 32, 64 queries over 131072 keys, d = 128. */
size_t sla_backward_workspace_size(const sla_problem* p);

sla_status sla_backward(const sla_problem* p, const void* q, const void* k, const void* v,
                        const float* alpha, const void* dout, const int32_t* block_idx,
                        float* dq, float* dk, float* dv, float* dalpha, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- allocation-free decode
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. sla_forward_cached without the workspace
 * arguments: its workspace is a fixed device array inside the library,
 * SLA_NOALLOC_SCRATCH_BYTES long, one per GPU, which each GPU the library runs on holds from
 * the code object's load until the process ends. The call allocates and frees nothing; its
 * kernels, outputs and conventions are those of sla_forward_cached, and the result is the
 * same bit for bit. The array of the CURRENT device is used (`stream` must belong to it);
 * its address is looked up on the first call on each device. Returns SLA_ERR_SCRATCH, with
 * nothing enqueued, when sla_cached_workspace_size(p) exceeds the array (decode shapes up to
 * e.g. 128 heads x 64 queries over 131072 keys with top_k 64 fit). Every call on one GPU
 * shares that GPU's array and nothing in it must start cleared: calls ordered on one stream
 * are safe, but calls that may overlap on one GPU (different streams or threads without
 * ordering between them) race and give undefined results. */
#define SLA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

sla_status sla_forward_cached_noalloc(const sla_problem* p, const void* q, const void* k,
                                      const void* v, const float* proj_q, const float* alpha,
                                      const void* cache, void* o, int32_t* block_idx,
                                      hipStream_t stream);

/* ---------------------------------------------------------------- diagnostics
 * Not part of the method: one 32 x 32 x 64 product C = A B of E4M3 codes (a: 32 x 64 row-major,
 * b: 64 x 32 row-major, device bytes; no NaN codes) computed twice on the GPU, with the scaled
 * fp8 matrix instruction (unit scales) into c_fp8 and with the bf16 matrix instruction on the
 * same values (exact operands and products) into c_bf16, both fp32 32 x 32 row-major. It
 * measures how the fp8 instruction accumulates products of different magnitude, which decides
 * the quantised forward's choice of instruction for Q K^T (see sla_forward_fp8). */
sla_status sla_diag_fp8_mfma(const uint8_t* a, const uint8_t* b, float* c_fp8, float* c_bf16,
                             hipStream_t stream);

/* Not part of the method: the matrix-core throughput this GPU reaches, for rooflines measured
 * against the instruction rather than the published peak. Launches `blocks` workgroups of four
 * waves; each wave issues 4 * iters 32x32x16 bf16 matrix products in four independent chains
 * (32768 FLOP each: blocks * 16 * iters * 32768 FLOP in all) and every thread writes one
 * float to sink (device, blocks * 256 floats, caller-owned). The caller times the launch on
 * `stream` (for example with events). SLA_ERR_NULL for a NULL sink, SLA_ERR_SHAPE for blocks or
 * iters <= 0; nothing is enqueued then. */
sla_status sla_diag_mfma_rate(float* sink, int blocks, int iters, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* sla_status_string(sla_status s);

#ifdef __cplusplus
}
#endif
#endif /* SLA_H */
