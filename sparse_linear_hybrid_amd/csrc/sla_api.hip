// C ABI entry points (include/sla.h): argument validation, workspace plan and the launch
// sequence. Validation happens before anything is enqueued.
#include <algorithm>

#include "common.h"
#include "kernels.h"

using namespace sla;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

sla_status check_problem(const sla_problem* p) {
  if (!p) return SLA_ERR_NULL;
  if (p->batch < 1 || p->heads < 1 || p->n_q < 1 || p->n_kv < 1) return SLA_ERR_SHAPE;
  if (p->in_dtype != SLA_F32 && p->in_dtype != SLA_BF16) return SLA_ERR_DTYPE;
  if (p->out_dtype != SLA_F32 && p->out_dtype != SLA_BF16) return SLA_ERR_DTYPE;
  if (p->head_dim != 64 && p->head_dim != 128) return SLA_ERR_UNSUPPORTED;
  if (p->block != kBlock) return SLA_ERR_UNSUPPORTED;
  const long long nbq = (p->n_q + kBlock - 1) / kBlock;
  const long long nbk = (p->n_kv + kBlock - 1) / kBlock;
  if (nbk > kMaxKeyBlocks) return SLA_ERR_UNSUPPORTED;
  // grid sizes: one workgroup per (batch*head, query block) must fit a 1-D grid
  const long long rows = (long long)p->batch * p->heads * nbq;
  if (rows > 0x7fffffffLL || (long long)p->batch * p->heads > 65535) return SLA_ERR_SHAPE;
  if (p->top_k < 0 || p->top_k > nbk) return SLA_ERR_TOPK;
  return SLA_OK;
}

sla_status check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* x : ps)
    if (!x) return SLA_ERR_NULL;
  for (const void* x : ps)
    if (!aligned16(x)) return SLA_ERR_ALIGN;
  return SLA_OK;
}

// Workspace plan of the forward entry points, with the cache path decided (Plan::few).
Plan forward_plan(const sla_problem& p) {
  Plan s = make_plan(p);
  plan_few_path(s);
  return s;
}

// The forward variants: SLA2 (learnable router), its fp8 sparse branch, SLA2 with the
// training-free router (proj_q / proj_k unused and may be NULL), and the piecewise forward
// (learnable router; exact routed blocks plus the Taylor tail; alpha unused and may be NULL).
enum class Fwd { kSla, kFp8, kTaylor, kPisa };

sla_status forward_impl(const sla_problem* p, const void* q, const void* k, const void* v,
                        const float* proj_q, const float* proj_k, const float* alpha, void* o,
                        int32_t* block_idx, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, Fwd mode, hipEvent_t* ev) {
  sla_status st = check_problem(p);
  if (st != SLA_OK) return st;
  if (mode == Fwd::kFp8 && p->in_dtype != SLA_BF16) return SLA_ERR_DTYPE;
  switch (mode) {
    case Fwd::kTaylor: st = check_ptrs({q, k, v, alpha, o}); break;
    case Fwd::kPisa: st = check_ptrs({q, k, v, proj_q, proj_k, o}); break;
    default: st = check_ptrs({q, k, v, proj_q, proj_k, alpha, o}); break;
  }
  if (st != SLA_OK) return st;
  if (block_idx && !aligned16(block_idx)) return SLA_ERR_ALIGN;
  const Plan s = forward_plan(*p);
  // Only the learnable router's bf16 forward takes the cache path; the Taylor router's
  // forward keeps the per-block layout (SLA_VARIANT_TAYLOR).
  const bool few = s.few && mode == Fwd::kSla;
  const size_t need = mode == Fwd::kFp8    ? s.total_fp8
                      : mode == Fwd::kPisa ? s.total_pisa
                      : few                ? s.total_few
                                           : s.total_fwd;
  if (!workspace || workspace_bytes < need) return SLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SLA_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  auto mark = [&](int e) { return ev ? hipEventRecord(ev[e], stream) : hipSuccess; };
  auto ok = [](hipError_t e) { return e == hipSuccess; };
  if (few && mode == Fwd::kSla) {
    // Few query blocks over a long key sequence (SPLA page, section 2.2: the unselected blocks'
    // linear term is the total minus the selected blocks' term, so no per-block summary is
    // stored): build the summary cache (k~, S_tot, z_tot) in the workspace with one pass over
    // K and V, route against it, and run the cached forward, whose exact branch forms the
    // selected blocks' summaries from the tiles it reads. Stages: the cache build is the
    // key/value stage, the complement and quantisation stages are empty.
    char* cache = ws + s.few_cache;
    char* dws = ws + s.few_dec;
    const DecodePlan d = make_decode_plan(s);
    const CachePlan c = make_cache_plan(s);
    int32_t* idx = block_idx ? block_idx : reinterpret_cast<int32_t*>(dws + d.idx);
    if (!ok(mark(2 * SLA_STAGE_KV_SUMMARY))) return SLA_ERR_HIP;
    if (!ok(launch_kv_cache_update(s, k, v, proj_k, 0, cache, ws + s.few_cws, stream)))
      return SLA_ERR_HIP;
    if (!ok(mark(2 * SLA_STAGE_KV_SUMMARY + 1))) return SLA_ERR_HIP;
    if (!ok(mark(2 * SLA_STAGE_ROUTE))) return SLA_ERR_HIP;
    if (!ok(launch_route_cached(s, q, proj_q, reinterpret_cast<const double*>(cache + c.kt),
                                (size_t)s.D, (size_t)s.BH * s.D, idx,
                                reinterpret_cast<double*>(dws + d.qt),
                                reinterpret_cast<double*>(dws + d.scores), stream)))
      return SLA_ERR_HIP;
    if (!ok(mark(2 * SLA_STAGE_ROUTE + 1))) return SLA_ERR_HIP;
    for (int stg : {SLA_STAGE_COMPLEMENT, SLA_STAGE_QUANT})
      if (!ok(mark(2 * stg)) || !ok(mark(2 * stg + 1))) return SLA_ERR_HIP;
    if (!ok(mark(2 * SLA_STAGE_SPARSE))) return SLA_ERR_HIP;
    if (!ok(launch_decode(s, q, k, v, idx, alpha, cache, o, dws, stream))) return SLA_ERR_HIP;
    if (!ok(mark(2 * SLA_STAGE_SPARSE + 1))) return SLA_ERR_HIP;
    return SLA_OK;
  }
  int32_t* idx = block_idx ? block_idx : reinterpret_cast<int32_t*>(ws + s.idx);
  if (!ok(mark(2 * SLA_STAGE_KV_SUMMARY))) return SLA_ERR_HIP;
  if (mode == Fwd::kPisa) {
    if (!ok(launch_pisa_stats(s, k, v, proj_k, ws, stream))) return SLA_ERR_HIP;
  } else if (!ok(launch_kv_summary(s, k, v, mode == Fwd::kTaylor ? nullptr : proj_k, ws,
                                   stream, /*fp8=*/mode == Fwd::kFp8))) {
    return SLA_ERR_HIP;
  }
  if (!ok(mark(2 * SLA_STAGE_KV_SUMMARY + 1))) return SLA_ERR_HIP;
  if (!ok(mark(2 * SLA_STAGE_ROUTE))) return SLA_ERR_HIP;
  // the complement's routed-block bitmap comes out of the top-k pass (the piecewise tail
  // builds its own)
  uint32_t* bits = mode == Fwd::kPisa ? nullptr : reinterpret_cast<uint32_t*>(ws + s.selbits);
  if (mode == Fwd::kTaylor) {
    if (!ok(launch_route_taylor(s, q, k, idx, bits, ws, stream))) return SLA_ERR_HIP;
  } else if (!ok(launch_route(s, q, k, proj_q, proj_k, idx, bits, ws, /*pool_k=*/false,
                              stream))) {
    return SLA_ERR_HIP;
  }
  if (!ok(mark(2 * SLA_STAGE_ROUTE + 1))) return SLA_ERR_HIP;
  if (!ok(mark(2 * SLA_STAGE_COMPLEMENT))) return SLA_ERR_HIP;
  if (mode == Fwd::kPisa) {
    if (!ok(launch_pisa_tail(s, q, idx, ws, stream))) return SLA_ERR_HIP;
  } else if (!ok(launch_complement(s, idx, ws, stream))) {
    return SLA_ERR_HIP;
  }
  if (!ok(mark(2 * SLA_STAGE_COMPLEMENT + 1))) return SLA_ERR_HIP;
  // fp8: K and V were quantised by the key/value pass, and the quantised sparse kernel
  // quantises Q itself, so the quantisation stage is empty on every path
  if (!ok(mark(2 * SLA_STAGE_QUANT))) return SLA_ERR_HIP;
  if (!ok(mark(2 * SLA_STAGE_QUANT + 1))) return SLA_ERR_HIP;
  if (!ok(mark(2 * SLA_STAGE_SPARSE))) return SLA_ERR_HIP;
  hipError_t e;
  switch (mode) {
    case Fwd::kFp8: e = launch_sparse_fp8(s, q, idx, alpha, o, ws, stream); break;
    case Fwd::kPisa: e = launch_sparse_pisa(s, q, k, idx, o, ws, stream); break;
    default: e = launch_sparse(s, q, k, idx, alpha, o, ws, stream); break;
  }
  if (!ok(e)) return SLA_ERR_HIP;
  if (!ok(mark(2 * SLA_STAGE_SPARSE + 1))) return SLA_ERR_HIP;
  return SLA_OK;
}

}  // namespace

extern "C" {

size_t sla_workspace_size(const sla_problem* p, int variant) {
  if (check_problem(p) != SLA_OK) return 0;
  const Plan s = forward_plan(*p);
  switch (variant) {
    case SLA_VARIANT_FORWARD:   // also the routers' layout (their buffers lead both layouts)
      return s.few ? std::max(s.total_few, s.total_route) : s.total_fwd;
    case SLA_VARIANT_TAYLOR: return s.total_fwd;
    case SLA_VARIANT_FP8: return s.total_fp8;
    case SLA_VARIANT_PISA: return s.total_pisa;
    default: return 0;
  }
}

sla_status sla_route(const sla_problem* p, const void* q, const void* k, const float* proj_q,
                     const float* proj_k, int32_t* block_idx, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  sla_status st = check_problem(p);
  if (st != SLA_OK) return st;
  st = check_ptrs({q, k, proj_q, proj_k, block_idx});
  if (st != SLA_OK) return st;
  const Plan s = make_plan(*p);
  if (!workspace || workspace_bytes < s.total_route) return SLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SLA_ERR_ALIGN;
  if (launch_route(s, q, k, proj_q, proj_k, block_idx, nullptr, static_cast<char*>(workspace),
                   /*pool_k=*/true, stream) != hipSuccess)
    return SLA_ERR_HIP;
  return SLA_OK;
}

sla_status sla_forward(const sla_problem* p, const void* q, const void* k, const void* v,
                       const float* proj_q, const float* proj_k, const float* alpha, void* o,
                       int32_t* block_idx, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  return forward_impl(p, q, k, v, proj_q, proj_k, alpha, o, block_idx, workspace,
                      workspace_bytes, stream, Fwd::kSla, nullptr);
}

sla_status sla_forward_fp8(const sla_problem* p, const void* q, const void* k, const void* v,
                           const float* proj_q, const float* proj_k, const float* alpha, void* o,
                           int32_t* block_idx, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  return forward_impl(p, q, k, v, proj_q, proj_k, alpha, o, block_idx, workspace,
                      workspace_bytes, stream, Fwd::kFp8, nullptr);
}

sla_status sla_forward_profiled(const sla_problem* p, const void* q, const void* k,
                                const void* v, const float* proj_q, const float* proj_k,
                                const float* alpha, void* o, int32_t* block_idx,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                int flags, hipEvent_t* events) {
  Fwd mode;
  switch (flags) {
    case 0: mode = Fwd::kSla; break;
    case SLA_PROFILE_FP8: mode = Fwd::kFp8; break;
    case SLA_PROFILE_TAYLOR: mode = Fwd::kTaylor; break;
    case SLA_PROFILE_PISA: mode = Fwd::kPisa; break;
    default: return SLA_ERR_UNSUPPORTED;
  }
  return forward_impl(p, q, k, v, proj_q, proj_k, alpha, o, block_idx, workspace,
                      workspace_bytes, stream, mode, events);
}

sla_status sla_route_taylor(const sla_problem* p, const void* q, const void* k,
                            int32_t* block_idx, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  sla_status st = check_problem(p);
  if (st != SLA_OK) return st;
  st = check_ptrs({q, k, block_idx});
  if (st != SLA_OK) return st;
  const Plan s = make_plan(*p);
  if (!workspace || workspace_bytes < s.total_route) return SLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SLA_ERR_ALIGN;
  if (launch_route_taylor(s, q, k, block_idx, nullptr, static_cast<char*>(workspace), stream) !=
      hipSuccess)
    return SLA_ERR_HIP;
  return SLA_OK;
}

sla_status sla_forward_taylor(const sla_problem* p, const void* q, const void* k, const void* v,
                              const float* alpha, void* o, int32_t* block_idx, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  return forward_impl(p, q, k, v, nullptr, nullptr, alpha, o, block_idx, workspace,
                      workspace_bytes, stream, Fwd::kTaylor, nullptr);
}

sla_status sla_forward_pisa(const sla_problem* p, const void* q, const void* k, const void* v,
                            const float* proj_q, const float* proj_k, void* o,
                            int32_t* block_idx, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  return forward_impl(p, q, k, v, proj_q, proj_k, nullptr, o, block_idx, workspace,
                      workspace_bytes, stream, Fwd::kPisa, nullptr);
}

sla_status sla_workspace_region(const sla_problem* p, int variant, int region, size_t* offset,
                                size_t* bytes) {
  const sla_status st = check_problem(p);
  if (st != SLA_OK) return st;
  if (!offset || !bytes) return SLA_ERR_NULL;
  const Plan s = forward_plan(*p);
  const size_t BH = s.BH, D = s.D, nbq = s.nbq, nbk = s.nbk;
  switch (region) {
    case SLA_WS_Q8: *offset = s.q8; *bytes = BH * nbq * kBlock * D * 2; break;
    case SLA_WS_K8: *offset = s.k8; *bytes = BH * nbk * kBlock * D * 2; break;
    case SLA_WS_V8: *offset = s.v8; *bytes = BH * nbk * kBlock * D; break;
    case SLA_WS_EQ: *offset = s.sq8; *bytes = BH * nbq * 4; break;
    case SLA_WS_EK: *offset = s.sk8; *bytes = BH * nbk * 4; break;
    case SLA_WS_EV: *offset = s.sv8; *bytes = BH * nbk * 4; break;
    case SLA_WS_SCORES: *offset = s.scores; *bytes = BH * nbq * nbk * 8; break;
    case SLA_WS_SC: *offset = s.sc; *bytes = BH * nbq * D * D * 2; break;
    case SLA_WS_ZC: *offset = s.zc; *bytes = BH * nbq * D * 4; break;
    case SLA_WS_HBAR: *offset = s.hbar; *bytes = BH * D * D * 2; break;
    case SLA_WS_CENT_HI: *offset = s.cent_hi; *bytes = BH * (size_t)s.npad * D * 2; break;
    case SLA_WS_CENT_LO: *offset = s.cent_lo; *bytes = BH * (size_t)s.npad * D * 2; break;
    case SLA_WS_VSUM: *offset = s.vsum; *bytes = BH * D * (size_t)s.npad * 2; break;
    default: return SLA_ERR_SHAPE;
  }
  const bool fp8_region = region <= SLA_WS_EV;
  const bool pisa_region = region >= SLA_WS_HBAR;
  const bool linear_region = region == SLA_WS_SC || region == SLA_WS_ZC;
  if (variant != SLA_VARIANT_FORWARD && variant != SLA_VARIANT_FP8 &&
      variant != SLA_VARIANT_PISA && variant != SLA_VARIANT_TAYLOR)
    return SLA_ERR_SHAPE;
  if (fp8_region && variant != SLA_VARIANT_FP8) return SLA_ERR_SHAPE;
  if (pisa_region && variant != SLA_VARIANT_PISA) return SLA_ERR_SHAPE;
  if (linear_region && variant == SLA_VARIANT_PISA) return SLA_ERR_SHAPE;
  // the cache path of sla_forward keeps no scores and no per-query-block complement
  if (s.few && variant == SLA_VARIANT_FORWARD && (linear_region || region == SLA_WS_SCORES))
    return SLA_ERR_UNSUPPORTED;
  return SLA_OK;
}

size_t sla_kv_cache_size(const sla_problem* p) {
  if (check_problem(p) != SLA_OK) return 0;
  return make_cache_plan(make_plan(*p)).bytes;
}

size_t sla_kv_cache_workspace_size(const sla_problem* p, int32_t n_done) {
  if (check_problem(p) != SLA_OK || n_done < 0 || n_done > p->n_kv) return 0;
  const size_t b = cache_update_ws_bytes(make_plan(*p), n_done);
  return b > 0 ? b : 256;
}

sla_status sla_kv_cache_update(const sla_problem* p, const void* k, const void* v,
                               const float* proj_k, int32_t n_done, void* cache,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  sla_status st = check_problem(p);
  if (st != SLA_OK) return st;
  if (p->in_dtype != SLA_BF16) return SLA_ERR_DTYPE;
  if (n_done < 0 || n_done > p->n_kv) return SLA_ERR_SHAPE;
  st = check_ptrs({k, v, proj_k, cache});
  if (st != SLA_OK) return st;
  const Plan s = make_plan(*p);
  if (!workspace || workspace_bytes < cache_update_ws_bytes(s, n_done)) return SLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SLA_ERR_ALIGN;
  if (launch_kv_cache_update(s, k, v, proj_k, n_done, static_cast<char*>(cache),
                             static_cast<char*>(workspace), stream) != hipSuccess)
    return SLA_ERR_HIP;
  return SLA_OK;
}

size_t sla_cached_workspace_size(const sla_problem* p) {
  if (check_problem(p) != SLA_OK) return 0;
  return make_decode_plan(make_plan(*p)).bytes;
}

sla_status sla_forward_cached(const sla_problem* p, const void* q, const void* k, const void* v,
                              const float* proj_q, const float* alpha, const void* cache,
                              void* o, int32_t* block_idx, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  sla_status st = check_problem(p);
  if (st != SLA_OK) return st;
  if (p->in_dtype != SLA_BF16) return SLA_ERR_DTYPE;
  st = check_ptrs({q, k, v, proj_q, alpha, cache, o});
  if (st != SLA_OK) return st;
  if (block_idx && !aligned16(block_idx)) return SLA_ERR_ALIGN;
  const Plan s = make_plan(*p);
  const DecodePlan d = make_decode_plan(s);
  if (!workspace || workspace_bytes < d.bytes) return SLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SLA_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  const char* cc = static_cast<const char*>(cache);
  const CachePlan c = make_cache_plan(s);
  int32_t* idx = block_idx ? block_idx : reinterpret_cast<int32_t*>(ws + d.idx);
  if (launch_route_cached(s, q, proj_q, reinterpret_cast<const double*>(cc + c.kt),
                          (size_t)s.D, (size_t)s.BH * s.D, idx,
                          reinterpret_cast<double*>(ws + d.qt),
                          reinterpret_cast<double*>(ws + d.scores), stream) != hipSuccess)
    return SLA_ERR_HIP;
  if (launch_decode(s, q, k, v, idx, alpha, cc, o, ws, stream) != hipSuccess) return SLA_ERR_HIP;
  return SLA_OK;
}

size_t sla_backward_workspace_size(const sla_problem* p) {
  if (check_problem(p) != SLA_OK) return 0;
  return make_bwd_plan(make_plan(*p)).bytes;
}

sla_status sla_backward(const sla_problem* p, const void* q, const void* k, const void* v,
                        const float* alpha, const void* dout, const int32_t* block_idx,
                        float* dq, float* dk, float* dv, float* dalpha, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  sla_status st = check_problem(p);
  if (st != SLA_OK) return st;
  if (p->in_dtype != SLA_BF16) return SLA_ERR_DTYPE;
  st = check_ptrs({q, k, v, alpha, dout, dq, dk, dv, dalpha});
  if (st != SLA_OK) return st;
  if (p->top_k > 0) {   // with no routed block the index list is empty and may be NULL
    st = check_ptrs({block_idx});
    if (st != SLA_OK) return st;
  }
  const Plan s = make_plan(*p);
  if (!workspace || workspace_bytes < make_bwd_plan(s).bytes) return SLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SLA_ERR_ALIGN;
  if (launch_backward(s, q, k, v, alpha, dout, block_idx, dq, dk, dv, dalpha,
                      static_cast<char*>(workspace), stream) != hipSuccess)
    return SLA_ERR_HIP;
  return SLA_OK;
}

const char* sla_status_string(sla_status s) {
  switch (s) {
    case SLA_OK: return "ok";
    case SLA_ERR_NULL: return "a required pointer is NULL";
    case SLA_ERR_SHAPE: return "a size is out of range";
    case SLA_ERR_DTYPE: return "unsupported dtype";
    case SLA_ERR_TOPK: return "top_k out of range";
    case SLA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SLA_ERR_WORKSPACE: return "workspace missing or too small";
    case SLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SLA_ERR_HIP: return "kernel launch failed";
    case SLA_ERR_SCRATCH: return "problem needs more than the allocation-free scratch array";
  }
  return "unknown status";
}

}  // extern "C"
