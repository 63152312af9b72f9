"""MI355X-native (gfx950) SLA2 sparse-linear attention forward.

The computation lives in libsla.so (HIP kernels behind the C ABI of include/sla.h);
``sla`` is its ctypes binding. The library is loaded on first use; every entry point raises if it is not built.
"""
from .sla import (SlaError, STATUS, Problem, make_problem, workspace_size, sla_route, sla_forward,
                  sla_forward_fp8, sla_forward_profiled, library, LIB_PATH, EXPORTS,
                  STAGES, workspace_region, WS_REGIONS, kv_cache_size, sla_kv_cache_update,
                  cached_workspace_size, sla_forward_cached, sla_route_taylor,
                  sla_forward_taylor, sla_forward_pisa, VARIANT_FORWARD, VARIANT_FP8,
                  VARIANT_PISA, VARIANT_TAYLOR, sla_forward_cached_noalloc, NOALLOC_SCRATCH_BYTES,
                  sla_backward, sla_backward_workspace_size, sla_diag_fp8_mfma,
                  sla_diag_mfma_rate)
from .autograd import sla_attention, SLAAttention

__all__ = ["SlaError", "STATUS", "Problem", "make_problem", "workspace_size", "sla_route", "sla_forward",
           "sla_forward_fp8", "sla_forward_profiled", "library", "LIB_PATH", "EXPORTS", "STAGES",
           "workspace_region", "WS_REGIONS", "kv_cache_size", "sla_kv_cache_update",
           "cached_workspace_size", "sla_forward_cached", "sla_route_taylor",
           "sla_forward_taylor", "sla_forward_pisa", "VARIANT_FORWARD", "VARIANT_FP8",
           "VARIANT_PISA", "VARIANT_TAYLOR", "sla_forward_cached_noalloc", "NOALLOC_SCRATCH_BYTES",
           "sla_backward", "sla_backward_workspace_size", "sla_diag_fp8_mfma",
           "sla_diag_mfma_rate", "sla_attention", "SLAAttention"]
