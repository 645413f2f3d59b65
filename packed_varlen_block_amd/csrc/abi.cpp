// Status strings, version and workspace sizing for the C ABI.
#include <cstddef>
#include <cstdint>

#include "pvb.h"

namespace pvb {
size_t attn_fwd_workspace_bytes(int32_t T, int32_t n_seg);
size_t attn_bwd_workspace_bytes(int32_t T, int32_t H, int32_t d, int32_t n_seg, int32_t grad_dtype);
size_t cross_bwd_workspace_bytes(int32_t T_q, int32_t T_k, int32_t H, int32_t n_seg);
}  // namespace pvb

extern "C" size_t pvb_varlen_attn_workspace_bytes(int32_t T, int32_t H, int32_t d, int32_t n_seg,
                                                  int32_t bwd, int32_t grad_dtype) {
  if (T < 0 || H <= 0 || n_seg < 0 || (d != 64 && d != 128)) return 0;
  if (bwd) {
    if (grad_dtype != PVB_BF16 && grad_dtype != PVB_F32) return 0;
    return pvb::attn_bwd_workspace_bytes(T, H, d, n_seg, grad_dtype);
  }
  return pvb::attn_fwd_workspace_bytes(T, n_seg);
}

extern "C" size_t pvb_varlen_cross_attn_workspace_bytes(int32_t T_q, int32_t T_k, int32_t H, int32_t d,
                                                        int32_t n_seg, int32_t bwd, int32_t grad_dtype) {
  if (T_q < 0 || T_k < 0 || H <= 0 || n_seg < 0 || (d != 64 && d != 128)) return 0;
  if (bwd) {
    if (grad_dtype != PVB_BF16 && grad_dtype != PVB_F32) return 0;
    return pvb::cross_bwd_workspace_bytes(T_q, T_k, H, n_seg);
  }
  return pvb::attn_fwd_workspace_bytes(T_q, n_seg);
}

extern "C" const char* pvb_status_string(int32_t status) {
  switch (status) {
    case PVB_OK: return "ok";
    case PVB_E_INVALID_ARG: return "invalid argument";
    case PVB_E_OVERSIZED: return "sample longer than the capacity";
    case PVB_E_OVERFLOW: return "count or offset overflows int32";
    case PVB_E_BAD_CU_SEQLENS: return "bad cu_seqlens (first != 0, decreasing, or last != T)";
    case PVB_E_WORKSPACE: return "workspace missing or too small";
    case PVB_E_UNSUPPORTED: return "unsupported size or head dimension";
    case PVB_E_HIP: return "HIP runtime error";
    case PVB_E_NO_TARGETS: return "no eligible targets (the mean has no denominator)";
    default: return "unknown status";
  }
}

extern "C" const char* pvb_version(void) { return "pvb 0.1.0 gfx950"; }
