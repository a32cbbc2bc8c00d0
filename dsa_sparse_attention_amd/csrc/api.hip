// Host-side plumbing of the C ABI: geometry, status strings, error reporting.
#include <math.h>

#include <string>

#include "common.hpp"

namespace dsa {

static thread_local std::string g_last_error;

dsa_status fail(dsa_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

dsa_status check_geometry(const dsa_geometry* g) {
  if (!g) return fail(DSA_ERR_INVALID_ARGUMENT, "geometry pointer is NULL");
  if (g->region_size != kRegion || g->proxy_dim != kProxy || g->n_groups != kGroups ||
      g->n_idx_heads != kIdxHeads || g->n_q_heads != kQHeads || g->head_dim != kHeadDim)
    return fail(DSA_ERR_UNSUPPORTED,
                "geometry differs from the compiled one (region 8, proxy 256, groups 4, indexer "
                "heads 16, query heads 64, head_dim 192)");
  if (g->topk < 1 || g->topk > kMaxTopk)
    return fail(DSA_ERR_UNSUPPORTED, "topk must be in [1, 512]");
  if (!(g->softmax_scale > 0.0f) || !isfinite(g->softmax_scale))
    return fail(DSA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and positive");
  return DSA_OK;
}

dsa_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(DSA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return DSA_OK;
}

}  // namespace dsa

extern "C" {

dsa_status dsa_geometry_default(dsa_geometry* g) {
  if (!g) return dsa::fail(DSA_ERR_INVALID_ARGUMENT, "geometry pointer is NULL");
  g->region_size = dsa::kRegion;
  g->proxy_dim = dsa::kProxy;
  g->n_groups = dsa::kGroups;
  g->n_idx_heads = dsa::kIdxHeads;
  g->n_q_heads = dsa::kQHeads;
  g->head_dim = dsa::kHeadDim;
  g->topk = dsa::kMaxTopk;
  g->softmax_scale = (float)(1.0 / sqrt((double)dsa::kHeadDim));
  return DSA_OK;
}

const char* dsa_status_string(int s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported geometry or size";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DSA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* dsa_last_error(void) { return dsa::g_last_error.c_str(); }

}  // extern "C"
