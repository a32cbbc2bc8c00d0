// Host-side plumbing of the C ABI: geometry, status strings, error reporting.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

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

dsa_status paged_map(const char* who, const dsa_page_table* pt, CacheMap* m) {
  if (!pt || !pt->block_table) return fail(DSA_ERR_INVALID_ARGUMENT, std::string(who) + ": page table or block table is NULL");
  if (pt->max_pages <= 0 || pt->n_pages <= 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, std::string(who) + ": max_pages and n_pages must be positive");
  if (pt->n_pages > kMaxPages || (int64_t)pt->max_pages * kPageRegions * kRegion > (int64_t)1 << 31)
    return fail(DSA_ERR_UNSUPPORTED, std::string(who) + ": more than 2^25 pages or 2^31 positions per sequence");
  m->bt = pt->block_table;
  m->R = (int64_t)pt->max_pages * kPageRegions;
  m->bt_stride = pt->max_pages;
  m->n_pages = pt->n_pages;
  return DSA_OK;
}

dsa_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(DSA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return DSA_OK;
}

// ---- instrumentation ----
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
  bool done;
};
static std::atomic<bool> g_prof_on{false};
static std::mutex g_prof_mu;
static std::vector<ProfRec> g_prof_recs;
static std::vector<hipEvent_t> g_prof_pool;
constexpr size_t kProfMaxRecs = 8192;

static hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  // timing only: no system-scope fence on record, which would write back and
  // invalidate the caches between the kernels being timed
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

ProfScope::ProfScope(const char* name, hipStream_t s) : rec(-1), stream(s) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (g_prof_recs.size() >= kProfMaxRecs) return;
  ProfRec r{name, prof_event(), prof_event(), false};
  if (!r.a || !r.b || hipEventRecord(r.a, s) != hipSuccess) return;
  g_prof_recs.push_back(r);
  rec = (int)g_prof_recs.size() - 1;
}

ProfScope::~ProfScope() {
  if (rec < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if ((size_t)rec < g_prof_recs.size() && hipEventRecord(g_prof_recs[rec].b, stream) == hipSuccess)
    g_prof_recs[rec].done = true;
}

}  // namespace dsa

extern "C" {

dsa_status dsa_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(dsa::g_prof_mu);
  for (auto& r : dsa::g_prof_recs) {
    (void)hipEventSynchronize(r.b);
    dsa::g_prof_pool.push_back(r.a);
    dsa::g_prof_pool.push_back(r.b);
  }
  dsa::g_prof_recs.clear();
  dsa::g_prof_on.store(on != 0);
  return DSA_OK;
}

dsa_status dsa_profile_kernel_stats(const char* kernel, double* total_ms, int32_t* launches) {
  if (!kernel || !total_ms || !launches)
    return dsa::fail(DSA_ERR_INVALID_ARGUMENT, "dsa_profile_kernel_stats: NULL pointer");
  std::lock_guard<std::mutex> lk(dsa::g_prof_mu);
  double tot = 0.0;
  int32_t n = 0;
  for (auto& r : dsa::g_prof_recs) {
    if (!r.done || strcmp(r.name, kernel) != 0) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return dsa::fail(DSA_ERR_HIP, "event synchronize failed");
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return dsa::fail(DSA_ERR_HIP, "event elapsed failed");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return DSA_OK;
}

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
