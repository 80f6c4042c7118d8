// C ABI of the library: host-side validation, workspace carving and launch sequencing.
// Nothing is enqueued before every argument has been checked; no exception leaves this file.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>

#include "../../include/park.h"
#include "park_internal.h"

namespace {

thread_local std::string g_last_error;

park_status fail(park_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
park_status fail(park_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

park_status ok() {
  g_last_error.clear();
  return PARK_OK;
}

park_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PARK_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Bump allocator over the caller's workspace; with a null base it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

park_status check_shape(const park_shape* s, park::Dims* out) {
  if (!s) return fail(PARK_EINVAL, "shape is NULL");
  if (s->heads < 1 || s->heads > 65535) return fail(PARK_EINVAL, "heads must be in [1, 65535], got %lld", (long long)s->heads);
  if (s->n < 1 || s->n >= (int64_t(1) << 24)) return fail(PARK_EINVAL, "n must be in [1, 2^24), got %lld", (long long)s->n);
  if (s->d != 64 && s->d != 128) return fail(PARK_EUNSUPPORTED, "d must be 64 or 128, got %lld", (long long)s->d);
  if (s->dtype != PARK_F32 && s->dtype != PARK_BF16) return fail(PARK_EUNSUPPORTED, "dtype must be PARK_F32 or PARK_BF16");
  *out = park::Dims{s->heads, s->n, s->d, s->dtype == PARK_BF16 ? 1 : 0};
  return PARK_OK;
}

park_status check_clusters(const park::Dims& s, int64_t c, const char* name) {
  if (c < 1 || c > park::kMaxClusters || c > s.N)
    return fail(PARK_EINVAL, "%s must be in [1, min(n, %d)], got %lld", name, park::kMaxClusters, (long long)c);
  return PARK_OK;
}

park_status check_ptr(const void* p, const char* name, size_t align) {
  if (!p) return fail(PARK_EINVAL, "%s is NULL", name);
  if (!aligned(p, align)) return fail(PARK_EINVAL, "%s must be %zu-byte aligned", name, align);
  return PARK_OK;
}

#define PARK_TRY(expr)               \
  do {                               \
    park_status _st = (expr);        \
    if (_st != PARK_OK) return _st;  \
  } while (0)

float resolve_scale(float scale, int64_t d) { return scale > 0.f ? scale : 1.0f / std::sqrt((float)d); }

// ---------------------------------------------------------------------------------------------
// Workspace plans (shared by the size query and the carving)
// ---------------------------------------------------------------------------------------------

struct MetricWs {
  double* partial;
};
MetricWs plan_metric(Carver& cv, const park::Dims& s) {
  MetricWs w;
  w.partial = cv.take<double>(s.bf16 ? park::metric_partial_count(s) : 1);
  return w;
}

struct ClusterWs {
  double* cand_norm;
  float* cand_y;
  double* kpp_psum;
  int32_t* kpp_sync;
  int32_t* table;
  void* g;
  float* b;
  double* fuse_sum = nullptr;   // fused Euclidean Lloyd step: per work-group member sums
  int32_t* fuse_cnt = nullptr;  // and member counts (NULL: the step runs unfused)
};
ClusterWs plan_cluster(Carver& cv, const park::Dims& s, int C, bool qrkc) {
  ClusterWs w;
  if (!qrkc) {
    const int P = park::fused_parts(s, C);
    if (P > 0) {
      w.fuse_sum = cv.take<double>((size_t)s.H * P * C * s.D);
      w.fuse_cnt = cv.take<int32_t>((size_t)s.H * P * C);
    }
  }
  const size_t S = (size_t)park::kpp_candidates(s.N, C);
  w.cand_norm = cv.take<double>((size_t)s.H * S);
  w.cand_y = qrkc ? cv.take<float>((size_t)s.H * S * s.D) : nullptr;
  w.kpp_psum = cv.take<double>((size_t)s.H * C * 16 * 2);
  w.kpp_sync = cv.take<int32_t>((size_t)s.H * C * 3 + 1);
  w.table = cv.take<int32_t>(park::sort_table_ints(s, C));
  w.g = s.bf16 ? (void*)cv.take<uint16_t>((size_t)(s.H * C * s.D)) : (void*)cv.take<float>((size_t)(s.H * C * s.D));
  w.b = cv.take<float>((size_t)(s.H * C));
  return w;
}

struct MapWs {
  uint16_t* khat;
  float* logn;
  int32_t* chunk_base;
  float* partial;
};
MapWs plan_map(Carver& cv, const park::Dims& s, int cq, int ck) {
  MapWs w;
  w.khat = cv.take<uint16_t>((size_t)(s.H * ck * s.D));
  w.logn = cv.take<float>((size_t)(s.H * ck));
  w.chunk_base = cv.take<int32_t>((size_t)(s.H * (cq + 1)));
  w.partial = cv.take<float>((size_t)(s.H * park::pama_max_chunks(s, cq) * ck));
  return w;
}

// Estimator maps: centroid-query rows (CC, CF), the map workspace sized for the query rows used
// (FC, CC, FF) and the CF passes' per-chunk pairs and row offsets.
struct EstWs {
  uint16_t* qrows = nullptr;
  int32_t* qperm = nullptr;
  int32_t* qoff = nullptr;
  float* cf_part = nullptr;
  float* cf_off = nullptr;
  MapWs map;
};
EstWs plan_estimator(Carver& cv, const park::Dims& s, int cq, int ck, int mode) {
  EstWs w;
  if (mode == PARK_EST_CC || mode == PARK_EST_CF) {
    w.qrows = cv.take<uint16_t>((size_t)(s.H * cq * s.D));
    w.qperm = cv.take<int32_t>((size_t)(s.H * cq));
    w.qoff = cv.take<int32_t>((size_t)(s.H * (cq + 1)));
  }
  if (mode == PARK_EST_CF) {
    w.cf_part = cv.take<float>((size_t)(s.H * park::cf_chunks(s) * cq * 2));
    w.cf_off = cv.take<float>((size_t)(s.H * cq));
  } else if (mode == PARK_EST_CC) {
    park::Dims sq = s;
    sq.N = cq;
    w.map = plan_map(cv, sq, cq, ck);
  } else {
    w.map = plan_map(cv, s, cq, ck);
  }
  return w;
}
size_t estimator_ws_bytes(const park::Dims& s, int cq, int ck) {
  size_t m = 0;
  for (int mode = PARK_EST_FC; mode <= PARK_EST_FF; ++mode) {
    Carver c(nullptr);
    plan_estimator(c, s, cq, ck, mode);
    m = c.off > m ? c.off : m;
  }
  return m;
}

struct AttnWs {
  int32_t* tile_base;
  int32_t* runs;  // per (head, query cluster): the runs of its selected keys, run and key counts
};
AttnWs plan_attn(Carver& cv, const park::Dims& s, int cq, int ck) {
  AttnWs w;
  w.tile_base = cv.take<int32_t>((size_t)(s.H * (2 * cq + 1)));
  w.runs = cv.take<int32_t>(park::attn_run_ints(s, cq, ck));
  return w;
}

struct ForwardWs {
  float* metric;
  int32_t *q_labels, *q_perm, *q_offsets, *k_labels, *k_perm, *k_offsets;
  float* map;
  int32_t *counts, *cols;
  int64_t* sel_keys;
  MetricWs mt;
  ClusterWs qc, kc;
  MapWs mw;
  AttnWs aw;
};
ForwardWs plan_forward(Carver& cv, const park::Dims& s, const park_params& p) {
  ForwardWs w;
  const size_t hn = (size_t)(s.H * s.N);
  w.metric = cv.take<float>((size_t)(s.H * s.D * s.D));
  w.q_labels = cv.take<int32_t>(hn);
  w.q_perm = cv.take<int32_t>(hn);
  w.q_offsets = cv.take<int32_t>((size_t)(s.H * (p.cq + 1)));
  w.k_labels = cv.take<int32_t>(hn);
  w.k_perm = cv.take<int32_t>(hn);
  w.k_offsets = cv.take<int32_t>((size_t)(s.H * (p.ck + 1)));
  w.map = cv.take<float>((size_t)(s.H * p.cq * p.ck));
  w.counts = cv.take<int32_t>((size_t)(s.H * p.cq));
  w.cols = cv.take<int32_t>((size_t)(s.H * p.cq * p.ck));
  w.sel_keys = cv.take<int64_t>((size_t)(s.H * p.cq));
  w.mt = plan_metric(cv, s);
  w.qc = plan_cluster(cv, s, p.cq, false);
  w.kc = plan_cluster(cv, s, p.ck, p.kmetric == PARK_QRKC);
  w.mw = plan_map(cv, s, p.cq, p.ck);
  w.aw = plan_attn(cv, s, p.cq, p.ck);
  return w;
}

park_status check_params(const park::Dims& s, const park_params* p, bool need_iters) {
  if (!p) return fail(PARK_EINVAL, "params is NULL");
  PARK_TRY(check_clusters(s, p->cq, "cq"));
  PARK_TRY(check_clusters(s, p->ck, "ck"));
  if (p->iters < (need_iters ? 1 : 0) || p->iters > 100000)
    return fail(PARK_EINVAL, "iters must be in [%d, 100000], got %d", need_iters ? 1 : 0, p->iters);
  if (!(p->p > 0.0 && p->p <= 1.0)) return fail(PARK_EINVAL, "p must be in (0, 1], got %g", p->p);
  if (p->kmetric != PARK_EUCLID && p->kmetric != PARK_QRKC) return fail(PARK_EINVAL, "kmetric must be PARK_EUCLID or PARK_QRKC");
  if (p->init != PARK_INIT_KMEANSPP && p->init != PARK_INIT_WARM && p->init != PARK_INIT_SUBSET)
    return fail(PARK_EINVAL, "init must be PARK_INIT_KMEANSPP, PARK_INIT_WARM or PARK_INIT_SUBSET");
  if (p->init == PARK_INIT_SUBSET && (p->subset_stride < 1 || p->subset_phase < 0 || p->subset_phase >= p->subset_stride))
    return fail(PARK_EINVAL, "subset updates need subset_stride >= 1 and 0 <= subset_phase < subset_stride, got %d, %d",
                p->subset_stride, p->subset_phase);
  if (std::isnan(p->scale)) return fail(PARK_EINVAL, "scale is NaN");
  return PARK_OK;
}

park_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return PARK_OK;
  if (ws_bytes < need) return fail(PARK_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", ws_bytes, need);
  if (!ws) return fail(PARK_EINVAL, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(PARK_EINVAL, "workspace must be 256-byte aligned");
  return PARK_OK;
}

size_t forward_ws_bytes(const park::Dims& s, const park_params& p) {
  Carver cv(nullptr);
  plan_forward(cv, s, p);
  return cv.off;
}

// Lloyd iterations shared by park_cluster and park_forward: (g, b) of the current centroids, then
// per iteration assign -> stable sort -> update (which also prepares (g, b) for the next one). A
// Euclidean bf16 side with at most 128 clusters runs the fused step instead (same labels; means
// from per-tile fp32 sums added in fp64) and sorts once at the end.
// With stride > 1 (a subset update) only the rows phase, phase + stride, ... are re-assigned; the
// others keep the labels already in `labels`, which are first clamped into [0, C).
hipError_t run_lloyd(const park::Dims& s, const void* x, const float* metric, int C, int iters, float* cent,
                     int32_t* labels, int32_t* perm, int32_t* offsets, const ClusterWs& w, hipStream_t st,
                     int stride = 1, int phase = 0) {
  if (iters == 0) return hipSuccess;
  hipError_t e = park::launch_update(s, x, C, nullptr, nullptr, cent, 0, metric, w.g, w.b, st);
  if (metric == nullptr && stride == 1 && w.fuse_sum != nullptr) {
    // Euclidean side with few clusters: assignment and member means in one pass per iteration,
    // the cluster order once after the last
    for (int it = 0; it < iters && e == hipSuccess; ++it) {
      e = park::launch_lloyd_fused(s, x, C, w.g, w.b, labels, w.fuse_sum, w.fuse_cnt, cent, st);
      if (e == hipSuccess) e = park::launch_update(s, x, C, nullptr, nullptr, cent, 0, nullptr, w.g, w.b, st);
    }
    if (e == hipSuccess) e = park::launch_sort(s, C, labels, w.table, perm, offsets, st);
    return e;
  }
  if (e == hipSuccess && stride > 1) e = park::launch_clamp_labels(s, C, labels, st);
  for (int it = 0; it < iters && e == hipSuccess; ++it) {
    e = park::launch_assign(s, x, C, w.g, w.b, labels, st, stride, phase);
    if (e == hipSuccess) e = park::launch_sort(s, C, labels, w.table, perm, offsets, st);
    if (e == hipSuccess) e = park::launch_update(s, x, C, perm, offsets, cent, 1, metric, w.g, w.b, st);
  }
  return e;
}

// A helper stream per device (default priority, created on first use and kept for the process):
// park_forward runs the query-side Lloyd iterations on it, concurrently with the key side on the
// caller's stream (the query side streams its data from HBM while the key side's assignment is
// bound by the matrix cores). Fork and join go through events, so the caller's stream still orders
// every launch of the call, also under stream capture.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
std::map<int, SideStream> g_side;

// Returns the device's helper stream with g_side_mu held by `lock`.
hipError_t side_stream(std::unique_lock<std::mutex>& lock, SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  lock = std::unique_lock<std::mutex>(g_side_mu);
  SideStream& ss = g_side[dev];
  if (!ss.stream) {
    SideStream n;
    e = hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    ss = n;
  }
  *out = &ss;
  return hipSuccess;
}

// Scratch of park_sparse_attn_noalloc: static device memory of a fixed size, one copy per GPU,
// held until the process ends. Host code never uses the array's name as an address: on each device
// its address comes from hipGetSymbolAddress once (with that device current) and is kept here.
constexpr size_t kNoAllocScratchBytes = size_t(96) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;

// The current device's scratch address (nullptr and an error on failure).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return hipSuccess;
}

park::KppArgs kpp_args(const void* x, const float* metric, int C, int side, float* cent, const ClusterWs& w) {
  return park::KppArgs{x, metric, C, side, cent, w.cand_norm, w.cand_y, w.kpp_psum, w.kpp_sync};
}

}  // namespace

extern "C" {

const char* park_version(void) { return "park-mi355x 0.1.0 (gfx950)"; }

const char* park_status_string(int32_t status) {
  switch (status) {
    case PARK_OK: return "PARK_OK";
    case PARK_EINVAL: return "PARK_EINVAL";
    case PARK_EUNSUPPORTED: return "PARK_EUNSUPPORTED";
    case PARK_EWORKSPACE: return "PARK_EWORKSPACE";
    case PARK_EHIP: return "PARK_EHIP";
    default: return "PARK_UNKNOWN";
  }
}

const char* park_last_error(void) { return g_last_error.c_str(); }

void park_debug_force_seed_timeout(int32_t on) { park::g_force_seed_timeout.store(on != 0 ? 1 : 0); }

size_t park_workspace_bytes(int32_t entry, const park_shape* shape, const park_params* params) {
  try {
    park::Dims s;
    if (check_shape(shape, &s) != PARK_OK) return 0;
    Carver cv(nullptr);
    switch (entry) {
      case PARK_ENTRY_METRIC:
        plan_metric(cv, s);
        return cv.off;
      case PARK_ENTRY_CLUSTER_Q:
      case PARK_ENTRY_CLUSTER_K: {
        if (!params) return 0;
        const int C = entry == PARK_ENTRY_CLUSTER_Q ? params->cq : params->ck;
        if (check_clusters(s, C, "clusters") != PARK_OK) return 0;
        plan_cluster(cv, s, C, entry == PARK_ENTRY_CLUSTER_K && params->kmetric == PARK_QRKC);
        return cv.off;
      }
      case PARK_ENTRY_RETRIEVE_MAP:
        if (!params || check_clusters(s, params->cq, "cq") != PARK_OK || check_clusters(s, params->ck, "ck") != PARK_OK) return 0;
        plan_map(cv, s, params->cq, params->ck);
        return cv.off;
      case PARK_ENTRY_SELECT_TOPP:
        return 0;
      case PARK_ENTRY_SPARSE_ATTN:
        if (!params || check_clusters(s, params->cq, "cq") != PARK_OK || check_clusters(s, params->ck, "ck") != PARK_OK) return 0;
        plan_attn(cv, s, params->cq, params->ck);
        return cv.off;
      case PARK_ENTRY_SPARSE_ATTN_WEIGHTED:
        if (!params || check_clusters(s, params->cq, "cq") != PARK_OK || check_clusters(s, params->ck, "ck") != PARK_OK) return 0;
        plan_attn(cv, s, params->cq, params->ck);
        return cv.off;
      case PARK_ENTRY_ESTIMATOR:
        if (!params || check_clusters(s, params->cq, "cq") != PARK_OK || check_clusters(s, params->ck, "ck") != PARK_OK) return 0;
        return estimator_ws_bytes(s, params->cq, params->ck);
      case PARK_ENTRY_FORWARD:
        if (check_params(s, params, true) != PARK_OK) return 0;
        return forward_ws_bytes(s, *params);
      case PARK_ENTRY_MERGE:
        if (!params || check_clusters(s, params->cq, "cq") != PARK_OK || params->ck < 1 ||
            params->ck > park::kMaxClusters)
          return 0;
        cv.take<int32_t>(park::merge_ws_ints(s.H, params->cq, params->ck));
        return cv.off;
      default:
        return 0;
    }
  } catch (...) {
    return 0;
  }
}

park_status park_qrkc_metric(const park_shape* shape, const void* q, float* metric, void* ws, size_t ws_bytes,
                             void* stream) {
  try {
    park::Dims s;
    PARK_TRY(check_shape(shape, &s));
    PARK_TRY(check_ptr(q, "q", 16));
    PARK_TRY(check_ptr(metric, "metric", 4));
    Carver meas(nullptr);
    plan_metric(meas, s);
    PARK_TRY(check_ws(ws, ws_bytes, meas.off));
    Carver cv(ws);
    MetricWs w = plan_metric(cv, s);
    return hip_check(park::launch_metric(s, q, metric, w.partial, (hipStream_t)stream), "park_qrkc_metric");
  } catch (...) {
    return fail(PARK_EHIP, "park_qrkc_metric: internal error");
  }
}

park_status park_cluster(const park_shape* shape, const void* x, int32_t metric, const float* qmetric,
                         int32_t n_clusters, int32_t iters, int32_t init, uint64_t seed, int32_t side, float* centroids,
                         int32_t* labels, int32_t* perm, int32_t* offsets, int32_t* status, void* ws, size_t ws_bytes,
                         void* stream) {
  try {
    park::Dims s;
    PARK_TRY(check_shape(shape, &s));
    PARK_TRY(check_ptr(x, "x", 16));
    PARK_TRY(check_clusters(s, n_clusters, "n_clusters"));
    if (metric != PARK_EUCLID && metric != PARK_QRKC) return fail(PARK_EINVAL, "metric must be PARK_EUCLID or PARK_QRKC");
    if (metric == PARK_QRKC) PARK_TRY(check_ptr(qmetric, "qmetric", 4));
    if (iters < 0 || iters > 100000) return fail(PARK_EINVAL, "iters must be in [0, 100000], got %d", iters);
    if (init != PARK_INIT_KMEANSPP && init != PARK_INIT_WARM) return fail(PARK_EINVAL, "init must be PARK_INIT_KMEANSPP or PARK_INIT_WARM");
    if (side != PARK_SIDE_Q && side != PARK_SIDE_K) return fail(PARK_EINVAL, "side must be PARK_SIDE_Q or PARK_SIDE_K");
    PARK_TRY(check_ptr(centroids, "centroids", 4));
    if (status && !aligned(status, 4)) return fail(PARK_EINVAL, "status must be 4-byte aligned");
    if (iters > 0) {
      PARK_TRY(check_ptr(labels, "labels", 4));
      PARK_TRY(check_ptr(perm, "perm", 4));
      PARK_TRY(check_ptr(offsets, "offsets", 4));
    }
    Carver meas(nullptr);
    plan_cluster(meas, s, n_clusters, metric == PARK_QRKC);
    PARK_TRY(check_ws(ws, ws_bytes, meas.off));
    Carver cv(ws);
    ClusterWs w = plan_cluster(cv, s, n_clusters, metric == PARK_QRKC);
    const float* mp = metric == PARK_QRKC ? qmetric : nullptr;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (init == PARK_INIT_KMEANSPP) {
      const park::KppArgs a = kpp_args(x, mp, n_clusters, side, centroids, w);
      e = park::launch_kpp(s, &a, 1, seed, status, st);
    }
    if (e == hipSuccess) e = run_lloyd(s, x, mp, n_clusters, iters, centroids, labels, perm, offsets, w, st);
    return hip_check(e, "park_cluster");
  } catch (...) {
    return fail(PARK_EHIP, "park_cluster: internal error");
  }
}

park_status park_cluster_subset(const park_shape* shape, const void* x, int32_t metric, const float* qmetric,
                                int32_t n_clusters, int32_t iters, int32_t stride, int32_t phase, float* centroids,
                                int32_t* labels, int32_t* perm, int32_t* offsets, void* ws, size_t ws_bytes,
                                void* stream) {
  try {
    park::Dims s;
    PARK_TRY(check_shape(shape, &s));
    PARK_TRY(check_ptr(x, "x", 16));
    PARK_TRY(check_clusters(s, n_clusters, "n_clusters"));
    if (metric != PARK_EUCLID && metric != PARK_QRKC) return fail(PARK_EINVAL, "metric must be PARK_EUCLID or PARK_QRKC");
    if (metric == PARK_QRKC) PARK_TRY(check_ptr(qmetric, "qmetric", 4));
    if (iters < 1 || iters > 100000) return fail(PARK_EINVAL, "iters must be in [1, 100000], got %d", iters);
    if (stride < 1 || phase < 0 || phase >= stride)
      return fail(PARK_EINVAL, "need stride >= 1 and 0 <= phase < stride, got %d, %d", stride, phase);
    PARK_TRY(check_ptr(centroids, "centroids", 4));
    PARK_TRY(check_ptr(labels, "labels", 4));
    PARK_TRY(check_ptr(perm, "perm", 4));
    PARK_TRY(check_ptr(offsets, "offsets", 4));
    Carver meas(nullptr);
    plan_cluster(meas, s, n_clusters, metric == PARK_QRKC);
    PARK_TRY(check_ws(ws, ws_bytes, meas.off));
    Carver cv(ws);
    ClusterWs w = plan_cluster(cv, s, n_clusters, metric == PARK_QRKC);
    return hip_check(run_lloyd(s, x, metric == PARK_QRKC ? qmetric : nullptr, n_clusters, iters, centroids, labels,
                               perm, offsets, w, (hipStream_t)stream, stride, phase),
                     "park_cluster_subset");
  } catch (...) {
    return fail(PARK_EHIP, "park_cluster_subset: internal error");
  }
}

park_status park_retrieve_map(const park_shape* shape, const void* q, const int32_t* q_perm, const int32_t* q_offsets,
                              int32_t cq, const float* k_centroids, const int32_t* k_offsets, int32_t ck, float scale,
                              float* map, void* ws, size_t ws_bytes, void* stream) {
  try {
    park::Dims s;
    PARK_TRY(check_shape(shape, &s));
    PARK_TRY(check_ptr(q, "q", 16));
    PARK_TRY(check_ptr(q_perm, "q_perm", 4));
    PARK_TRY(check_ptr(q_offsets, "q_offsets", 4));
    PARK_TRY(check_ptr(k_centroids, "k_centroids", 4));
    PARK_TRY(check_ptr(k_offsets, "k_offsets", 4));
    PARK_TRY(check_ptr(map, "map", 4));
    PARK_TRY(check_clusters(s, cq, "cq"));
    PARK_TRY(check_clusters(s, ck, "ck"));
    if (std::isnan(scale)) return fail(PARK_EINVAL, "scale is NaN");
    Carver meas(nullptr);
    plan_map(meas, s, cq, ck);
    PARK_TRY(check_ws(ws, ws_bytes, meas.off));
    Carver cv(ws);
    MapWs w = plan_map(cv, s, cq, ck);
    return hip_check(park::launch_pama(s, q, q_perm, q_offsets, cq, k_centroids, k_offsets, ck,
                                       resolve_scale(scale, s.D), map, w.khat, w.logn, w.chunk_base, w.partial,
                                       (hipStream_t)stream),
                     "park_retrieve_map");
  } catch (...) {
    return fail(PARK_EHIP, "park_retrieve_map: internal error");
  }
}

park_status park_estimator_map(const park_shape* shape, const void* q, const void* k, const int32_t* q_perm,
                               const int32_t* q_offsets, int32_t cq, const float* q_centroids, const int32_t* k_perm,
                               const int32_t* k_offsets, int32_t ck, const float* k_centroids, int32_t mode,
                               float scale, float* map, void* ws, size_t ws_bytes, void* stream) {
  try {
    park::Dims s;
    PARK_TRY(check_shape(shape, &s));
    if (mode < PARK_EST_FC || mode > PARK_EST_FF) return fail(PARK_EINVAL, "mode must be a park_estimator, got %d", mode);
    if (mode != PARK_EST_FC && !s.bf16) return fail(PARK_EUNSUPPORTED, "estimator modes CC, CF and FF need bf16 data");
    PARK_TRY(check_clusters(s, cq, "cq"));
    PARK_TRY(check_clusters(s, ck, "ck"));
    if (std::isnan(scale)) return fail(PARK_EINVAL, "scale is NaN");
    const bool full_q = mode == PARK_EST_FC || mode == PARK_EST_FF;
    const bool full_k = mode == PARK_EST_CF || mode == PARK_EST_FF;
    PARK_TRY(check_ptr(q_offsets, "q_offsets", 4));
    if (full_q) {
      PARK_TRY(check_ptr(q, "q", 16));
      PARK_TRY(check_ptr(q_perm, "q_perm", 4));
    } else {
      PARK_TRY(check_ptr(q_centroids, "q_centroids", 4));
    }
    if (full_k) {
      PARK_TRY(check_ptr(k, "k", 16));
      PARK_TRY(check_ptr(k_perm, "k_perm", 4));
    } else {
      PARK_TRY(check_ptr(k_centroids, "k_centroids", 4));
    }
    PARK_TRY(check_ptr(k_offsets, "k_offsets", 4));
    PARK_TRY(check_ptr(map, "map", 4));
    PARK_TRY(check_ws(ws, ws_bytes, estimator_ws_bytes(s, cq, ck)));
    Carver cv(ws);
    EstWs w = plan_estimator(cv, s, cq, ck, mode);
    hipStream_t st = (hipStream_t)stream;
    const float sc = resolve_scale(scale, s.D);
    hipError_t e = hipSuccess;
    park::Dims sq = s;
    const void* qr = q;
    const int32_t* qp = q_perm;
    const int32_t* qo = q_offsets;
    if (!full_q) {  // one bf16 centroid row per query cluster
      sq.N = cq;
      e = park::launch_centroid_queries(s.H, cq, (int)s.D, q_centroids, q_offsets, w.qrows, w.qperm, w.qoff, st);
      qr = w.qrows;
      qp = w.qperm;
      qo = w.qoff;
    }
    if (e == hipSuccess) {
      if (mode == PARK_EST_CF)
        e = park::launch_cf_map(s, w.qrows, q_offsets, cq, k, k_perm, k_offsets, ck, sc, map, w.cf_part, w.cf_off, st);
      else if (full_k)
        e = park::launch_block_mass(sq, qr, qp, qo, cq, k, s.N, k_perm, k_offsets, ck, sc, map, w.map.chunk_base,
                                    w.map.partial, st);
      else
        e = park::launch_pama(sq, qr, qp, qo, cq, k_centroids, k_offsets, ck, sc, map, w.map.khat, w.map.logn,
                              w.map.chunk_base, w.map.partial, st);
    }
    return hip_check(e, "park_estimator_map");
  } catch (...) {
    return fail(PARK_EHIP, "park_estimator_map: internal error");
  }
}

park_status park_select_topp(const float* map, int64_t heads, int32_t cq, int32_t ck, const int32_t* k_offsets,
                             double p, uint8_t* mask, int32_t* counts, int32_t* cols, int64_t* sel_keys,
                             void* stream) {
  try {
    if (heads < 1 || heads > 65535) return fail(PARK_EINVAL, "heads must be in [1, 65535]");
    if (cq < 1 || cq > park::kMaxClusters) return fail(PARK_EINVAL, "cq must be in [1, %d]", park::kMaxClusters);
    if (ck < 1 || ck > park::kMaxClusters) return fail(PARK_EINVAL, "ck must be in [1, %d]", park::kMaxClusters);
    if (!(p > 0.0 && p <= 1.0)) return fail(PARK_EINVAL, "p must be in (0, 1], got %g", p);
    PARK_TRY(check_ptr(map, "map", 4));
    PARK_TRY(check_ptr(k_offsets, "k_offsets", 4));
    PARK_TRY(check_ptr(counts, "counts", 4));
    PARK_TRY(check_ptr(cols, "cols", 4));
    if (sel_keys) PARK_TRY(check_ptr(sel_keys, "sel_keys", 8));
    return hip_check(park::launch_select_topp(map, heads, cq, ck, k_offsets, p, mask, counts, cols, sel_keys,
                                              (hipStream_t)stream),
                     "park_select_topp");
  } catch (...) {
    return fail(PARK_EHIP, "park_select_topp: internal error");
  }
}

park_status park_select_topk(const float* map, int64_t heads, int32_t cq, int32_t ck, const int32_t* k_offsets,
                             double rho, uint8_t* mask, int32_t* counts, int32_t* cols, int64_t* sel_keys,
                             void* stream) {
  try {
    if (heads < 1 || heads > 65535) return fail(PARK_EINVAL, "heads must be in [1, 65535]");
    if (cq < 1 || cq > park::kMaxClusters) return fail(PARK_EINVAL, "cq must be in [1, %d]", park::kMaxClusters);
    if (ck < 1 || ck > park::kMaxClusters) return fail(PARK_EINVAL, "ck must be in [1, %d]", park::kMaxClusters);
    if (!(rho >= 0.0 && rho <= 1.0)) return fail(PARK_EINVAL, "rho must be in [0, 1], got %g", rho);
    PARK_TRY(check_ptr(map, "map", 4));
    PARK_TRY(check_ptr(k_offsets, "k_offsets", 4));
    PARK_TRY(check_ptr(counts, "counts", 4));
    PARK_TRY(check_ptr(cols, "cols", 4));
    if (sel_keys) PARK_TRY(check_ptr(sel_keys, "sel_keys", 8));
    return hip_check(park::launch_select_topk(map, heads, cq, ck, k_offsets, rho, mask, counts, cols, sel_keys,
                                              (hipStream_t)stream),
                     "park_select_topk");
  } catch (...) {
    return fail(PARK_EHIP, "park_select_topk: internal error");
  }
}

park_status park_select_sip(const float* map, int64_t heads, int32_t cq, int32_t ck, const int32_t* k_offsets,
                            double rho, uint64_t seed, uint8_t* mask, int32_t* counts, int32_t* cols,
                            int64_t* sel_keys, float* log_w, void* stream) {
  try {
    if (heads < 1 || heads > 65535) return fail(PARK_EINVAL, "heads must be in [1, 65535]");
    if (cq < 1 || cq > park::kMaxClusters) return fail(PARK_EINVAL, "cq must be in [1, %d]", park::kMaxClusters);
    if (ck < 1 || ck > park::kMaxClusters) return fail(PARK_EINVAL, "ck must be in [1, %d]", park::kMaxClusters);
    if (!(rho >= 0.0 && rho <= 1.0)) return fail(PARK_EINVAL, "rho must be in [0, 1], got %g", rho);
    PARK_TRY(check_ptr(map, "map", 4));
    PARK_TRY(check_ptr(k_offsets, "k_offsets", 4));
    PARK_TRY(check_ptr(counts, "counts", 4));
    PARK_TRY(check_ptr(cols, "cols", 4));
    PARK_TRY(check_ptr(log_w, "log_w", 4));
    if (sel_keys) PARK_TRY(check_ptr(sel_keys, "sel_keys", 8));
    return hip_check(park::launch_select_sip(map, heads, cq, ck, k_offsets, rho, seed, mask, counts, cols, sel_keys,
                                             log_w, (hipStream_t)stream),
                     "park_select_sip");
  } catch (...) {
    return fail(PARK_EHIP, "park_select_sip: internal error");
  }
}

namespace {
park_status sparse_attn_impl(const char* name, const park_shape* shape, const void* q, const void* k, const void* v,
                             const int32_t* q_perm, const int32_t* q_offsets, int32_t cq, const int32_t* k_perm,
                             const int32_t* k_offsets, int32_t ck, const int32_t* counts, const int32_t* cols,
                             const float* log_w, float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                             void* stream) {
  park::Dims s;
  PARK_TRY(check_shape(shape, &s));
  PARK_TRY(check_ptr(q, "q", 16));
  PARK_TRY(check_ptr(k, "k", 16));
  PARK_TRY(check_ptr(v, "v", 16));
  PARK_TRY(check_ptr(out, "out", 16));
  PARK_TRY(check_ptr(q_perm, "q_perm", 4));
  PARK_TRY(check_ptr(q_offsets, "q_offsets", 4));
  PARK_TRY(check_ptr(k_perm, "k_perm", 4));
  PARK_TRY(check_ptr(k_offsets, "k_offsets", 4));
  PARK_TRY(check_ptr(counts, "counts", 4));
  PARK_TRY(check_ptr(cols, "cols", 4));
  if (log_w) PARK_TRY(check_ptr(log_w, "log_w", 4));
  if (lse) PARK_TRY(check_ptr(lse, "lse", 4));
  PARK_TRY(check_clusters(s, cq, "cq"));
  PARK_TRY(check_clusters(s, ck, "ck"));
  if (std::isnan(scale)) return fail(PARK_EINVAL, "scale is NaN");
  Carver meas(nullptr);
  plan_attn(meas, s, cq, ck);
  PARK_TRY(check_ws(ws, ws_bytes, meas.off));
  Carver cv(ws);
  AttnWs w = plan_attn(cv, s, cq, ck);
  return hip_check(park::launch_sparse_attn(s, q, k, v, q_perm, q_offsets, cq, k_perm, k_offsets, ck, counts, cols,
                                            log_w, resolve_scale(scale, s.D), out, lse, w.tile_base, w.runs,
                                            nullptr, (hipStream_t)stream),
                   name);
}
}  // namespace

park_status park_sparse_attn(const park_shape* shape, const void* q, const void* k, const void* v, const int32_t* q_perm,
                             const int32_t* q_offsets, int32_t cq, const int32_t* k_perm, const int32_t* k_offsets,
                             int32_t ck, const int32_t* counts, const int32_t* cols, float scale, void* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream) {
  try {
    return sparse_attn_impl("park_sparse_attn", shape, q, k, v, q_perm, q_offsets, cq, k_perm, k_offsets, ck, counts,
                            cols, nullptr, scale, out, lse, ws, ws_bytes, stream);
  } catch (...) {
    return fail(PARK_EHIP, "park_sparse_attn: internal error");
  }
}

park_status park_sparse_attn_noalloc(const park_shape* shape, const void* q, const void* k, const void* v,
                                     const int32_t* q_perm, const int32_t* q_offsets, int32_t cq, const int32_t* k_perm,
                                     const int32_t* k_offsets, int32_t ck, const int32_t* counts, const int32_t* cols,
                                     float scale, void* out, float* lse, void* stream) {
  try {
    park::Dims s;
    PARK_TRY(check_shape(shape, &s));
    PARK_TRY(check_clusters(s, cq, "cq"));
    PARK_TRY(check_clusters(s, ck, "ck"));
    Carver meas(nullptr);
    plan_attn(meas, s, cq, ck);
    if (meas.off > kNoAllocScratchBytes)
      return fail(PARK_EWORKSPACE,
                  "park_sparse_attn_noalloc: this shape needs %zu bytes of scratch, more than the %zu bytes it holds "
                  "(use park_sparse_attn with a workspace)",
                  meas.off, kNoAllocScratchBytes);
    void* ptr = nullptr;
    PARK_TRY(hip_check(scratch_address(&ptr), "park_sparse_attn_noalloc: scratch address"));
    return sparse_attn_impl("park_sparse_attn_noalloc", shape, q, k, v, q_perm, q_offsets, cq, k_perm, k_offsets, ck,
                            counts, cols, nullptr, scale, out, lse, ptr, kNoAllocScratchBytes, stream);
  } catch (...) {
    return fail(PARK_EHIP, "park_sparse_attn_noalloc: internal error");
  }
}

park_status park_sparse_attn_weighted(const park_shape* shape, const void* q, const void* k, const void* v,
                                      const int32_t* q_perm, const int32_t* q_offsets, int32_t cq,
                                      const int32_t* k_perm, const int32_t* k_offsets, int32_t ck,
                                      const int32_t* counts, const int32_t* cols, const float* log_w, float scale,
                                      void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  try {
    if (!log_w) return fail(PARK_EINVAL, "log_w is NULL");
    return sparse_attn_impl("park_sparse_attn_weighted", shape, q, k, v, q_perm, q_offsets, cq, k_perm, k_offsets,
                            ck, counts, cols, log_w, scale, out, lse, ws, ws_bytes, stream);
  } catch (...) {
    return fail(PARK_EHIP, "park_sparse_attn_weighted: internal error");
  }
}

park_status park_merge_clusters(int64_t heads, int64_t n, int32_t cq, int32_t ck, int32_t bm, const int32_t* q_perm,
                                const int32_t* q_offsets, const int32_t* k_offsets, const int32_t* counts,
                                const int32_t* cols, int32_t* group, int32_t* m_perm, int32_t* m_offsets,
                                int32_t* m_counts, int32_t* m_cols, void* ws, size_t ws_bytes, void* stream) {
  try {
    if (heads < 1 || heads > 65535) return fail(PARK_EINVAL, "heads must be in [1, 65535]");
    if (n < 1 || n >= (int64_t(1) << 24)) return fail(PARK_EINVAL, "n must be in [1, 2^24), got %lld", (long long)n);
    if (cq < 1 || cq > park::kMaxClusters || cq > n) return fail(PARK_EINVAL, "cq must be in [1, min(n, %d)]", park::kMaxClusters);
    if (ck < 1 || ck > park::kMaxClusters) return fail(PARK_EINVAL, "ck must be in [1, %d]", park::kMaxClusters);
    if (bm < 1) return fail(PARK_EINVAL, "bm must be >= 1, got %d", bm);
    PARK_TRY(check_ptr(q_perm, "q_perm", 4));
    PARK_TRY(check_ptr(q_offsets, "q_offsets", 4));
    PARK_TRY(check_ptr(k_offsets, "k_offsets", 4));
    PARK_TRY(check_ptr(counts, "counts", 4));
    PARK_TRY(check_ptr(cols, "cols", 4));
    PARK_TRY(check_ptr(group, "group", 4));
    PARK_TRY(check_ptr(m_perm, "m_perm", 4));
    PARK_TRY(check_ptr(m_offsets, "m_offsets", 4));
    PARK_TRY(check_ptr(m_counts, "m_counts", 4));
    PARK_TRY(check_ptr(m_cols, "m_cols", 4));
    if (m_perm == q_perm || m_cols == cols || m_offsets == q_offsets || m_counts == counts)
      return fail(PARK_EINVAL, "the merged clustering must not overlap its inputs");
    const size_t need = park::merge_ws_ints(heads, cq, ck) * sizeof(int32_t);
    PARK_TRY(check_ws(ws, ws_bytes, need));
    return hip_check(park::launch_merge(heads, n, cq, ck, bm, q_perm, q_offsets, k_offsets, counts, cols, group, m_perm,
                                        m_offsets, m_counts, m_cols, static_cast<int32_t*>(ws), (hipStream_t)stream),
                     "park_merge_clusters");
  } catch (...) {
    return fail(PARK_EHIP, "park_merge_clusters: internal error");
  }
}

park_status park_permute_rows(const park_shape* shape, const void* x, const int32_t* perm, void* out, void* stream) {
  try {
    park::Dims s;
    PARK_TRY(check_shape(shape, &s));
    PARK_TRY(check_ptr(x, "x", 16));
    PARK_TRY(check_ptr(perm, "perm", 4));
    PARK_TRY(check_ptr(out, "out", 16));
    if (x == out) return fail(PARK_EINVAL, "x and out must not overlap");
    return hip_check(park::launch_permute(s, x, perm, out, 0, (hipStream_t)stream), "park_permute_rows");
  } catch (...) {
    return fail(PARK_EHIP, "park_permute_rows: internal error");
  }
}

park_status park_unpermute_rows(const park_shape* shape, const void* x, const int32_t* perm, void* out, void* stream) {
  try {
    park::Dims s;
    PARK_TRY(check_shape(shape, &s));
    PARK_TRY(check_ptr(x, "x", 16));
    PARK_TRY(check_ptr(perm, "perm", 4));
    PARK_TRY(check_ptr(out, "out", 16));
    if (x == out) return fail(PARK_EINVAL, "x and out must not overlap");
    return hip_check(park::launch_permute(s, x, perm, out, 1, (hipStream_t)stream), "park_unpermute_rows");
  } catch (...) {
    return fail(PARK_EHIP, "park_unpermute_rows: internal error");
  }
}

park_status park_forward(const park_shape* shape, const void* q, const void* k, const void* v, void* out,
                         const park_params* params, float* q_centroids, float* k_centroids,
                         const park_forward_outputs* outputs, void* ws, size_t ws_bytes, void* stream) {
  try {
    park::Dims s;
    PARK_TRY(check_shape(shape, &s));
    PARK_TRY(check_params(s, params, true));
    PARK_TRY(check_ptr(q, "q", 16));
    PARK_TRY(check_ptr(k, "k", 16));
    PARK_TRY(check_ptr(v, "v", 16));
    PARK_TRY(check_ptr(out, "out", 16));
    PARK_TRY(check_ptr(q_centroids, "q_centroids", 4));
    PARK_TRY(check_ptr(k_centroids, "k_centroids", 4));
    park_forward_outputs o;
    std::memset(&o, 0, sizeof(o));
    if (outputs) o = *outputs;
    const void* opt[] = {o.metric, o.q_labels, o.q_perm, o.q_offsets, o.k_labels, o.k_perm, o.k_offsets,
                         o.map, o.counts, o.cols, o.lse, o.status};
    for (const void* ptr : opt)
      if (ptr && !aligned(ptr, 4)) return fail(PARK_EINVAL, "forward outputs must be 4-byte aligned");
    if (o.sel_keys && !aligned(o.sel_keys, 8)) return fail(PARK_EINVAL, "sel_keys must be 8-byte aligned");
    if (o.stats && !aligned(o.stats, 8)) return fail(PARK_EINVAL, "stats must be 8-byte aligned");
    const park_params& p = *params;
    const bool subset = p.init == PARK_INIT_SUBSET;
    if (subset && (!o.q_labels || !o.k_labels))
      return fail(PARK_EINVAL, "PARK_INIT_SUBSET needs outputs->q_labels and outputs->k_labels (the previous labels)");
    PARK_TRY(check_ws(ws, ws_bytes, forward_ws_bytes(s, p)));
    Carver cv(ws);
    ForwardWs w = plan_forward(cv, s, p);
    hipStream_t st = (hipStream_t)stream;
    float* M = o.metric ? o.metric : w.metric;
    int32_t* ql = o.q_labels ? o.q_labels : w.q_labels;
    int32_t* qp = o.q_perm ? o.q_perm : w.q_perm;
    int32_t* qo = o.q_offsets ? o.q_offsets : w.q_offsets;
    int32_t* kl = o.k_labels ? o.k_labels : w.k_labels;
    int32_t* kp = o.k_perm ? o.k_perm : w.k_perm;
    int32_t* ko = o.k_offsets ? o.k_offsets : w.k_offsets;
    float* map = o.map ? o.map : w.map;
    int32_t* counts = o.counts ? o.counts : w.counts;
    int32_t* cols = o.cols ? o.cols : w.cols;
    int64_t* sk = o.sel_keys ? o.sel_keys : w.sel_keys;
    const float scale = resolve_scale(p.scale, s.D);
    const bool qrkc = p.kmetric == PARK_QRKC;

    hipError_t e = hipSuccess;
    if (qrkc) e = park::launch_metric(s, q, M, w.mt.partial, st);
    if (e == hipSuccess && p.init == PARK_INIT_KMEANSPP) {
      // both sides seeded in one launch (one workgroup per head and side)
      const park::KppArgs a[2] = {kpp_args(q, nullptr, p.cq, PARK_SIDE_Q, q_centroids, w.qc),
                                  kpp_args(k, qrkc ? M : nullptr, p.ck, PARK_SIDE_K, k_centroids, w.kc)};
      e = park::launch_kpp(s, a, 2, p.seed, o.status, st);
    }
    if (e == hipSuccess) {
      // query side on the helper stream, key side on the caller's, joined before the map
      std::unique_lock<std::mutex> lock;
      SideStream* ss = nullptr;
      e = side_stream(lock, &ss);
      if (e == hipSuccess) e = hipEventRecord(ss->fork, st);
      if (e == hipSuccess) e = hipStreamWaitEvent(ss->stream, ss->fork, 0);
      const int stride = subset ? p.subset_stride : 1, phase = subset ? p.subset_phase : 0;
      if (e == hipSuccess)
        e = run_lloyd(s, q, nullptr, p.cq, p.iters, q_centroids, ql, qp, qo, w.qc, ss->stream, stride, phase);
      if (e == hipSuccess) e = hipEventRecord(ss->join, ss->stream);
      if (e == hipSuccess)
        e = run_lloyd(s, k, qrkc ? M : nullptr, p.ck, p.iters, k_centroids, kl, kp, ko, w.kc, st, stride, phase);
      if (e == hipSuccess) e = hipStreamWaitEvent(st, ss->join, 0);
    }
    if (e == hipSuccess)
      e = park::launch_pama(s, q, qp, qo, p.cq, k_centroids, ko, p.ck, scale, map, w.mw.khat, w.mw.logn,
                            w.mw.chunk_base, w.mw.partial, st);
    if (e == hipSuccess)
      e = park::launch_select_topp(map, s.H, p.cq, p.ck, ko, p.p, o.mask, counts, cols, sk, st);
    if (e == hipSuccess)
      e = park::launch_sparse_attn(s, q, k, v, qp, qo, p.cq, kp, ko, p.ck, counts, cols, nullptr, scale, out, o.lse,
                                   w.aw.tile_base, w.aw.runs, reinterpret_cast<int64_t*>(o.stats), st);
    return hip_check(e, "park_forward");
  } catch (...) {
    return fail(PARK_EHIP, "park_forward: internal error");
  }
}

}  // extern "C"
