// Internal launcher interface between the C ABI layer and the kernels. Every launcher enqueues
// on `stream` and returns hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace park {

struct Dims {
  int64_t H, N, D;
  int bf16;  // 1: bf16 data, 0: fp32 data
};

constexpr int kMaxClusters = 2048;
constexpr int kMetricChunk = 4096;  // tokens per partial second-moment block
constexpr int kSortChunk = 1024;    // tokens per counting-sort chunk (one wave)
constexpr int kPamaRows = 256;      // query rows per PAMA work item
constexpr int kAttnBM = 128;        // query rows per attention work item

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int kpp_candidates(int64_t n, int c) {
  int64_t s = 8 * (int64_t)c;
  if (s < 4096) s = 4096;
  return (int)(s < n ? s : n);
}

// metric.hip
hipError_t launch_metric(const Dims& s, const void* q, float* metric, double* partial, hipStream_t st);
size_t metric_partial_count(const Dims& s);

// kmeans.hip
// Bits of the optional device status word (PARK_DEVSTATUS_* of the C ABI).
constexpr int kSeedTimeout = 1;  // a bounded wait of the cooperative k-means++ seeding gave up
// Failure-handling hook: while non-zero, every cooperative seeding launch starts with its failure
// flag raised, so each bounded wait gives up at once and the status bit is set.
extern std::atomic<int> g_force_seed_timeout;
struct KppArgs {
  const void* x;        // [H, N, D] data of the side
  const float* metric;  // [H, D, D] query metric (QRKC side) or NULL (Euclidean)
  int C;                // clusters
  int side;             // random stream id
  float* cent;          // [H, C, D] output centroids
  double* xx;           // workspace [H, S] candidate norms
  float* y;             // workspace [H, S, D] candidate metric products (QRKC side)
  double* psum;         // workspace [H, C, 16, 2] per-part sums of the cooperative seeding
  int* sync;            // workspace [H, C, 3] step flags of the cooperative seeding
};
// k-means++ seeding of one or two sides in a single launch.
// status (device, may be NULL): kSeedTimeout is or-ed in when a cooperative exchange timed out.
hipError_t launch_kpp(const Dims& s, const KppArgs* sides, int nsides, uint64_t seed, int* status, hipStream_t st);
// Fused Euclidean Lloyd step (bf16, D = 64 or 128, at most 128 clusters): labels of every point
// and the member means into cent (empty clusters keep theirs); the consumed form (g, b) is then
// recomputed by launch_update. fused_parts gives the work-groups per head (0: not applicable);
// psum holds H * parts * C * D doubles, pcnt H * parts * C ints.
constexpr int kFuseCUs = 256;      // work-groups per layer the split aims at (one per CU)
constexpr int kFuseMaxParts = 32;  // work-groups per head at most
int fused_parts(const Dims& s, int C);
hipError_t launch_lloyd_fused(const Dims& s, const void* x, int C, const void* g, const float* b, int32_t* labels,
                              double* psum, int32_t* pcnt, float* cent, hipStream_t st);
// Centroid means (do_update) and the consumed form (g, b) of the centroids for the next assignment.
hipError_t launch_update(const Dims& s, const void* x, int C, const int32_t* perm, const int32_t* offsets, float* cent,
                         int do_update, const float* metric, void* g, float* b, hipStream_t st);
// Assignment of the rows phase, phase + stride, ... (all rows by default); other labels untouched.
hipError_t launch_assign(const Dims& s, const void* x, int C, const void* g, const float* b, int32_t* labels,
                         hipStream_t st, int stride = 1, int phase = 0);
// Labels outside [0, C) become 0 (caller-provided labels of a subset update).
hipError_t launch_clamp_labels(const Dims& s, int C, int32_t* labels, hipStream_t st);
hipError_t launch_sort(const Dims& s, int C, const int32_t* labels, int32_t* table, int32_t* perm,
                       int32_t* offsets, hipStream_t st);
size_t sort_table_ints(const Dims& s, int C);

// pama.hip
hipError_t launch_pama(const Dims& s, const void* q, const int32_t* q_perm, const int32_t* q_offsets, int cq,
                       const float* k_cent, const int32_t* k_offsets, int ck, float scale, float* map,
                       void* khat, float* logn, int32_t* chunk_base, float* partial, hipStream_t st);
int64_t pama_max_chunks(const Dims& s, int cq);
// Block masses over every key (bf16 data): map[h, i, j] = mean over the rows of query cluster i of
// the softmax mass (over all nk keys) that falls on key cluster j. Workspace as launch_pama.
// CF estimator map: centroid rows [H, cq, D] bf16 against every key; part holds H * cf_chunks(s) * cq
// (reference, sum) pairs, off H * cq floats.
int64_t cf_chunks(const Dims& s);
hipError_t launch_cf_map(const Dims& s, const void* rows, const int32_t* q_offsets, int cq, const void* k,
                         const int32_t* k_perm, const int32_t* k_offsets, int ck, float scale, float* map, float* part,
                         float* off, hipStream_t st);
hipError_t launch_block_mass(const Dims& s, const void* q, const int32_t* q_perm, const int32_t* q_offsets, int cq,
                             const void* k, int64_t nk, const int32_t* k_perm, const int32_t* k_offsets, int ck,
                             float scale, float* map, int32_t* chunk_base, float* partial, hipStream_t st);
// bf16 centroid rows [H, C, D]; one row per non-empty cluster of q_offsets (perm, offsets).
hipError_t launch_centroid_queries(int64_t H, int C, int D, const float* cent, const int32_t* q_offsets, void* rows,
                                   int32_t* perm, int32_t* offsets, hipStream_t st);

// select.hip
hipError_t launch_select_topp(const float* map, int64_t H, int cq, int ck, const int32_t* k_offsets, double p,
                              uint8_t* mask, int32_t* counts, int32_t* cols, int64_t* sel_keys, hipStream_t st);
hipError_t launch_select_topk(const float* map, int64_t H, int cq, int ck, const int32_t* k_offsets, double rho,
                              uint8_t* mask, int32_t* counts, int32_t* cols, int64_t* sel_keys, hipStream_t st);
hipError_t launch_select_sip(const float* map, int64_t H, int cq, int ck, const int32_t* k_offsets, double rho,
                             uint64_t seed, uint8_t* mask, int32_t* counts, int32_t* cols, int64_t* sel_keys,
                             float* log_w, hipStream_t st);

// attn.hip
hipError_t launch_sparse_attn(const Dims& s, const void* q, const void* k, const void* v, const int32_t* q_perm,
                              const int32_t* q_offsets, int cq, const int32_t* k_perm, const int32_t* k_offsets,
                              int ck, const int32_t* counts, const int32_t* cols, const float* log_w, float scale,
                              void* out, float* lse, int32_t* tile_base, int32_t* runs, int64_t* stats,
                              hipStream_t st);
int64_t attn_max_tiles(const Dims& s, int cq);
// ints of the run workspace: per (head, query cluster) the runs of its selected keys (at most ck,
// three ints each) + [H, cq] run counts + [H, cq] key counts + [H, cq] non-empty selected blocks.
// stats (device, may be NULL): the eight int64 of park_stats.
size_t attn_run_ints(const Dims& s, int cq, int ck);

// merge.hip
// Tile-aware merging of query clusters (cost ceil(n / bm) * selected keys per group); outputs a
// query clustering with cq slots. Workspace: merge_ws_ints(H, cq, ck) int32.
size_t merge_ws_ints(int64_t H, int cq, int ck);
hipError_t launch_merge(int64_t H, int64_t N, int cq, int ck, int bm, const int32_t* q_perm, const int32_t* q_offsets,
                        const int32_t* k_offsets, const int32_t* counts, const int32_t* cols, int32_t* group,
                        int32_t* m_perm, int32_t* m_offsets, int32_t* m_counts, int32_t* m_cols, int32_t* ws,
                        hipStream_t st);

// permute.hip
hipError_t launch_permute(const Dims& s, const void* x, const int32_t* perm, void* out, int inverse,
                          hipStream_t st);

}  // namespace park
