/*
 * park.h - C ABI of the MI355X (gfx950) PARK block retrieval + block-sparse attention library.
 *
 * Method: "PARK: Accurate Block Retrieval for Sparse Attention in Video Diffusion Transformers".
 * Per attention head: cluster queries with Euclidean K-means and keys with K-means under a metric
 * derived from the current queries (QRKC), order tokens cluster by cluster, build the PAMA
 * block-importance map (every query's softmax over the key centroids, averaged within its query
 * cluster), cut each map row at top-p cumulative mass, and run attention only over the selected
 * (query cluster, key cluster) pairs.
 *
 * Conventions for every entry point:
 *   - Tensors are device pointers to dense row-major arrays; X of a park_shape is [heads, n, d].
 *   - The caller owns every buffer, including the workspace (size from park_workspace_bytes).
 *     The library allocates no device memory and keeps no state between calls.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null stream).
 *   - Arguments are validated on the host before anything is enqueued; on error nothing is
 *     enqueued and park_last_error() holds a message. Device faults surface at the caller's next
 *     synchronisation. No C++ exception crosses this interface.
 *   - Supported: d in {64, 128}; dtype PARK_F32 or PARK_BF16; 1 <= clusters <= min(n, 2048);
 *     1 <= n < 2^24; all pointers 16-byte aligned.
 *   - Ties and reductions are resolved in a fixed order: results are deterministic run to run.
 */
#ifndef PARK_H
#define PARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PARK_OK = 0,
  PARK_EINVAL = 1,       /* bad argument (null pointer, size out of range, misalignment) */
  PARK_EUNSUPPORTED = 2, /* valid but not supported here (d, dtype) */
  PARK_EWORKSPACE = 3,   /* workspace smaller than park_workspace_bytes() */
  PARK_EHIP = 4          /* a HIP launch or runtime call failed */
} park_status;

typedef enum { PARK_F32 = 0, PARK_BF16 = 1 } park_dtype;
typedef enum { PARK_EUCLID = 0, PARK_QRKC = 1 } park_metric;
typedef enum { PARK_INIT_KMEANSPP = 0, PARK_INIT_WARM = 1, PARK_INIT_SUBSET = 2 } park_init;
typedef enum { PARK_SIDE_Q = 0, PARK_SIDE_K = 1 } park_side;
/* Query/key representations of a block map (PARK, thelatestinai.com page, Table 1): F = full
 * (every original query or key), C = centroid. FC is the PAMA map. */
typedef enum { PARK_EST_FC = 0, PARK_EST_CC = 1, PARK_EST_CF = 2, PARK_EST_FF = 3 } park_estimator;

typedef struct {
  int64_t heads; /* independent attention heads */
  int64_t n;     /* tokens per head */
  int64_t d;     /* head dimension: 64 or 128 */
  int32_t dtype; /* park_dtype of Q, K, V and the attention output */
} park_shape;

typedef struct {
  int32_t cq;      /* query clusters (NQ on the PARK pages, Tables 7-8) */
  int32_t ck;      /* key clusters (NK) */
  int32_t iters;   /* Lloyd iterations per clustering, >= 1 for park_forward */
  double p;        /* top-p threshold, 0 < p <= 1 (PARK page, Table 1: p = 0.9) */
  float scale;     /* softmax scale; <= 0 selects 1/sqrt(d) */
  uint64_t seed;   /* k-means++ seed */
  int32_t kmetric; /* park_metric of the key clustering: PARK_QRKC (default) or PARK_EUCLID */
  int32_t init;    /* park_init: PARK_INIT_KMEANSPP, or PARK_INIT_WARM to start from the
                      centroids already in the caller's centroid buffers, or PARK_INIT_SUBSET: a
                      warm start that re-assigns only a subset of the tokens (see park_forward) */
  int32_t subset_stride; /* PARK_INIT_SUBSET: every subset_stride-th token is re-assigned, */
  int32_t subset_phase;  /* starting at token subset_phase (0 <= phase < stride); else unused */
} park_params;

/* Entry identifiers for park_workspace_bytes. */
enum {
  PARK_ENTRY_METRIC = 0,
  PARK_ENTRY_CLUSTER_Q = 1, /* park_cluster with cq clusters, Euclidean */
  PARK_ENTRY_CLUSTER_K = 2, /* park_cluster with ck clusters, metric kmetric */
  PARK_ENTRY_RETRIEVE_MAP = 3,
  PARK_ENTRY_SELECT_TOPP = 4,
  PARK_ENTRY_SPARSE_ATTN = 5,
  PARK_ENTRY_FORWARD = 6,
  PARK_ENTRY_ESTIMATOR = 7,  /* park_estimator_map, any mode */
  PARK_ENTRY_SPARSE_ATTN_WEIGHTED = 8,
  PARK_ENTRY_MERGE = 9 /* park_merge_clusters: shape->heads, params->cq, params->ck */
};

/* Workspace bytes an entry needs for this shape and these parameters (0 on invalid input). */
size_t park_workspace_bytes(int32_t entry, const park_shape* shape, const park_params* params);

/* Human-readable name of a status code (static string). */
const char* park_status_string(int32_t status);

/* Detail of the last error on the calling thread ("" when none). */
const char* park_last_error(void);

/* Library version string. */
const char* park_version(void);

/* Bits of the optional device status word (int32) that park_cluster and park_forward take. The
 * library only sets bits (atomic or), never clears them: the caller zeroes the word before the
 * calls it wants to check and reads it after synchronising. */
enum {
  /* a bounded wait of the cooperative k-means++ seeding gave up (a part of the launch did not
   * answer within ~30 ms): every later wait of that launch returned at once, so the seeded
   * centroids, and all that follows from them in this call, are not the seeding the draws define */
  PARK_DEVSTATUS_SEED_TIMEOUT = 1
};

/* Failure-handling hook for tests: while `on` is non-zero, every cooperative seeding launch of this
 * process starts with its failure flag raised, so each of its bounded waits gives up at once, the
 * launch ends normally with wrong centroids, and PARK_DEVSTATUS_SEED_TIMEOUT is set. Not for
 * production use. */
void park_debug_force_seed_timeout(int32_t on);

/*
 * QRKC key metric. PARK page, Figure 2 caption and abstract: keys are transformed with a metric
 * derived from the current queries so that keys with similar QK scores group together. Reading:
 * M_h = (1/n) sum_t q_t q_t^T, so (k - c)^T M (k - c) is the mean over the current queries of the
 * squared QK-score difference (q.k - q.c)^2.
 *   q      [heads, n, d] of shape->dtype
 *   metric [heads, d, d] float32 output (symmetric)
 */
park_status park_qrkc_metric(const park_shape* shape, const void* q, float* metric, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * K-means clustering of one token side (PARK page, Figure 2 caption: queries with Euclidean
 * K-means, keys with the query-derived metric).
 *   x          [heads, n, d] of shape->dtype: queries or keys
 *   metric     PARK_EUCLID, or PARK_QRKC with qmetric = [heads, d, d] float32 from
 *              park_qrkc_metric (NULL for PARK_EUCLID)
 *   n_clusters C, 1 <= C <= min(n, 2048)
 *   iters      Lloyd iterations (assign, then update) >= 0
 *   init       PARK_INIT_KMEANSPP: seeded k-means++ over the strided candidate rows
 *              floor(i*n/S), S = min(n, max(4096, 8C)), draws from the SplitMix64 counter stream
 *              (seed, head, side); PARK_INIT_WARM: start from the values in `centroids`
 *   side       park_side, selects the random stream
 *   centroids  [heads, C, d] float32, output (input too for PARK_INIT_WARM): after the last
 *              update each centroid is the mean of its members; empty clusters keep their value
 *   labels     [heads, n] int32: cluster of each token from the last assignment
 *   perm       [heads, n] int32: token at each cluster-ordered position (stable: tokens of one
 *              cluster keep their original order)
 *   offsets    [heads, C + 1] int32: cluster j occupies positions offsets[j] .. offsets[j+1]-1
 * Assignment: label(x) = argmin_j b_j - 2 x.g_j, lowest j on ties, with (g_j, b_j) the consumed
 * centroid: Euclidean g_j = c_j (bf16-rounded for bf16 data), b_j = |g_j|^2; QRKC g_j = M c_j
 * (fp32, then bf16 for bf16 data), b_j = c_j^T M c_j. With iters == 0 only the centroids are
 * written and labels/perm/offsets may be NULL.
 *   status     optional device int32 (NULL: not reported): PARK_DEVSTATUS_* bits are or-ed in
 *              when the seeding's cooperative exchange fails (see PARK_DEVSTATUS_SEED_TIMEOUT)
 */
park_status park_cluster(const park_shape* shape, const void* x, int32_t metric, const float* qmetric,
                         int32_t n_clusters, int32_t iters, int32_t init, uint64_t seed, int32_t side,
                         float* centroids, int32_t* labels, int32_t* perm, int32_t* offsets, int32_t* status,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * Subset update of a clustering between anchor steps (HyperVAttention page, abstract: hybrid
 * clustering runs the full clustering only at anchor steps and updates a subset of the tokens at
 * the steps in between). Reading of the subset: the tokens phase, phase + stride, phase + 2 stride,
 * ...; a caller that advances phase by one per denoising step refreshes every token once per stride
 * steps. Each of the `iters` iterations re-assigns the subset's tokens against the consumed form of
 * the current centroids (as park_cluster), keeps the other tokens' labels, and sets every centroid
 * to the mean of its members under the combined labels over the current values of all tokens
 * (empty clusters keep their value).
 *   x, metric, qmetric, n_clusters  as park_cluster
 *   iters      >= 1
 *   stride     >= 1 (1: every token, i.e. warm-started Lloyd iterations); 0 <= phase < stride
 *   centroids  [heads, C, d] float32, input and output (the previous step's centroids)
 *   labels     [heads, n] int32, input and output (the previous step's labels; values outside
 *              [0, C) are taken as cluster 0)
 *   perm, offsets  outputs as park_cluster
 * Workspace: park_workspace_bytes(PARK_ENTRY_CLUSTER_Q or _K, ...) as park_cluster.
 */
park_status park_cluster_subset(const park_shape* shape, const void* x, int32_t metric, const float* qmetric,
                                int32_t n_clusters, int32_t iters, int32_t stride, int32_t phase,
                                float* centroids, int32_t* labels, int32_t* perm, int32_t* offsets, void* ws,
                                size_t ws_bytes, void* stream);

/*
 * PAMA block-importance map (PARK page, Figure 2 caption and abstract: each original query keeps
 * its own softmax over the key centroids; the distributions are averaged within each query block).
 *   q            [heads, n, d] queries in original token order
 *   q_perm, q_offsets  query clustering from park_cluster (cq clusters)
 *   k_centroids  [heads, ck, d] float32 key centroids (bf16-rounded on use for bf16 data)
 *   k_offsets    [heads, ck + 1] key cluster offsets (sizes n_j)
 *   scale        softmax scale (<= 0 selects 1/sqrt(d))
 *   map          [heads, cq, ck] float32 output: A[i, j] = mean over queries t of block i of
 *                softmax_j(scale * q_t.c_j + ln n_j); empty key clusters get 0; empty query
 *                blocks give a zero row.
 */
park_status park_retrieve_map(const park_shape* shape, const void* q, const int32_t* q_perm,
                              const int32_t* q_offsets, int32_t cq, const float* k_centroids,
                              const int32_t* k_offsets, int32_t ck, float scale, float* map, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * Row-wise top-p cut of the map (PARK page, Table 1 caption: top-p block retrieval, p = 0.9).
 * Per row: order key clusters by importance (descending, ties to the lower index) and keep the
 * shortest prefix whose cumulative importance (summed in fp64) reaches p. p >= 1 keeps every
 * non-empty key cluster; a row whose total stays below p keeps every block with positive
 * importance; empty key clusters are never kept; an all-zero row keeps nothing.
 *   map       [heads, cq, ck] float32
 *   k_offsets [heads, ck + 1]
 *   mask      [heads, cq, ck] uint8 output (1 = kept), may be NULL
 *   counts    [heads, cq] int32 output: kept clusters per row
 *   cols      [heads, cq, ck] int32 output: kept cluster ids of row i in ascending order in
 *             cols[h, i, 0 .. counts[h, i]-1] (row-padded layout)
 *   sel_keys  [heads, cq] int64 output: keys row i attends to (sum of kept cluster sizes), may be NULL
 */
park_status park_select_topp(const float* map, int64_t heads, int32_t cq, int32_t ck,
                             const int32_t* k_offsets, double p, uint8_t* mask, int32_t* counts,
                             int32_t* cols, int64_t* sel_keys, void* stream);

/*
 * Block map under one of the four query/key representations of PARK Table 1 (thelatestinai.com
 * page; Table 4 compares the same four): row i is the mean over the queries of query cluster i of a
 * distribution over key clusters j:
 *   PARK_EST_FC  softmax_j(s q.c_j + ln n_j) of each original query (the PAMA map, as
 *                park_retrieve_map);
 *   PARK_EST_CC  the same for the query cluster's centroid instead of its queries;
 *   PARK_EST_CF  the softmax mass of the query centroid over all keys that falls on cluster j;
 *   PARK_EST_FF  the dense softmax mass of each original query that falls on cluster j (the exact
 *                block importance; N^2 d work per head).
 * Centroids enter as consumed by the matrix cores (bf16-rounded); CC, CF and FF need bf16 data
 * (PARK_EUNSUPPORTED otherwise). Arguments a mode does not read may be NULL:
 *   q, q_perm                  FC, FF        k, k_perm       CF, FF
 *   q_centroids [heads, cq, d] float32: CC, CF    k_centroids [heads, ck, d] float32: FC, CC
 *   q_offsets, k_offsets       every mode
 *   map        [heads, cq, ck] float32 output; an empty query cluster gets a zero row
 * Workspace: park_workspace_bytes(PARK_ENTRY_ESTIMATOR, shape, params with cq, ck).
 */
park_status park_estimator_map(const park_shape* shape, const void* q, const void* k, const int32_t* q_perm,
                               const int32_t* q_offsets, int32_t cq, const float* q_centroids,
                               const int32_t* k_perm, const int32_t* k_offsets, int32_t ck,
                               const float* k_centroids, int32_t mode, float scale, float* map, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * Row-wise top-k cut at a fixed retrieval ratio (PARK, thelatestinai.com page, Table 10 caption:
 * top-k block retrieval at rho = 0.1). Per head, k = ceil(rho * C_ne) of the C_ne non-empty key
 * clusters, clamped to [1, C_ne]; every row with positive importance keeps the k non-empty key
 * clusters of highest importance (ties to the lower index); a row without positive importance
 * (empty query cluster) keeps nothing. Arguments and outputs as park_select_topp; rho in [0, 1].
 */
park_status park_select_topk(const float* map, int64_t heads, int32_t cq, int32_t ck,
                             const int32_t* k_offsets, double rho, uint8_t* mask, int32_t* counts,
                             int32_t* cols, int64_t* sel_keys, void* stream);

/*
 * Sampling with inclusion-probability weighting (AB-Attention page, SIP paragraph: blocks are
 * sampled according to their estimated importance instead of being truncated, and each sampled
 * block is reweighted by the inverse of its inclusion probability, so that one sparse pass
 * estimates dense attention). Per row i of head h, with m = the top-k budget of park_select_topk
 * at ratio rho (the expected number of sampled blocks) and a_j the map row with empty key clusters
 * and non-positive entries at 0:
 *   pi_j = min(1, kappa a_j), kappa such that sum_j pi_j = m (every positive block has pi = 1 when
 *   m reaches their number; computed in fp64 from the fp32 map);
 *   u_j  = 53 high bits of the first SplitMix64 output seeded with
 *          seed ^ (h << 32) ^ (2 << 24) ^ (i * ck + j), times 2^-53;
 *   block j is kept iff u_j < pi_j, with log weight ln(1 / pi_j).
 * Arguments and outputs as park_select_topk, plus
 *   seed   the draws' seed (h is the head index within this call)
 *   log_w  [heads, cq, ck] float32 output: ln(1 / pi_j) for kept blocks, 0 elsewhere; pass it to
 *          park_sparse_attn_weighted together with counts and cols.
 */
park_status park_select_sip(const float* map, int64_t heads, int32_t cq, int32_t ck,
                            const int32_t* k_offsets, double rho, uint64_t seed, uint8_t* mask,
                            int32_t* counts, int32_t* cols, int64_t* sel_keys, float* log_w,
                            void* stream);

/*
 * Attention over the selected blocks only (PARK abstract: attention computed only within the
 * retrieved blocks). Every query of cluster i attends to the keys of the clusters in
 * cols[h, i, 0 .. counts[h, i]-1]; the softmax is renormalised over those keys.
 *   q, k, v    [heads, n, d] in original token order (fp32 data is rounded to bf16 on load;
 *              the products run on bf16 MFMA with fp32 accumulation)
 *   q_perm/q_offsets, k_perm/k_offsets  clusterings from park_cluster
 *   out        [heads, n, d] of shape->dtype, original token order
 *   lse        [heads, n] float32 log-sum-exp of the scaled scores over the selected keys, or NULL
 */
park_status park_sparse_attn(const park_shape* shape, const void* q, const void* k, const void* v,
                             const int32_t* q_perm, const int32_t* q_offsets, int32_t cq,
                             const int32_t* k_perm, const int32_t* k_offsets, int32_t ck,
                             const int32_t* counts, const int32_t* cols, float scale, void* out,
                             float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * park_sparse_attn without a workspace argument and without any allocation, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * it). Arguments, results and errors as park_sparse_attn. Its scratch (the per-cluster key runs and
 * the work order) is a static device array of 96 MiB on every GPU the library runs on, held until
 * the process ends; shapes that need more (park_workspace_bytes(PARK_ENTRY_SPARSE_ATTN, ...) above
 * 96 MiB, e.g. heads * cq * (3 ck + 7) * 4 bytes at large cq and ck) are refused with
 * PARK_EWORKSPACE before anything is enqueued. Every call overwrites what it reads of the scratch
 * before reading it (nothing needs clearing), and all calls on one GPU share it: calls that overlap
 * on one GPU (on different streams, or from different threads) race and must be serialised by the
 * caller.
 */
park_status park_sparse_attn_noalloc(const park_shape* shape, const void* q, const void* k, const void* v,
                                     const int32_t* q_perm, const int32_t* q_offsets, int32_t cq,
                                     const int32_t* k_perm, const int32_t* k_offsets, int32_t ck,
                                     const int32_t* counts, const int32_t* cols, float scale, void* out,
                                     float* lse, void* stream);

/*
 * Block-weighted attention over the selected blocks (AB-Attention page, SIP paragraph: sampled blocks
 * reweighted by the inverse of their inclusion probability). As park_sparse_attn, except that every
 * key of selected block j of row i enters the softmax with weight w = exp(log_w[h, i, j]):
 *   O_t = sum_{j in S} w_j sum_{k in j} e^{s q_t.k} v_k / sum_{j in S} w_j sum_{k in j} e^{s q_t.k},
 * i.e. each of those logits gains log_w[h, i, j]; lse is the log of the denominator.
 *   log_w  [heads, cq, ck] float32, read at the selected (i, j) only (from park_select_sip, or any
 *          finite log weights)
 * Workspace: park_workspace_bytes(PARK_ENTRY_SPARSE_ATTN_WEIGHTED, ...): the gather lists plus one
 * float32 logit offset per listed key, [heads, cq, n].
 */
park_status park_sparse_attn_weighted(const park_shape* shape, const void* q, const void* k, const void* v,
                                      const int32_t* q_perm, const int32_t* q_offsets, int32_t cq,
                                      const int32_t* k_perm, const int32_t* k_offsets, int32_t ck,
                                      const int32_t* counts, const int32_t* cols, const float* log_w,
                                      float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                                      void* stream);

/*
 * Tile-aware merging of query clusters (HyperVAttention page, abstract: merging clusters so as to
 * lower the CTA-aligned execution cost puts idle tile capacity to use, and the merged queries attend
 * to the union of the selections). Reading of the cost: a group of n queries whose selection holds
 * L keys costs ceil(n / bm) * L (its tiles of bm queries, each over every selected key). Parallel
 * agglomeration: each round every group proposes the partner of largest positive gain
 * cost(a) + cost(b) - cost(a u b) (ties to the lower index) and mutual proposals merge into the
 * lower index; the rounds end when no pair gains. Empty query clusters stay alone.
 *   q_perm [heads, n], q_offsets [heads, cq + 1]  the query clustering (park_cluster)
 *   k_offsets [heads, ck + 1]                     key cluster sizes
 *   counts [heads, cq], cols [heads, cq, ck]      the selection (park_select_topp / _topk)
 *   bm        queries per tile of the cost (the attention's work item: 384 for bf16 data)
 *   group     [heads, cq] output: merged slot of every query cluster
 *   m_perm, m_offsets, m_counts, m_cols  outputs, the merged groups as a query clustering and its
 *             selection with cq slots: slot g < G is the g-th group in increasing order of its
 *             lowest cluster, its queries cluster by cluster in increasing cluster order (each
 *             in q_perm order), its selection the ascending union; slots G .. cq - 1 are empty.
 *             Pass them to park_sparse_attn in place of q_perm, q_offsets, counts, cols.
 * Workspace: park_workspace_bytes(PARK_ENTRY_MERGE, ...): a selection bitset per cluster and head.
 * Cost: per round, cq^2 bitset intersections of ck / 32 words per head.
 */
park_status park_merge_clusters(int64_t heads, int64_t n, int32_t cq, int32_t ck, int32_t bm,
                                const int32_t* q_perm, const int32_t* q_offsets, const int32_t* k_offsets,
                                const int32_t* counts, const int32_t* cols, int32_t* group, int32_t* m_perm,
                                int32_t* m_offsets, int32_t* m_counts, int32_t* m_cols, void* ws,
                                size_t ws_bytes, void* stream);

/*
 * Cluster-contiguous gather and its inverse (the "Clustered" token ordering of PARK Tables 1/10).
 *   park_permute_rows:   out[h, p, :] = x[h, perm[h, p], :]
 *   park_unpermute_rows: out[h, perm[h, p], :] = x[h, p, :]
 * x and out are [heads, n, d] of shape->dtype and must not overlap.
 */
park_status park_permute_rows(const park_shape* shape, const void* x, const int32_t* perm, void* out,
                              void* stream);
park_status park_unpermute_rows(const park_shape* shape, const void* x, const int32_t* perm, void* out,
                                void* stream);

/* Optional outputs of park_forward (any field may be NULL; then the value stays in the workspace). */
typedef struct {
  float* metric;       /* [heads, d, d] */
  int32_t* q_labels;   /* [heads, n] */
  int32_t* q_perm;     /* [heads, n] */
  int32_t* q_offsets;  /* [heads, cq + 1] */
  int32_t* k_labels;   /* [heads, n] */
  int32_t* k_perm;     /* [heads, n] */
  int32_t* k_offsets;  /* [heads, ck + 1] */
  float* map;          /* [heads, cq, ck] */
  uint8_t* mask;       /* [heads, cq, ck] */
  int32_t* counts;     /* [heads, cq] */
  int32_t* cols;       /* [heads, cq, ck] */
  int64_t* sel_keys;   /* [heads, cq] */
  float* lse;          /* [heads, n] */
  int32_t* status;     /* one int32: PARK_DEVSTATUS_* bits or-ed in (see park_cluster) */
  struct park_stats* stats; /* selection and work statistics of the call (see park_stats) */
} park_forward_outputs;

/* Statistics of one park_forward call, written to device memory (totals over all heads). Token
 * density = pairs / (heads n^2); block density = blocks / live_blocks; the attention computes
 * 4 d FLOPs per pair and its matrix cores 4 d per padded pair. */
typedef struct park_stats {
  int64_t pairs;        /* selected (query, key) pairs: sum over query clusters of n_q(i) * L(i) */
  int64_t padded_pairs; /* pairs the matrix cores run: queries of a cluster rounded up to the 32 of a
                           wave, its selected keys to whole key tiles */
  int64_t blocks;       /* selected (query cluster, key cluster) blocks, both clusters non-empty */
  int64_t live_blocks;  /* non-empty query clusters x non-empty key clusters */
  int64_t work_items;   /* attention work items (tiles of up to 384 queries of one cluster) */
  int64_t tokens;       /* heads * n */
  int64_t reserved[2];
} park_stats;

/*
 * The whole path for one layer (PARK page, abstract: retrieve the important blocks of each head's
 * attention, then compute attention only within them; Figure 2 caption: Euclidean K-means on the
 * queries, K-means under the query-derived metric on the keys, the PAMA map, top-p): QRKC metric,
 * both clusterings, PAMA map, top-p, block-sparse attention. q_centroids [heads, cq, d] and
 * k_centroids [heads, ck, d] are caller state, outputs of every call and inputs of the warm modes:
 *   PARK_INIT_KMEANSPP  seeded k-means++ on both sides, then params->iters Lloyd iterations;
 *   PARK_INIT_WARM      params->iters Lloyd iterations from the caller's centroids (a later
 *                       denoising step reusing the previous step's clustering: PARK,
 *                       thelatestinai.com page, Table 9 recomputes the retrieval only at some steps);
 *   PARK_INIT_SUBSET    params->iters subset updates (park_cluster_subset) from the caller's
 *                       centroids and labels: outputs->q_labels and outputs->k_labels are then
 *                       required and hold the previous step's labels on entry.
 * The query side uses random stream PARK_SIDE_Q, the key side PARK_SIDE_K. The query-side
 * iterations run on a helper stream forked from and joined back into `stream` by events.
 */
park_status park_forward(const park_shape* shape, const void* q, const void* k, const void* v, void* out,
                         const park_params* params, float* q_centroids, float* k_centroids,
                         const park_forward_outputs* outputs, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PARK_H */
