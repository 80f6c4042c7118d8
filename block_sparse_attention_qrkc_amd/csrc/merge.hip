// Tile-aware merging of query clusters (HyperVAttention page, abstract: merging clusters that lowers
// the CTA-aligned execution cost fills idle tile capacity; the merged queries attend to the union of
// the selections).
//
// Cost of a group of n queries whose selected key clusters hold L keys: ceil(n / bm) * L (its tiles
// of bm queries, each running over every selected key). Parallel agglomeration: every round each
// group proposes the partner of largest positive gain cost(a) + cost(b) - cost(a u b), ties to the
// lower index, and groups that propose each other merge into the lower index; rounds end when no
// pair gains. The gain is symmetric, so the pair of largest gain always proposes itself and every
// round that can merge does.
//
// merge_decide: one work-group per head; selections are bitsets over the key clusters (workspace),
// sizes and group state live in LDS. merge_apply: one work-group per (cluster, head) copies the
// cluster's queries to their place in the merged order.
#include "park_common.h"
#include "park_internal.h"

namespace park {

namespace {

constexpr int kMergeThreads = 1024;

__device__ __forceinline__ int64_t tile_cost(int64_t n, int64_t keys, int bm) { return ((n + bm - 1) / bm) * keys; }

// sum of the key-cluster sizes over the set bits of a & b
__device__ __forceinline__ int64_t weighted_and(const uint32_t* __restrict__ a, const uint32_t* __restrict__ b,
                                                int W, const int* __restrict__ nk) {
  int64_t s = 0;
  for (int w = 0; w < W; ++w) {
    uint32_t m = a[w] & b[w];
    while (m) {
      const int j = __ffs(m) - 1;
      s += nk[w * 32 + j];
      m &= m - 1;
    }
  }
  return s;
}

// Per head: the merge decisions, then the layout of the merged clustering.
//   bits   [H, cq, W] uint32 workspace (W = ceil(ck / 32))
//   dst    [H, cq] int32 workspace: first merged position of each cluster's queries
//   group  [H, cq]: merged group (slot) of each cluster; m_offsets [H, cq + 1], m_counts [H, cq],
//   m_cols [H, cq, ck] (ascending), as a query clustering with cq slots (slots past the groups empty)
__global__ __launch_bounds__(kMergeThreads) void merge_decide(const int32_t* __restrict__ q_offsets,
                                                              const int32_t* __restrict__ k_offsets,
                                                              const int32_t* __restrict__ counts,
                                                              const int32_t* __restrict__ cols, int cq, int ck,
                                                              int bm, uint32_t* __restrict__ bits,
                                                              int32_t* __restrict__ dst, int32_t* __restrict__ group,
                                                              int32_t* __restrict__ m_offsets,
                                                              int32_t* __restrict__ m_counts,
                                                              int32_t* __restrict__ m_cols) {
  __shared__ int nk[kMaxClusters];       // key-cluster sizes
  __shared__ int nq[kMaxClusters];       // queries of the group rooted at i (of cluster i at first)
  __shared__ int64_t gl[kMaxClusters];   // keys the group rooted at i selects
  __shared__ int parent[kMaxClusters];   // parent[i] == i: i is a root
  __shared__ int best[kMaxClusters];     // proposal of root i this round (-1: none)
  __shared__ unsigned long long bkey[kMaxClusters];  // (gain << 12) | (4095 - partner), 0: none
  __shared__ int slot[kMaxClusters];     // merged slot of root i
  __shared__ int gq[kMaxClusters];       // queries of slot g
  __shared__ int scratch[17];
  __shared__ int merged;
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int W = (ck + 31) / 32;
  const int32_t* qo = q_offsets + (int64_t)h * (cq + 1);
  const int32_t* ko = k_offsets + (int64_t)h * (ck + 1);
  uint32_t* B = bits + (int64_t)h * cq * W;
  for (int j = tid; j < ck; j += kMergeThreads) nk[j] = max(ko[j + 1] - ko[j], 0);
  for (int i = tid; i < cq; i += kMergeThreads) {
    nq[i] = max(qo[i + 1] - qo[i], 0);
    parent[i] = i;
    for (int w = 0; w < W; ++w) B[(int64_t)i * W + w] = 0u;
  }
  __syncthreads();
  // selection bitsets of the non-empty query clusters (an empty one selects nothing)
  for (int i = tid; i < cq; i += kMergeThreads) {
    int64_t L = 0;
    if (nq[i] > 0) {
      int c = counts[(int64_t)h * cq + i];
      c = c < 0 ? 0 : (c > ck ? ck : c);
      const int32_t* row = cols + ((int64_t)h * cq + i) * ck;
      for (int m = 0; m < c; ++m) {
        const int j = row[m];
        if (j < 0 || j >= ck) continue;
        const uint32_t bit = 1u << (j & 31);
        uint32_t* wd = B + (int64_t)i * W + (j >> 5);
        if (!(*wd & bit)) {
          *wd |= bit;
          L += nk[j];
        }
      }
    }
    gl[i] = L;
  }
  __syncthreads();
  for (;;) {
    // proposals, one pair (a < b) of non-empty roots per thread at a time: each side keeps its
    // largest positive gain, ties to the lower partner, by a 64-bit max on (gain, 4095 - partner)
    // (gains stay below 2^50: at most N^2 with N < 2^24; partners below 2048)
    for (int i = tid; i < cq; i += kMergeThreads) bkey[i] = 0ull;
    if (tid == 0) merged = 0;
    __syncthreads();
    for (int64_t e = tid; e < (int64_t)cq * cq; e += kMergeThreads) {
      const int a = (int)(e / cq), b = (int)(e % cq);
      if (b <= a || parent[a] != a || parent[b] != b || nq[a] == 0 || nq[b] == 0) continue;
      const int64_t un = gl[a] + gl[b] - weighted_and(B + (int64_t)a * W, B + (int64_t)b * W, W, nk);
      const int64_t g = tile_cost(nq[a], gl[a], bm) + tile_cost(nq[b], gl[b], bm) -
                        tile_cost((int64_t)nq[a] + nq[b], un, bm);
      if (g > 0) {
        atomicMax(&bkey[a], ((unsigned long long)g << 12) | (unsigned long long)(4095 - b));
        atomicMax(&bkey[b], ((unsigned long long)g << 12) | (unsigned long long)(4095 - a));
      }
    }
    __syncthreads();
    for (int i = tid; i < cq; i += kMergeThreads) best[i] = bkey[i] ? 4095 - (int)(bkey[i] & 4095ull) : -1;
    __syncthreads();
    // mutual proposals merge into the lower index (pairs are disjoint: one proposal per root)
    for (int a = tid; a < cq; a += kMergeThreads) {
      const int b = best[a];
      if (b > a && best[b] == a) {
        const int64_t un = gl[a] + gl[b] - weighted_and(B + (int64_t)a * W, B + (int64_t)b * W, W, nk);
        for (int w = 0; w < W; ++w) B[(int64_t)a * W + w] |= B[(int64_t)b * W + w];
        nq[a] += nq[b];
        gl[a] = un;
        parent[b] = a;
        atomicAdd(&merged, 1);
      }
    }
    __syncthreads();
    if (merged == 0) break;
    __syncthreads();
  }
  // Roots in increasing order are the slots (slot of root i = number of roots below i; every thread
  // takes two consecutive clusters, cq <= 2048); each cluster's root by following parents (a merged
  // root points to the lower root it joined, so chains end at the group's lowest cluster).
  constexpr int PER = (kMaxClusters + kMergeThreads - 1) / kMergeThreads;
  int isroot[PER];
  int local = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = tid * PER + q;
    isroot[q] = i < cq && parent[i] == i;
    local += isroot[q];
  }
  int total;
  int run = block_exclusive_scan(local, scratch, &total);
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = tid * PER + q;
    if (isroot[q]) slot[i] = run++;
  }
  for (int g = tid; g < cq; g += kMergeThreads) gq[g] = 0;
  __syncthreads();
  for (int i = tid; i < cq; i += kMergeThreads) {
    int r = i;
    while (parent[r] != r) r = parent[r];
    group[(int64_t)h * cq + i] = slot[r];
    best[i] = r;  // reuse: root of cluster i
    if (r == i) gq[slot[i]] = nq[i];  // the root holds its group's query count
  }
  __syncthreads();
  // slot offsets (slots past the groups are empty) and each cluster's first merged position:
  // the clusters of a group follow each other in increasing index order
  if (tid == 0) {
    int acc = 0;
    for (int g = 0; g < cq; ++g) {
      m_offsets[(int64_t)h * (cq + 1) + g] = acc;
      acc += g < total ? gq[g] : 0;
    }
    m_offsets[(int64_t)h * (cq + 1) + cq] = acc;
    for (int g = 0; g < total; ++g) gq[g] = m_offsets[(int64_t)h * (cq + 1) + g];  // running cursor
    for (int i = 0; i < cq; ++i) {
      const int g = slot[best[i]];
      dst[(int64_t)h * cq + i] = gq[g];
      gq[g] += max(qo[i + 1] - qo[i], 0);
    }
  }
  // selections of the slots: the set bits of the root's bitset, ascending
  for (int i = tid; i < cq; i += kMergeThreads) {
    if (parent[i] != i) continue;
    const int g = slot[i];
    int32_t* out = m_cols + ((int64_t)h * cq + g) * ck;
    int c = 0;
    for (int w = 0; w < W; ++w) {
      uint32_t m = B[(int64_t)i * W + w];
      while (m) {
        out[c++] = w * 32 + __ffs(m) - 1;
        m &= m - 1;
      }
    }
    m_counts[(int64_t)h * cq + g] = c;
  }
  for (int g = total + tid; g < cq; g += kMergeThreads) m_counts[(int64_t)h * cq + g] = 0;
}

// One work-group per (cluster, head): the cluster's queries, in their clustered order, to their
// merged positions.
__global__ __launch_bounds__(256) void merge_apply(const int32_t* __restrict__ q_perm,
                                                   const int32_t* __restrict__ q_offsets, int64_t N, int cq,
                                                   const int32_t* __restrict__ dst, int32_t* __restrict__ m_perm) {
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int32_t* qo = q_offsets + (int64_t)h * (cq + 1);
  const int a = qo[i], b = qo[i + 1];
  const int d = dst[(int64_t)h * cq + i];
  for (int t = a + (int)threadIdx.x; t < b; t += 256) m_perm[(int64_t)h * N + d + (t - a)] = q_perm[(int64_t)h * N + t];
}

}  // namespace

size_t merge_ws_ints(int64_t H, int cq, int ck) { return (size_t)(H * cq) * (size_t)((ck + 31) / 32) + (size_t)(H * cq); }

hipError_t launch_merge(int64_t H, int64_t N, int cq, int ck, int bm, const int32_t* q_perm, const int32_t* q_offsets,
                        const int32_t* k_offsets, const int32_t* counts, const int32_t* cols, int32_t* group,
                        int32_t* m_perm, int32_t* m_offsets, int32_t* m_counts, int32_t* m_cols, int32_t* ws,
                        hipStream_t st) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws);
  int32_t* dst = ws + (size_t)(H * cq) * (size_t)((ck + 31) / 32);
  merge_decide<<<(unsigned)H, kMergeThreads, 0, st>>>(q_offsets, k_offsets, counts, cols, cq, ck, bm, bits, dst, group,
                                                     m_offsets, m_counts, m_cols);
  merge_apply<<<dim3((unsigned)cq, (unsigned)H), 256, 0, st>>>(q_perm, q_offsets, N, cq, dst, m_perm);
  return hipGetLastError();
}

}  // namespace park
