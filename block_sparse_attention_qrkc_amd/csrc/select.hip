// Row-wise cuts of the block map: top-p (PARK page, Table 1 caption: top-p retrieval at p = 0.9)
// and top-k at a fixed retrieval ratio (Table 10 caption: rho = 0.1; k = ceil(rho * C_ne) of the
// head's C_ne non-empty key blocks, at least 1).
// One workgroup per (row, head): bitonic sort of 64-bit keys (importance bits, complemented index;
// empty key blocks get key 0 and sort last) in LDS; top-p takes fp64 prefix sums in sorted order
// and the shortest prefix reaching p, top-k the first k; then an ordered compaction of the kept
// cluster ids.
#include "park_common.h"
#include "park_internal.h"

namespace park {

namespace {

constexpr int kSelThreads = 256;

// rho < 0: top-p with p; rho >= 0: top-k at ratio rho
__global__ __launch_bounds__(kSelThreads) void select_topp_kernel(const float* __restrict__ map, int cq, int ck,
                                                                  const int32_t* __restrict__ k_off, double p,
                                                                  double rho,
                                                                  uint8_t* __restrict__ mask,
                                                                  int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ cols,
                                                                  int64_t* __restrict__ sel_keys) {
  __shared__ uint64_t keys[kMaxClusters];
  __shared__ uint8_t keep[kMaxClusters];
  __shared__ double dscratch[17];
  __shared__ int iscratch[17];
  __shared__ int64_t lscratch[17];
  __shared__ int kstar;
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const float* row = map + ((int64_t)h * cq + i) * ck;
  const int32_t* ko = k_off + (int64_t)h * (ck + 1);
  int P2 = 1;
  while (P2 < ck) P2 <<= 1;

  const bool topk = rho >= 0.0;
  int any_pos = 0, live = 0;
  for (int j = tid; j < P2; j += kSelThreads) {
    uint64_t key = 0;
    if (j < ck && ko[j + 1] > ko[j]) {
      uint32_t bits = __float_as_uint(row[j]);
      if (bits & 0x80000000u) bits = 0;  // -0 (or a negative) counts as zero importance
      if (bits) any_pos = 1;
      ++live;
      key = ((uint64_t)bits << 32) | (uint64_t)(~(uint32_t)j);
    }
    keys[j] = key;
    if (j < ck) keep[j] = 0;
  }
  if (tid == 0) kstar = 0x7FFFFFFF;
  any_pos = __syncthreads_or(any_pos);
  int n_live = 0;
  if (topk) {
    int tot;
    (void)block_exclusive_scan(live, iscratch, &tot);
    n_live = tot;
  }

  if (any_pos && (topk || p < 1.0)) {
    // descending sort: larger importance first, equal importance -> lower index first
    for (int k = 2; k <= P2; k <<= 1) {
      for (int jj = k >> 1; jj > 0; jj >>= 1) {
        for (int idx = tid; idx < P2; idx += kSelThreads) {
          const int ixj = idx ^ jj;
          if (ixj > idx) {
            const uint64_t a = keys[idx], b = keys[ixj];
            const bool up = (idx & k) == 0;
            if ((a < b) == up) {
              keys[idx] = b;
              keys[ixj] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    if (topk) {
      // the first k sorted entries (all of them non-empty key blocks)
      int k = (int)ceil(rho * (double)n_live - 1e-9);
      k = k < 1 ? 1 : (k > n_live ? n_live : k);
      for (int e = tid; e < k; e += kSelThreads) keep[~(uint32_t)(keys[e] & 0xFFFFFFFFu)] = 1;
    } else {
    // fp64 prefix sums in sorted order: thread t owns sorted positions [t*per, t*per + per)
    const int per = (P2 + kSelThreads - 1) / kSelThreads;
    const int b0 = tid * per;
    double local = 0.0;
    for (int e = 0; e < per; ++e)
      if (b0 + e < P2) local += (double)__uint_as_float((uint32_t)(keys[b0 + e] >> 32));
    double total;
    double run = block_exclusive_scan(local, dscratch, &total);
    for (int e = 0; e < per; ++e) {
      if (b0 + e < P2) {
        run += (double)__uint_as_float((uint32_t)(keys[b0 + e] >> 32));
        if (run >= p) {
          atomicMin(&kstar, b0 + e);
          break;
        }
      }
    }
    __syncthreads();
    const int ks = kstar;
    if (ks != 0x7FFFFFFF) {
      for (int e = tid; e <= ks; e += kSelThreads) keep[~(uint32_t)(keys[e] & 0xFFFFFFFFu)] = 1;
    } else {
      for (int j = tid; j < ck; j += kSelThreads) keep[j] = row[j] > 0.f;
    }
    }
  } else if (any_pos) {
    // p >= 1: every non-empty key cluster
    for (int j = tid; j < ck; j += kSelThreads) keep[j] = 1;
  }
  __syncthreads();
  // never keep empty key clusters; ordered compaction
  const int per = (ck + kSelThreads - 1) / kSelThreads;
  const int j0 = tid * per;
  int local = 0;
  int64_t lkeys = 0;
  for (int e = 0; e < per; ++e) {
    const int j = j0 + e;
    if (j < ck) {
      const int n = ko[j + 1] - ko[j];
      if (n == 0) keep[j] = 0;
      if (keep[j]) {
        ++local;
        lkeys += n;
      }
    }
  }
  int total;
  int pos = block_exclusive_scan(local, iscratch, &total);
  int64_t ktotal;
  (void)block_exclusive_scan(lkeys, lscratch, &ktotal);
  int32_t* crow = cols + ((int64_t)h * cq + i) * ck;
  uint8_t* mrow = mask ? mask + ((int64_t)h * cq + i) * ck : nullptr;
  for (int e = 0; e < per; ++e) {
    const int j = j0 + e;
    if (j < ck) {
      if (keep[j]) crow[pos++] = j;
      if (mrow) mrow[j] = keep[j];
    }
  }
  if (tid == 0) {
    counts[(int64_t)h * cq + i] = total;
    if (sel_keys) sel_keys[(int64_t)h * cq + i] = ktotal;
  }
}

}  // namespace

hipError_t launch_select_topp(const float* map, int64_t H, int cq, int ck, const int32_t* k_offsets, double p,
                              uint8_t* mask, int32_t* counts, int32_t* cols, int64_t* sel_keys, hipStream_t st) {
  select_topp_kernel<<<dim3((unsigned)cq, (unsigned)H), kSelThreads, 0, st>>>(map, cq, ck, k_offsets, p, -1.0, mask,
                                                                               counts, cols, sel_keys);
  return hipGetLastError();
}

hipError_t launch_select_topk(const float* map, int64_t H, int cq, int ck, const int32_t* k_offsets, double rho,
                              uint8_t* mask, int32_t* counts, int32_t* cols, int64_t* sel_keys, hipStream_t st) {
  select_topp_kernel<<<dim3((unsigned)cq, (unsigned)H), kSelThreads, 0, st>>>(map, cq, ck, k_offsets, 1.0, rho, mask,
                                                                               counts, cols, sel_keys);
  return hipGetLastError();
}

}  // namespace park
