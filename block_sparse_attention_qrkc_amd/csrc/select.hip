// Row-wise cuts of the block map: top-p (PARK page, Table 1 caption: top-p retrieval at p = 0.9),
// top-k at a fixed retrieval ratio (Table 10 caption: rho = 0.1; k = ceil(rho * C_ne) of the
// head's C_ne non-empty key blocks, at least 1), and sampling with inclusion-probability weighting
// (AB-Attention page, SIP paragraph) with the top-k budget as the expected number of blocks.
// One workgroup per (row, head): bitonic sort of 64-bit keys (importance bits, complemented index;
// empty key blocks get key 0 and sort last) in LDS; top-p takes fp64 prefix sums in sorted order
// and the shortest prefix reaching p, top-k the first k, SIP water-fills the inclusion
// probabilities over the sorted importances and draws one uniform per block; then an ordered
// compaction of the kept cluster ids.
#include "park_common.h"
#include "park_internal.h"

namespace park {

namespace {

constexpr int kSelThreads = 256;
constexpr int kSelTopP = 0, kSelTopK = 1, kSelSip = 2;
constexpr uint64_t kSipStream = 2;  // stream id of the block sampling (k-means++ uses 0 and 1)

// mode kSelTopP: top-p with p; kSelTopK: top-k at ratio rho; kSelSip: sampling with the top-k
// budget at ratio rho, drawing from the counter stream of `seed`, log weights into log_w
__global__ __launch_bounds__(kSelThreads) void select_topp_kernel(const float* __restrict__ map, int cq, int ck,
                                                                  const int32_t* __restrict__ k_off, int mode,
                                                                  double p, double rho, uint64_t seed,
                                                                  uint8_t* __restrict__ mask,
                                                                  int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ cols,
                                                                  int64_t* __restrict__ sel_keys,
                                                                  float* __restrict__ log_w) {
  __shared__ uint64_t keys[kMaxClusters];
  __shared__ uint8_t keep[kMaxClusters];
  __shared__ float lw[kMaxClusters];
  __shared__ double dscratch[17];
  __shared__ int iscratch[17];
  __shared__ int64_t lscratch[17];
  __shared__ int kstar;
  __shared__ double kappa;
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const float* row = map + ((int64_t)h * cq + i) * ck;
  const int32_t* ko = k_off + (int64_t)h * (ck + 1);
  int P2 = 1;
  while (P2 < ck) P2 <<= 1;

  const bool topk = mode != kSelTopP;  // top-k and SIP share the budget k and the sort
  int any_pos = 0, live = 0, npos = 0;
  for (int j = tid; j < P2; j += kSelThreads) {
    uint64_t key = 0;
    if (j < ck && ko[j + 1] > ko[j]) {
      uint32_t bits = __float_as_uint(row[j]);
      if (bits & 0x80000000u) bits = 0;  // -0 (or a negative) counts as zero importance
      if (bits) {
        any_pos = 1;
        ++npos;
      }
      ++live;
      key = ((uint64_t)bits << 32) | (uint64_t)(~(uint32_t)j);
    }
    keys[j] = key;
    if (j < ck) {
      keep[j] = 0;
      lw[j] = 0.f;
    }
  }
  if (tid == 0) kstar = 0x7FFFFFFF;
  any_pos = __syncthreads_or(any_pos);
  int n_live = 0, n_pos = 0;
  if (topk) {
    int tot;
    (void)block_exclusive_scan(live, iscratch, &tot);
    n_live = tot;
    (void)block_exclusive_scan(npos, iscratch, &tot);
    n_pos = tot;
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
    int k = (int)ceil(rho * (double)n_live - 1e-9);
    k = k < 1 ? 1 : (k > n_live ? n_live : k);
    if (mode == kSelTopK) {
      // the first k sorted entries (all of them non-empty key blocks)
      for (int e = tid; e < k; e += kSelThreads) keep[~(uint32_t)(keys[e] & 0xFFFFFFFFu)] = 1;
    } else if (mode == kSelSip) {
      // inclusion probabilities pi = min(1, kappa a) summing to k over the n_pos positive blocks
      // (sorted positions 0 .. n_pos-1): the t largest are capped at 1 for the smallest t with
      // (k - t) a_t <= sum_{e >= t} a_e, and then kappa = (k - t) / sum_{e >= t} a_e. t = k - 1
      // always qualifies (exactly: its rest includes a_t), so rounding cannot leave t undecided.
      int tcap = n_pos;  // k >= n_pos: every positive block has pi = 1
      double kap = 0.0;
      if (k < n_pos) {
        const int per = (P2 + kSelThreads - 1) / kSelThreads;
        const int b0 = tid * per;
        double local = 0.0;
        for (int e = 0; e < per; ++e)
          if (b0 + e < P2) local += (double)__uint_as_float((uint32_t)(keys[b0 + e] >> 32));
        double total;
        double run = block_exclusive_scan(local, dscratch, &total);
        int my_t = -1;
        double my_kap = 0.0;
        for (int e = 0; e < per; ++e) {
          const int t = b0 + e;
          if (t >= n_pos) break;
          const double a = (double)__uint_as_float((uint32_t)(keys[t] >> 32));
          const double rest = total - run;
          if (t == k - 1 || (double)(k - t) * a <= rest) {
            my_t = t;
            my_kap = (double)(k - t) / rest;
            atomicMin(&kstar, t);
            break;
          }
          run += a;
        }
        __syncthreads();
        if (my_t == kstar) kappa = my_kap;  // exactly one thread holds the smallest t
        __syncthreads();
        tcap = kstar;
        kap = kappa;
      }
      for (int e = tid; e < n_pos; e += kSelThreads) {
        const double a = (double)__uint_as_float((uint32_t)(keys[e] >> 32));
        const int j = (int)~(uint32_t)(keys[e] & 0xFFFFFFFFu);
        const double pi = e < tcap ? 1.0 : fmin(1.0, kap * a);
        const uint64_t key = seed ^ ((uint64_t)h << 32) ^ (kSipStream << 24) ^ ((uint64_t)i * (uint64_t)ck + (uint64_t)j);
        const double u = (double)(splitmix_first(key) >> 11) * 0x1.0p-53;
        if (u < pi) {
          keep[j] = 1;
          lw[j] = pi < 1.0 ? (float)(-log(pi)) : 0.f;
        }
      }
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
  float* lrow = log_w ? log_w + ((int64_t)h * cq + i) * ck : nullptr;
  for (int e = 0; e < per; ++e) {
    const int j = j0 + e;
    if (j < ck) {
      if (keep[j]) crow[pos++] = j;
      if (mrow) mrow[j] = keep[j];
      if (lrow) lrow[j] = keep[j] ? lw[j] : 0.f;
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
  select_topp_kernel<<<dim3((unsigned)cq, (unsigned)H), kSelThreads, 0, st>>>(
      map, cq, ck, k_offsets, kSelTopP, p, 0.0, 0, mask, counts, cols, sel_keys, nullptr);
  return hipGetLastError();
}

hipError_t launch_select_topk(const float* map, int64_t H, int cq, int ck, const int32_t* k_offsets, double rho,
                              uint8_t* mask, int32_t* counts, int32_t* cols, int64_t* sel_keys, hipStream_t st) {
  select_topp_kernel<<<dim3((unsigned)cq, (unsigned)H), kSelThreads, 0, st>>>(
      map, cq, ck, k_offsets, kSelTopK, 1.0, rho, 0, mask, counts, cols, sel_keys, nullptr);
  return hipGetLastError();
}

hipError_t launch_select_sip(const float* map, int64_t H, int cq, int ck, const int32_t* k_offsets, double rho,
                             uint64_t seed, uint8_t* mask, int32_t* counts, int32_t* cols, int64_t* sel_keys,
                             float* log_w, hipStream_t st) {
  select_topp_kernel<<<dim3((unsigned)cq, (unsigned)H), kSelThreads, 0, st>>>(
      map, cq, ck, k_offsets, kSelSip, 1.0, rho, seed, mask, counts, cols, sel_keys, log_w);
  return hipGetLastError();
}

}  // namespace park
