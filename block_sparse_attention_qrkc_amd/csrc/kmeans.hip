// K-means for both token sides (PARK page, Figure 2 caption: queries under Euclidean K-means, keys
// under the query-derived metric M):
//   * k-means++ seeding (Arthur & Vassilvitskii 2007) over strided candidate rows, in fp64, with
//     draws from a SplitMix64 counter stream (Steele, Lea & Flood 2014);
//   * assignment: label = argmin_j b_j - 2 x.g_j on bf16 MFMA (fp32 accumulation), lowest j on ties;
//   * stable counting sort of the labels into cluster-contiguous order;
//   * update: fixed-order fp64 member means stored as fp32, followed by the consumed form (g, b)
//     of every centroid for the next assignment.
#include "park_common.h"
#include "park_internal.h"

namespace park {

namespace {

// ------------------------------------------------------------------------------------------------
// k-means++ seeding
// ------------------------------------------------------------------------------------------------

__device__ __forceinline__ uint64_t splitmix_first(uint64_t seed) {
  uint64_t z = seed + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ double kpp_uniform(uint64_t seed, int head, int side, int m) {
  const uint64_t key = seed ^ ((uint64_t)head << 32) ^ ((uint64_t)side << 24) ^ (uint64_t)m;
  return (double)(splitmix_first(key) >> 11) * 0x1.0p-53;
}

__device__ __forceinline__ int64_t cand_row(int i, int S, int64_t N) { return ((int64_t)i * N) / S; }

// Squared norm of every candidate: |x|^2 (Euclidean) or x^T M x (QRKC), fp64.
template <typename T, int D>
__global__ __launch_bounds__(256) void kpp_cand_norm(const T* __restrict__ X, int64_t N, int S,
                                                     const float* __restrict__ M, double* __restrict__ out) {
  const int h = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= S) return;
  const T* x = X + ((int64_t)h * N + cand_row(i, S, N)) * D;
  float xv[D];
#pragma unroll
  for (int a0 = 0; a0 < D; a0 += 8) load8_f32(x + a0, xv + a0);
  double s = 0.0;
  if (M == nullptr) {
#pragma unroll
    for (int a = 0; a < D; ++a) s += (double)xv[a] * (double)xv[a];
  } else {
    const float* Mh = M + (int64_t)h * D * D;
    for (int a = 0; a < D; ++a) {
      double y = 0.0;
#pragma unroll 16
      for (int b = 0; b < D; ++b) y += (double)Mh[a * D + b] * (double)xv[b];
      s += (double)xv[a] * y;
    }
  }
  out[(int64_t)h * S + i] = s;
}

constexpr int kKppThreads = 1024;
constexpr int kKppMaxPer = 16;  // candidates per thread (S <= 16384)

// One workgroup per head. Thread t owns candidates [t*P, t*P + P). D2 is kept in registers.
template <typename T, int D>
__global__ __launch_bounds__(kKppThreads) void kpp_seed(const T* __restrict__ X, int64_t N, int S, int C,
                                                        const float* __restrict__ M,
                                                        const double* __restrict__ cand_norm, uint64_t seed,
                                                        int side, float* __restrict__ cent) {
  __shared__ double cvec[D];
  __shared__ double yvec[D];
  __shared__ double red[kKppThreads / kWave];
  __shared__ double scan_scratch[17];
  __shared__ double cc_shared;
  __shared__ int pick;
  __shared__ int fallback;

  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int l = lane_id();
  const int w = tid / kWave;
  const int P = (S + kKppThreads - 1) / kKppThreads;
  const int base = tid * P;
  const T* Xh = X + (int64_t)h * N * D;
  const float* Mh = M ? M + (int64_t)h * D * D : nullptr;
  const double* xx = cand_norm + (int64_t)h * S;

  double d2[kKppMaxPer];
  double own_xx[kKppMaxPer];
  uint32_t taken = 0;
#pragma unroll
  for (int k = 0; k < kKppMaxPer; ++k) {
    d2[k] = 0.0;
    own_xx[k] = (k < P && base + k < S) ? xx[base + k] : 0.0;
  }

  for (int m = 0; m < C; ++m) {
    // ---- choose candidate t
    if (m == 0) {
      if (tid == 0) {
        int t0 = (int)(kpp_uniform(seed, h, side, 0) * (double)S);
        pick = t0 < S ? t0 : S - 1;
      }
      __syncthreads();
    } else {
      double local = 0.0;
#pragma unroll
      for (int k = 0; k < kKppMaxPer; ++k)
        if (k < P) local += d2[k];
      double total;
      const double ex = block_exclusive_scan(local, scan_scratch, &total);
      if (tid == 0) {
        pick = S;
        fallback = 0;
      }
      __syncthreads();
      if (total > 0.0) {
        const double v = kpp_uniform(seed, h, side, m) * total;
        // owner: the first thread whose range reaches past v
        if (ex + local > v) atomicMin(&pick, tid);
        __syncthreads();
        const int owner = pick;
        __syncthreads();
        if (owner >= kKppThreads && tid == 0) fallback = S + 1;  // rounding left v past every range
        if (tid == owner) {
          double run = ex;
          int found = -1, last_pos = -1;
#pragma unroll
          for (int k = 0; k < kKppMaxPer; ++k) {
            if (k < P && found < 0 && d2[k] > 0.0) {
              last_pos = k;
              run += d2[k];
              if (run > v) found = k;
            }
          }
          if (found < 0) found = last_pos;
          if (found >= 0)
            pick = base + found;
          else
            fallback = owner * P + 1;  // no mass in the owner's range: take the last one before it
        }
        __syncthreads();
        if (fallback) {
          const int limit = fallback - 1;
          if (tid == 0) pick = -1;
          __syncthreads();
          int lastk = -1;
#pragma unroll
          for (int k = 0; k < kKppMaxPer; ++k)
            if (k < P && base + k < limit && d2[k] > 0.0) lastk = base + k;
          if (lastk >= 0) atomicMax(&pick, lastk);
          __syncthreads();
          if (tid == 0 && pick < 0) pick = 0;
          __syncthreads();
        }
      } else {
        // every D^2 is zero: lowest candidate not yet chosen
        int first = S;
#pragma unroll
        for (int k = kKppMaxPer - 1; k >= 0; --k)
          if (k < P && base + k < S && !((taken >> k) & 1u)) first = base + k;
        if (first < S) atomicMin(&pick, first);
        __syncthreads();
      }
    }
    const int t = pick;
    const int64_t row = cand_row(t, S, N);
    // ---- centre c = x_t, y = M c (or c), cc = c.y
    for (int a = tid; a < D; a += kKppThreads) {
      const float cv = load_f32(Xh + row * D, a);
      cvec[a] = (double)cv;
      cent[((int64_t)h * C + m) * D + a] = cv;
    }
    __syncthreads();
    if (Mh != nullptr) {
      // thread (a, part): 8 threads per output row, 16 products each for D = 128
      constexpr int kParts = 8;
      const int a = tid / kParts;
      const int part = tid % kParts;
      double y = 0.0;
      if (a < D) {
        const int b0 = part * (D / kParts);
#pragma unroll
        for (int b = 0; b < D / kParts; ++b) y += (double)Mh[a * D + b0 + b] * cvec[b0 + b];
      }
#pragma unroll
      for (int o = 1; o < kParts; o <<= 1) y += __shfl_xor(y, o, kWave);
      if (a < D && part == 0) yvec[a] = y;
    } else {
      for (int a = tid; a < D; a += kKppThreads) yvec[a] = cvec[a];
    }
    __syncthreads();
    {
      double s = (tid < D) ? cvec[tid] * yvec[tid] : 0.0;
      s = wave_sum_f64(s);
      if (l == 0) red[w] = s;
      __syncthreads();
      if (tid == 0) {
        double c2 = 0.0;
        for (int q = 0; q < kKppThreads / kWave; ++q) c2 += red[q];
        cc_shared = c2;
      }
      __syncthreads();
    }
    const double cc = cc_shared;
    // ---- D^2 update: dist = xx - 2 x.y + cc
#pragma unroll
    for (int k = 0; k < kKppMaxPer; ++k) {
      if (k < P && base + k < S) {
        const int i = base + k;
        if (i == t) {
          taken |= 1u << k;
          d2[k] = 0.0;
        } else if (!((taken >> k) & 1u)) {
          const T* x = Xh + cand_row(i, S, N) * D;
          double dot = 0.0;
          for (int a0 = 0; a0 < D; a0 += 8) {
            float xv[8];
            load8_f32(x + a0, xv);
#pragma unroll
            for (int e = 0; e < 8; ++e) dot += (double)xv[e] * yvec[a0 + e];
          }
          double dist = own_xx[k] - 2.0 * dot + cc;
          dist = dist > 0.0 ? dist : 0.0;
          d2[k] = (m == 0 || dist < d2[k]) ? dist : d2[k];
        }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------------
// Update (optional) + consumed centroid form
// ------------------------------------------------------------------------------------------------

// One workgroup per (cluster, head). With do_update, c_j = fp32(fp64 mean of members in sorted
// order); empty clusters keep their value. Then g_j, b_j for the next assignment:
//   Euclidean: g = c (bf16-rounded for bf16 data), b = fp32(sum g^2)
//   QRKC:      y = M c (fp64), g = fp32(y) (then bf16), b = fp32(c.y)
template <typename T, int D>
__global__ __launch_bounds__(256) void update_consume(const T* __restrict__ X, int64_t N, int C,
                                                      const int32_t* __restrict__ perm,
                                                      const int32_t* __restrict__ offsets, float* __restrict__ cent,
                                                      int do_update, const float* __restrict__ M, void* g_out,
                                                      float* __restrict__ b_out, int bf16) {
  constexpr int TPR = D / 2;        // threads per row (2 dims each)
  constexpr int RG = 256 / TPR;     // row groups
  __shared__ double part[RG][D];
  __shared__ float cvec[D];
  __shared__ double red[4];
  const int j = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int l = lane_id();
  float* cj = cent + ((int64_t)h * C + j) * D;
  int n = 0;
  if (do_update) {
    const int beg = offsets[(int64_t)h * (C + 1) + j];
    const int end = offsets[(int64_t)h * (C + 1) + j + 1];
    n = end - beg;
    if (n > 0) {
      const int dp = tid % TPR;
      const int rg = tid / TPR;
      const T* Xh = X + (int64_t)h * N * D;
      const int32_t* ph = perm + (int64_t)h * N;
      double s0 = 0.0, s1 = 0.0;
      for (int r = beg + rg; r < end; r += RG) {
        const T* x = Xh + (int64_t)ph[r] * D + 2 * dp;
        s0 += (double)load_f32(x, 0);
        s1 += (double)load_f32(x, 1);
      }
      part[rg][2 * dp] = s0;
      part[rg][2 * dp + 1] = s1;
      __syncthreads();
      if (tid < D) {
        double s = 0.0;
#pragma unroll
        for (int q = 0; q < RG; ++q) s += part[q][tid];
        const float c = (float)(s / (double)n);
        cj[tid] = c;
        cvec[tid] = c;
      }
    }
  }
  if (n == 0 && tid < D) cvec[tid] = cj[tid];
  __syncthreads();
  double term = 0.0;
  if (tid < D) {
    const int64_t gi = ((int64_t)h * C + j) * D + tid;
    float gv;
    if (M == nullptr) {
      gv = cvec[tid];
      if (bf16) gv = bf16_bits_to_f32(f32_to_bf16_bits(gv));
      term = (double)gv * (double)gv;
    } else {
      const float* Mr = M + (int64_t)h * D * D + (int64_t)tid * D;
      double y = 0.0;
      for (int b = 0; b < D; ++b) y += (double)Mr[b] * (double)cvec[b];
      gv = (float)y;
      if (bf16) gv = bf16_bits_to_f32(f32_to_bf16_bits(gv));
      term = (double)cvec[tid] * y;
    }
    if (bf16)
      static_cast<uint16_t*>(g_out)[gi] = (uint16_t)(__float_as_uint(gv) >> 16);
    else
      static_cast<float*>(g_out)[gi] = gv;
  }
  term = wave_sum_f64(term);
  if (l == 0) red[tid / kWave] = term;
  __syncthreads();
  if (tid == 0) {
    double s = 0.0;
    for (int q = 0; q < 4; ++q) s += red[q];
    b_out[(int64_t)h * C + j] = (float)s;
  }
}

// ------------------------------------------------------------------------------------------------
// Assignment
// ------------------------------------------------------------------------------------------------

constexpr int kAsgChunk = 128;  // centroids staged in LDS at a time

// bf16 data. Each wave owns PT*32 points held as MFMA B operands; centroid tiles of 32 rows are
// the A operands. The accumulator starts at -b_j/2, so it holds x.g_j - b_j/2 and the label is the
// argmax (lowest j on ties).
template <int D, int PT>
__global__ __launch_bounds__(256) void assign_bf16(const uint16_t* __restrict__ X, int64_t N, int C,
                                                   const uint16_t* __restrict__ G, const float* __restrict__ b,
                                                   int32_t* __restrict__ labels) {
  constexpr int KS = D / 16;
  constexpr int STR = D + 8;  // padded LDS row (bf16 elements)
  __shared__ __attribute__((aligned(16))) uint16_t gl[kAsgChunk * STR];
  __shared__ float hb[kAsgChunk];
  const int h = blockIdx.y;
  const int l = lane_id();
  const int w = threadIdx.x / kWave;
  const int hl = l / 32;
  const int64_t p_base = (int64_t)blockIdx.x * (4 * 32 * PT) + (int64_t)w * 32 * PT;
  const uint16_t* Xh = X + (int64_t)h * N * D;
  const uint16_t* Gh = G + (int64_t)h * C * D;
  const float* bh = b + (int64_t)h * C;

  u32x4_t xb[PT][KS];
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) {
    const int64_t p = p_base + pt * 32 + l % 32;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (p < N) v = *reinterpret_cast<const u32x4_t*>(Xh + p * D + kk * 16 + hl * 8);
      xb[pt][kk] = v;
    }
  }
  float best[PT];
  int bidx[PT];
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) {
    best[pt] = -INFINITY;
    bidx[pt] = 0;
  }
  for (int c0 = 0; c0 < C; c0 += kAsgChunk) {
    // stage centroids [c0, c0 + 128) and -b/2
    for (int e = threadIdx.x; e < kAsgChunk * (D / 8); e += 256) {
      const int r = e / (D / 8);
      const int c8 = e % (D / 8);
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (c0 + r < C) v = *reinterpret_cast<const u32x4_t*>(Gh + (int64_t)(c0 + r) * D + c8 * 8);
      *reinterpret_cast<u32x4_t*>(&gl[r * STR + c8 * 8]) = v;
    }
    for (int r = threadIdx.x; r < kAsgChunk; r += 256) hb[r] = (c0 + r < C) ? -0.5f * bh[c0 + r] : -INFINITY;
    __syncthreads();
    const int ntile = (C - c0 + 31) / 32 < kAsgChunk / 32 ? (C - c0 + 31) / 32 : kAsgChunk / 32;
    for (int ct = 0; ct < ntile; ++ct) {
      f32x16_t acc[PT];
      f32x16_t init;
#pragma unroll
      for (int i = 0; i < 16; ++i) init[i] = hb[ct * 32 + (i / 4) * 8 + hl * 4 + i % 4];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) acc[pt] = init;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&gl[(ct * 32 + l % 32) * STR + kk * 16 + hl * 8]);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = mfma32(a, xb[pt][kk], acc[pt]);
      }
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = c0 + ct * 32 + (i / 4) * 8 + hl * 4 + i % 4;
          if (acc[pt][i] > best[pt]) {
            best[pt] = acc[pt][i];
            bidx[pt] = j;
          }
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) {
    const float ob = __shfl_xor(best[pt], 32, kWave);
    const int oi = __shfl_xor(bidx[pt], 32, kWave);
    if (ob > best[pt] || (ob == best[pt] && oi < bidx[pt])) bidx[pt] = oi;
    const int64_t p = p_base + pt * 32 + l % 32;
    if (hl == 0 && p < N) labels[(int64_t)h * N + p] = bidx[pt];
  }
}

// fp32 data: one thread per point, fp64 dot products against fp32 centroids staged in LDS.
template <int D>
__global__ __launch_bounds__(256) void assign_f32(const float* __restrict__ X, int64_t N, int C,
                                                  const float* __restrict__ G, const float* __restrict__ b,
                                                  int32_t* __restrict__ labels) {
  constexpr int CH = 32;
  __shared__ float gl[CH * D];
  __shared__ float bl[CH];
  const int h = blockIdx.y;
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float* x = X + ((int64_t)h * N + (p < N ? p : 0)) * D;
  double best = INFINITY;
  int bi = 0;
  for (int c0 = 0; c0 < C; c0 += CH) {
    for (int e = threadIdx.x; e < CH * D; e += 256) {
      const int r = e / D;
      gl[e] = (c0 + r < C) ? G[((int64_t)h * C + c0 + r) * D + e % D] : 0.f;
    }
    for (int r = threadIdx.x; r < CH; r += 256) bl[r] = (c0 + r < C) ? b[(int64_t)h * C + c0 + r] : 0.f;
    __syncthreads();
    const int nc = C - c0 < CH ? C - c0 : CH;
    for (int r = 0; r < nc; ++r) {
      double dot = 0.0;
      for (int a = 0; a < D; ++a) dot += (double)x[a] * (double)gl[r * D + a];
      const double f = (double)bl[r] - 2.0 * dot;
      if (f < best) {
        best = f;
        bi = c0 + r;
      }
    }
    __syncthreads();
  }
  if (p < N) labels[(int64_t)h * N + p] = bi;
}

// ------------------------------------------------------------------------------------------------
// Stable counting sort: per-chunk histograms -> per-head scan -> ordered scatter
// ------------------------------------------------------------------------------------------------

__global__ __launch_bounds__(64) void sort_hist(const int32_t* __restrict__ labels, int64_t N, int C, int nchunk,
                                                int32_t* __restrict__ table) {
  __shared__ int cnt[kMaxClusters];
  const int h = blockIdx.y;
  const int ch = blockIdx.x;
  for (int c = threadIdx.x; c < C; c += 64) cnt[c] = 0;
  __syncthreads();
  const int64_t t0 = (int64_t)ch * kSortChunk;
  const int32_t* lh = labels + (int64_t)h * N;
  for (int e = threadIdx.x; e < kSortChunk; e += 64) {
    const int64_t t = t0 + e;
    if (t < N) atomicAdd(&cnt[lh[t]], 1);
  }
  __syncthreads();
  int32_t* out = table + ((int64_t)h * nchunk + ch) * C;
  for (int c = threadIdx.x; c < C; c += 64) out[c] = cnt[c];
}

// Per head: table[chunk][c] <- number of tokens placed before chunk's first token of cluster c
// (offsets included); offsets[c] = tokens with label < c.
__global__ __launch_bounds__(1024) void sort_scan(int32_t* __restrict__ table, int nchunk, int C,
                                                  int32_t* __restrict__ offsets) {
  __shared__ int tot[kMaxClusters];
  __shared__ int scratch[17];
  const int h = blockIdx.x;
  int32_t* th = table + (int64_t)h * nchunk * C;
  for (int c = threadIdx.x; c < C; c += 1024) {
    int run = 0;
    for (int k = 0; k < nchunk; ++k) {
      const int v = th[(int64_t)k * C + c];
      th[(int64_t)k * C + c] = run;
      run += v;
    }
    tot[c] = run;
  }
  __syncthreads();
  // exclusive scan of tot over clusters: each thread a contiguous segment
  const int per = (C + 1023) / 1024;
  const int c_beg = threadIdx.x * per;
  int local = 0;
  for (int k = 0; k < per; ++k)
    if (c_beg + k < C) local += tot[c_beg + k];
  int total;
  int run = block_exclusive_scan(local, scratch, &total);
  for (int k = 0; k < per; ++k) {
    const int c = c_beg + k;
    if (c < C) {
      const int v = tot[c];
      tot[c] = run;
      offsets[(int64_t)h * (C + 1) + c] = run;
      run += v;
    }
  }
  if (threadIdx.x == 0) offsets[(int64_t)h * (C + 1) + C] = total;
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += 1024) {
    const int o = tot[c];
    for (int k = 0; k < nchunk; ++k) th[(int64_t)k * C + c] += o;
  }
}

// One wave per chunk: tokens are placed in order, 64 at a time; lanes with equal labels are
// ranked by lane index, which keeps the original order inside each cluster.
__global__ __launch_bounds__(64) void sort_scatter(const int32_t* __restrict__ labels, int64_t N, int C,
                                                   int nchunk, const int32_t* __restrict__ table,
                                                   int32_t* __restrict__ perm) {
  __shared__ int cursor[kMaxClusters];
  const int h = blockIdx.y;
  const int ch = blockIdx.x;
  const int l = lane_id();
  const int32_t* base = table + ((int64_t)h * nchunk + ch) * C;
  for (int c = l; c < C; c += 64) cursor[c] = base[c];
  __syncthreads();
  const int32_t* lh = labels + (int64_t)h * N;
  int32_t* ph = perm + (int64_t)h * N;
  const uint64_t lt_mask = (l == 0) ? 0ull : (~0ull >> (64 - l));
  for (int r = 0; r < kSortChunk / 64; ++r) {
    const int64_t t = (int64_t)ch * kSortChunk + r * 64 + l;
    const bool valid = t < N;
    const int lab = valid ? lh[t] : -1;
    uint64_t active = __ballot(valid);
    int pos = 0;
    while (active) {
      const int leader = __ffsll((unsigned long long)active) - 1;
      const int lead_lab = __shfl(lab, leader, kWave);
      const uint64_t same = __ballot(lab == lead_lab) & active;
      const int c0 = cursor[lead_lab];
      if (lab == lead_lab && valid) pos = c0 + __popcll(same & lt_mask);
      __syncthreads();  // every lane has read cursor before the leader advances it
      if (l == leader) cursor[lead_lab] = c0 + __popcll(same);
      __syncthreads();
      active &= ~same;
    }
    if (valid) ph[pos] = (int32_t)t;
  }
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------------------

hipError_t launch_kpp(const Dims& s, const void* x, const float* metric, int C, uint64_t seed, int side,
                      float* cent, double* cand_norm, hipStream_t st) {
  const int S = kpp_candidates(s.N, C);
  const dim3 g1((unsigned)ceil_div(S, 256), (unsigned)s.H);
#define PARK_KPP(T, D)                                                                                 \
  kpp_cand_norm<T, D><<<g1, 256, 0, st>>>(static_cast<const T*>(x), s.N, S, metric, cand_norm);       \
  kpp_seed<T, D><<<(unsigned)s.H, kKppThreads, 0, st>>>(static_cast<const T*>(x), s.N, S, C, metric, \
                                                         cand_norm, seed, side, cent);
  if (s.bf16) {
    if (s.D == 128) {
      PARK_KPP(uint16_t, 128)
    } else {
      PARK_KPP(uint16_t, 64)
    }
  } else {
    if (s.D == 128) {
      PARK_KPP(float, 128)
    } else {
      PARK_KPP(float, 64)
    }
  }
#undef PARK_KPP
  return hipGetLastError();
}

hipError_t launch_consume(const Dims& s, const void* x, int C, const int32_t* perm, const int32_t* offsets,
                          float* cent, int do_update, const float* metric, void* g, float* b, hipStream_t st) {
  const dim3 grid((unsigned)C, (unsigned)s.H);
#define PARK_UPD(T, D)                                                                                         \
  update_consume<T, D><<<grid, 256, 0, st>>>(static_cast<const T*>(x), s.N, C, perm, offsets, cent, do_update, \
                                             metric, g, b, s.bf16);
  if (s.bf16) {
    if (s.D == 128) {
      PARK_UPD(uint16_t, 128)
    } else {
      PARK_UPD(uint16_t, 64)
    }
  } else {
    if (s.D == 128) {
      PARK_UPD(float, 128)
    } else {
      PARK_UPD(float, 64)
    }
  }
#undef PARK_UPD
  return hipGetLastError();
}

hipError_t launch_assign(const Dims& s, const void* x, int C, const void* g, const float* b, int32_t* labels,
                         hipStream_t st) {
  if (s.bf16) {
    constexpr int PT = 2;
    const dim3 grid((unsigned)ceil_div(s.N, 4 * 32 * PT), (unsigned)s.H);
    if (s.D == 128)
      assign_bf16<128, PT><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x), s.N, C,
                                                 static_cast<const uint16_t*>(g), b, labels);
    else
      assign_bf16<64, PT><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x), s.N, C,
                                                static_cast<const uint16_t*>(g), b, labels);
  } else {
    const dim3 grid((unsigned)ceil_div(s.N, 256), (unsigned)s.H);
    if (s.D == 128)
      assign_f32<128><<<grid, 256, 0, st>>>(static_cast<const float*>(x), s.N, C, static_cast<const float*>(g), b,
                                            labels);
    else
      assign_f32<64><<<grid, 256, 0, st>>>(static_cast<const float*>(x), s.N, C, static_cast<const float*>(g), b,
                                           labels);
  }
  return hipGetLastError();
}

size_t sort_table_ints(const Dims& s, int C) { return (size_t)(s.H * ceil_div(s.N, kSortChunk) * C); }

hipError_t launch_sort(const Dims& s, int C, const int32_t* labels, int32_t* table, int32_t* perm,
                       int32_t* offsets, hipStream_t st) {
  const int nchunk = (int)ceil_div(s.N, kSortChunk);
  const dim3 grid((unsigned)nchunk, (unsigned)s.H);
  sort_hist<<<grid, 64, 0, st>>>(labels, s.N, C, nchunk, table);
  sort_scan<<<(unsigned)s.H, 1024, 0, st>>>(table, nchunk, C, offsets);
  sort_scatter<<<grid, 64, 0, st>>>(labels, s.N, C, nchunk, table, perm);
  return hipGetLastError();
}

}  // namespace park
