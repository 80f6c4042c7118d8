// Block-sparse attention over the selected (query cluster, key cluster) pairs (PARK abstract:
// attention is computed only within the retrieved blocks).
//
// Schedule: a work item is one tile of 256 (bf16) or 128 (fp32) queries of one query cluster. The
// original key rows of the key clusters a query cluster selected are gathered once into one list
// (the cluster's virtual key sequence), so key tiles are full MFMA tiles except the last one of each
// item, however small the individual clusters are.
//
// Per wave of 32 queries and key tile: S^T = K Q^T and O^T += V^T P^T run on 32x32x16 bf16 MFMA with
// fp32 accumulation, and an online softmax in exp2 form keeps one reference max and sum per query.
// Outputs are written straight to the queries' original rows.
#include <type_traits>

#include "park_common.h"
#include "park_internal.h"

namespace park {

namespace {

// Per head, the work list in longest-first order (the schedule step of the PARK page: per query
// cluster a list of bm-query work items; clusters with more selected keys first, so that the last
// work items dealt to a CU are the short ones). Clusters are sorted by their gathered key count,
// descending, ties by lower index; ord[k] is the k-th cluster in that order and tb[k] the number of
// work items before it, tb[cq] the total. Per head the layout is tb[0 .. cq], then ord[0 .. cq-1].
__global__ __launch_bounds__(1024) void attn_order(const int32_t* __restrict__ q_offsets,
                                                   const int32_t* __restrict__ glen, int cq, int bm,
                                                   int32_t* __restrict__ tile_base) {
  __shared__ uint64_t keys[kMaxClusters];
  __shared__ int scratch[17];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* off = q_offsets + (int64_t)h * (cq + 1);
  const int32_t* gl = glen + (int64_t)h * cq;
  int32_t* tb = tile_base + (int64_t)h * (2 * cq + 1);
  int32_t* ord = tb + cq + 1;
  int P2 = 1;
  while (P2 < cq) P2 <<= 1;
  // key: gathered key count, then the complemented cluster index; padding (key 0) sorts last
  for (int j = tid; j < P2; j += 1024)
    keys[j] = j < cq ? ((uint64_t)(uint32_t)max(gl[j], 0) << 32) | (uint64_t)(~(uint32_t)j) : 0;
  __syncthreads();
  for (int k = 2; k <= P2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int idx = tid; idx < P2; idx += 1024) {
        const int ixj = idx ^ jj;
        if (ixj > idx) {
          const uint64_t a = keys[idx], b = keys[ixj];
          if ((a < b) == ((idx & k) == 0)) {
            keys[idx] = b;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  // thread t owns sorted positions [t * per, t * per + per)
  const int per = (cq + 1023) / 1024;
  const int k0 = tid * per;
  int local = 0;
  for (int k = k0; k < min(k0 + per, cq); ++k) {
    const int i = (int)~(uint32_t)(keys[k] & 0xFFFFFFFFu);
    local += (max(off[i + 1] - off[i], 0) + bm - 1) / bm;
  }
  int total;
  int run = block_exclusive_scan(local, scratch, &total);
  for (int k = k0; k < min(k0 + per, cq); ++k) {
    const int i = (int)~(uint32_t)(keys[k] & 0xFFFFFFFFu);
    tb[k] = run;
    ord[k] = i;
    run += (max(off[i + 1] - off[i], 0) + bm - 1) / bm;
  }
  if (tid == 0) tb[cq] = total;
}

// Per (query cluster i, head h): the keys of the selected key clusters, in selection order, form the
// cluster's virtual key sequence. Key cluster j occupies the k_perm positions ko[j] .. ko[j+1]-1, so
// the sequence is a list of runs of consecutive k_perm positions: consecutive selected clusters
// whose ranges touch (every cluster between them empty) share one run. Virtual key v of run r
// (rv[r] <= v < rv[r+1]) is the key at k_perm position v + rd[r]. Per (h, i) the region of
// run_stride(ck) ints holds rv[0 .. R] (rv[R] = the sequence length), rd[0 .. R-1] and, for the
// weighted form, rb[0 .. R-1] = the run's logit offset in raw-score units (runs then stay one per
// cluster, since clusters carry their own weights). Column entries outside [0, ck) or with offsets
// outside [0, N] contribute nothing; the sequence is cut at N keys (reached only when a cluster is
// listed twice).
__host__ __device__ constexpr int64_t run_stride(int ck) { return ((3 * (int64_t)ck + 1) + 3) & ~int64_t(3); }

__global__ __launch_bounds__(256) void attn_runs(const int32_t* __restrict__ counts, const int32_t* __restrict__ cols,
                                                 const int32_t* __restrict__ k_offsets, int64_t N, int cq, int ck,
                                                 const float* __restrict__ log_w, float inv_scale,
                                                 int32_t* __restrict__ runs, int32_t* __restrict__ nrun,
                                                 int32_t* __restrict__ glen, int32_t* __restrict__ nblk) {
  __shared__ int scratch[17];
  __shared__ int last_hi[4];  // per wave: end position of its last non-empty entry, -1 if none
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int l = lane_id();
  const int w = tid / kWave;
  int cnt = counts[(int64_t)h * cq + i];
  cnt = cnt < 0 ? 0 : (cnt > ck ? ck : cnt);
  const int32_t* crow = cols + ((int64_t)h * cq + i) * ck;
  const int32_t* ko = k_offsets + (int64_t)h * (ck + 1);
  const float* lwrow = log_w ? log_w + ((int64_t)h * cq + i) * ck : nullptr;
  int32_t* rv = runs + ((int64_t)h * cq + i) * run_stride(ck);
  int32_t* rd = rv + ck + 1;
  float* rb = reinterpret_cast<float*>(rv + 2 * ck + 1);
  int64_t base = 0;  // keys of the entries before this chunk
  int R = 0;         // runs started before this chunk
  int kept = 0;      // runs that start before N
  int carry = -1;    // end position of the last non-empty entry before this chunk
  int blocks = 0;    // selected non-empty key clusters
  for (int m0 = 0; m0 < cnt; m0 += 256) {
    const int m = m0 + tid;
    int lo = 0, len = 0;
    float bias = 0.f;
    if (m < cnt) {
      const int j = crow[m];
      if (j >= 0 && j < ck) {
        const int64_t a = ko[j], b = ko[j + 1];
        if (a >= 0 && b > a && b <= N) {
          lo = (int)a;
          len = (int)(b - a);
        }
        if (lwrow) bias = lwrow[j] * inv_scale;
      }
    }
    const bool ne = len > 0;
    // end position of the previous non-empty entry: within the wave from the nearest lower lane,
    // else from the waves before, else from the chunks before
    const uint64_t bal = __ballot(ne);
    const uint64_t below = bal & ((1ull << l) - 1ull);
    const int src = below ? 63 - __clzll((unsigned long long)below) : 0;
    const int hi_below = __shfl(lo + len, src, kWave);
    const int hi_last = __shfl(lo + len, bal ? 63 - __clzll((unsigned long long)bal) : 0, kWave);
    if (l == 0) last_hi[w] = bal ? hi_last : -1;
    __syncthreads();
    int prev = carry;
    for (int q = 0; q < w; ++q) prev = last_hi[q] >= 0 ? last_hi[q] : prev;
    if (below) prev = hi_below;
    int chunk_last = carry;
    for (int q = 0; q < 4; ++q) chunk_last = last_hi[q] >= 0 ? last_hi[q] : chunk_last;
    const bool start = ne && (lwrow != nullptr || prev != lo);
    int tot_len, tot_start;
    const int pre_len = block_exclusive_scan(len, scratch, &tot_len);
    const int pre_start = block_exclusive_scan(start ? 1 : 0, scratch, &tot_start);
    const int64_t v0 = base + pre_len;
    const bool write = start && v0 < N;
    if (write) {
      const int r = R + pre_start;
      rv[r] = (int)v0;
      rd[r] = lo - (int)v0;
      if (lwrow) rb[r] = bias;
    }
    kept += __syncthreads_count(write);
    blocks += __syncthreads_count(ne);
    base += tot_len;
    R += tot_start;
    carry = chunk_last;
  }
  if (tid == 0) {
    const int L = (int)min<int64_t>(base, N);
    rv[kept] = L;
    nrun[(int64_t)h * cq + i] = kept;
    glen[(int64_t)h * cq + i] = L;
    nblk[(int64_t)h * cq + i] = blocks;
  }
}

// Totals of the selection (park_stats). attn_stats_head: one work-group per head writes the head's
// five partial totals (pairs, padded pairs, blocks, live query clusters x live key clusters, work
// items) to part[h * 8 ..]; attn_stats_sum adds them over the heads in head order (deterministic).
// bn = keys per tile of the kernel.
__global__ __launch_bounds__(256) void attn_stats_head(const int32_t* __restrict__ q_offsets,
                                                       const int32_t* __restrict__ k_offsets, int cq, int ck,
                                                       const int32_t* __restrict__ glen,
                                                       const int32_t* __restrict__ nblk,
                                                       const int32_t* __restrict__ tile_base, int bn,
                                                       int64_t* __restrict__ part) {
  __shared__ int64_t red[5][4];
  const int h = blockIdx.x;
  const int32_t* qo = q_offsets + (int64_t)h * (cq + 1);
  const int32_t* ko = k_offsets + (int64_t)h * (ck + 1);
  int64_t acc[5] = {0, 0, 0, 0, 0};  // pairs, padded, blocks, live query clusters, live key clusters
  for (int i = threadIdx.x; i < cq; i += 256) {
    const int64_t nq = qo[i + 1] - qo[i];
    const int64_t L = glen[(int64_t)h * cq + i];
    acc[0] += nq * L;
    acc[1] += ((nq + 31) / 32) * 32 * ((L + bn - 1) / bn) * bn;
    acc[2] += nq > 0 ? nblk[(int64_t)h * cq + i] : 0;
    acc[3] += nq > 0;
  }
  for (int j = threadIdx.x; j < ck; j += 256) acc[4] += ko[j + 1] > ko[j];
  const int l = lane_id(), w = threadIdx.x / kWave;
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    int64_t v = acc[q];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    if (l == 0) red[q][w] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t t[5];
    for (int q = 0; q < 5; ++q) t[q] = ((red[q][0] + red[q][1]) + red[q][2]) + red[q][3];
    int64_t* o = part + (int64_t)h * 8;
    o[0] = t[0];
    o[1] = t[1];
    o[2] = t[2];
    o[3] = t[3] * t[4];
    o[4] = tile_base[(int64_t)h * (2 * cq + 1) + cq];
  }
}

__global__ __launch_bounds__(64) void attn_stats_sum(const int64_t* __restrict__ part, int64_t H, int64_t N,
                                                     int64_t* __restrict__ stats) {
  const int q = threadIdx.x;
  if (q < 5) {
    int64_t v = 0;
    for (int64_t h = 0; h < H; ++h) v += part[h * 8 + q];
    stats[q] = v;
  } else if (q == 5) {
    stats[5] = H * N;
  } else if (q < 8) {
    stats[q] = 0;
  }
}

__device__ __forceinline__ int find_tile(const int32_t* tb, int cq, int c) {
  int lo = 0, hi = cq;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tb[mid] <= c)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// The bf16 attention's work queue: hpre[h] = work items of the heads before h (hpre[H] = all), and
// the queue counter cleared.
__global__ __launch_bounds__(1024) void attn_queue_prep(const int32_t* __restrict__ tile_base, int64_t H, int cq,
                                                        int64_t* __restrict__ hpre,
                                                        unsigned long long* __restrict__ qctr) {
  __shared__ int64_t scratch[17];
  const int tid = threadIdx.x;
  const int64_t per = (H + 1023) / 1024;
  const int64_t h0 = tid * per, h1 = min(h0 + per, H);
  int64_t local = 0;
  for (int64_t h = h0; h < h1; ++h) local += tile_base[h * (2 * cq + 1) + cq];
  int64_t total;
  int64_t run = block_exclusive_scan(local, scratch, &total);
  for (int64_t h = h0; h < h1; ++h) {
    hpre[h] = run;
    run += tile_base[h * (2 * cq + 1) + cq];
  }
  if (tid == 0) hpre[H] = total;
  if (tid == 0) qctr[0] = 0ull;
}

template <typename T>
__device__ __forceinline__ void store_out4(T* p, float a, float b, float c, float d);
template <>
[[maybe_unused]] __device__ __forceinline__ void store_out4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
  u32x2_t v;
  v[0] = pack_bf16x2(a, b);
  v[1] = pack_bf16x2(c, d);
  *reinterpret_cast<u32x2_t*>(p) = v;
}
template <>
__device__ __forceinline__ void store_out4<float>(float* p, float a, float b, float c, float d) {
  f32x4_t v = {a, b, c, d};
  *reinterpret_cast<f32x4_t*>(p) = v;
}

constexpr int kBN = 64;

template <typename T, int D>
__global__ __launch_bounds__(256) void sparse_attn_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                          const T* __restrict__ V, int64_t N,
                                                          const int32_t* __restrict__ q_perm,
                                                          const int32_t* __restrict__ q_off, int cq,
                                                          const int32_t* __restrict__ tile_base,
                                                          const int32_t* __restrict__ k_perm, int ck,
                                                          const int32_t* __restrict__ runs,
                                                          const int32_t* __restrict__ glen, int weighted,
                                                          float scale, T* __restrict__ out,
                                                          float* __restrict__ lse) {
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int KSTR = D + 8;
  constexpr int VSTR = kBN + 8;
  __shared__ __attribute__((aligned(16))) uint16_t ks[kBN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VSTR];
  __shared__ int32_t krow[kBN];
  __shared__ float kbias[kBN];  // per-key logit offsets (block weights) in raw-score units

  const int h = blockIdx.y;
  const int c = blockIdx.x;
  const int32_t* tb = tile_base + (int64_t)h * (2 * cq + 1);
  if (c >= tb[cq]) return;
  const int ti = find_tile(tb, cq, c);
  const int i = tb[cq + 1 + ti];
  const int tid = threadIdx.x;
  const int l = lane_id();
  const int w = tid / kWave;
  const int hl = l / 32;
  const int32_t* qo = q_off + (int64_t)h * (cq + 1);
  const int qbeg = qo[i] + (c - tb[ti]) * kAttnBM;
  const int qend = min(qbeg + kAttnBM, qo[i + 1]);
  const int32_t* rv = runs + ((int64_t)h * cq + i) * run_stride(ck);
  const int32_t* rd = rv + ck + 1;
  const float* brow = weighted ? reinterpret_cast<const float*>(rv + 2 * ck + 1) : nullptr;
  const int32_t* kp = k_perm + (int64_t)h * N;
  const int L = glen[(int64_t)h * cq + i];
  int cr = 0;  // run of this thread's key (threads < kBN; keys advance by kBN per tile)
  const T* Qh = Q + (int64_t)h * N * D;
  const T* Kh = K + (int64_t)h * N * D;
  const T* Vh = V + (int64_t)h * N * D;

  // B operand of S^T = K Q^T: query column l%32, dims kk*16 + hl*8 .. +7
  const int qpos = qbeg + w * 32 + l % 32;
  const bool qok = qpos < qend;
  const int qrow = qok ? q_perm[(int64_t)h * N + qpos] : 0;
  u32x4_t qb[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (qok) v = load8_bf16<T>(Qh + (int64_t)qrow * D + kk * 16 + hl * 8);
    qb[kk] = v;
  }
  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  const float sl2 = scale * 1.4426950408889634f;
  float m_run = -INFINITY;  // running max of raw scores
  float l_run = 0.f;        // this lane's share of the running sum
  // A-operand row of S^T held by lane l: physical key of MFMA row l%32 (see below)
  const int r = l % 32;
  const int prow = ((r / 4) % 2) * 16 + (r / 8) * 4 + r % 4;

  for (int v0 = 0; v0 < L; v0 += kBN) {
    if (tid < kBN) {
      const int v = v0 + tid;
      int row = -1;
      float bias = 0.f;
      if (v < L) {
        while (rv[cr + 1] <= v) ++cr;
        row = kp[v + rd[cr]];
        if (brow) bias = brow[cr];
      }
      krow[tid] = row;
      kbias[tid] = bias;
    }
    __syncthreads();
    // K tile, row-major
    for (int u = tid; u < kBN * (D / 8); u += 256) {
      const int kr = u / (D / 8), c8 = u % (D / 8);
      const int row = krow[kr];
      u32x4_t val = {0u, 0u, 0u, 0u};
      if (row >= 0) val = load8_bf16<T>(Kh + (int64_t)row * D + c8 * 8);
      *reinterpret_cast<u32x4_t*>(&ks[kr * KSTR + c8 * 8]) = val;
    }
    // V tile, transposed: vt[dim][key], two keys per 32-bit LDS write
    for (int u = tid; u < (kBN / 2) * (D / 8); u += 256) {
      const int pr = u % (kBN / 2), c8 = u / (kBN / 2);
      const int r0 = krow[2 * pr], r1 = krow[2 * pr + 1];
      u32x4_t a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (r0 >= 0) a = load8_bf16<T>(Vh + (int64_t)r0 * D + c8 * 8);
      if (r1 >= 0) b = load8_bf16<T>(Vh + (int64_t)r1 * D + c8 * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (a[q] & 0xFFFFu) | (b[q] << 16);
        const uint32_t hi = (a[q] >> 16) | (b[q] & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(&vt[(c8 * 8 + 2 * q) * VSTR + 2 * pr]) = lo;
        *reinterpret_cast<uint32_t*>(&vt[(c8 * 8 + 2 * q + 1) * VSTR + 2 * pr]) = hi;
      }
    }
    __syncthreads();

    // S^T for two 32-key subtiles. MFMA row r of subtile st is physical key
    // 32*st + ((r/4)%2)*16 + (r/8)*4 + r%4, so accumulator element i of lane l holds the score of
    // key 32*st + hl*16 + i against query l%32.
    f32x16_t sacc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[st][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&ks[(st * 32 + prow) * KSTR + kk * 16 + hl * 8]);
        sacc[st] = mfma32(a, qb[kk], sacc[st]);
      }
    }
    if (brow) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[st][e] += kbias[st * 32 + hl * 16 + e];
    }
    const int nvalid = L - v0;  // keys with index < nvalid in this tile are real
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kt = st * 32 + hl * 16 + e;
        if (kt < nvalid) mx = fmaxf(mx, sacc[st][e]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f((m_run - m_new) * sl2);
    const float mb = m_new * sl2;
    float psum = 0.f;
    u32x4_t pb[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float pv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kt = st * 32 + hl * 16 + e;
        pv[e] = kt < nvalid ? exp2f(sacc[st][e] * sl2 - mb) : 0.f;
        psum += pv[e];
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int q = 0; q < 4; ++q) pb[st][kh][q] = pack_bf16x2(pv[kh * 8 + 2 * q], pv[kh * 8 + 2 * q + 1]);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
    // O^T += V^T P^T: k-step (st, kh) pairs key 32*st + hl*16 + kh*8 + e with k index hl*8 + e
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const u32x4_t a =
              *reinterpret_cast<const u32x4_t*>(&vt[(dt * 32 + l % 32) * VSTR + st * 32 + hl * 16 + kh * 8]);
          o[dt] = mfma32(a, pb[st][kh], o[dt]);
        }
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (qok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T* orow = out + ((int64_t)h * N + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = dt * 32 + g4 * 8 + hl * 4;
        store_out4<T>(orow + d0, o[dt][g4 * 4] * inv, o[dt][g4 * 4 + 1] * inv, o[dt][g4 * 4 + 2] * inv,
                      o[dt][g4 * 4 + 3] * inv);
      }
    if (lse != nullptr && hl == 0)
      lse[(int64_t)h * N + qrow] = l_tot > 0.f ? m_run * scale + logf(l_tot) : -INFINITY;
  }
}


// ------------------------------------------------------------------------------------------------
// bf16 kernel: key/value tiles are copied HBM -> LDS with gfx950 direct buffer loads (no register
// staging) into a ring of stages, so copies run several tiles ahead of the MFMA work. Rows stay
// row-major in LDS with their 16-byte chunks XOR-swizzled by row (bank spread); V^T operands come
// from the transposing LDS read (each lane of a 16-lane group receives 4 keys of one column).
// ------------------------------------------------------------------------------------------------

// 384-query work items: twelve waves x 32 queries share one work-group per CU (three waves per
// SIMD, 168 registers each), so each key/value tile copied to LDS serves up to 384 queries and each
// SIMD has three waves to interleave matrix-core, vector and LDS work. Tiles (32 keys for d = 128,
// 64 for d = 64) are copied by eight of the waves (1 KB of K and of V per wave and copy) through a
// ring of four stages three tiles ahead; a wave waits only for the copies of the tile it is about to
// read (a counted vmcnt, then a plain barrier: a fenced barrier would also wait for the copies still
// in flight). A d = 128 work item of at most 192 queries (the ragged last item of a query cluster)
// runs a second form: 64-key tiles, and two groups of six waves on the same queries, each group
// one 32-key half of every tile; the second group's partial output, reference and sum are merged
// into the first's at the end. The busiest SIMD of such an item then computes half the sub-tiles it
// would compute alone (one wave per SIMD runs at well under a third of three waves' rate).
constexpr int kBf16BM = 384;                      // queries per work item
[[maybe_unused]] constexpr int kBf16BN = 32;      // keys per matrix-core sub-tile for d = 128
[[maybe_unused]] constexpr int kBf16TK = 64;      // keys per copied tile in the split form (and for d = 64)
[[maybe_unused]] constexpr int kBf16NST = 4;      // LDS stages of the ring
[[maybe_unused]] constexpr int kBf16SplitQ = 192; // d = 128 items of at most this many queries split their keys

// The lane id through an opaque read, which the compiler can neither reuse across nor hoist out of
// the code that needs it.
__device__ __forceinline__ int lane_id_opaque() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

// vmcnt(n) & lgkmcnt(0), then a plain workgroup barrier
template <int VM>
__device__ __forceinline__ void wait_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (0x7 << 4) | ((VM >> 4) << 14));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// f(integral_constant<I>) for I = B .. E-1 in order while it returns true
template <int B, int E, typename F>
__device__ __forceinline__ bool unroll_while(F&& f) {
  if constexpr (B < E) {
    if (!f(std::integral_constant<int, B>{})) return false;
    return unroll_while<B + 1, E>(f);
  } else {
    return true;
  }
}

// LDS reads the kernel writes out itself, each block ending by waiting for its reads. The compiler
// cannot tell which LDS the transposing read builtin reads, nor order a read of the index lists
// against the direct HBM -> LDS copies of later tiles, and would wait for every copy in flight
// before such a read; the explicit counted waits and barriers already order them.
// Four 16-byte reads at consecutive 16-byte offsets.
template <int OFF>
__device__ __forceinline__ void lds_read4_b128(u32x4_t (&r)[4], uint32_t a) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%5\n\t"
      "ds_read_b128 %1, %4 offset:%6\n\t"
      "ds_read_b128 %2, %4 offset:%7\n\t"
      "ds_read_b128 %3, %4 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a), "i"(OFF), "i"(OFF + 16), "i"(OFF + 32), "i"(OFF + 48)
      : "memory");
}
template <int OFF>
__device__ __forceinline__ void lds_read4x_b128(u32x4_t (&r)[4], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%8\n\t"
      "ds_read_b128 %1, %5 offset:%8\n\t"
      "ds_read_b128 %2, %6 offset:%8\n\t"
      "ds_read_b128 %3, %7 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF)
      : "memory");
}
template <int OFF>
__device__ __forceinline__ void tr_read8(u32x2_t (&r)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
      "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
      "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
      "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
      "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
      "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
      "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
      "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(OFF)
      : "memory");
}
// One dword.
[[maybe_unused]] __device__ __forceinline__ int lds_read_b32(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
// Two dwords.
[[maybe_unused]] __device__ __forceinline__ u32x2_t lds_read_b64(uint32_t addr) {
  u32x2_t v;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
// One dword written (the counted waits and barriers order it).
[[maybe_unused]] __device__ __forceinline__ void lds_write_b32(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// W: every gather-list key carries a logit offset (the log weight of its block, in raw-score
// units), copied into LDS with the tile and added to the scores
template <int D, bool W>
__global__ __launch_bounds__(768, 1) void sparse_attn_bf16(const uint16_t* __restrict__ Q,
                                                         const uint16_t* __restrict__ K,
                                                         const uint16_t* __restrict__ V, int64_t N,
                                                         const int32_t* __restrict__ q_perm,
                                                         const int32_t* __restrict__ q_off, int cq,
                                                         const int32_t* __restrict__ tile_base,
                                                         const int32_t* __restrict__ k_perm, int ck,
                                                         const int32_t* __restrict__ runs,
                                                         const int32_t* __restrict__ nrun,
                                                         const int32_t* __restrict__ glen, float scale,
                                                         uint16_t* __restrict__ out, float* __restrict__ lse,
                                                         const int64_t* __restrict__ hpre,
                                                         unsigned long long* __restrict__ qctr, int64_t H) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = 12;
  constexpr int NWC = 8;  // copier waves
  constexpr int NST = kBf16NST;
  constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3: raw (untyped) access
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int CPR = D / 8;
  constexpr int ROWB = D * 2;
  constexpr int NSC = D == 64 ? 2 : 1;          // 32-key sub-tiles a wave computes at once
  constexpr bool SPLIT = D == 128;              // ragged items may split their keys over two wave groups
  constexpr int RPB = 1024 / ROWB;              // rows per 1 KB wave load
  // the ring (K and V) for the largest tiles (64 keys); the split form's merge reuses it: 17 KB per
  // wave of the second group (its 64 output accumulators, then reference and sum, as one 16-byte
  // row per lane each)
  constexpr int MERGEB = SPLIT ? 6 * 17 * 1024 : 0;
  constexpr int RINGB = 2 * NST * 64 * ROWB > MERGEB ? 2 * NST * 64 * ROWB : MERGEB;
  __shared__ __attribute__((aligned(1024))) uint8_t stages[RINGB];
  // the query cluster's runs (see attn_runs), one record per run r: {rd[r], rv[r + 1]}, so that one
  // LDS read gives a lane the run's offset and its end; the weighted form keeps rb[r] apart
  __shared__ __attribute__((aligned(16))) int32_t s_run[kMaxClusters * 2];
  __shared__ __attribute__((aligned(16))) int32_t s_rb[W ? kMaxClusters : 1];
  // weighted form: per tile, the logit offset of each of the tile's keys (lane l: key l % BN),
  // written when the tile's entries are loaded and read when it is computed
  __shared__ __attribute__((aligned(16))) float bring[W ? 2 * NST : 1][kWave];
  // gather-list entries of the tiles in flight (see load_idx)
  __shared__ __attribute__((aligned(16))) int32_t idxs[NST][kWave];

  // Persistent work-groups, one per CU, take the work items in order from one queue: the heads one
  // after the other, each head's items longest-first. All CUs then work on about one head at a
  // time, whose key/value rows (39 MB at the Wan shape) stay in the 256 MB memory-side cache;
  // eight per-XCD queues of five heads each (consecutive items of a head sharing an XCD's L2)
  // measured 2 % slower. The last items are the last head's shortest.
  __shared__ int64_t s_item;
  const int64_t T = hpre[H];
  for (;;) {
  if (threadIdx.x == 0) {
    const int64_t v = (int64_t)atomicAdd(&qctr[0], 1ull);
    s_item = v < T ? v : -1;
  }
  __syncthreads();
  const int64_t gi = __builtin_amdgcn_readfirstlane(s_item);
  if (gi < 0) break;
  int hlo = 0, hhi = (int)H;  // the item's head: the largest h with hpre[h] <= gi
  while (hhi - hlo > 1) {
    const int mid = (hlo + hhi) >> 1;
    if (hpre[mid] <= gi)
      hlo = mid;
    else
      hhi = mid;
  }
  const int h = hlo;
  const int c = (int)(gi - hpre[h]);
  const int32_t* tb = tile_base + (int64_t)h * (2 * cq + 1);
  const int ti = find_tile(tb, cq, c);
  const int i = tb[cq + 1 + ti];
  const int l = lane_id_opaque();  // derived per item, not kept live across the item loop
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const bool copier = w < NWC;
  const bool indexer = w == NWC;  // the first wave without copies resolves the tiles' key rows
  const int wc = copier ? w : NWC - 1;
  const int hl = l / 32;
  const int32_t* qo = q_off + (int64_t)h * (cq + 1);
  const int qbeg = qo[i] + (c - tb[ti]) * kBf16BM;
  const int qend = min(qbeg + kBf16BM, qo[i + 1]);
  // split form: wave 6 g + j takes query group j and sub-tile g of every tile
  const bool split = SPLIT && qend - qbeg <= kBf16SplitQ;
  const int grp = split ? w / 6 : 0;
  const int qw = split ? w - 6 * grp : w;
  const bool active = qbeg + qw * 32 < qend;  // this wave has at least one query
  const int L = glen[(int64_t)h * cq + i];
  const int R = nrun[(int64_t)h * cq + i];
  {
    const int32_t* rg = runs + ((int64_t)h * cq + i) * run_stride(ck);
    for (int e = threadIdx.x; e < R; e += NW * kWave) {
      s_run[e * 2] = rg[ck + 1 + e];
      s_run[e * 2 + 1] = rg[e + 1];
      if constexpr (W) s_rb[e] = rg[2 * ck + 1 + e];
    }
  }
  const uint16_t* Qh = Q + (int64_t)h * N * D;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + (int64_t)h * N * D), (short)0, (int)(uint32_t)(N * ROWB), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(V + (int64_t)h * N * D), (short)0, (int)(uint32_t)(N * ROWB), kBufferFlags);

  const int qpos = qbeg + qw * 32 + l % 32;
  const bool qok = qpos < qend;
  const int qrow = q_perm[(int64_t)h * N + min(qpos, qend - 1)];
  u32x4_t qb[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(Qh + (int64_t)qrow * D + kk * 16 + hl * 8);
    const u32x4_t z = {0u, 0u, 0u, 0u};
    qb[kk] = qok ? v : z;
  }

  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  const float sl2 = scale * 1.4426950408889634f;
  // Softmax reference: m_ref is set from the first tile's scores and only raised when a tile's
  // weights 2^(sl2 (s - m_ref)) would exceed 2^40 in one lane's sum; any reference works for the
  // final O / l and the fp32 accumulators have range to spare, so almost no tile rescales O.
  constexpr float kRaise = 1099511627776.0f;  // 2^40
  float m_ref = -INFINITY;
  float l_run = 0.f;

  // The tile loop for tiles of TK keys: 32 for d = 128 outside the split form, 64 in it (each group
  // of waves one half) and for d = 64.
  auto run = [&](auto TKc) __attribute__((always_inline)) {
    constexpr int BN = decltype(TKc)::value;
    // the lane-derived values are derived again in each form (an opaque read of the lane id), so
    // that the two forms' copies are not kept live across both: the 168-register budget is tight
    const int l = lane_id_opaque();
    const int hl = l / 32;
    constexpr int NSUB = BN / 32;                 // 32-key sub-tiles per tile
    static_assert(NSUB == NSC || (SPLIT && NSUB == 2), "a wave computes all sub-tiles, or one in the split form");
    constexpr int TILEB = BN * ROWB;              // one K (or V) tile
    // K and V of a stage side by side while every stage offset fits the LDS reads' 16-bit offset
    // field, else the K ring followed by the V ring
    constexpr bool INTER = 2 * NST * TILEB <= 65536;
    constexpr int KSTR = INTER ? 2 * TILEB : TILEB;  // bytes from one stage's K to the next
    constexpr int VOFF = INTER ? TILEB : NST * TILEB; // a stage's V past its K
    constexpr int LOADS = TILEB / (1024 * NWC);    // 1 KB loads per wave per tile, for K and for V
    static_assert(LOADS >= 1, "tile smaller than one load per wave");
    constexpr int CP = 2 * LOADS;                 // copies per wave per tile
    // load slots: slot q of this lane copies tile row trow[q], logical chunk (l % CPR) ^ swizzle, into
    // physical chunk l % CPR of the wave's 1 KB block (w * LOADS + q)
    int trow[LOADS], lbyte[LOADS];
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
      trow[q] = (wc * LOADS + q) * RPB + l / CPR;
      lbyte[q] = ((l % CPR) ^ chunk_swz<CPR>(trow[q])) * 16;
    }
    const int nt = (L + BN - 1) / BN;
    // Gather-list entries of tile x reach LDS (set x % NST, one 256-byte region per wave, lane l
    // holding entry x * BN + l % BN) by a direct load in iteration x - 2 NST + 1; the lane's entry is
    // read into a register at the end of iteration x - NST, ready for the copies of iteration
    // x - NST + 1.
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(k_perm + (int64_t)h * N), (short)0, (int)(uint32_t)(N * 4), kBufferFlags);
    constexpr int IL = 1;  // index loads per wave and tile
    // Cursor of this lane's key through the runs: keys advance by BN per tile, so the run index only
    // grows (the run record is read again per tile, which keeps the cursor to one register).
    __syncthreads();  // run records in LDS
    int cr = 0;
    const uint32_t run_base = (uint32_t)(size_t)((PARK_LDS int32_t*)s_run);
    const uint32_t rb_base = (uint32_t)(size_t)((PARK_LDS int32_t*)s_rb);
    const uint32_t bring_base = (uint32_t)(size_t)((PARK_LDS float*)&bring[0][0]);
    auto load_idx = [&](int set, int tile) __attribute__((always_inline)) {
      if (!indexer) return;
      const int li = lane_id_opaque();  // the lane id read again: no register held for it
      const int v = tile * BN + li % BN;
      int off = (int)(N * 4);  // past the buffer's range: reads 0 (a valid row; its scores are masked)
      float bias = 0.f;
      if (v < L) {
        u32x2_t rec = lds_read_b64(run_base + (uint32_t)cr * 8u);
        while (v >= (int)rec[1]) {  // rec[1]: first key after run cr (< L for every run but the last)
          ++cr;
          rec = lds_read_b64(run_base + (uint32_t)cr * 8u);
        }
        off = (v + (int)rec[0]) * 4;
        if constexpr (W) bias = __int_as_float(lds_read_b32(rb_base + (uint32_t)cr * 4u));
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (PARK_LDS void*)&idxs[set][0], 4, off, 0, 0, 0);
      if constexpr (W) lds_write_b32(bring_base + (uint32_t)((tile % (2 * NST)) * kWave + li) * 4u, bias);
    };
    // entries of this lane's copy rows trow[q] = trow[0] + q RPB
    const uint32_t ibase = (uint32_t)(size_t)((PARK_LDS int32_t*)&idxs[0][trow[0]]);
    auto read_idx = [&](int set, int(&nr)[LOADS]) __attribute__((always_inline)) {
      if (!copier) return;  // only the copier waves use the entries
#pragma unroll
      for (int q = 0; q < LOADS; ++q) nr[q] = lds_read_b32(ibase + (uint32_t)((set * kWave + q * RPB) * 4));
    };
    int nnext[LOADS];  // gather-list rows of this lane's copies in the next issue
#pragma unroll
    for (int q = 0; q < LOADS; ++q) nnext[q] = 0;
    auto issue = [&](const int(&nrow)[LOADS], int slot, int tile) __attribute__((always_inline)) {
      if (!copier) return;
#pragma unroll
      for (int q = 0; q < LOADS; ++q) {
        const int boff = slot * KSTR + (w * LOADS + q) * 1024;
        const int voff = (int)((uint32_t)nrow[q] * ROWB + lbyte[q]);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (PARK_LDS void*)(stages + boff), 16, voff, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (PARK_LDS void*)(stages + VOFF + boff), 16, voff, 0, 0, 0);
      }
      (void)tile;
    };

    const int r = l % 32;
    const int prow = ((r / 4) % 2) * 16 + (r / 8) * 4 + r % 4;
    const int g16 = l / 16, i16 = l % 16;
    const bf16x2_t ones = as_bf16x2(0x3F803F80u);

    // per-lane byte offsets of the LDS operand reads within a stage (K, and V past VOFF), computed
    // once; a wave of the split form's second group reads the second sub-tile of every tile
    const int sub0 = grp * 32;
    int kofs[NSC][KS], vofs[DT][NSC][2][2];
#pragma unroll
    for (int st = 0; st < NSC; ++st) {
      const int R = sub0 + st * 32 + prow;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) kofs[st][kk] = R * ROWB + ((2 * kk + hl) ^ chunk_swz<CPR>(R)) * 16;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int D0 = dt * 32 + 16 * (g16 & 1);
      const int cc = (D0 + 4 * (i16 % 4)) / 8;
      const int half = (i16 % 4) & 1;
#pragma unroll
      for (int st = 0; st < NSC; ++st)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int R1 = sub0 + st * 32 + 16 * (g16 >> 1) + 8 * kh + i16 / 4;
          const int R2 = R1 + 4;
          vofs[dt][st][kh][0] = VOFF + R1 * ROWB + (cc ^ chunk_swz<CPR>(R1)) * 16 + half * 8;
          vofs[dt][st][kh][1] = VOFF + R2 * ROWB + (cc ^ chunk_swz<CPR>(R2)) * 16 + half * 8;
        }
    }

    static_assert((NST - 1) * KSTR <= 65535, "stage offsets fit the LDS reads' 16-bit offset field");
    // scores of one tile: its eight K operand reads in two blocks of four, each followed by its MFMAs
    const uint32_t sbase = (uint32_t)(size_t)((PARK_LDS uint8_t*)stages);
    static_assert(KS * NSC == 8, "eight K reads per computed sub-tile set");
    // The accumulators start at 0, or (weighted form) at the keys' logit offsets, which the tile's
    // entries brought into LDS: accumulator e of sub-tile st is key v0 + st * 32 + hl * 16 + e.
    auto s_tile = [&](auto OFFc, f32x16_t(&sa)[NSC], int v0) __attribute__((always_inline)) {
      constexpr int OFF = decltype(OFFc)::value;
      if constexpr (W) {
        const int tile = v0 / BN, sub = v0 % BN;
#pragma unroll
        for (int st = 0; st < NSC; ++st) {
          u32x4_t b[4];
          const uint32_t ba =
              bring_base + (uint32_t)((tile % (2 * NST)) * kWave + sub + st * 32 + (lane_id_opaque() / 32) * 16) * 4u;
          lds_read4_b128<0>(b, ba);
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t u = b[q][e];
              sa[st][q * 4 + e] = __uint_as_float(u);
            }
        }
      } else {
#pragma unroll
        for (int st = 0; st < NSC; ++st)
#pragma unroll
          for (int e = 0; e < 16; ++e) sa[st][e] = 0.f;
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t a[4];
        u32x4_t ka[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int idx = hh * 4 + j;
          a[j] = sbase + kofs[idx / KS][idx % KS];
        }
        lds_read4x_b128<OFF>(ka, a);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int idx = hh * 4 + j;
          sa[idx / KS] = mfma32(ka[j], qb[idx % KS], sa[idx / KS]);
        }
      }
    };
    // the mask of keys past the list end; v0 = the first key
    auto adjust = [&](f32x16_t(&sa)[NSC], int v0) __attribute__((always_inline)) {
      const int nvalid = L - v0;
      if (__builtin_expect(nvalid < NSC * 32, 0)) {
        // accumulator e of sub-tile st is key v0 + st * 32 + hl * 16 + e (hl read again: no register held)
        const int lim = nvalid - (lane_id_opaque() / 32) * 16;
#pragma unroll
        for (int st = 0; st < NSC; ++st)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (st * 32 + e >= lim) sa[st][e] = -INFINITY;
      }
    };
    auto tile_max = [&](const f32x16_t(&sa)[NSC]) __attribute__((always_inline)) {
      float mx = sa[0][0];
#pragma unroll
      for (int st = 0; st < NSC; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sa[st][e]);
      return fmaxf(mx, __shfl_xor(mx, 32, kWave));
    };
    auto weights = [&](const f32x16_t(&sa)[NSC], u32x4_t(&pb)[NSC][2]) __attribute__((always_inline)) {
      const float mb = m_ref * sl2;
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NSC; ++st) {
        float pv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[st][e], sl2, -mb));
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t pk = pack_bf16x2(pv[kh * 8 + 2 * q], pv[kh * 8 + 2 * q + 1]);
            pb[st][kh][q] = pk;
            s4[q] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pk), ones, s4[q], false);
          }
      }
      return (s4[0] + s4[1]) + (s4[2] + s4[3]);
    };
    // V^T operands of a tile: two blocks of eight reads, each followed by its P V MFMAs
    auto pv_tile = [&](auto OFFc, const u32x4_t(&pb)[NSC][2]) __attribute__((always_inline)) {
      constexpr int OFF = decltype(OFFc)::value;
      constexpr int DG = 2 / NSC;
#pragma unroll
      for (int d0 = 0; d0 < DT; d0 += DG) {
        uint32_t a[8];
        u32x2_t r[8];
#pragma unroll
        for (int x = 0; x < DG; ++x)
#pragma unroll
          for (int st = 0; st < NSC; ++st)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
              for (int z = 0; z < 2; ++z) a[((x * NSC + st) * 2 + kh) * 2 + z] = sbase + vofs[d0 + x][st][kh][z];
        tr_read8<OFF>(r, a);
#pragma unroll
        for (int x = 0; x < DG; ++x)
#pragma unroll
          for (int st = 0; st < NSC; ++st)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
              const int j = ((x * NSC + st) * 2 + kh) * 2;
              const u32x4_t va = u32x4_t{r[j][0], r[j][1], r[j + 1][0], r[j + 1][1]};
              o[d0 + x] = mfma32(va, pb[st][kh], o[d0 + x]);
            }
      }
    };

    // one sub-tile set of the stage at LDS offset OFF (its V past VOFF), first key v0; `first`: the
    // wave's first set, which sets the softmax reference
    auto compute = [&](auto OFFc, int v0, bool first) __attribute__((always_inline)) {
      f32x16_t sc[NSC];
      s_tile(OFFc, sc, v0);
      adjust(sc, v0);
      if (first) m_ref = tile_max(sc);
      u32x4_t pb[NSC][2];
      float ps = weights(sc, pb);
      if (__builtin_amdgcn_ballot_w64(!(ps <= kRaise))) {
        // rare: the scores are computed again (the tile is still in LDS), so they need not stay
        // live through the softmax
        f32x16_t s2[NSC];
        s_tile(OFFc, s2, v0);
        adjust(s2, v0);
        const float m_new = fmaxf(m_ref, tile_max(s2));
        const float alpha = __builtin_amdgcn_exp2f((m_ref - m_new) * sl2);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
        m_ref = m_new;
        ps = weights(s2, pb);
      }
      l_run += ps;
      pv_tile(OFFc, pb);
    };

    if (nt > 0) {
      // prologue: entries of tiles 0 .. NST-1 (one wait of the indexer, then a barrier), then, once
      // every copier has read them, those of tiles NST .. 2 NST-2 into the sets just read, then the
      // copies of tiles 0 .. NST-2 into stages 0 .. NST-2
#pragma unroll
      for (int x = 0; x < NST; ++x) load_idx(x, x);
      if (indexer) __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) & lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      int n0[NST][LOADS];
#pragma unroll
      for (int x = 0; x < NST; ++x) read_idx(x, n0[x]);
      // the indexer's next loads land in sets 0 .. NST-2: every copier has read them first (the
      // reads wait for their data), else a late copier could take a later tile's entries
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
#pragma unroll
      for (int x = NST; x < 2 * NST - 1; ++x) load_idx(x % NST, x);
#pragma unroll
      for (int x = 0; x < NST - 1; ++x) issue(n0[x], x, x);
#pragma unroll
      for (int q = 0; q < LOADS; ++q) nnext[q] = n0[NST - 1][q];
    }
    // Iteration t (stage SL = t % NST): wait until tile t landed, copy tile t + NST - 1 into the stage
    // tile t - 1 used, load the entries of tile t + 2 NST - 1, compute tile t, read the entries of
    // tile t + NST. Copier waves: tile t was copied in iteration t - NST + 1 (or in the prologue),
    // after which each of the NST - 2 iterations since issued CP copies. Indexer: the entries of tile
    // t + NST were loaded in iteration t - NST + 1 (or in the prologue), after which NST - 2 index
    // loads followed; its wait before the barrier lets every wave read them at the end of iteration
    // t. The other waves issue no vector-memory operations in the loop.
    for (int t = 0; t < nt; t += NST) {
      const bool go_on = unroll_while<0, NST>([&](auto SLc) __attribute__((always_inline)) {
        constexpr int SL = decltype(SLc)::value;
        constexpr int XS = (SL + NST - 1) % NST;
        const int tt = t + SL;
        if (tt >= nt) return false;
        if (indexer)
          wait_barrier<(NST - 2) * IL>();
        else
          wait_barrier<(NST - 2) * CP>();
        issue(nnext, XS, tt + NST - 1);
        load_idx(XS, tt + 2 * NST - 1);
        // the tile's sub-tiles (split form: this wave's half, if it holds a key of the list)
        const int v0 = tt * BN + sub0;
        if (active && v0 < L) compute(std::integral_constant<int, SL * KSTR>{}, v0, tt == 0);
        read_idx(SL, nnext);
        return true;
      });
      if (!go_on) break;
    }
  };
  if constexpr (D == 64) {
    run(std::integral_constant<int, 64>{});
  } else {
    if (split)
      run(std::integral_constant<int, 64>{});
    else
      run(std::integral_constant<int, 32>{});
  }
  // drain the copies still in flight before the ring is reused or the work-group's LDS handed to
  // another
  __builtin_amdgcn_s_waitcnt(0x0F70);
  // lane-derived values derived again rather than kept live through the tile loop
  {
    const int l = lane_id_opaque();
    const int hl = l / 32;
    const int qpos = qbeg + qw * 32 + l % 32;
    const bool qok = qpos < qend;
    if (split) {
      // merge the second group's (O, reference, sum) into the first's: with m = max(m0, m1),
      // O = O0 2^(sl2 (m0 - m)) + O1 2^(sl2 (m1 - m)) and the same for the sums; a group that met
      // no key of the list has m = -inf and weight 0
      f32x4_t* mrow = reinterpret_cast<f32x4_t*>(stages) + qw * 17 * kWave + l;
      __syncthreads();  // every wave is done with the ring
      if (grp == 1 && active) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            mrow[(dt * 4 + g4) * kWave] = f32x4_t{o[dt][g4 * 4], o[dt][g4 * 4 + 1], o[dt][g4 * 4 + 2], o[dt][g4 * 4 + 3]};
        mrow[16 * kWave] = f32x4_t{m_ref, l_run, 0.f, 0.f};
      }
      __syncthreads();
      if (grp == 0 && active) {
        const f32x4_t ml = mrow[16 * kWave];
        const float m = fmaxf(m_ref, ml[0]);
        const float a0 = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_ref - m) * sl2);
        const float a1 = ml[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((ml[0] - m) * sl2);
        l_run = l_run * a0 + ml[1] * a1;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4_t v = mrow[(dt * 4 + g4) * kWave];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[dt][g4 * 4 + e] = o[dt][g4 * 4 + e] * a0 + v[e] * a1;
          }
        m_ref = m;
      }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
    if (qok && grp == 0) {
      const int qrow = q_perm[(int64_t)h * N + qpos];
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      uint16_t* orow = out + ((int64_t)h * N + qrow) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = dt * 32 + g4 * 8 + hl * 4;
          store_out4<uint16_t>(orow + d0, o[dt][g4 * 4] * inv, o[dt][g4 * 4 + 1] * inv, o[dt][g4 * 4 + 2] * inv,
                               o[dt][g4 * 4 + 3] * inv);
        }
      if (lse != nullptr && hl == 0)
        lse[(int64_t)h * N + qrow] = l_tot > 0.f ? m_ref * scale + logf(l_tot) : -INFINITY;
    }
  }
  __syncthreads();  // the item's LDS is free for the next one
  }
#endif
}


}  // namespace

int64_t attn_max_tiles(const Dims& s, int cq) { return ceil_div(s.N, s.bf16 ? kBf16BM : kAttnBM) + cq; }

size_t attn_run_ints(const Dims& s, int cq, int ck) {
  // + per-head partial statistics: 8 int64 per head, after an alignment of up to 4 bytes; then the
  // work queue: H + 1 int64 head offsets and a uint64 counter
  return (size_t)(s.H * cq) * (size_t)run_stride(ck) + 3 * (size_t)(s.H * cq) + 16 * (size_t)s.H + 1 +
         2 * ((size_t)s.H + 1) + 2;
}

hipError_t launch_sparse_attn(const Dims& s, const void* q, const void* k, const void* v, const int32_t* q_perm,
                              const int32_t* q_offsets, int cq, const int32_t* k_perm, const int32_t* k_offsets,
                              int ck, const int32_t* counts, const int32_t* cols, const float* log_w, float scale,
                              void* out, float* lse, int32_t* tile_base, int32_t* runs, int64_t* stats,
                              hipStream_t st) {
  int32_t* nrun = runs + (size_t)(s.H * cq) * (size_t)run_stride(ck);
  int32_t* glen = nrun + s.H * cq;
  int32_t* nblk = glen + s.H * cq;
  // per-head partial statistics: 8 int64 per head after the counts, aligned up to 8 bytes
  int64_t* spart = reinterpret_cast<int64_t*>((reinterpret_cast<uintptr_t>(nblk + s.H * cq) + 7) & ~uintptr_t(7));
  const int weighted = log_w != nullptr;
  attn_runs<<<dim3((unsigned)cq, (unsigned)s.H), 256, 0, st>>>(counts, cols, k_offsets, s.N, cq, ck, log_w,
                                                               1.f / scale, runs, nrun, glen, nblk);
  attn_order<<<(unsigned)s.H, 1024, 0, st>>>(q_offsets, glen, cq, s.bf16 ? kBf16BM : kAttnBM, tile_base);
  int64_t* hpre = spart + 8 * s.H;
  unsigned long long* qctr = reinterpret_cast<unsigned long long*>(hpre + s.H + 1);
  if (s.bf16) attn_queue_prep<<<1, 1024, 0, st>>>(tile_base, s.H, cq, hpre, qctr);
  if (stats) {
    attn_stats_head<<<(unsigned)s.H, 256, 0, st>>>(q_offsets, k_offsets, cq, ck, glen, nblk, tile_base,
                                                   s.bf16 && s.D == 128 ? kBf16BN : kBN, spart);
    attn_stats_sum<<<1, 64, 0, st>>>(spart, s.H, s.N, stats);
  }
  const dim3 grid((unsigned)attn_max_tiles(s, cq), (unsigned)s.H);
#define PARK_ATTN(T, D)                                                                                          \
  sparse_attn_kernel<T, D><<<grid, 256, 0, st>>>(static_cast<const T*>(q), static_cast<const T*>(k),            \
                                                 static_cast<const T*>(v), s.N, q_perm, q_offsets, cq, tile_base, \
                                                 k_perm, ck, runs, glen, weighted, scale, static_cast<T*>(out), lse);
#define PARK_BF16ATTN(D, W)                                                                                  \
  sparse_attn_bf16<D, W><<<ncu, 768, 0, st>>>(qh, kh, vh, s.N, q_perm, q_offsets, cq, tile_base, k_perm, ck, runs, \
                                            nrun, glen, scale, oh, lse, hpre, qctr, s.H);
  if (s.bf16) {
    // one persistent work-group per CU
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (ncu < 1) ncu = 1;
    const uint16_t* qh = static_cast<const uint16_t*>(q);
    const uint16_t* kh = static_cast<const uint16_t*>(k);
    const uint16_t* vh = static_cast<const uint16_t*>(v);
    uint16_t* oh = static_cast<uint16_t*>(out);
    if (s.D == 128) {
      if (weighted) {
        PARK_BF16ATTN(128, true)
      } else {
        PARK_BF16ATTN(128, false)
      }
    } else {
      if (weighted) {
        PARK_BF16ATTN(64, true)
      } else {
        PARK_BF16ATTN(64, false)
      }
    }
  } else {
    if (s.D == 128) {
      PARK_ATTN(float, 128)
    } else {
      PARK_ATTN(float, 64)
    }
  }
#undef PARK_BF16ATTN
#undef PARK_ATTN
  return hipGetLastError();
}

}  // namespace park
