// PAMA block-importance map (PARK page, Figure 2 caption and abstract): every original query keeps
// its own softmax over the key centroids (logit scale*q.c_j + ln n_j), and the distributions are
// averaged within each query cluster.
//
// Work item = up to 256 consecutive cluster-ordered queries of one query cluster. bf16 data: four
// waves, each handling four 16-query tiles with 16x16x32 MFMA (queries = A rows, centroids = B
// columns), so every centroid fragment loaded feeds four MFMAs.
// Pass 1 keeps a running (reference, sum) per query with one exp2 per logit; pass 2 recomputes
// the logits and adds the normalised weights into per-wave column sums in LDS. Partial column sums of each
// work item are then summed per cluster in fixed order in fp64 and divided by the cluster size.
#include "park_common.h"
#include "park_internal.h"

namespace park {

namespace {

// Per head: chunk_base[i] = work items of query clusters before i; chunk_base[cq] = total.
__global__ __launch_bounds__(1024) void pama_chunks(const int32_t* __restrict__ q_offsets, int cq,
                                                    int32_t* __restrict__ chunk_base) {
  __shared__ int scratch[17];
  const int h = blockIdx.x;
  const int32_t* off = q_offsets + (int64_t)h * (cq + 1);
  int32_t* cb = chunk_base + (int64_t)h * (cq + 1);
  const int per = (cq + 1023) / 1024;
  const int i0 = threadIdx.x * per;
  int local = 0;
  for (int k = 0; k < per; ++k)
    if (i0 + k < cq) local += (off[i0 + k + 1] - off[i0 + k] + kPamaRows - 1) / kPamaRows;
  int total;
  int run = block_exclusive_scan(local, scratch, &total);
  for (int k = 0; k < per; ++k) {
    if (i0 + k < cq) {
      cb[i0 + k] = run;
      run += (off[i0 + k + 1] - off[i0 + k] + kPamaRows - 1) / kPamaRows;
    }
  }
  if (threadIdx.x == 0) cb[cq] = total;
}

// Consumed key centroids (bf16-rounded) and log2 n_j (-inf for empty clusters).
__global__ __launch_bounds__(256) void pama_prep(const float* __restrict__ k_cent, const int32_t* __restrict__ k_off,
                                                 int ck, int D, uint16_t* __restrict__ khat,
                                                 float* __restrict__ logn) {
  const int h = blockIdx.y;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tot = (int64_t)ck * D;
  if (e < tot) khat[(int64_t)h * tot + e] = (uint16_t)f32_to_bf16_bits(k_cent[(int64_t)h * tot + e]);
  if (e < ck) {
    const int n = k_off[(int64_t)h * (ck + 1) + e + 1] - k_off[(int64_t)h * (ck + 1) + e];
    logn[(int64_t)h * ck + e] = n > 0 ? log2f((float)n) : -INFINITY;
  }
}

constexpr int kPamaTW = 4;  // 16-query tiles per MFMA group of a wave

__device__ __forceinline__ int find_item(const int32_t* cb, int cq, int c) {
  // largest i with cb[i] <= c and cb[i+1] > c
  int lo = 0, hi = cq;  // cb[lo] <= c < cb[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cb[mid] <= c)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Work item = up to 256 consecutive cluster-ordered queries (four waves of 64). Column tiles (16
// key centroids, or with FULL 16 keys in cluster order) pass through LDS: each tile is fetched from
// memory once per work-group, one 16-byte piece per thread, into a ring of two buffers (one barrier
// per tile), and every wave reads its MFMA B fragments from there. Rows of a staged tile are
// padded by 16 bytes, so that the 16 column lanes of a fragment read hit distinct banks.
template <int D, bool FULL, int TW>
__global__ __launch_bounds__(256) void pama_bf16(const uint16_t* __restrict__ Q, int64_t N,
                                                 const int32_t* __restrict__ q_perm,
                                                 const int32_t* __restrict__ q_off, int cq,
                                                 const uint16_t* __restrict__ khat, const float* __restrict__ logn,
                                                 int ck, float scale, const int32_t* __restrict__ chunk_base,
                                                 int max_chunks, float* __restrict__ partial,
                                                 const uint16_t* __restrict__ K, int64_t Nk,
                                                 const int32_t* __restrict__ k_perm,
                                                 const int32_t* __restrict__ k_off) {
  constexpr int KS = D / 32;
  // a wave's 64 rows run as 4 / TW groups of TW 16-query tiles (each B fragment feeds TW MFMAs)
  static_assert(TW == 1 || TW == 2 || TW == 4, "tiles per group");
  constexpr int RS = D + 8;      // staged row stride in bf16 elements (16 bytes of padding)
  constexpr int PPR = D / 8;     // 16-byte pieces per row
  __shared__ float colsum[4][kMaxClusters];
  __shared__ float lns[FULL ? 1 : kMaxClusters];
  __shared__ int koff[FULL ? kMaxClusters + 1 : 1];
  __shared__ __attribute__((aligned(16))) uint16_t btile[2][16 * RS];
  const int h = blockIdx.y;
  const int c = blockIdx.x;
  const int32_t* cb = chunk_base + (int64_t)h * (cq + 1);
  if (c >= cb[cq]) return;
  const int i = find_item(cb, cq, c);
  const int32_t* off = q_off + (int64_t)h * (cq + 1);
  const int row0 = off[i] + (c - cb[i]) * kPamaRows;
  const int row_end = min(row0 + kPamaRows, off[i + 1]);
  const int tid = threadIdx.x;
  const int l = lane_id();
  const int w = tid / kWave;
  const int g = l / 16;  // lane group: rows g*4 .. g*4+3 of a tile
  const uint16_t* Qh = Q + (int64_t)h * N * D;
  const int32_t* ph = q_perm + (int64_t)h * N;
  const uint16_t* kh = khat + (int64_t)h * ck * D;
  const uint16_t* Kh = FULL ? K + (int64_t)h * Nk * D : nullptr;
  const int32_t* kph = FULL ? k_perm + (int64_t)h * Nk : nullptr;
  // columns: the key centroids, or (FULL) every key in cluster order, whose weights are summed per
  // key cluster
  const int64_t ncol = FULL ? Nk : ck;
  const int nct = (int)((ncol + 15) / 16);
  for (int j = tid; j < 4 * kMaxClusters; j += 256) (&colsum[0][0])[j] = 0.f;
  if constexpr (FULL) {
    for (int j = tid; j <= ck; j += 256) koff[j] = k_off[(int64_t)h * (ck + 1) + j];
  } else {
    for (int j = tid; j < ck; j += 256) lns[j] = logn[(int64_t)h * ck + j];
  }
  // staging: thread tid < 16 * PPR fetches piece tid % PPR of row tid / PPR of a column tile (rows
  // past the last column are clamped; their weight is -inf)
  const bool stager = tid < 16 * PPR;
  const int sr = tid / PPR, sp = tid % PPR;
  auto gload = [&](int ct) __attribute__((always_inline)) {
    const int64_t j = min((int64_t)ct * 16 + sr, ncol - 1);
    const uint16_t* src = FULL ? Kh + (int64_t)kph[j] * D : kh + j * D;
    return *reinterpret_cast<const u32x4_t*>(src + sp * 8);
  };
  auto sstore = [&](int buf, u32x4_t v) __attribute__((always_inline)) {
    *reinterpret_cast<u32x4_t*>(&btile[buf][sr * RS + sp * 8]) = v;
  };
  // the weight of this lane's column in tile ct (log2 n_j; FULL: 0), -inf past the last column
  auto weight = [&](int ct) __attribute__((always_inline)) {
    const int64_t j = (int64_t)ct * 16 + l % 16;
    if constexpr (FULL)
      return j < ncol ? 0.f : -INFINITY;
    else
      return j < ncol ? lns[j] : -INFINITY;
  };
  // One sweep over the column tiles; body(ct, bv, ln) runs on the waves that hold rows. Every wave
  // takes part in the staging and the barriers.
  auto sweep = [&](bool active, auto&& body) __attribute__((always_inline)) {
    u32x4_t nxt = {0u, 0u, 0u, 0u};
    if (stager) {
      sstore(0, gload(0));
      nxt = gload(min(1, nct - 1));
    }
    for (int ct = 0; ct < nct; ++ct) {
      // tile ct is in buffer ct & 1; every wave is done with tile ct - 1, whose buffer is refilled
      __syncthreads();
      if (stager && ct + 1 < nct) {
        sstore((ct + 1) & 1, nxt);
        nxt = gload(min(ct + 2, nct - 1));
      }
      if (active) {
        u32x4_t bv[KS];
        const uint16_t* bt = &btile[ct & 1][(l % 16) * RS + g * 8];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) bv[kk] = *reinterpret_cast<const u32x4_t*>(bt + kk * 32);
        body(ct, bv, weight(ct));
      }
    }
    __syncthreads();  // the buffers are free for the next sweep
  };

  constexpr float kRaise = 16.f;
  // logit scale in base 2 (kept above 1e-30 so that its reciprocal is finite; below that every
  // logit is log2 n_j to within 1e-28 anyway)
  const float c1 = fmaxf(scale * 1.4426950408889634f, 1e-30f);
  const float ic1 = 1.f / c1;
  int cl = 0;  // FULL: the key cluster of this lane's column (advances with the tiles)
  for (int grp = 0; grp < 4 / TW; ++grp) {
    const int w0 = row0 + w * 64 + grp * 16 * TW;  // this group's first row
    const bool active = w0 < row_end;
    // A operands: query row w0 + t*16 + l%16, dims kk*32 + g*8 .. +7
    u32x4_t qa[TW][KS];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const int r = w0 + t * 16 + l % 16;
      const bool ok = r < row_end;
      const uint16_t* qrow = Qh + (int64_t)(ok ? ph[r] : 0) * D;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (ok) v = *reinterpret_cast<const u32x4_t*>(qrow + kk * 32 + g * 8);
        qa[t][kk] = v;
      }
    }
    // Logits in base 2: lg2 = acc * c1 + log2(n_j), acc = q . c_j. Pass 1 keeps, per lane and row,
    // a reference r and the sum of 2^(lg2 - r) over this lane's columns; the row's accumulators
    // start at nr = -r / c1 instead of 0, so that acc * c1 + log2(n_j) is already lg2 - r: one
    // fma, one exp2 and one add per logit. r is raised only when a logit exceeds it by more than
    // kRaise (the first tile, or rarely later); the raised rows then take their logit computed
    // again from zero accumulators, so that the new reference is exact. nr starts at 1e30: every
    // finite logit raises it, and an empty column (-inf) never meets inf - inf.
    float nr[TW][4], s[TW][4];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        nr[t][e] = 1e30f;
        s[t][e] = 0.f;
      }
    sweep(active, [&](int ct, const u32x4_t* bv, float ln) __attribute__((always_inline)) {
      float d[TW][4], dmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        f32x4_t acc = {nr[t][0], nr[t][1], nr[t][2], nr[t][3]};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) acc = mfma16(qa[t][kk], bv[kk], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          d[t][e] = __builtin_fmaf(acc[e], c1, ln);
          dmax = fmaxf(dmax, d[t][e]);
        }
      }
      if (__builtin_expect(__ballot(dmax > kRaise) != 0, 0)) {
#pragma unroll
        for (int t = 0; t < TW; ++t) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) acc = mfma16(qa[t][kk], bv[kk], acc);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (d[t][e] > kRaise) {
              const float lg = __builtin_fmaf(acc[e], c1, ln);
              s[t][e] *= __builtin_amdgcn_exp2f(-__builtin_fmaf(nr[t][e], c1, lg));  // 2^(r - lg2)
              nr[t][e] = -lg * ic1;
              d[t][e] = 0.f;
            }
        }
      }
#pragma unroll
      for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[t][e] += __builtin_amdgcn_exp2f(d[t][e]);
    });
    // merge (reference, sum) across the 16 lanes (columns) of each group; the row's offset
    // off = r + log2(sum) makes 2^(lg2 - off) its normalised weight (off = +inf for rows that are
    // out of range, whose weights are then 0); pass 2 starts its accumulators at -off / c1
    float roff[TW][4];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float rr = -nr[t][e] * c1;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const float ro = __shfl_xor(rr, o, kWave);
          const float so = __shfl_xor(s[t][e], o, kWave);
          const float rn = fmaxf(rr, ro);
          s[t][e] = s[t][e] * __builtin_amdgcn_exp2f(rr - rn) + so * __builtin_amdgcn_exp2f(ro - rn);
          rr = rn;
        }
        const bool ok = (w0 + t * 16 + g * 4 + e) < row_end && s[t][e] > 0.f;
        roff[t][e] = ok ? -(rr + log2f(s[t][e])) * ic1 : -INFINITY;
      }
    }
    // pass 2: accumulate normalised weights 2^(lg2 - off) into the wave's column sums (the
    // accumulators start at roff = -off / c1, -inf for rows out of range)
    cl = 0;
    sweep(active, [&](int ct, const u32x4_t* bv, float ln) __attribute__((always_inline)) {
      const int64_t j = (int64_t)ct * 16 + l % 16;
      float cs = 0.f;
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        f32x4_t acc = {roff[t][0], roff[t][1], roff[t][2], roff[t][3]};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) acc = mfma16(qa[t][kk], bv[kk], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) cs += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[e], c1, ln));
      }
      cs += __shfl_xor(cs, 16, kWave);
      cs += __shfl_xor(cs, 32, kWave);
      if constexpr (FULL) {
        while (cl < ck && koff[cl + 1] <= j) ++cl;
        if (g == 0 && j < ncol) atomicAdd(&colsum[w][cl], cs);
      } else {
        if (g == 0 && j < ncol) colsum[w][j] += cs;
      }
    });
  }
  float* out = partial + ((int64_t)h * max_chunks + c) * ck;
  for (int j = tid; j < ck; j += 256) out[j] = ((colsum[0][j] + colsum[1][j]) + colsum[2][j]) + colsum[3][j];
}

// fp32 data: one thread per query row, fp64 logits and weights, block-wide column sums.
template <int D>
__global__ __launch_bounds__(256) void pama_f32(const float* __restrict__ Q, int64_t N,
                                                const int32_t* __restrict__ q_perm, const int32_t* __restrict__ q_off,
                                                int cq, const float* __restrict__ k_cent,
                                                const int32_t* __restrict__ k_off, int ck, float scale,
                                                const int32_t* __restrict__ chunk_base, int max_chunks,
                                                float* __restrict__ partial) {
  __shared__ double red[4];
  const int h = blockIdx.y;
  const int c = blockIdx.x;
  const int32_t* cb = chunk_base + (int64_t)h * (cq + 1);
  if (c >= cb[cq]) return;
  const int i = find_item(cb, cq, c);
  const int32_t* off = q_off + (int64_t)h * (cq + 1);
  const int r = off[i] + (c - cb[i]) * kPamaRows + threadIdx.x;
  const bool ok = r < off[i + 1];
  const float* q = Q + ((int64_t)h * N + (ok ? q_perm[(int64_t)h * N + r] : 0)) * D;
  const float* kc = k_cent + (int64_t)h * ck * D;
  const int32_t* ko = k_off + (int64_t)h * (ck + 1);
  double m = -INFINITY, s = 0.0;
  for (int j = 0; j < ck; ++j) {
    const int n = ko[j + 1] - ko[j];
    if (n == 0) continue;
    double dot = 0.0;
    for (int a = 0; a < D; ++a) dot += (double)q[a] * (double)kc[j * D + a];
    const double lg = (double)scale * dot + log((double)n);
    if (lg > m) {
      s = s * exp(m - lg) + 1.0;
      m = lg;
    } else {
      s += exp(lg - m);
    }
  }
  float* out = partial + ((int64_t)h * max_chunks + c) * ck;
  for (int j = 0; j < ck; ++j) {
    const int n = ko[j + 1] - ko[j];
    double wv = 0.0;
    if (ok && n > 0) {
      double dot = 0.0;
      for (int a = 0; a < D; ++a) dot += (double)q[a] * (double)kc[j * D + a];
      wv = exp((double)scale * dot + log((double)n) - m) / s;
    }
    wv = wave_sum_f64(wv);
    if (lane_id() == 0) red[threadIdx.x / kWave] = wv;
    __syncthreads();
    if (threadIdx.x == 0) out[j] = (float)(((red[0] + red[1]) + red[2]) + red[3]);
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void pama_reduce(const float* __restrict__ partial, const int32_t* __restrict__ q_off,
                                                   const int32_t* __restrict__ chunk_base, int cq, int ck,
                                                   int max_chunks, float* __restrict__ map) {
  const int h = blockIdx.y;
  const int i = blockIdx.x;
  const int32_t* cb = chunk_base + (int64_t)h * (cq + 1);
  const int n = q_off[(int64_t)h * (cq + 1) + i + 1] - q_off[(int64_t)h * (cq + 1) + i];
  float* row = map + ((int64_t)h * cq + i) * ck;
  for (int j = threadIdx.x; j < ck; j += 256) {
    double s = 0.0;
    for (int c = cb[i]; c < cb[i + 1]; ++c) s += (double)partial[((int64_t)h * max_chunks + c) * ck + j];
    row[j] = n > 0 ? (float)(s / (double)n) : 0.f;
  }
}

}  // namespace

int64_t pama_max_chunks(const Dims& s, int cq) { return ceil_div(s.N, kPamaRows) + cq; }

hipError_t launch_pama(const Dims& s, const void* q, const int32_t* q_perm, const int32_t* q_offsets, int cq,
                       const float* k_cent, const int32_t* k_offsets, int ck, float scale, float* map, void* khat,
                       float* logn, int32_t* chunk_base, float* partial, hipStream_t st) {
  const int maxc = (int)pama_max_chunks(s, cq);
  pama_chunks<<<(unsigned)s.H, 1024, 0, st>>>(q_offsets, cq, chunk_base);
  const dim3 grid((unsigned)maxc, (unsigned)s.H);
  if (s.bf16) {
    const dim3 pg((unsigned)ceil_div((int64_t)ck * s.D, 256), (unsigned)s.H);
    pama_prep<<<pg, 256, 0, st>>>(k_cent, k_offsets, ck, (int)s.D, static_cast<uint16_t*>(khat), logn);
    if (s.D == 128)
      pama_bf16<128, false, kPamaTW><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(q), s.N, q_perm, q_offsets, cq,
                                                  static_cast<const uint16_t*>(khat), logn, ck, scale, chunk_base,
                                                  maxc, partial, nullptr, 0, nullptr, nullptr);
    else
      pama_bf16<64, false, kPamaTW><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(q), s.N, q_perm, q_offsets, cq,
                                                 static_cast<const uint16_t*>(khat), logn, ck, scale, chunk_base,
                                                 maxc, partial, nullptr, 0, nullptr, nullptr);
  } else {
    if (s.D == 128)
      pama_f32<128><<<grid, 256, 0, st>>>(static_cast<const float*>(q), s.N, q_perm, q_offsets, cq, k_cent,
                                          k_offsets, ck, scale, chunk_base, maxc, partial);
    else
      pama_f32<64><<<grid, 256, 0, st>>>(static_cast<const float*>(q), s.N, q_perm, q_offsets, cq, k_cent,
                                         k_offsets, ck, scale, chunk_base, maxc, partial);
  }
  pama_reduce<<<dim3((unsigned)cq, (unsigned)s.H), 256, 0, st>>>(partial, q_offsets, chunk_base, cq, ck, maxc, map);
  return hipGetLastError();
}

namespace {
// Centroid queries for the centroid-query estimators: rows[h][i] = bf16(cent[h][i]) (as consumed by
// the MFMA); each non-empty query cluster owns one row (perm lists them in order, offsets count
// them), an empty one owns none, so its map row stays zero.
__global__ __launch_bounds__(1024) void centroid_queries(const float* __restrict__ cent, int C, int D,
                                                         const int32_t* __restrict__ q_offsets,
                                                         uint16_t* __restrict__ rows, int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ offsets) {
  __shared__ int scratch[17];
  const int h = blockIdx.x;
  const int32_t* qo = q_offsets + (int64_t)h * (C + 1);
  for (int64_t e = threadIdx.x; e < (int64_t)C * D; e += 1024)
    rows[(int64_t)h * C * D + e] = (uint16_t)f32_to_bf16_bits(cent[(int64_t)h * C * D + e]);
  const int per = (C + 1023) / 1024;
  const int i0 = threadIdx.x * per;
  int local = 0;
  for (int k = 0; k < per; ++k)
    if (i0 + k < C) local += qo[i0 + k + 1] > qo[i0 + k];
  int total;
  int run = block_exclusive_scan(local, scratch, &total);
  for (int k = 0; k < per; ++k) {
    const int i = i0 + k;
    if (i < C) {
      offsets[(int64_t)h * (C + 1) + i] = run;
      if (qo[i + 1] > qo[i]) perm[(int64_t)h * C + run++] = i;
    }
  }
  if (threadIdx.x == 0) offsets[(int64_t)h * (C + 1) + C] = total;
}
}  // namespace

hipError_t launch_centroid_queries(int64_t H, int C, int D, const float* cent, const int32_t* q_offsets, void* rows,
                                   int32_t* perm, int32_t* offsets, hipStream_t st) {
  centroid_queries<<<(unsigned)H, 1024, 0, st>>>(cent, C, D, q_offsets, static_cast<uint16_t*>(rows), perm, offsets);
  return hipGetLastError();
}

hipError_t launch_block_mass(const Dims& s, const void* q, const int32_t* q_perm, const int32_t* q_offsets, int cq,
                             const void* k, int64_t nk, const int32_t* k_perm, const int32_t* k_offsets, int ck,
                             float scale, float* map, int32_t* chunk_base, float* partial, hipStream_t st) {
  const int maxc = (int)pama_max_chunks(s, cq);
  pama_chunks<<<(unsigned)s.H, 1024, 0, st>>>(q_offsets, cq, chunk_base);
  const dim3 grid((unsigned)maxc, (unsigned)s.H);
  const uint16_t* qh = static_cast<const uint16_t*>(q);
  const uint16_t* kh = static_cast<const uint16_t*>(k);
  if (s.D == 128)
    pama_bf16<128, true, kPamaTW><<<grid, 256, 0, st>>>(qh, s.N, q_perm, q_offsets, cq, nullptr, nullptr, ck, scale, chunk_base,
                                               maxc, partial, kh, nk, k_perm, k_offsets);
  else
    pama_bf16<64, true, kPamaTW><<<grid, 256, 0, st>>>(qh, s.N, q_perm, q_offsets, cq, nullptr, nullptr, ck, scale, chunk_base,
                                              maxc, partial, kh, nk, k_perm, k_offsets);
  pama_reduce<<<dim3((unsigned)cq, (unsigned)s.H), 256, 0, st>>>(partial, q_offsets, chunk_base, cq, ck, maxc, map);
  return hipGetLastError();
}


// Centroid-query / full-key map (the CF estimator: the query centroid's softmax over every key,
// summed per key cluster). Rows are the Cq bf16 centroid rows of a head, few against N keys, so the
// work is split over the keys: a first pass keeps per (row, 1024-key chunk) a running (reference,
// sum) in base 2, a merge folds the chunks in order into each row's offset r + log2(sum), and a
// second pass gives each work-group eight key clusters, walks their keys in cluster order and
// writes each (row, cluster) mass directly (lane sums reduced in a fixed order, no atomics).
namespace {
constexpr int kCfChunk = 1024;   // key positions per first-pass work-group
constexpr int kCfClusters = 8;   // key clusters per second-pass work-group
constexpr int kCfTW = 2;         // 16-row tiles per wave

// A operands of row tile rt: centroid row rt * 16 + l % 16 (clamped), dims kk * 32 + g * 8 .. +7
template <int KS>
__device__ __forceinline__ void cf_rows(const uint16_t* R, int cq, int rt, int l, int g, u32x4_t* qa) {
  const int r = min(rt * 16 + l % 16, cq - 1);
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) qa[kk] = *reinterpret_cast<const u32x4_t*>(R + (int64_t)r * (KS * 32) + kk * 32 + g * 8);
}

// B operands of the key at cluster-order position pos (clamped to the last key)
template <int KS>
__device__ __forceinline__ void cf_key(const uint16_t* Kh, const int32_t* kp, int64_t nk, int64_t pos, int g,
                                       u32x4_t* bv) {
  const int64_t row = kp[pos < nk ? pos : nk - 1];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) bv[kk] = *reinterpret_cast<const u32x4_t*>(Kh + row * (KS * 32) + kk * 32 + g * 8);
}

template <int D>
__global__ __launch_bounds__(256) void cf_lse(const uint16_t* __restrict__ rows, int cq,
                                              const uint16_t* __restrict__ K, int64_t N,
                                              const int32_t* __restrict__ k_perm, float c1, int nchunk,
                                              float* __restrict__ part) {
  constexpr int KS = D / 32;
  constexpr float kRaise = 16.f;
  const int h = blockIdx.y, ch = blockIdx.x;
  const int l = lane_id(), w = threadIdx.x / kWave, g = l / 16;
  const uint16_t* Rh = rows + (int64_t)h * cq * D;
  const uint16_t* Kh = K + (int64_t)h * N * D;
  const int32_t* kp = k_perm + (int64_t)h * N;
  const int64_t p0 = (int64_t)ch * kCfChunk;
  const int nkt = (int)((min<int64_t>(p0 + kCfChunk, N) - p0 + 15) / 16);
  const int nrt = (cq + 15) / 16;
  for (int rt0 = w * kCfTW; rt0 < nrt; rt0 += 4 * kCfTW) {
    u32x4_t qa[kCfTW][KS];
#pragma unroll
    for (int t = 0; t < kCfTW; ++t) cf_rows<KS>(Rh, cq, rt0 + t, l, g, qa[t]);
    float r[kCfTW][4], s[kCfTW][4];
#pragma unroll
    for (int t = 0; t < kCfTW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r[t][e] = -1e30f;
        s[t][e] = 0.f;
      }
    for (int kt = 0; kt < nkt; ++kt) {
      const int64_t pos = p0 + kt * 16 + l % 16;
      u32x4_t bv[KS];
      cf_key<KS>(Kh, kp, N, pos, g, bv);
      const float ln = pos < N ? 0.f : -INFINITY;
      float lg[kCfTW][4], dmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < kCfTW; ++t) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) acc = mfma16(qa[t][kk], bv[kk], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lg[t][e] = __builtin_fmaf(acc[e], c1, ln);
          dmax = fmaxf(dmax, lg[t][e] - r[t][e]);
        }
      }
      if (__builtin_expect(__ballot(dmax > kRaise) != 0, 0)) {
#pragma unroll
        for (int t = 0; t < kCfTW; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (lg[t][e] - r[t][e] > kRaise) {
              s[t][e] *= __builtin_amdgcn_exp2f(r[t][e] - lg[t][e]);
              r[t][e] = lg[t][e];
            }
      }
#pragma unroll
      for (int t = 0; t < kCfTW; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[t][e] += __builtin_amdgcn_exp2f(lg[t][e] - r[t][e]);
    }
#pragma unroll
    for (int t = 0; t < kCfTW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const float ro = __shfl_xor(r[t][e], o, kWave);
          const float so = __shfl_xor(s[t][e], o, kWave);
          const float rn = fmaxf(r[t][e], ro);
          s[t][e] = s[t][e] * __builtin_amdgcn_exp2f(r[t][e] - rn) + so * __builtin_amdgcn_exp2f(ro - rn);
          r[t][e] = rn;
        }
        const int row = (rt0 + t) * 16 + g * 4 + e;
        if (l % 16 == 0 && row < cq) {
          float* dst = part + (((int64_t)h * nchunk + ch) * cq + row) * 2;
          dst[0] = r[t][e];
          dst[1] = s[t][e];
        }
      }
  }
}

// Per row: fold the chunks' (reference, sum) pairs in chunk order into off = r + log2(sum).
__global__ __launch_bounds__(256) void cf_merge(const float* __restrict__ part, int nchunk, int cq,
                                                float* __restrict__ off) {
  const int h = blockIdx.y;
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= cq) return;
  float r = -1e30f, s = 0.f;
  for (int c = 0; c < nchunk; ++c) {
    const float* p = part + (((int64_t)h * nchunk + c) * cq + row) * 2;
    const float rc = p[0], sc = p[1];
    const float rn = fmaxf(r, rc);
    s = s * __builtin_amdgcn_exp2f(r - rn) + sc * __builtin_amdgcn_exp2f(rc - rn);
    r = rn;
  }
  off[(int64_t)h * cq + row] = s > 0.f ? r + log2f(s) : INFINITY;
}

template <int D>
__global__ __launch_bounds__(256) void cf_mass(const uint16_t* __restrict__ rows, const int32_t* __restrict__ q_off,
                                               int cq, const uint16_t* __restrict__ K, int64_t N,
                                               const int32_t* __restrict__ k_perm,
                                               const int32_t* __restrict__ k_off, int ck, float c1,
                                               const float* __restrict__ off, float* __restrict__ map) {
  constexpr int KS = D / 32;
  const int h = blockIdx.y;
  const int j0 = blockIdx.x * kCfClusters, j1 = min(j0 + kCfClusters, ck);
  const int l = lane_id(), w = threadIdx.x / kWave, g = l / 16;
  const uint16_t* Rh = rows + (int64_t)h * cq * D;
  const uint16_t* Kh = K + (int64_t)h * N * D;
  const int32_t* kp = k_perm + (int64_t)h * N;
  const int32_t* ko = k_off + (int64_t)h * (ck + 1);
  const int32_t* qo = q_off + (int64_t)h * (cq + 1);
  const int nrt = (cq + 15) / 16;
  for (int rt0 = w * kCfTW; rt0 < nrt; rt0 += 4 * kCfTW) {
    u32x4_t qa[kCfTW][KS];
    float ro[kCfTW][4];
#pragma unroll
    for (int t = 0; t < kCfTW; ++t) {
      cf_rows<KS>(Rh, cq, rt0 + t, l, g, qa[t]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = (rt0 + t) * 16 + g * 4 + e;
        ro[t][e] = row < cq ? off[(int64_t)h * cq + row] : INFINITY;
      }
    }
    for (int j = j0; j < j1; ++j) {
      const int a = max(ko[j], 0), b = (int)min<int64_t>(ko[j + 1], N);  // malformed offsets stay in range
      float cs[kCfTW][4];
#pragma unroll
      for (int t = 0; t < kCfTW; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) cs[t][e] = 0.f;
      for (int p = a; p < b; p += 16) {
        const int pos = p + l % 16;
        u32x4_t bv[KS];
        cf_key<KS>(Kh, kp, N, pos, g, bv);
        const bool ok = pos < b;
#pragma unroll
        for (int t = 0; t < kCfTW; ++t) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) acc = mfma16(qa[t][kk], bv[kk], acc);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = __builtin_amdgcn_exp2f(acc[e] * c1 - ro[t][e]);
            cs[t][e] += ok ? v : 0.f;
          }
        }
      }
#pragma unroll
      for (int t = 0; t < kCfTW; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) cs[t][e] += __shfl_xor(cs[t][e], o, kWave);
          const int row = (rt0 + t) * 16 + g * 4 + e;
          if (l % 16 == 0 && row < cq) map[((int64_t)h * cq + row) * ck + j] = qo[row + 1] > qo[row] ? cs[t][e] : 0.f;
        }
    }
  }
}
}  // namespace

int64_t cf_chunks(const Dims& s) { return ceil_div(s.N, kCfChunk); }

hipError_t launch_cf_map(const Dims& s, const void* rows, const int32_t* q_offsets, int cq, const void* k,
                         const int32_t* k_perm, const int32_t* k_offsets, int ck, float scale, float* map, float* part,
                         float* off, hipStream_t st) {
  const int nchunk = (int)cf_chunks(s);
  const float c1 = scale * 1.4426950408889634f;
  const uint16_t* rh = static_cast<const uint16_t*>(rows);
  const uint16_t* kh = static_cast<const uint16_t*>(k);
  const dim3 g1((unsigned)nchunk, (unsigned)s.H), g2((unsigned)ceil_div(cq, 256), (unsigned)s.H),
      g3((unsigned)ceil_div(ck, kCfClusters), (unsigned)s.H);
  if (s.D == 128) {
    cf_lse<128><<<g1, 256, 0, st>>>(rh, cq, kh, s.N, k_perm, c1, nchunk, part);
    cf_merge<<<g2, 256, 0, st>>>(part, nchunk, cq, off);
    cf_mass<128><<<g3, 256, 0, st>>>(rh, q_offsets, cq, kh, s.N, k_perm, k_offsets, ck, c1, off, map);
  } else {
    cf_lse<64><<<g1, 256, 0, st>>>(rh, cq, kh, s.N, k_perm, c1, nchunk, part);
    cf_merge<<<g2, 256, 0, st>>>(part, nchunk, cq, off);
    cf_mass<64><<<g3, 256, 0, st>>>(rh, q_offsets, cq, kh, s.N, k_perm, k_offsets, ck, c1, off, map);
  }
  return hipGetLastError();
}

}  // namespace park
