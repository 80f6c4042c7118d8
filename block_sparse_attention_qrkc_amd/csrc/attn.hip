// Block-sparse attention over the selected (query cluster, key cluster) pairs (PARK abstract:
// attention is computed only within the retrieved blocks).
//
// Schedule: a work item is one 128-query tile of one query cluster. The key clusters a query
// cluster selected are merged into runs of contiguous cluster-ordered key positions, and the runs
// are concatenated into one virtual key sequence, so key tiles of 64 are full MFMA tiles except the
// last one of each item, however small the individual clusters are.
//
// Kernel: four waves x 32 queries. Per 64-key tile, keys and values are gathered through the key
// permutation into LDS (values transposed), S^T = K Q^T and O^T += V^T P^T run on 32x32x16 bf16
// MFMA with fp32 accumulation, and an online softmax in exp2 form keeps one running max and sum per
// query. Outputs are written straight to the queries' original rows.
#include "park_common.h"
#include "park_internal.h"

namespace park {

namespace {

// Per head: tile_base[i] = tiles of query clusters before i; tile_base[cq] = total.
__global__ __launch_bounds__(1024) void attn_tiles(const int32_t* __restrict__ q_offsets, int cq,
                                                   int32_t* __restrict__ tile_base) {
  __shared__ int scratch[17];
  const int h = blockIdx.x;
  const int32_t* off = q_offsets + (int64_t)h * (cq + 1);
  int32_t* tb = tile_base + (int64_t)h * (cq + 1);
  const int per = (cq + 1023) / 1024;
  const int i0 = threadIdx.x * per;
  int local = 0;
  for (int k = 0; k < per; ++k)
    if (i0 + k < cq) local += (off[i0 + k + 1] - off[i0 + k] + kAttnBM - 1) / kAttnBM;
  int total;
  int run = block_exclusive_scan(local, scratch, &total);
  for (int k = 0; k < per; ++k) {
    if (i0 + k < cq) {
      tb[i0 + k] = run;
      run += (off[i0 + k + 1] - off[i0 + k] + kAttnBM - 1) / kAttnBM;
    }
  }
  if (threadIdx.x == 0) tb[cq] = total;
}

// Per (query cluster, head): runs of contiguous key positions. Layout of one row's record
// (stride 2*ck + 3 ints): [0] = number of runs R, [1 .. R+1] = virtual starts (the last one is the
// total key count), [ck + 2 .. ck + 2 + R) = key-position starts.
__global__ __launch_bounds__(256) void attn_runs(const int32_t* __restrict__ counts, const int32_t* __restrict__ cols,
                                                 const int32_t* __restrict__ k_offsets, int cq, int ck,
                                                 int32_t* __restrict__ runs) {
  __shared__ int iscratch[17];
  __shared__ int iscratch2[17];
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  int cnt = counts[(int64_t)h * cq + i];
  cnt = cnt < 0 ? 0 : (cnt > ck ? ck : cnt);
  const int32_t* crow = cols + ((int64_t)h * cq + i) * ck;
  const int32_t* ko = k_offsets + (int64_t)h * (ck + 1);
  int32_t* rec = runs + ((int64_t)h * cq + i) * (2 * ck + 3);
  const int per = (cnt + 255) / 256;
  const int m0 = tid * per;
  int nflag = 0, len = 0;
  for (int e = 0; e < per; ++e) {
    const int m = m0 + e;
    if (m < cnt) {
      const int j = crow[m];
      const bool jok = j >= 0 && j < ck;
      const int a = jok ? ko[j] : 0, b = jok ? ko[j + 1] : 0;
      if (b > a) {
        len += b - a;
        bool start = true;
        if (m > 0) {
          const int jp = crow[m - 1];
          if (jp >= 0 && jp < ck && ko[jp + 1] > ko[jp] && ko[jp + 1] == a) start = false;
        }
        nflag += start;
      }
    }
  }
  int nruns, total_len;
  int rid = block_exclusive_scan(nflag, iscratch, &nruns);
  int vpos = block_exclusive_scan(len, iscratch2, &total_len);
  for (int e = 0; e < per; ++e) {
    const int m = m0 + e;
    if (m < cnt) {
      const int j = crow[m];
      const bool jok = j >= 0 && j < ck;
      const int a = jok ? ko[j] : 0, b = jok ? ko[j + 1] : 0;
      if (b > a) {
        bool start = true;
        if (m > 0) {
          const int jp = crow[m - 1];
          if (jp >= 0 && jp < ck && ko[jp + 1] > ko[jp] && ko[jp + 1] == a) start = false;
        }
        if (start) {
          rec[1 + rid] = vpos;
          rec[ck + 2 + rid] = a;
          ++rid;
        }
        vpos += b - a;
      }
    }
  }
  if (tid == 0) {
    rec[0] = nruns;
    rec[1 + nruns] = total_len;
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

template <typename T>
__device__ __forceinline__ void store_out4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store_out4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
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
                                                          const int32_t* __restrict__ k_perm,
                                                          const int32_t* __restrict__ tile_base,
                                                          const int32_t* __restrict__ runs, int ck, float scale,
                                                          T* __restrict__ out, float* __restrict__ lse) {
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int KSTR = D + 8;
  constexpr int VSTR = kBN + 8;
  __shared__ __attribute__((aligned(16))) uint16_t ks[kBN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VSTR];
  __shared__ int32_t krow[kBN];
  __shared__ int32_t run_v[kMaxClusters + 1];
  __shared__ int32_t run_k[kMaxClusters];

  const int h = blockIdx.y;
  const int c = blockIdx.x;
  const int32_t* tb = tile_base + (int64_t)h * (cq + 1);
  if (c >= tb[cq]) return;
  const int i = find_tile(tb, cq, c);
  const int tid = threadIdx.x;
  const int l = lane_id();
  const int w = tid / kWave;
  const int hl = l / 32;
  const int32_t* qo = q_off + (int64_t)h * (cq + 1);
  const int qbeg = qo[i] + (c - tb[i]) * kAttnBM;
  const int qend = min(qbeg + kAttnBM, qo[i + 1]);
  const int32_t* rec = runs + ((int64_t)h * cq + i) * (2 * ck + 3);
  const int nr = rec[0];
  for (int e = tid; e <= nr; e += 256) run_v[e] = rec[1 + e];
  for (int e = tid; e < nr; e += 256) run_k[e] = rec[ck + 2 + e];
  const T* Qh = Q + (int64_t)h * N * D;
  const T* Kh = K + (int64_t)h * N * D;
  const T* Vh = V + (int64_t)h * N * D;
  const int32_t* kp = k_perm + (int64_t)h * N;

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
  __syncthreads();
  const int L = run_v[nr];
  // A-operand row of S^T held by lane l: physical key of MFMA row l%32 (see below)
  const int r = l % 32;
  const int prow = ((r / 4) % 2) * 16 + (r / 8) * 4 + r % 4;

  for (int v0 = 0; v0 < L; v0 += kBN) {
    if (tid < kBN) {
      const int v = v0 + tid;
      int row = -1;
      if (v < L) {
        int lo = 0, hi = nr;  // run_v[lo] <= v < run_v[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (run_v[mid] <= v)
            lo = mid;
          else
            hi = mid;
        }
        row = kp[run_k[lo] + (v - run_v[lo])];
      }
      krow[tid] = row;
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

}  // namespace

int64_t attn_max_tiles(const Dims& s, int cq) { return ceil_div(s.N, kAttnBM) + cq; }

hipError_t launch_sparse_attn(const Dims& s, const void* q, const void* k, const void* v, const int32_t* q_perm,
                              const int32_t* q_offsets, int cq, const int32_t* k_perm, const int32_t* k_offsets,
                              int ck, const int32_t* counts, const int32_t* cols, float scale, void* out, float* lse,
                              int32_t* tile_base, int32_t* runs, hipStream_t st) {
  attn_tiles<<<(unsigned)s.H, 1024, 0, st>>>(q_offsets, cq, tile_base);
  attn_runs<<<dim3((unsigned)cq, (unsigned)s.H), 256, 0, st>>>(counts, cols, k_offsets, cq, ck, runs);
  const dim3 grid((unsigned)attn_max_tiles(s, cq), (unsigned)s.H);
#define PARK_ATTN(T, D)                                                                                          \
  sparse_attn_kernel<T, D><<<grid, 256, 0, st>>>(static_cast<const T*>(q), static_cast<const T*>(k),            \
                                                 static_cast<const T*>(v), s.N, q_perm, q_offsets, cq, k_perm, \
                                                 tile_base, runs, ck, scale, static_cast<T*>(out), lse);
  if (s.bf16) {
    if (s.D == 128) {
      PARK_ATTN(uint16_t, 128)
    } else {
      PARK_ATTN(uint16_t, 64)
    }
  } else {
    if (s.D == 128) {
      PARK_ATTN(float, 128)
    } else {
      PARK_ATTN(float, 64)
    }
  }
#undef PARK_ATTN
  return hipGetLastError();
}

}  // namespace park
