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


// ------------------------------------------------------------------------------------------------
// bf16 kernel: key/value tiles are copied HBM -> LDS with gfx950 direct loads (no register staging),
// double-buffered so the copy of tile t+1 overlaps the MFMA work on tile t. Rows stay row-major in
// LDS with their 16-byte chunks XOR-swizzled by row (bank spread); V^T operands come from the
// transposing LDS read (each lane of a 16-lane group receives 4 keys of one column).
// ------------------------------------------------------------------------------------------------

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
#define PARK_LDS __attribute__((address_space(3)))

template <int CPR>
__device__ __forceinline__ int chunk_swz(int r) {
  return CPR == 16 ? ((r & 7) | (((r >> 4) & 1) << 3)) : (r & 7);
}

// vmcnt(0): wait until this wave's vector-memory operations (including LDS-direct loads) are done
#define PARK_WAIT_VMEM() __builtin_amdgcn_s_waitcnt(0x0F70)

template <int D>
struct AttnTileLoader {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int ROWB = D * 2;         // bytes per row
  static constexpr int TILEB = kBN * ROWB;   // bytes per K (or V) tile
  static constexpr int RPB = 1024 / ROWB;    // rows per 1 KB wave load
  static constexpr int LOADS = TILEB / 4096; // wave loads per wave per tile (4 waves)
};

constexpr int kAttnMaxRuns = 1024;  // runs kept in LDS by the direct-load kernel

template <int D>
__global__ __launch_bounds__(256, 2) void sparse_attn_bf16(const uint16_t* __restrict__ Q,
                                                           const uint16_t* __restrict__ K,
                                                           const uint16_t* __restrict__ V, int64_t N,
                                                           const int32_t* __restrict__ q_perm,
                                                           const int32_t* __restrict__ q_off, int cq,
                                                           const int32_t* __restrict__ k_perm,
                                                           const int32_t* __restrict__ tile_base,
                                                           const int32_t* __restrict__ runs, int ck, float scale,
                                                           uint16_t* __restrict__ out, float* __restrict__ lse) {
  using TL = AttnTileLoader<D>;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int CPR = TL::CPR;
  constexpr int ROWB = TL::ROWB;
  constexpr int TILEB = TL::TILEB;
  constexpr int RPB = TL::RPB;
  constexpr int LOADS = TL::LOADS;
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[TILEB];
  __shared__ int32_t run_v[kAttnMaxRuns + 1];
  __shared__ int32_t run_k[kAttnMaxRuns];

  const int h = blockIdx.y;
  const int c = blockIdx.x;
  const int32_t* tb = tile_base + (int64_t)h * (cq + 1);
  if (c >= tb[cq]) return;
  const int i = find_tile(tb, cq, c);
  const int l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int hl = l / 32;
  const int32_t* qo = q_off + (int64_t)h * (cq + 1);
  const int qbeg = qo[i] + (c - tb[i]) * kAttnBM;
  const int qend = min(qbeg + kAttnBM, qo[i + 1]);
  const int32_t* rec = runs + ((int64_t)h * cq + i) * (2 * ck + 3);
  const int nr = rec[0];
  for (int e = threadIdx.x; e <= nr; e += 256) run_v[e] = rec[1 + e];
  for (int e = threadIdx.x; e < nr; e += 256) run_k[e] = rec[ck + 2 + e];
  const uint16_t* Qh = Q + (int64_t)h * N * D;
  const uint16_t* Kh = K + (int64_t)h * N * D;
  const uint16_t* Vh = V + (int64_t)h * N * D;
  const int32_t* kp = k_perm + (int64_t)h * N;

  const int qpos = qbeg + w * 32 + l % 32;
  const bool qok = qpos < qend;
  const int qrow = qok ? q_perm[(int64_t)h * N + qpos] : 0;
  u32x4_t qb[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (qok) v = *reinterpret_cast<const u32x4_t*>(Qh + (int64_t)qrow * D + kk * 16 + hl * 8);
    qb[kk] = v;
  }
  __syncthreads();
  const int L = run_v[nr];

  // load slots: slot q of this lane copies tile row trow[q], logical chunk lchunk[q], into physical
  // chunk l % CPR of the wave's 1 KB block (w * LOADS + q)
  int trow[LOADS], cur[LOADS], lchunk[LOADS], nrow[LOADS];
#pragma unroll
  for (int q = 0; q < LOADS; ++q) {
    trow[q] = (w * LOADS + q) * RPB + l / CPR;
    cur[q] = 0;
    lchunk[q] = (l % CPR) ^ chunk_swz<CPR>(trow[q]);
  }
  // rows of the keys of tile starting at v0 (keys past the end read row 0: finite, masked)
  auto fetch_rows = [&](int v0) {
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
      const int v = v0 + trow[q];
      int pos = -1;
      if (v < L) {
        while (run_v[cur[q] + 1] <= v) ++cur[q];
        pos = run_k[cur[q]] + (v - run_v[cur[q]]);
      }
      nrow[q] = pos >= 0 ? kp[pos] : 0;
    }
  };
  auto issue = [&](uint8_t* kbuf, uint8_t* vbuf) {
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
      const int64_t goff = (int64_t)nrow[q] * D + lchunk[q] * 8;
      const int boff = (w * LOADS + q) * 1024;
      __builtin_amdgcn_global_load_lds(Kh + goff, (PARK_LDS void*)(kbuf + boff), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(Vh + goff, (PARK_LDS void*)(vbuf + boff), 16, 0, 0);
    }
  };

  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  const float sl2 = scale * 1.4426950408889634f;
  // softmax reference: the running max is only raised when a score exceeds it by more than
  // 8 / sl2 (p stays below 2^8), which skips almost every rescale of O
  const float thresh = 8.0f / sl2;
  float m_ref = -INFINITY;
  float l_run = 0.f;
  const int r = l % 32;
  const int prow = ((r / 4) % 2) * 16 + (r / 8) * 4 + r % 4;
  const int g16 = l / 16, i16 = l % 16;

  auto compute = [&](const uint8_t* kt, const uint8_t* vt, int v0) {
    f32x16_t sacc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int R = st * 32 + prow;
      const uint8_t* krow = kt + R * ROWB;
      const int sw = chunk_swz<CPR>(R);
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[st][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(krow + ((2 * kk + hl) ^ sw) * 16);
        sacc[st] = mfma32(a, qb[kk], sacc[st]);
      }
    }
    const int nvalid = L - v0;
    if (nvalid < kBN) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (st * 32 + hl * 16 + e >= nvalid) sacc[st][e] = -INFINITY;
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[st][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const bool raise = mx > m_ref + thresh;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float m_new = raise ? mx : m_ref;
      const float alpha = __builtin_amdgcn_exp2f((m_ref - m_new) * sl2);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
      m_ref = m_new;
    }
    const float mb = m_ref * sl2;
    u32x4_t pb[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float pv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[st][e], sl2, -mb));
        l_run += pv[e];
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int q = 0; q < 4; ++q) pb[st][kh][q] = pack_bf16x2(pv[kh * 8 + 2 * q], pv[kh * 8 + 2 * q + 1]);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int D0 = dt * 32 + 16 * (g16 & 1);
      const int cc = (D0 + 4 * (i16 % 4)) / 8;
      const int half = (i16 % 4) & 1;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int R1 = st * 32 + 16 * (g16 >> 1) + 8 * kh + i16 / 4;
          const int R2 = R1 + 4;
          const s16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (PARK_LDS s16x4_t*)(vt + R1 * ROWB + (cc ^ chunk_swz<CPR>(R1)) * 16 + half * 8));
          const s16x4_t t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (PARK_LDS s16x4_t*)(vt + R2 * ROWB + (cc ^ chunk_swz<CPR>(R2)) * 16 + half * 8));
          const u32x2_t a1 = __builtin_bit_cast(u32x2_t, t1);
          const u32x2_t a2 = __builtin_bit_cast(u32x2_t, t2);
          const u32x4_t a = {a1[0], a1[1], a2[0], a2[1]};
          o[dt] = mfma32(a, pb[st][kh], o[dt]);
        }
    }
  };

  // pipeline: rows of tile t+2 are fetched while tile t+1 is copied and tile t is computed
  const int nt = (L + kBN - 1) / kBN;
  if (nt > 0) {
    fetch_rows(0);
    issue(kb0, vb0);
    if (nt > 1) fetch_rows(kBN);
  }
  for (int t = 0; t < nt; t += 2) {
    PARK_WAIT_VMEM();
    __syncthreads();
    if (t + 1 < nt) {
      issue(kb1, vb1);
      if (t + 2 < nt) fetch_rows((t + 2) * kBN);
    }
    compute(kb0, vb0, t * kBN);
    if (t + 1 < nt) {
      PARK_WAIT_VMEM();
      __syncthreads();
      if (t + 2 < nt) {
        issue(kb0, vb0);
        if (t + 3 < nt) fetch_rows((t + 3) * kBN);
      }
      compute(kb1, vb1, (t + 1) * kBN);
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (qok) {
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
  if (s.bf16 && ck > kAttnMaxRuns) {
    // more selectable clusters than the direct-load kernel keeps runs for: register-staged kernel
    if (s.D == 128) {
      PARK_ATTN(uint16_t, 128)
    } else {
      PARK_ATTN(uint16_t, 64)
    }
  } else if (s.bf16) {
    const uint16_t* qh = static_cast<const uint16_t*>(q);
    const uint16_t* kh = static_cast<const uint16_t*>(k);
    const uint16_t* vh = static_cast<const uint16_t*>(v);
    uint16_t* oh = static_cast<uint16_t*>(out);
    if (s.D == 128)
      sparse_attn_bf16<128><<<grid, 256, 0, st>>>(qh, kh, vh, s.N, q_perm, q_offsets, cq, k_perm, tile_base, runs, ck,
                                                   scale, oh, lse);
    else
      sparse_attn_bf16<64><<<grid, 256, 0, st>>>(qh, kh, vh, s.N, q_perm, q_offsets, cq, k_perm, tile_base, runs, ck,
                                                  scale, oh, lse);
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
