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

// Per (query cluster, head): the original key rows of the selected key clusters, concatenated in
// selection order: gather[(h * cq + i) * N + v] for v < glen[h * cq + i]. Column entries outside
// [0, ck) or with offsets outside [0, N] contribute nothing; the list is cut at N keys.
__global__ __launch_bounds__(256) void attn_gather(const int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ cols,
                                                   const int32_t* __restrict__ k_offsets,
                                                   const int32_t* __restrict__ k_perm, int64_t N, int cq, int ck,
                                                   const float* __restrict__ log_w, float inv_scale,
                                                   int32_t* __restrict__ gather, int32_t* __restrict__ glen,
                                                   float* __restrict__ gbias) {
  __shared__ int scratch[17];
  __shared__ int c_start[256], c_len[256], c_dst[256];
  __shared__ float c_bias[256];
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int l = lane_id();
  const int w = tid / kWave;
  int cnt = counts[(int64_t)h * cq + i];
  cnt = cnt < 0 ? 0 : (cnt > ck ? ck : cnt);
  const int32_t* crow = cols + ((int64_t)h * cq + i) * ck;
  const int32_t* ko = k_offsets + (int64_t)h * (ck + 1);
  const int32_t* kp = k_perm + (int64_t)h * N;
  int32_t* dst = gather + ((int64_t)h * cq + i) * N;
  float* bdst = log_w ? gbias + ((int64_t)h * cq + i) * N : nullptr;
  const float* lwrow = log_w ? log_w + ((int64_t)h * cq + i) * ck : nullptr;
  int64_t base = 0;
  for (int m0 = 0; m0 < cnt; m0 += 256) {
    const int m = m0 + tid;
    int a = 0, len = 0;
    float bias = 0.f;
    if (m < cnt) {
      const int j = crow[m];
      if (j >= 0 && j < ck) {
        const int64_t lo = ko[j], hi = ko[j + 1];
        if (lo >= 0 && hi > lo && hi <= N) {
          a = (int)lo;
          len = (int)(hi - lo);
        }
        if (lwrow) bias = lwrow[j] * inv_scale;
      }
    }
    int tot;
    const int pre = block_exclusive_scan(len, scratch, &tot);
    c_start[tid] = a;
    c_len[tid] = len;
    c_dst[tid] = (int)min<int64_t>(base + pre, N);
    c_bias[tid] = bias;
    __syncthreads();
    // each wave copies two clusters at a time, four 64-key rows of each in flight
    const int nloc = min(256, cnt - m0);
    for (int e0 = w; e0 < nloc; e0 += 8) {
      int s0[2], d0[2], ln[2];
      float cb[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int e = e0 + 4 * x;
        s0[x] = e < nloc ? c_start[e] : 0;
        d0[x] = e < nloc ? c_dst[e] : 0;
        ln[x] = e < nloc ? (int)min<int64_t>(c_len[e], N - d0[x]) : 0;
        cb[x] = e < nloc ? c_bias[e] : 0.f;
      }
      const int lmax = max(ln[0], ln[1]);
      for (int u0 = 0; u0 < lmax; u0 += 4 * kWave) {
        int v[2][4];
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int u = u0 + k * kWave + l;
            v[x][k] = kp[s0[x] + min(u, max(ln[x] - 1, 0))];  // clamped: every load is issued
          }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int u = u0 + k * kWave + l;
            if (u < ln[x]) {
              dst[d0[x] + u] = v[x][k];
              if (bdst) bdst[d0[x] + u] = cb[x];
            }
          }
      }
    }
    base += tot;
    __syncthreads();
  }
  if (tid == 0) glen[(int64_t)h * cq + i] = (int)min<int64_t>(base, N);
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
                                                          const int32_t* __restrict__ gather,
                                                          const int32_t* __restrict__ glen,
                                                          const float* __restrict__ gbias, float scale,
                                                          T* __restrict__ out, float* __restrict__ lse) {
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
  const int32_t* rows = gather + ((int64_t)h * cq + i) * N;
  const float* brow = gbias ? gbias + ((int64_t)h * cq + i) * N : nullptr;
  const int L = glen[(int64_t)h * cq + i];
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
      krow[tid] = v < L ? rows[v] : -1;
      kbias[tid] = (brow && v < L) ? brow[v] : 0.f;
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

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
#define PARK_LDS __attribute__((address_space(3)))

// Chunk swizzle of LDS row r. Two read patterns must be bank-conflict free:
//  - K (ds_read_b128): a 16-lane group reads one logical chunk of rows {0-3, 16-19, 4-7, 20-23}
//    (or the same set + 8), so those 16 rows need distinct swizzles (and, for 8-lane phases,
//    distinct low 3 bits within {0-3, 16-19} and within {4-7, 20-23});
//  - V (ds_read_b64_tr_b16): a half-wave reads an aligned group of four chunks from four
//    consecutive rows 4a..4a+3 (a quarter-wave: two chunks), so bits 2-3 (and bits 1-2) of the
//    swizzle must differ across those four rows.
// D = 128 (16 chunks per row): sw = 2 (g ^ 2g) ^ ((r >> 2) & 1) * 2 ^ ((r >> 4) & 1), g = r & 3,
// i.e. {0, 6, 12, 10} by r & 3 with the bit-0/bit-1 flips separating the row quartets.
// D = 64 (8 chunks, two rows per 256-byte bank sweep): rows of equal parity in a K group need
// distinct swizzles, rows r and r + 2 of a V quartet need different bit 2.
template <int CPR>
__device__ __forceinline__ int chunk_swz(int r) {
  if constexpr (CPR == 16) {
    const int g = r & 3;
    return (2 * (g ^ (g << 1))) ^ (((r >> 2) & 1) << 1) ^ ((r >> 4) & 1);
  } else {
    return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 4) & 1);
  }
}

// Work-group -> tile mapping that keeps neighbouring tiles (the tiles of one query cluster read
// the same key/value rows) on one XCD: work-groups are dealt to the 8 XCDs round-robin, so XCD x
// receives ids x, x + 8, ...; those are given the x-th contiguous range of tiles.
[[maybe_unused]] __device__ __forceinline__ void xcd_tile(int& h, int& c) {
  const int nx = gridDim.x;
  const int G = nx * gridDim.y;
  const int b = blockIdx.x + blockIdx.y * nx;
  const int x = b & 7, per = G >> 3, rem = G & 7;
  const int L = x * per + min(x, rem) + (b >> 3);
  h = L / nx;
  c = L - h * nx;
}

// 384-query tiles: twelve waves x 32 queries share one work-group per CU (three waves per SIMD,
// 168 registers each), so each key/value tile copied to LDS serves 384 queries and each SIMD has
// three waves to interleave matrix-core, vector and LDS work. Tiles of 32 keys (d = 128; 64 for
// d = 64) are copied by eight of the waves, 1 KB of K and of V each, through a ring of four stages
// three tiles ahead; a wave waits only for the copies of the tile it is about to read (a counted
// vmcnt, then a plain barrier: a fenced barrier would also wait for the copies still in flight).
constexpr int kBf16BM = 384;  // queries per work item
[[maybe_unused]] constexpr int kBf16BN = 32;   // keys per tile for d = 128
[[maybe_unused]] constexpr int kBf16NST = 4;   // LDS stages of one tile (K and V)

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
__device__ __forceinline__ int lds_read_b32(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
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
                                                         const int32_t* __restrict__ gather,
                                                         const int32_t* __restrict__ glen,
                                                         const float* __restrict__ gbias, float scale,
                                                         uint16_t* __restrict__ out, float* __restrict__ lse) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = 12;
  constexpr int NWC = 8;  // copier waves
  constexpr int NST = kBf16NST;
  constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3: raw (untyped) access
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int CPR = D / 8;
  constexpr int ROWB = D * 2;
  constexpr int BN = D == 64 ? 64 : kBf16BN;
  constexpr int NSUB = BN / 32;                 // 32-key sub-tiles
  constexpr int TILEB = BN * ROWB;              // one K (or V) tile
  constexpr int BIASB = W ? 256 : 0;            // per wave: the tile's key offsets (lanes l % BN)
  constexpr int STAGEB = 2 * TILEB + NWC * BIASB;  // K, V, then the key offsets
  constexpr int RPB = 1024 / ROWB;              // rows per 1 KB wave load
  constexpr int LOADS = TILEB / (1024 * NWC);    // 1 KB loads per wave per tile, for K and for V
  static_assert(LOADS >= 1, "tile smaller than one load per wave");
  constexpr int CP = 2 * LOADS + (W ? 1 : 0);   // copies per wave per tile
  __shared__ __attribute__((aligned(1024))) uint8_t stages[NST * STAGEB];

  int h, c;
  xcd_tile(h, c);
  const int32_t* tb = tile_base + (int64_t)h * (2 * cq + 1);
  if (c >= tb[cq]) return;
  const int ti = find_tile(tb, cq, c);
  const int i = tb[cq + 1 + ti];
  const int l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const bool copier = w < NWC;
  const int wc = copier ? w : NWC - 1;
  const int hl = l / 32;
  const int32_t* qo = q_off + (int64_t)h * (cq + 1);
  const int qbeg = qo[i] + (c - tb[ti]) * kBf16BM;
  const int qend = min(qbeg + kBf16BM, qo[i + 1]);
  const bool active = qbeg + w * 32 < qend;  // this wave has at least one query
  const int32_t* rows = gather + ((int64_t)h * cq + i) * N;
  const int L = glen[(int64_t)h * cq + i];
  const uint16_t* Qh = Q + (int64_t)h * N * D;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + (int64_t)h * N * D), (short)0, (int)(uint32_t)(N * ROWB), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(V + (int64_t)h * N * D), (short)0, (int)(uint32_t)(N * ROWB), kBufferFlags);
  // key offsets past the list end read as 0 (the range check of the buffer resource)
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W ? gbias + ((int64_t)h * cq + i) * N : nullptr), (short)0, (int)(uint32_t)(W ? L * 4 : 0),
      kBufferFlags);

  const int qpos = qbeg + w * 32 + l % 32;
  const bool qok = qpos < qend;
  const int qrow = q_perm[(int64_t)h * N + min(qpos, qend - 1)];
  u32x4_t qb[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(Qh + (int64_t)qrow * D + kk * 16 + hl * 8);
    const u32x4_t z = {0u, 0u, 0u, 0u};
    qb[kk] = qok ? v : z;
  }

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
  static_assert(LOADS == 1, "one 1 KB copy per wave and tile");
  __shared__ __attribute__((aligned(16))) int32_t idxs[NST][NWC][kWave];
  const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc((void*)rows, (short)0, (int)(uint32_t)(L * 4),
                                                                       kBufferFlags);
  constexpr int IL = 1;  // index loads per wave and tile
  auto load_idx = [&](int set, int tile) __attribute__((always_inline)) {
    if (!copier) return;
    // entries past the list end read as 0 (a valid row; its scores are masked)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (PARK_LDS void*)&idxs[set][wc][0], 4, (tile * BN + l % BN) * 4, 0, 0,
                                             0);
  };
  const uint32_t ibase = (uint32_t)(size_t)((PARK_LDS int32_t*)&idxs[0][wc][trow[0]]);
  auto read_idx = [&](int set) __attribute__((always_inline)) {
    return lds_read_b32(ibase + (uint32_t)(set * NWC * kWave * 4));
  };
  int nnext = 0;  // gather-list row of this lane's copy in the next issue
  auto issue = [&](int nrow0, int slot, int tile) __attribute__((always_inline)) {
    if (!copier) return;
    const int nrow[1] = {nrow0};
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
      const int boff = slot * STAGEB + (w * LOADS + q) * 1024;
      const int voff = (int)((uint32_t)nrow[q] * ROWB + lbyte[q]);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (PARK_LDS void*)(stages + boff), 16, voff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (PARK_LDS void*)(stages + boff + TILEB), 16, voff, 0, 0, 0);
    }
    if constexpr (W) {
      const int boff = slot * STAGEB + 2 * TILEB + wc * BIASB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (PARK_LDS void*)(stages + boff), 4, (tile * BN + l % BN) * 4, 0,
                                               0, 0);
    }
  };

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
  const int r = l % 32;
  const int prow = ((r / 4) % 2) * 16 + (r / 8) * 4 + r % 4;
  const int g16 = l / 16, i16 = l % 16;
  const bf16x2_t ones = as_bf16x2(0x3F803F80u);

  // per-lane byte offsets of the LDS operand reads within a K (V) tile, computed once
  int kofs[NSUB][KS], vofs[DT][NSUB][2][2];
#pragma unroll
  for (int st = 0; st < NSUB; ++st) {
    const int R = st * 32 + prow;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kofs[st][kk] = R * ROWB + ((2 * kk + hl) ^ chunk_swz<CPR>(R)) * 16;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int D0 = dt * 32 + 16 * (g16 & 1);
    const int cc = (D0 + 4 * (i16 % 4)) / 8;
    const int half = (i16 % 4) & 1;
#pragma unroll
    for (int st = 0; st < NSUB; ++st)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int R1 = st * 32 + 16 * (g16 >> 1) + 8 * kh + i16 / 4;
        const int R2 = R1 + 4;
        vofs[dt][st][kh][0] = R1 * ROWB + (cc ^ chunk_swz<CPR>(R1)) * 16 + half * 8;
        vofs[dt][st][kh][1] = R2 * ROWB + (cc ^ chunk_swz<CPR>(R2)) * 16 + half * 8;
      }
  }

  static_assert((NST - 1) * STAGEB + TILEB + 64 <= 65535, "stage offsets fit the LDS reads' 16-bit offset field");
  // scores of one tile: its eight K operand reads in two blocks of four, each followed by its MFMAs
  const uint32_t sbase = (uint32_t)(size_t)((PARK_LDS uint8_t*)stages);
  static_assert(KS * NSUB == 8, "eight K reads per tile");
  auto s_tile = [&](auto OFFc, f32x16_t(&sa)[NSUB]) __attribute__((always_inline)) {
    constexpr int OFF = decltype(OFFc)::value;
#pragma unroll
    for (int st = 0; st < NSUB; ++st)
#pragma unroll
      for (int e = 0; e < 16; ++e) sa[st][e] = 0.f;
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
  // key offsets (weighted form) and the mask of keys past the list end
  auto adjust = [&](auto OFFc, f32x16_t(&sa)[NSUB], int v0) __attribute__((always_inline)) {
    if constexpr (W) {
      constexpr int OFF = decltype(OFFc)::value;  // the stage
#pragma unroll
      for (int st = 0; st < NSUB; ++st) {
        u32x4_t b[4];
        const uint32_t ba = sbase + 2 * TILEB + (w % NWC) * BIASB + (st * 32 + hl * 16) * 4;
        if constexpr (OFF + 48 <= 65535) {
          lds_read4_b128<OFF>(b, ba);
        } else {
          lds_read4_b128<0>(b, ba + OFF);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) sa[st][q * 4 + e] += __uint_as_float(b[q][e]);
      }
    }
    const int nvalid = L - v0;
    if (__builtin_expect(nvalid < BN, 0)) {
      const int lim = nvalid - hl * 16;  // accumulator e of sub-tile st is key st * 32 + hl * 16 + e
#pragma unroll
      for (int st = 0; st < NSUB; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (st * 32 + e >= lim) sa[st][e] = -INFINITY;
    }
  };
  auto tile_max = [&](const f32x16_t(&sa)[NSUB]) __attribute__((always_inline)) {
    float mx = sa[0][0];
#pragma unroll
    for (int st = 0; st < NSUB; ++st)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sa[st][e]);
    return fmaxf(mx, __shfl_xor(mx, 32, kWave));
  };
  auto weights = [&](const f32x16_t(&sa)[NSUB], u32x4_t(&pb)[NSUB][2]) __attribute__((always_inline)) {
    const float mb = m_ref * sl2;
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NSUB; ++st) {
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
  auto pv_tile = [&](auto OFFc, const u32x4_t(&pb)[NSUB][2]) __attribute__((always_inline)) {
    constexpr int OFF = decltype(OFFc)::value;
    constexpr int DG = 2 / NSUB;
#pragma unroll
    for (int d0 = 0; d0 < DT; d0 += DG) {
      uint32_t a[8];
      u32x2_t r[8];
#pragma unroll
      for (int x = 0; x < DG; ++x)
#pragma unroll
        for (int st = 0; st < NSUB; ++st)
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int z = 0; z < 2; ++z) a[((x * NSUB + st) * 2 + kh) * 2 + z] = sbase + vofs[d0 + x][st][kh][z];
      tr_read8<OFF>(r, a);
#pragma unroll
      for (int x = 0; x < DG; ++x)
#pragma unroll
        for (int st = 0; st < NSUB; ++st)
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            const int j = ((x * NSUB + st) * 2 + kh) * 2;
            const u32x4_t va = u32x4_t{r[j][0], r[j][1], r[j + 1][0], r[j + 1][1]};
            o[d0 + x] = mfma32(va, pb[st][kh], o[d0 + x]);
          }
    }
  };

  if (nt > 0) {
    // prologue: entries of tiles 0 .. NST-1 (one wait), then those of tiles NST .. 2 NST-2 into the
    // sets just read, then the copies of tiles 0 .. NST-2 into stages 0 .. NST-2
#pragma unroll
    for (int x = 0; x < NST; ++x) load_idx(x, x);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    int n0[NST];
#pragma unroll
    for (int x = 0; x < NST; ++x) n0[x] = read_idx(x);
#pragma unroll
    for (int x = NST; x < 2 * NST - 1; ++x) load_idx(x % NST, x);
#pragma unroll
    for (int x = 0; x < NST - 1; ++x) issue(n0[x], x, x);
    nnext = n0[NST - 1];
  }
  // Iteration t (stage SL = t % NST): wait until tile t landed, copy tile t + NST - 1 into the stage
  // tile t - 1 used, load the entries of tile t + 2 NST - 1, compute tile t, read the entries of
  // tile t + NST. Tile t was copied in iteration t - NST + 1, after which each of the NST - 2
  // iterations since issued CP + IL vector-memory operations (copies, then the index load), or in
  // the prologue, after which at least NST - 2 tiles' CP copies were issued; the entries read at the
  // end of iteration t were loaded before those copies. Copier waves only issue copies; the waits
  // hold trivially for the others.
  for (int t = 0; t < nt; t += NST) {
    const bool go_on = unroll_while<0, NST>([&](auto SLc) __attribute__((always_inline)) {
      constexpr int SL = decltype(SLc)::value;
      constexpr int XS = (SL + NST - 1) % NST;
      const int tt = t + SL;
      if (tt >= nt) return false;
      if (tt < NST - 1)
        wait_barrier<(NST - 2) * CP>();
      else
        wait_barrier<(NST - 2) * (CP + IL)>();
      issue(nnext, XS, tt + NST - 1);
      load_idx(XS, tt + 2 * NST - 1);
      if (active) {
        f32x16_t sc[NSUB];
        s_tile(std::integral_constant<int, SL * STAGEB>{}, sc);
        adjust(std::integral_constant<int, SL * STAGEB>{}, sc, tt * BN);
        if (tt == 0) m_ref = tile_max(sc);
        u32x4_t pb[NSUB][2];
        float ps = weights(sc, pb);
        if (__builtin_amdgcn_ballot_w64(!(ps <= kRaise))) {
          // rare: the scores are computed again (the tile is still in LDS), so they need not stay
          // live through the softmax
          f32x16_t s2[NSUB];
          s_tile(std::integral_constant<int, SL * STAGEB>{}, s2);
          adjust(std::integral_constant<int, SL * STAGEB>{}, s2, tt * BN);
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
        pv_tile(std::integral_constant<int, SL * STAGEB + TILEB>{}, pb);
      }
      nnext = read_idx(SL);
      return true;
    });
    if (!go_on) break;
  }
  // drain the copies still in flight before the work-group's LDS can be handed to another
  __builtin_amdgcn_s_waitcnt(0x0F70);

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
#endif
}


}  // namespace

int64_t attn_max_tiles(const Dims& s, int cq) { return ceil_div(s.N, s.bf16 ? kBf16BM : kAttnBM) + cq; }

size_t attn_gather_ints(const Dims& s, int cq) { return (size_t)(s.H * cq) * (size_t)(s.N + 1); }

hipError_t launch_sparse_attn(const Dims& s, const void* q, const void* k, const void* v, const int32_t* q_perm,
                              const int32_t* q_offsets, int cq, const int32_t* k_perm, const int32_t* k_offsets,
                              int ck, const int32_t* counts, const int32_t* cols, const float* log_w, float scale,
                              void* out, float* lse, int32_t* tile_base, int32_t* gather, float* gbias,
                              hipStream_t st) {
  int32_t* glen = gather + (size_t)(s.H * cq) * (size_t)s.N;
  float* gb = log_w ? gbias : nullptr;
  attn_gather<<<dim3((unsigned)cq, (unsigned)s.H), 256, 0, st>>>(counts, cols, k_offsets, k_perm, s.N, cq, ck, log_w,
                                                                1.f / scale, gather, glen, gb);
  attn_order<<<(unsigned)s.H, 1024, 0, st>>>(q_offsets, glen, cq, s.bf16 ? kBf16BM : kAttnBM, tile_base);
  const dim3 grid((unsigned)attn_max_tiles(s, cq), (unsigned)s.H);
#define PARK_ATTN(T, D)                                                                                          \
  sparse_attn_kernel<T, D><<<grid, 256, 0, st>>>(static_cast<const T*>(q), static_cast<const T*>(k),            \
                                                 static_cast<const T*>(v), s.N, q_perm, q_offsets, cq, tile_base, \
                                                 gather, glen, gb, scale, static_cast<T*>(out), lse);
#define PARK_BF16ATTN(D, W)                                                                                            \
  sparse_attn_bf16<D, W><<<grid, 768, 0, st>>>(qh, kh, vh, s.N, q_perm, q_offsets, cq, tile_base, gather, glen, gb, \
                                             scale, oh, lse);
  if (s.bf16) {
    const uint16_t* qh = static_cast<const uint16_t*>(q);
    const uint16_t* kh = static_cast<const uint16_t*>(k);
    const uint16_t* vh = static_cast<const uint16_t*>(v);
    uint16_t* oh = static_cast<uint16_t*>(out);
    if (s.D == 128) {
      if (gb) {
        PARK_BF16ATTN(128, true)
      } else {
        PARK_BF16ATTN(128, false)
      }
    } else {
      if (gb) {
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
