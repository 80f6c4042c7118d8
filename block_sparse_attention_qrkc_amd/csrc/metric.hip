// QRKC key metric M_h = (1/n) sum_t q_t q_t^T (PARK page, Figure 2 caption: a key metric derived
// from the current queries). bf16 data: 32x32x16 MFMA over 4096-token blocks (the upper triangle
// of output tiles, mirrored) with fp32 accumulators flushed to fp64 every 256 tokens, then a
// fixed-order fp64 sum of the blocks. fp32 data: plain fp64 dot products.
#include "park_common.h"
#include "park_internal.h"

namespace park {

namespace {

constexpr int kSub = 64;     // tokens staged in LDS per step (two 32-row sub-tiles)
constexpr int kFlush = 256;  // tokens between fp32 -> fp64 flushes

// Upper-triangle 32x32 output tiles of one wave, grouped so that the wave's tiles share operands:
// f[] lists the 32-dimension blocks whose operands the wave reads, a[] / b[] index f[] per tile.
// D = 128: wave 0 (0,0) (0,1) (1,1); wave 1 (2,2) (2,3) (3,3); wave 2 (0,2) (0,3); wave 3 (1,2) (1,3).
// D = 64: wave 0 (0,0) (0,1) (1,1); the other waves only stage tokens.
template <int D, int W>
struct MetricTiles;
template <>
struct MetricTiles<128, 0> {
  static constexpr int n = 3, nf = 2, f[3] = {0, 1, 0}, a[3] = {0, 0, 1}, b[3] = {0, 1, 1};
};
template <>
struct MetricTiles<128, 1> {
  static constexpr int n = 3, nf = 2, f[3] = {2, 3, 0}, a[3] = {0, 0, 1}, b[3] = {0, 1, 1};
};
template <>
struct MetricTiles<128, 2> {
  static constexpr int n = 2, nf = 3, f[3] = {0, 2, 3}, a[3] = {0, 0, 0}, b[3] = {1, 2, 0};
};
template <>
struct MetricTiles<128, 3> {
  static constexpr int n = 2, nf = 3, f[3] = {1, 2, 3}, a[3] = {0, 0, 0}, b[3] = {1, 2, 0};
};
template <>
struct MetricTiles<64, 0> {
  static constexpr int n = 3, nf = 2, f[3] = {0, 1, 0}, a[3] = {0, 0, 1}, b[3] = {0, 1, 1};
};
template <int W>
struct MetricTiles<64, W> {
  static constexpr int n = 0, nf = 0, f[3] = {0, 0, 0}, a[3] = {0, 0, 0}, b[3] = {0, 0, 0};
};

// One wave's share of a block's partial sums Q^T Q (every wave stages tokens; wave W computes its
// tiles). Tokens pass through LDS kSub at a time in two buffers, each row's 16-byte chunks
// XOR-swizzled (chunk_swz); the MFMA operands of both factors have the same form, eight
// consecutive tokens of one dimension per lane, and come from transposing LDS reads
// (ds_read_b64_tr_b16, each lane of a 16-lane group receiving four tokens of one dimension). The
// tokens of a 16-deep MFMA step are the same permutation for both factors, so the contraction
// runs over every staged token once. The upper triangle of output tiles is computed and mirrored,
// so the result is exactly symmetric.
template <int D, int W>
__device__ __forceinline__ void metric_wave(const uint16_t* __restrict__ Qh, int64_t t_begin, int64_t t_end,
                                            double* __restrict__ out, uint8_t* stage) {
  using T = MetricTiles<D, W>;
  constexpr int NT = T::n, NF = T::nf;
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int ROWB = D * 2;     // bytes per staged row
  constexpr int BUFB = kSub * ROWB;
  constexpr int LOADS = kSub * CPR / 256;  // 16-byte loads per thread and step
  const int l = lane_id();
  const int g16 = l / 16, i16 = l % 16;

  f32x16_t acc[NT > 0 ? NT : 1];
  double acc64[NT > 0 ? NT : 1][16];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc[t][i] = 0.f;
      acc64[t][i] = 0.0;
    }
  // transposing-read offsets (within a buffer) of operand block f[x], sub-tile st, half kh, rows z
  uint32_t ofs[NF > 0 ? NF : 1][2][2][2];
#pragma unroll
  for (int x = 0; x < NF; ++x) {
    const int D0 = T::f[x] * 32 + 16 * (g16 & 1);
    const int cc = (D0 + 4 * (i16 % 4)) / 8;
    const int half = (i16 % 4) & 1;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int z = 0; z < 2; ++z) {
          const int R = st * 32 + 16 * (g16 >> 1) + 8 * kh + i16 / 4 + 4 * z;
          ofs[x][st][kh][z] = (uint32_t)(R * ROWB + (cc ^ chunk_swz<CPR>(R)) * 16 + half * 8);
        }
  }
  // staging: thread tid copies pieces e = tid + 256 q: row e / CPR, chunk e % CPR (rows past the
  // block end are stored as zeros; their loads read the last row). Two register sets alternate, so
  // the loads of a step are issued two steps before its LDS store.
  auto gload = [&](u32x4_t(&pre)[LOADS], int64_t t0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
      const int e = threadIdx.x + q * 256;
      const int64_t row = min(t0 + e / CPR, t_end - 1);
      pre[q] = *reinterpret_cast<const u32x4_t*>(Qh + row * D + (e % CPR) * 8);
    }
  };
  auto sstore = [&](const u32x4_t(&pre)[LOADS], int buf, int64_t t0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
      const int e = threadIdx.x + q * 256;
      const int r = e / CPR, c = e % CPR;
      u32x4_t v = pre[q];
      if (t0 + r >= t_end) v = u32x4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(stage + buf * BUFB + r * ROWB + (c ^ chunk_swz<CPR>(r)) * 16) = v;
    }
  };
  int since = 0;
  // one step: the tokens t0 .. t0 + kSub - 1 from `pre` into buffer `buf` (last read two steps
  // ago, before the previous step's barrier), the loads of step t0 + 2 kSub into `pre`, the MFMAs
  auto step = [&](u32x4_t(&pre)[LOADS], int buf, int64_t t0) __attribute__((always_inline)) {
    sstore(pre, buf, t0);
    __syncthreads();
    if (t0 + 2 * kSub < t_end) gload(pre, t0 + 2 * kSub);
    if constexpr (NT > 0) {
      const PARK_LDS uint8_t* sb = (const PARK_LDS uint8_t*)stage + buf * BUFB;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          u32x4_t fr[NF];
#pragma unroll
          for (int x = 0; x < NF; ++x) {
            const s16x4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PARK_LDS s16x4_t*)(sb + ofs[x][st][kh][0]));
            const s16x4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PARK_LDS s16x4_t*)(sb + ofs[x][st][kh][1]));
            const u32x2_t u0 = __builtin_bit_cast(u32x2_t, r0), u1 = __builtin_bit_cast(u32x2_t, r1);
            fr[x] = u32x4_t{u0[0], u0[1], u1[0], u1[1]};
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t] = mfma32(fr[T::a[t]], fr[T::b[t]], acc[t]);
        }
    }
    since += kSub;
    if (since >= kFlush) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          acc64[t][i] += (double)acc[t][i];
          acc[t][i] = 0.f;
        }
      since = 0;
    }
  };
  u32x4_t pa[LOADS], pb[LOADS];
  gload(pa, t_begin);
  if (t_begin + kSub < t_end) gload(pb, t_begin + kSub);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += 2 * kSub) {
    step(pa, 0, t0);
    if (t0 + kSub < t_end) step(pb, 1, t0 + kSub);
  }
  // element i of lane l in tile (A, B): row A * 32 + (i / 4) * 8 + (l / 32) * 4 + i % 4, column
  // B * 32 + l % 32; written at (row, col) and mirrored at (col, row) (diagonal tiles from their
  // upper triangle), so the block's partial is exactly symmetric
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int A = T::f[T::a[t]], B = T::f[T::b[t]];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = A * 32 + (i / 4) * 8 + (l / 32) * 4 + i % 4;
      const int col = B * 32 + l % 32;
      const double v = acc64[t][i] + (double)acc[t][i];
      if (A != B || row <= col) {
        out[row * D + col] = v;
        out[col * D + row] = v;
      }
    }
  }
}

// bf16 data: per block of kMetricChunk tokens the fp64 partial sums Q^T Q (a full, symmetric D x D
// matrix), then a fixed-order fp64 sum of the blocks (metric_reduce).
template <int D>
__global__ __launch_bounds__(256) void metric_partial_bf16(const uint16_t* __restrict__ Q, int64_t N,
                                                           double* __restrict__ part, int nchunk) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[2 * kSub * D * 2];
  const int h = blockIdx.y;
  const int chunk = blockIdx.x;
  const uint16_t* Qh = Q + (int64_t)h * N * D;
  const int64_t t_begin = (int64_t)chunk * kMetricChunk;
  const int64_t t_end = min(t_begin + (int64_t)kMetricChunk, N);
  double* out = part + ((int64_t)h * nchunk + chunk) * D * D;
  switch (__builtin_amdgcn_readfirstlane(threadIdx.x / kWave)) {
    case 0:
      metric_wave<D, 0>(Qh, t_begin, t_end, out, stage);
      break;
    case 1:
      metric_wave<D, 1>(Qh, t_begin, t_end, out, stage);
      break;
    case 2:
      metric_wave<D, 2>(Qh, t_begin, t_end, out, stage);
      break;
    default:
      metric_wave<D, 3>(Qh, t_begin, t_end, out, stage);
      break;
  }
}

__global__ __launch_bounds__(256) void metric_reduce(const double* __restrict__ part, int nchunk, int D, int64_t N,
                                                     float* __restrict__ metric) {
  const int h = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  const double* p = part + (int64_t)h * nchunk * D * D + e;
  double s = 0.0;
  for (int c = 0; c < nchunk; ++c) s += p[(int64_t)c * D * D];
  metric[(int64_t)h * D * D + e] = (float)(s / (double)N);
}

// fp32 data: one thread per (a, b) entry, exact-order fp64 sum over tokens.
__global__ __launch_bounds__(256) void metric_f32(const float* __restrict__ Q, int64_t N, int D,
                                                  float* __restrict__ metric) {
  const int h = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  const int a = e / D, b = e % D;
  const float* Qh = Q + (int64_t)h * N * D;
  double s = 0.0;
  for (int64_t t = 0; t < N; ++t) s += (double)Qh[t * D + a] * (double)Qh[t * D + b];
  metric[(int64_t)h * D * D + e] = (float)(s / (double)N);
}

}  // namespace

size_t metric_partial_count(const Dims& s) {
  return (size_t)(s.H * ceil_div(s.N, kMetricChunk) * s.D * s.D);
}

hipError_t launch_metric(const Dims& s, const void* q, float* metric, double* partial, hipStream_t st) {
  const int dd = (int)(s.D * s.D);
  if (!s.bf16) {
    metric_f32<<<dim3((unsigned)ceil_div(dd, 256), (unsigned)s.H), 256, 0, st>>>(
        static_cast<const float*>(q), s.N, (int)s.D, metric);
    return hipGetLastError();
  }
  const int nchunk = (int)ceil_div(s.N, kMetricChunk);
  const dim3 grid((unsigned)nchunk, (unsigned)s.H);
  if (s.D == 128)
    metric_partial_bf16<128><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(q), s.N, partial, nchunk);
  else
    metric_partial_bf16<64><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(q), s.N, partial, nchunk);
  metric_reduce<<<dim3((unsigned)ceil_div(dd, 256), (unsigned)s.H), 256, 0, st>>>(partial, nchunk, (int)s.D, s.N,
                                                                                  metric);
  return hipGetLastError();
}

}  // namespace park
