// QRKC key metric M_h = (1/n) sum_t q_t q_t^T (PARK page, Figure 2 caption: a key metric derived
// from the current queries). bf16 data: 32x32x16 MFMA over 4096-token blocks with fp32
// accumulators flushed to fp64 every 256 tokens, then a fixed-order fp64 sum of the blocks.
// fp32 data: plain fp64 dot products.
#include "park_common.h"
#include "park_internal.h"

namespace park {

namespace {

constexpr int kSub = 64;       // tokens staged in LDS per step
constexpr int kFlush = 256;    // tokens between fp32 -> fp64 flushes
constexpr int kLdsStride = kSub + 8;  // bf16 elements per transposed LDS row

template <int D>
__global__ __launch_bounds__(256) void metric_partial_bf16(const uint16_t* __restrict__ Q, int64_t N,
                                                           double* __restrict__ part, int nchunk) {
  constexpr int NB = D / 32;            // 32-wide dimension blocks
  constexpr int TPW = NB * NB / 4;      // output tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t qt[D * kLdsStride];  // [dim][token]
  const int h = blockIdx.y;
  const int chunk = blockIdx.x;
  const int l = lane_id();
  const int w = threadIdx.x / kWave;
  const uint16_t* Qh = Q + (int64_t)h * N * D;
  const int64_t t_begin = (int64_t)chunk * kMetricChunk;
  int64_t t_end = t_begin + kMetricChunk;
  if (t_end > N) t_end = N;

  f32x16_t acc[TPW];
  double acc64[TPW][16];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc[t][i] = 0.f;
      acc64[t][i] = 0.0;
    }
  }
  int since_flush = 0;
  // 16-byte loads per sub-block and thread; the next sub-block is loaded while this one is used
  // (rows past the block end are clamped to its last row and stored as zeros)
  constexpr int kLoads = kSub * D / 8 / 256;
  u32x4_t nxt[kLoads];
  auto fetch = [&](int64_t tn) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int e = threadIdx.x + q * 256;
      const int64_t row = tn + e % kSub < t_end ? tn + e % kSub : t_end - 1;
      nxt[q] = *reinterpret_cast<const u32x4_t*>(Qh + row * D + (e / kSub) * 8);
    }
  };
  fetch(t_begin);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kSub) {
    // stage 64 tokens transposed: qt[dim][token]
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int e = threadIdx.x + q * 256;
      const int r = e % kSub;
      const int c8 = e / kSub;
      u32x4_t val = nxt[q];
      if (t0 + r >= t_end) val = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        qt[(c8 * 8 + 2 * k2) * kLdsStride + r] = (uint16_t)(val[k2] & 0xFFFFu);
        qt[(c8 * 8 + 2 * k2 + 1) * kLdsStride + r] = (uint16_t)(val[k2] >> 16);
      }
    }
    __syncthreads();
    if (t0 + kSub < t_end) fetch(t0 + kSub);
#pragma unroll
    for (int ks = 0; ks < kSub / 16; ++ks) {
      const int tok = ks * 16 + (l / 32) * 8;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int id = w * TPW + t;
        const int ab = id / NB, bb = id % NB;
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&qt[(ab * 32 + l % 32) * kLdsStride + tok]);
        const u32x4_t b = *reinterpret_cast<const u32x4_t*>(&qt[(bb * 32 + l % 32) * kLdsStride + tok]);
        acc[t] = mfma32(a, b, acc[t]);
      }
    }
    __syncthreads();
    since_flush += kSub;
    if (since_flush >= kFlush) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          acc64[t][i] += (double)acc[t][i];
          acc[t][i] = 0.f;
        }
      }
      since_flush = 0;
    }
  }
  double* out = part + ((int64_t)h * nchunk + chunk) * D * D;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int id = w * TPW + t;
    const int ab = id / NB, bb = id % NB;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = ab * 32 + (i / 4) * 8 + (l / 32) * 4 + i % 4;
      const int col = bb * 32 + l % 32;
      out[row * D + col] = acc64[t][i] + (double)acc[t][i];
    }
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
