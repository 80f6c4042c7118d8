// K-means for both token sides (PARK page, Figure 2 caption: queries under Euclidean K-means, keys
// under the query-derived metric M):
//   * k-means++ seeding (Arthur & Vassilvitskii 2007) over strided candidate rows, in fp64, with
//     draws from a SplitMix64 counter stream (Steele, Lea & Flood 2014);
//   * assignment: label = argmin_j b_j - 2 x.g_j on bf16 MFMA (fp32 accumulation), lowest j on ties
//     (bf16 data: scores compared in their top 20 bits, see asg_key);
//   * stable counting sort of the labels into cluster-contiguous order;
//   * update: fixed-order fp64 member means stored as fp32, followed by the consumed form (g, b)
//     of every centroid for the next assignment.
#include <cfloat>

#include "park_common.h"
#include "park_internal.h"

namespace park {

namespace {

// ------------------------------------------------------------------------------------------------
// k-means++ seeding
// ------------------------------------------------------------------------------------------------

__device__ __forceinline__ double kpp_uniform(uint64_t seed, int head, int side, int m) {
  const uint64_t key = seed ^ ((uint64_t)head << 32) ^ ((uint64_t)side << 24) ^ (uint64_t)m;
  return (double)(splitmix_first(key) >> 11) * 0x1.0p-53;
}

// floor(i * N / S): i * N < 2^53 is exact in fp64, and the quotient's fractional part is at least 1/S,
// far above the division's rounding error, so the truncated fp64 quotient is the exact floor.
__device__ __forceinline__ int64_t cand_row(int i, int S, int64_t N) {
  return (int64_t)(((double)i * (double)N) / (double)S);
}

// Euclidean candidate norms xx_i = |x_i|^2 (fp64 sums of fp64 squares): block = 64 candidates,
// 4 threads each (a quarter of the dims per thread); rows staged in LDS.
template <typename T, int D>
__global__ __launch_bounds__(256) void kpp_prep(const T* __restrict__ X, int64_t N, int S, double* __restrict__ xx) {
  constexpr int XS = D + 1;  // padded row stride (floats)
  __shared__ float xs[64 * XS];
  __shared__ double part_s[4][64];
  const int h = blockIdx.y;
  const int i0 = blockIdx.x * 64;
  // rows staged 8 elements per load, all loads of a thread in flight together
#pragma unroll
  for (int k = 0; k < 64 * D / 8 / 256; ++k) {
    const int e = threadIdx.x + k * 256;
    const int r = e / (D / 8), a0 = (e % (D / 8)) * 8;
    float v[8];
    load8_f32(X + ((int64_t)h * N + cand_row(min(i0 + r, S - 1), S, N)) * D + a0, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) xs[r * XS + a0 + q] = i0 + r < S ? v[q] : 0.f;
  }
  __syncthreads();
  const int c = threadIdx.x % 64;   // candidate within the block
  const int q4 = threadIdx.x / 64;  // quarter of the dims (uniform per wave)
  constexpr int AQ = D / 4;
  const float* x = xs + c * XS;
  double acc = 0.0;
  for (int a = q4 * AQ; a < q4 * AQ + AQ; ++a) acc += (double)x[a] * (double)x[a];
  part_s[q4][c] = acc;
  __syncthreads();
  if (threadIdx.x < 64 && i0 + threadIdx.x < S)
    xx[(int64_t)h * S + i0 + threadIdx.x] =
        ((part_s[0][threadIdx.x] + part_s[1][threadIdx.x]) + part_s[2][threadIdx.x]) + part_s[3][threadIdx.x];
}

// QRKC candidate products with register tiles (y = M x and xx = x . y for 64 candidates per block):
// thread t computes the D / 16 outputs a = (D / 16) (t % 16) + {0 .. D / 16 - 1} of the four
// candidates 4 (t / 16) + {0..3}, accumulating over b = 0 .. D - 1 in order (fp32 FMA
// chains), reading 3 LDS vectors per 4 * D / 16 FMAs. xx: fp64 sums of fp64 products over the
// thread's outputs, then over the 16 output groups.
template <typename T, int D>
__global__ __launch_bounds__(256) void kpp_prep_tiled(const T* __restrict__ X, int64_t N, int S,
                                                      const float* __restrict__ M, double* __restrict__ xx,
                                                      float* __restrict__ y) {
  constexpr int OA = D / 16;  // outputs per thread
  extern __shared__ float kpt_lds[];
  float* ms = kpt_lds;          // [D][D]
  constexpr int XT = 68;         // padded stride of xs (16-byte aligned rows, fewer bank conflicts)
  float* xs = kpt_lds + D * D;  // [D][XT]: xs[b * XT + c] = x_c[b]
  const int h = blockIdx.y;
  const int i0 = blockIdx.x * 64;
  // all staging loads of a thread are issued before their LDS stores
  float v[64 * D / 8 / 256][8];
#pragma unroll
  for (int k = 0; k < 64 * D / 8 / 256; ++k) {
    const int e = threadIdx.x + k * 256;
    load8_f32(X + ((int64_t)h * N + cand_row(min(i0 + e / (D / 8), S - 1), S, N)) * D + (e % (D / 8)) * 8, v[k]);
  }
  f32x4_t mv4[D * D / 4 / 256];
#pragma unroll
  for (int k = 0; k < D * D / 4 / 256; ++k)
    mv4[k] = *reinterpret_cast<const f32x4_t*>(M + (int64_t)h * D * D + (threadIdx.x + k * 256) * 4);
#pragma unroll
  for (int k = 0; k < 64 * D / 8 / 256; ++k) {
    const int e = threadIdx.x + k * 256;
    const int c = e / (D / 8), b0 = (e % (D / 8)) * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) xs[(b0 + q) * XT + c] = i0 + c < S ? v[k][q] : 0.f;
  }
#pragma unroll
  for (int k = 0; k < D * D / 4 / 256; ++k) *reinterpret_cast<f32x4_t*>(ms + (threadIdx.x + k * 256) * 4) = mv4[k];
  __syncthreads();
  const int og = threadIdx.x % 16;  // output group
  const int cg = threadIdx.x / 16;  // candidate group
  float acc[4][OA];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int o = 0; o < OA; ++o) acc[q][o] = 0.f;
  for (int b = 0; b < D; ++b) {
    const f32x4_t xv = *reinterpret_cast<const f32x4_t*>(xs + b * XT + cg * 4);
    float mv[OA];  // M[b][a] == M[a][b]
#pragma unroll
    for (int o = 0; o < OA; o += 4) {
      const f32x4_t m4 = *reinterpret_cast<const f32x4_t*>(ms + b * D + og * OA + o);
      mv[o] = m4[0];
      mv[o + 1] = m4[1];
      mv[o + 2] = m4[2];
      mv[o + 3] = m4[3];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int o = 0; o < OA; ++o) acc[q][o] = __builtin_fmaf(mv[o], xv[q], acc[q][o]);
  }
  double part[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = cg * 4 + q;
    double sacc = 0.0;
#pragma unroll
    for (int o = 0; o < OA; ++o) sacc += (double)xs[(og * OA + o) * XT + c] * (double)acc[q][o];
    part[q] = sacc;
    if (i0 + c < S) {
      float* yr = y + ((int64_t)h * S + i0 + c) * D + og * OA;
#pragma unroll
      for (int o = 0; o < OA; o += 4) {
        const f32x4_t v = {acc[q][o], acc[q][o + 1], acc[q][o + 2], acc[q][o + 3]};
        *reinterpret_cast<f32x4_t*>(yr + o) = v;
      }
    }
  }
  // sum over the 16 output groups (16 consecutive lanes)
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) part[q] += __shfl_xor(part[q], o, kWave);
  if (og == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (i0 + cg * 4 + q < S) xx[(int64_t)h * S + i0 + cg * 4 + q] = part[q];
  }
}

// The same products for bf16 data on the matrix cores, 256 candidates per block: M (fp32) is split
// exactly into three bf16 parts (Mh = bf16(M), Mm = bf16(M - Mh), Ml = bf16(M - Mh - Mm); each
// difference is exact in fp32), staged in LDS, and y = Mh x + Mm x + Ml x accumulates the exact
// products in fp32 (32x32x16 MFMAs: dimensions of M as A rows, candidates as B columns; wave w
// takes 32 candidates). xx = x . y: fp64 sums of fp64 products, per lane over its outputs in tile
// order, then over the two half-waves.
template <int D>
__global__ __launch_bounds__(512) void kpp_prep_mfma(const uint16_t* __restrict__ X, int64_t N, int S,
                                                     const float* __restrict__ M, double* __restrict__ xx,
                                                     float* __restrict__ y) {
  constexpr int STR = D + 8;  // padded LDS row (bf16 elements)
  constexpr int KS = D / 16;  // 16-dimension MFMA steps
  constexpr int AT = D / 32;  // 32-dimension output tiles
  __shared__ __attribute__((aligned(16))) uint16_t ms[3][D * STR];
  const int h = blockIdx.y;
  const int l = lane_id();
  const int w = threadIdx.x / kWave;
  const int hl = l / 32;
  const float* Mh = M + (int64_t)h * D * D;
  for (int e = threadIdx.x; e < D * D / 4; e += 512) {
    const f32x4_t m4 = *reinterpret_cast<const f32x4_t*>(Mh + e * 4);
    const int r = (e * 4) / D, c = (e * 4) % D;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float m = m4[q];
      const uint32_t b0 = f32_to_bf16_bits(m);
      const float r1 = m - bf16_bits_to_f32(b0);
      const uint32_t b1 = f32_to_bf16_bits(r1);
      const float r2 = r1 - bf16_bits_to_f32(b1);
      ms[0][r * STR + c + q] = (uint16_t)b0;
      ms[1][r * STR + c + q] = (uint16_t)b1;
      ms[2][r * STR + c + q] = (uint16_t)f32_to_bf16_bits(r2);
    }
  }
  __syncthreads();
  const int cand = blockIdx.x * 256 + w * 32 + l % 32;  // this lane's candidate (B column)
  const bool ok = cand < S;
  const uint16_t* xr = X + ((int64_t)h * N + cand_row(min(cand, S - 1), S, N)) * D;
  f32x16_t acc[AT];
#pragma unroll
  for (int at = 0; at < AT; ++at)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[at][i] = 0.f;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(xr + kk * 16 + hl * 8);
#pragma unroll
    for (int at = 0; at < AT; ++at)
#pragma unroll
      for (int sp = 0; sp < 3; ++sp) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&ms[sp][(at * 32 + l % 32) * STR + kk * 16 + hl * 8]);
        acc[at] = mfma32(a, b, acc[at]);
      }
  }
  // element i of tile at: dimension at * 32 + (i / 4) * 8 + hl * 4 + i % 4 of this lane's candidate
  double part = 0.0;
  float* yr = y + ((int64_t)h * S + min(cand, S - 1)) * D;
#pragma unroll
  for (int at = 0; at < AT; ++at)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int a0 = at * 32 + g4 * 8 + hl * 4;
      const u32x2_t xv = *reinterpret_cast<const u32x2_t*>(xr + a0);
      const float xs[4] = {bf16_bits_to_f32(xv[0] & 0xFFFFu), bf16_bits_to_f32(xv[0] >> 16),
                           bf16_bits_to_f32(xv[1] & 0xFFFFu), bf16_bits_to_f32(xv[1] >> 16)};
#pragma unroll
      for (int q = 0; q < 4; ++q) part += (double)xs[q] * (double)acc[at][g4 * 4 + q];
      if (ok) {
        const f32x4_t v = {acc[at][g4 * 4], acc[at][g4 * 4 + 1], acc[at][g4 * 4 + 2], acc[at][g4 * 4 + 3]};
        *reinterpret_cast<f32x4_t*>(yr + a0) = v;
      }
    }
  part += __shfl_xor(part, 32, kWave);
  if (hl == 0 && ok) xx[(int64_t)h * S + cand] = part;
}

struct KppSide {
  const void* x;      // [H, N, D] data of this side
  const double* xx;   // [H, S] candidate norms
  const float* y;     // [H, S, D] candidate metric products (NULL: Euclidean, y = x)
  float* cent;        // [H, C, D] output
  int C, S, side;
};

constexpr int kKppThreads = 1024;
constexpr int kKppWaves = kKppThreads / kWave;

// Sum over aligned groups of G lanes (G = 8, 16 or 32); every lane of a group gets the group sum.
// Groups of 16 use DPP row rotations, groups of 8 a half-row mirror and quad permutations.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G == 16) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
    return v;
  } else if constexpr (G == 8) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    return v;
  } else {
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
  }
}

// One workgroup per (head, side); blockIdx.y selects the side. D^2 of the S candidates live in LDS.
// Per step: a block-wide prefix over D^2 (thread t owns candidates [t*P, t*P + P)) finds the sampled
// candidate; then every D^2 is lowered by the distance to the new centre,
// dist = xx_i - 2 x_i.y_t + xx_t. For the dot products LPR lanes read one candidate row together
// (16 bytes each, one cache line per 8 lanes), accumulate in fp32 and add across the group.
template <typename T, int D>
__global__ __launch_bounds__(kKppThreads) void kpp_seed(KppSide s0, KppSide s1, int64_t N, uint64_t seed) {
  constexpr int EPC = 16 / sizeof(T);      // elements per 16-byte chunk
  constexpr int LPR = D / EPC;             // lanes per candidate row
  constexpr int RPW = kWave / LPR;         // candidate rows per wave per round
  constexpr int RPB = kKppWaves * RPW;     // candidate rows per round
  constexpr int BATCH = 8;                 // rounds whose loads are in flight together
  extern __shared__ double d2s[];          // [S]
  __shared__ __attribute__((aligned(16))) float yf[D];
  __shared__ double wtot[kKppWaves];
  __shared__ double cc_s;
  __shared__ int pick;
  __shared__ uint32_t taken[16384 / 32];

  const KppSide sd = blockIdx.y == 0 ? s0 : s1;
  const int h = blockIdx.x;
  const int C = sd.C, S = sd.S;
  const int tid = threadIdx.x;
  const int l = lane_id();
  const int w = tid / kWave;
  const int P = (S + kKppThreads - 1) / kKppThreads;
  const int base = tid * P;
  const T* Xh = static_cast<const T*>(sd.x) + (int64_t)h * N * D;
  const double* xxh = sd.xx + (int64_t)h * S;
  const float* yh = sd.y ? sd.y + (int64_t)h * S * D : nullptr;
  for (int q = tid; q < 16384 / 32; q += kKppThreads) taken[q] = 0u;
  const int rounds = (S + RPB - 1) / RPB;
  const int my_chunk = l % LPR;
  const int my_row_in_wave = l / LPR;

  for (int m = 0; m < C; ++m) {
    if (m == 0) {
      if (tid == 0) {
        const int t0 = (int)(kpp_uniform(seed, h, sd.side, 0) * (double)S);
        pick = t0 < S ? t0 : S - 1;
      }
      __syncthreads();
    } else {
      double local = 0.0;
      for (int k = 0; k < P; ++k)
        if (base + k < S) local += d2s[base + k];
      const double inc = wave_inclusive_scan(local);
      if (l == kWave - 1) wtot[w] = inc;
      __syncthreads();  // A
      double total = 0.0;
#pragma unroll
      for (int q = 0; q < kKppWaves; ++q) total += wtot[q];
      if (total > 0.0) {
        const double v = kpp_uniform(seed, h, sd.side, m) * total;
        int owner_w = -1;
        double owner_pre = 0.0, run = 0.0;
#pragma unroll
        for (int q = 0; q < kKppWaves; ++q) {
          if (owner_w < 0 && run + wtot[q] > v) {
            owner_w = q;
            owner_pre = run;
          }
          run += wtot[q];
        }
        if (owner_w < 0) {  // v rounded onto the total: the last wave with mass
          run = 0.0;
          for (int q = 0; q < kKppWaves; ++q) {
            if (wtot[q] > 0.0) {
              owner_w = q;
              owner_pre = run;
            }
            run += wtot[q];
          }
        }
        if (w == owner_w) {
          const uint64_t hit = __ballot(owner_pre + inc > v);
          const int owner_l = hit ? __ffsll((unsigned long long)hit) - 1 : kWave - 1;
          if (l == owner_l) {
            double r2 = owner_pre + inc - local;
            int found = -1, last_pos = -1;
            for (int k = 0; k < P && base + k < S; ++k) {
              const double dk = d2s[base + k];
              if (dk > 0.0) {
                last_pos = k;
                r2 += dk;
                if (r2 > v) {
                  found = k;
                  break;
                }
              }
            }
            if (found < 0) found = last_pos;
            pick = found >= 0 ? base + found : -1;
          }
        }
      } else if (tid == 0) {
        pick = -1;
      }
      __syncthreads();  // B
      if (pick < 0) {
        // rounding left the sampler without a candidate: the last candidate with mass; or every
        // D^2 is zero: the lowest candidate not chosen yet
        const bool any_mass = total > 0.0;
        __syncthreads();
        if (tid == 0) pick = any_mass ? -1 : S;
        __syncthreads();
        for (int i = tid; i < S; i += kKppThreads) {
          if (any_mass) {
            if (d2s[i] > 0.0) atomicMax(&pick, i);
          } else if (!((taken[i >> 5] >> (i & 31)) & 1u)) {
            atomicMin(&pick, i);
          }
        }
        __syncthreads();
      }
    }
    const int t = pick;
    // centre: y = M x_t (or x_t); cc = xx_t
    {
      if (tid == 0) taken[t >> 5] |= 1u << (t & 31);
      const T* xt = Xh + cand_row(t, S, N) * D;
      for (int a = tid; a < D; a += kKppThreads) {
        const float xa = load_f32(xt, a);
        yf[a] = yh ? yh[(int64_t)t * D + a] : xa;
        sd.cent[((int64_t)h * C + m) * D + a] = xa;
      }
      if (tid == 0) cc_s = xxh[t];
    }
    __syncthreads();  // C
    const double cc = cc_s;
    float yc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) yc[e] = yf[my_chunk * EPC + e];
    for (int r0 = 0; r0 < rounds; r0 += BATCH) {
      u32x4_t xv[BATCH];
      double xxv[BATCH];
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int i = (r0 + b) * RPB + w * RPW + my_row_in_wave;
        u32x4_t v = {0u, 0u, 0u, 0u};
        double n2 = 0.0;
        if (r0 + b < rounds && i < S) {
          v = *reinterpret_cast<const u32x4_t*>(Xh + cand_row(i, S, N) * D + my_chunk * EPC);
          n2 = xxh[i];
        }
        xv[b] = v;
        xxv[b] = n2;
      }
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        float acc = 0.f;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc = __builtin_fmaf(__uint_as_float(xv[b][q] << 16), yc[2 * q], acc);
            acc = __builtin_fmaf(__uint_as_float(xv[b][q] & 0xFFFF0000u), yc[2 * q + 1], acc);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc = __builtin_fmaf(__uint_as_float(xv[b][q]), yc[q], acc);
        }
        acc = group_sum<LPR>(acc);
        const int i = (r0 + b) * RPB + w * RPW + my_row_in_wave;
        if (my_chunk == 0 && r0 + b < rounds && i < S) {
          double dist = xxv[b] - 2.0 * (double)acc + cc;
          dist = dist > 0.0 ? dist : 0.0;
          if (i == t)
            d2s[i] = 0.0;
          else if (m == 0 || dist < d2s[i])
            d2s[i] = dist;
        }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------------
// Cooperative k-means++ (bf16 data): the candidates of one (head, side) are split over G
// co-resident workgroups, each holding its share on chip for the whole seeding (one row per thread
// in registers, the rest in LDS), so a step touches no off-chip candidate data. Per step the parts
// publish their D^2 sums, the part holding the sampled prefix position finds the candidate and
// publishes it, and every part lowers its D^2 against the new centre. Launched cooperatively
// (all workgroups resident); every wait is bounded.
// Every exchanged value is its own message: a slot written once per step by one atomic store
// (relaxed, device scope) of a word that is never zero (a D^2 sum with its sign bit set, or a
// candidate index + 1), polled by the readers until it is non-zero. No value depends on other
// data published in the same kernel, so no fence is needed on either side.
// ------------------------------------------------------------------------------------------------

constexpr int kCoopMaxParts = 16;
// Threads per part: 512 (two waves per SIMD, room for the row and the update's registers) or,
// when a head's candidates do not fit on that many parts, 1024 (four waves per SIMD).
constexpr int kCoopThreads = 512;
constexpr int kCoopThreadsWide = 1024;
constexpr long long kSpinLimit = 1ll << 20;  // ~30 ms per wait; a normal wait takes microseconds

struct CoopSide {
  const uint16_t* x;  // [H, N, D]
  const double* xx;   // [H, S]
  const float* y;     // [H, S, D] or NULL (Euclidean)
  float* cent;        // [H, C, D]
  uint64_t* psum;     // [H, C, kCoopMaxParts, 2]: slot [m][part][0] = part's D^2 sum of step m, flagged
  int* sync;          // [H, C, 3]: [m][2] = candidate chosen at step m, + 1; then one failure flag
  int C, S, side, G, SP;
};

// Wait until *p != 0 and return it: relaxed polling (no cache maintenance per poll). A wait that
// runs out sets *fail, after which every wait of the launch returns at once (with 0), so a broken
// launch still ends promptly (with wrong centroids) instead of hanging.
__device__ __forceinline__ int spin_nonzero(int* p, int* fail) {
  long long n = 0;
  int v;
  while ((v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0) {
    if (__hip_atomic_load(fail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
    if (++n >= kSpinLimit) {
      __hip_atomic_store(fail, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return v;
}

// The same for two 64-bit slots written by one lane: both are polled in every round, so that the
// second costs no round trip of its own.
__device__ __forceinline__ void spin_slots(uint64_t* p, uint64_t* q, int* fail, uint64_t& a, uint64_t& c) {
  long long n = 0;
  for (;;) {
    a = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    c = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a != 0 && c != 0) break;
    if (__hip_atomic_load(fail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
    if (++n >= kSpinLimit) {
      __hip_atomic_store(fail, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// One DPP move of a double (both halves with the same control); lanes whose source lies outside
// the pattern, or whose row is masked off, read 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROWS, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROWS, 0xF, true);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// Inclusive sum over lanes 0..l of the wave: within each row of 16 by shifts of 1, 2, 4 and 8
// lanes, then the end of row 0 into row 1 and of row 2 into row 3, then the end of row 1 into
// rows 2 and 3 (register moves only, no LDS round trips).
__device__ __forceinline__ double wave_scan_dpp(double v) {
  v += dpp_f64<0x111, 0xF>(v);  // row_shr:1
  v += dpp_f64<0x112, 0xF>(v);  // row_shr:2
  v += dpp_f64<0x114, 0xF>(v);  // row_shr:4
  v += dpp_f64<0x118, 0xF>(v);  // row_shr:8
  v += dpp_f64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// The value of lane l - 1 (0 in lane 0): an inclusive scan turned exclusive without a subtraction.
__device__ __forceinline__ double wave_shr1(double v) { return dpp_f64<0x138, 0xF>(v); }  // wave_shr:1

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// H heads from head h0 on: the side pointers start at head h0, the draws use the head's own index.
// status (may be NULL): bit 0 is set at the end of the launch when any bounded wait of a side gave
// up, so a lost exchange reaches the caller instead of passing silently.
template <int D, int NT>
__global__ __launch_bounds__(NT) void kpp_coop(CoopSide s0, CoopSide s1, int H, int h0, int64_t N, uint64_t seed,
                                               int* status) {
  constexpr int kCoopWaves = NT / kWave;
  constexpr int ROW_U32 = D / 2;
  extern __shared__ uint32_t lrows[];  // [SP - threads][D / 2] bf16 pairs of the LDS-resident rows
  __shared__ __attribute__((aligned(16))) uint32_t yhi[D / 2];
  __shared__ __attribute__((aligned(16))) uint32_t ylo[D / 2];
  constexpr int CPR = D / 8;           // 16-byte pieces per row
  // per wave slot (register rows of waves 0.., then LDS rows of waves 0..): D^2 total, and its
  // exclusive prefix within the part in candidate order
  __shared__ double wsum[2 * kCoopWaves], wpre[2 * kCoopWaves];
  __shared__ int wmin[kCoopWaves];      // per wave: its first untaken candidate
  __shared__ int first_s, last_s;       // owner part: first candidate past the draw, last one with mass
  __shared__ double pre_s, v_s, cc_s;
  __shared__ int owner_s, pick_s;

  // decode (side, head, part) from an XCD-grouped order: work-groups are dealt to the 8 XCDs
  // round-robin, so XCD x receives ids x, x + 8, ...; those are given the x-th contiguous range of
  // (side, head, part), which keeps the parts of a head, which exchange partial sums every step, on
  // one XCD and its L2
  int b;
  {
    const int G = (int)gridDim.x;
    const int x = (int)blockIdx.x & 7, per = G >> 3, rem = G & 7;
    b = x * per + min(x, rem) + ((int)blockIdx.x >> 3);
  }
  const bool second = b >= H * s0.G;
  const CoopSide sd = second ? s1 : s0;
  if (second) b -= H * s0.G;
  const int h = b / sd.G;
  const int part = b % sd.G;
  const int C = sd.C, S = sd.S, G = sd.G, SP = sd.SP;
  const int tid = threadIdx.x;
  const int l = lane_id();
  const int w = tid / kWave;
  const int c0 = part * SP;                   // first candidate of this part
  const int cnt = min(SP, S - c0);            // candidates of this part
  const int nreg = min(cnt, NT);     // register-resident (thread tid: c0 + tid)
  const int nlds = cnt - nreg;                // LDS-resident (thread tid: c0 + 1024 + tid)
  const uint16_t* Xh = sd.x + (int64_t)h * N * D;
  const double* xxh = sd.xx + (int64_t)h * S;
  const float* yh = sd.y ? sd.y + (int64_t)h * S * D : nullptr;
  uint64_t* psum = sd.psum + (int64_t)h * C * kCoopMaxParts * 2;
  int* sync = sd.sync + (int64_t)h * C * 3;
  int* fail = sd.sync + (int64_t)H * C * 3;

  // on-chip candidate rows
  const bool has_r = tid < nreg;
  const bool has_l = tid < nlds;
  uint32_t xr[ROW_U32];
  {
    const int i = c0 + tid;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(Xh + (has_r ? cand_row(i, S, N) : 0) * D);
#pragma unroll
    for (int q = 0; q < ROW_U32; q += 4) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (has_r) v = *reinterpret_cast<const u32x4_t*>(src + q);
      xr[q] = v[0];
      xr[q + 1] = v[1];
      xr[q + 2] = v[2];
      xr[q + 3] = v[3];
    }
  }
  // LDS row r keeps its 16-byte piece p at position p ^ (r % CPR), so that the threads reading
  // their own rows piece by piece hit distinct banks
  for (int e = tid; e < nlds * CPR; e += NT) {
    const int r = e / CPR, p = e % CPR;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(Xh + cand_row(c0 + NT + r, S, N) * D);
    *reinterpret_cast<u32x4_t*>(&lrows[r * ROW_U32 + (p ^ (r % CPR)) * 4]) =
        *reinterpret_cast<const u32x4_t*>(src + p * 4);
  }
  const double xx_r = has_r ? xxh[c0 + tid] : 0.0;
  const double xx_l = has_l ? xxh[c0 + NT + tid] : 0.0;
  double d2r = 0.0, d2l = 0.0;
  bool taken_r = false, taken_l = false;
  __syncthreads();

  for (int m = 0; m < C; ++m) {
    int t;
    if (m == 0) {
      const int t0 = (int)(kpp_uniform(seed, h0 + h, sd.side, 0) * (double)S);
      t = t0 < S ? t0 : S - 1;
    } else {
      // ---- running D^2 sums inside each wave (candidate order: register rows of waves 0..7, then
      // LDS rows of waves 0..7), the wave totals, and each wave's first untaken candidate (register
      // rows precede LDS rows in candidate order)
      const double incr = wave_scan_dpp(d2r);
      const double incl = wave_scan_dpp(d2l);
      const uint64_t ur = __ballot(has_r && !taken_r);
      const uint64_t ul = __ballot(has_l && !taken_l);
      if (l == kWave - 1) {
        wsum[w] = incr;
        wsum[kCoopWaves + w] = incl;
      }
      if (l == 0) {
        wmin[w] = ur ? c0 + w * kWave + __ffsll((unsigned long long)ur) - 1
                     : (ul ? c0 + NT + w * kWave + __ffsll((unsigned long long)ul) - 1 : 0x7FFFFFFF);
        if (w == 0) {
          first_s = 0x7FFFFFFF;
          last_s = -1;
        }
      }
      __syncthreads();
      if (w == 0) {
        // slots of step m: [part][0] = D^2 sum with its sign bit set, [part][1] = first untaken + 1
        uint64_t* slots = psum + (int64_t)m * kCoopMaxParts * 2;
        const double u = kpp_uniform(seed, h0 + h, sd.side, m);
        // the wave slots' exclusive prefixes (for the search, if this part owns the draw), the
        // part's total and its first untaken candidate
        const double ws = l < 2 * kCoopWaves ? wsum[l] : 0.0;
        const double wi = wave_scan_dpp(ws);
        const double wx = wave_shr1(wi);
        if (l < 2 * kCoopWaves) wpre[l] = wx;
        const double pt = readlane_f64(wi, 2 * kCoopWaves - 1);
        int pf = l < kCoopWaves ? wmin[l] : 0x7FFFFFFF;
        // kCoopWaves <= 16: the minimum over row 0 by rotations of 1, 2, 4 and 8 lanes (row_ror)
        pf = min(pf, __builtin_amdgcn_update_dpp(pf, pf, 0x121, 0xF, 0xF, false));
        pf = min(pf, __builtin_amdgcn_update_dpp(pf, pf, 0x122, 0xF, 0xF, false));
        pf = min(pf, __builtin_amdgcn_update_dpp(pf, pf, 0x124, 0xF, 0xF, false));
        pf = min(pf, __builtin_amdgcn_update_dpp(pf, pf, 0x128, 0xF, 0xF, false));
        pf = __builtin_amdgcn_readfirstlane(pf);
        if (l == 0) {
          __hip_atomic_store(&slots[part * 2], (uint64_t)__double_as_longlong(pt) | (1ull << 63), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&slots[part * 2 + 1], (uint64_t)(uint32_t)pf + 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
        // the G part sums are read at once (lane q: part q) and scanned in the same order by every
        // part; a failed wait reads as an empty part
        double pq = 0.0;
        int fq = 0x7FFFFFFF;
        if (l < G) {
          uint64_t a, c;
          spin_slots(&slots[l * 2], &slots[l * 2 + 1], fail, a, c);
          pq = __longlong_as_double((long long)(a & ~(1ull << 63)));
          fq = c != 0 ? (int)(c - 1u) : 0x7FFFFFFF;
        }
        const double run = wave_scan_dpp(pq);  // inclusive prefix over parts
        const double total = readlane_f64(run, G - 1);
        int owner = -1;
        double v = 0.0, pre = 0.0;
        if (total > 0.0) {
          v = u * total;
          const uint64_t over = __ballot(l < G && run > v);
          if (over) {
            owner = __ffsll((unsigned long long)over) - 1;
          } else {  // v rounded onto the total: the last part with mass
            const uint64_t mass = __ballot(l < G && pq > 0.0);
            owner = 63 - __clzll((unsigned long long)mass);
          }
        }
        const double rx = wave_shr1(run);  // exclusive prefix over parts
        if (owner >= 0) pre = readlane_f64(rx, owner);
        if (l == 0) {
          owner_s = owner;
          pre_s = pre;
          v_s = v;
        }
        if (owner < 0) {
          // every D^2 is zero: the lowest candidate not chosen yet, over all parts
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) {
            const int f2 = __shfl_xor(fq, o, kWave);
            fq = f2 < fq ? f2 : fq;
          }
          if (l == 0) pick_s = fq < S ? fq : 0;
        }
      }
      __syncthreads();
      const int owner = owner_s;
      if (owner >= 0) {
        if (owner == part) {
          // per wave, the first candidate whose running sum exceeds v and the last one with mass
          // (rounding fallback), folded over the waves by LDS min / max
          const double v = v_s;
          const double pr = pre_s + wpre[w];
          const double pl = pre_s + wpre[kCoopWaves + w];
          const uint64_t hr = __ballot(d2r > 0.0 && pr + incr > v);
          const uint64_t hq = __ballot(d2l > 0.0 && pl + incl > v);
          const uint64_t mr = __ballot(d2r > 0.0);
          const uint64_t mq = __ballot(d2l > 0.0);
          if (l == 0) {
            const int rb = c0 + w * kWave, lb = c0 + NT + w * kWave;
            const int f = hr ? rb + __ffsll((unsigned long long)hr) - 1
                             : (hq ? lb + __ffsll((unsigned long long)hq) - 1 : 0x7FFFFFFF);
            const int la = mq ? lb + 63 - __clzll((unsigned long long)mq)
                              : (mr ? rb + 63 - __clzll((unsigned long long)mr) : -1);
            if (f != 0x7FFFFFFF) atomicMin(&first_s, f);
            if (la >= 0) atomicMax(&last_s, la);
          }
          __syncthreads();
          if (tid == 0) {
            int best = first_s;
            if (best == 0x7FFFFFFF) best = last_s >= 0 ? last_s : c0;
            // the flag carries the pick (+1, so that 0 means not yet)
            __hip_atomic_store(&sync[m * 3 + 2], best + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            pick_s = best;
          }
        } else if (tid == 0) {
          const int f = spin_nonzero(&sync[m * 3 + 2], fail);
          pick_s = f > 0 ? f - 1 : 0;  // 0 only after a failed wait (then the result is wrong anyway)
        }
        __syncthreads();
      }
      t = pick_s;
    }
    // ---- centre y_t as bf16 pairs (high part, remainder); part 0 writes the output centroid
    for (int a2 = tid; a2 < D / 2; a2 += NT) {
      const uint16_t* xt = Xh + cand_row(t, S, N) * D;
      const float x0 = bf16_bits_to_f32(xt[2 * a2]), x1 = bf16_bits_to_f32(xt[2 * a2 + 1]);
      const float y0 = yh ? yh[(int64_t)t * D + 2 * a2] : x0;
      const float y1 = yh ? yh[(int64_t)t * D + 2 * a2 + 1] : x1;
      const uint32_t h0 = f32_to_bf16_bits(y0), h1 = f32_to_bf16_bits(y1);
      yhi[a2] = h0 | (h1 << 16);
      ylo[a2] = f32_to_bf16_bits(y0 - bf16_bits_to_f32(h0)) | (f32_to_bf16_bits(y1 - bf16_bits_to_f32(h1)) << 16);
      if (part == 0) {
        sd.cent[((int64_t)h * C + m) * D + 2 * a2] = x0;
        sd.cent[((int64_t)h * C + m) * D + 2 * a2 + 1] = x1;
      }
    }
    if (tid == 0) cc_s = xxh[t];
    __syncthreads();
    const double cc = cc_s;
    // ---- lower D^2 against the new centre. Dot products on packed bf16 pairs (v_dot2_f32_bf16,
    // fp32 accumulation) against y split into a bf16 high part and a bf16 remainder.
    {
      float accr = 0.f, accl = 0.f, accr2 = 0.f, accl2 = 0.f;  // high and low parts of y
      const uint32_t* lrow = lrows + tid * ROW_U32;
#pragma unroll
      for (int q = 0; q < ROW_U32; q += 4) {
        const u32x4_t hv = *reinterpret_cast<const u32x4_t*>(&yhi[q]);
        const u32x4_t lv = *reinterpret_cast<const u32x4_t*>(&ylo[q]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t xe = xr[q + e], he = hv[e], le = lv[e];
          accr = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xe), as_bf16x2(he), accr, false);
          accr2 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xe), as_bf16x2(le), accr2, false);
        }
        if (has_l) {
          const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(lrow + (((q / 4) ^ (tid % CPR)) * 4));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t xe = xv[e], he = hv[e], le = lv[e];
            accl = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xe), as_bf16x2(he), accl, false);
            accl2 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xe), as_bf16x2(le), accl2, false);
          }
        }
      }
      accr += accr2;
      accl += accl2;
      if (has_r) {
        if (c0 + tid == t) {
          taken_r = true;
          d2r = 0.0;
        } else if (!taken_r) {
          double dist = xx_r - 2.0 * (double)accr + cc;
          dist = dist > 0.0 ? dist : 0.0;
          d2r = (m == 0 || dist < d2r) ? dist : d2r;
        }
      }
      if (has_l) {
        if (c0 + NT + tid == t) {
          taken_l = true;
          d2l = 0.0;
        } else if (!taken_l) {
          double dist = xx_l - 2.0 * (double)accl + cc;
          dist = dist > 0.0 ? dist : 0.0;
          d2l = (m == 0 || dist < d2l) ? dist : d2l;
        }
      }
    }
    __syncthreads();
  }
  if (tid == 0 && status != nullptr && __hip_atomic_load(fail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
    __hip_atomic_fetch_or(status, kSeedTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void fill_i32(int* p, int64_t n, int v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// ------------------------------------------------------------------------------------------------
// Update: member means, then the consumed centroid form (g, b) for the next assignment
// ------------------------------------------------------------------------------------------------

// One workgroup per (cluster, head). With do_update, c_j = fp32(fp64 mean of the members, summed
// in cluster order); empty clusters keep their value. Euclidean sides also write g_j (c_j, bf16-
// rounded for bf16 data) and b_j = fp32(sum g_j^2); QRKC sides get (g, b) from consume_qrkc.
template <typename T, int D>
__global__ __launch_bounds__(256) void centroid_mean(const T* __restrict__ X, int64_t N, int C,
                                                     const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ offsets, float* __restrict__ cent,
                                                     int do_update, int euclid, void* g_out, float* __restrict__ b_out,
                                                     int bf16) {
  constexpr int CPR = D / 8;     // 8-element pieces per row
  constexpr int RG = 256 / CPR;  // row groups
  __shared__ double part[RG][D];
  __shared__ double red[4];
  const int j = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  float* cj = cent + ((int64_t)h * C + j) * D;
  float c = 0.f;
  int n = 0;
  if (do_update) {
    const int beg = offsets[(int64_t)h * (C + 1) + j];
    const int end = offsets[(int64_t)h * (C + 1) + j + 1];
    n = end - beg;
    if (n > 0) {
      const int pc = tid % CPR;
      const int rg = tid / CPR;
      const T* Xh = X + (int64_t)h * N * D;
      const int32_t* ph = perm + (int64_t)h * N;
      double acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.0;
      // rows beg + rg + RG k in increasing k; U member indices, then U rows, in flight at a time
      constexpr int U = 8;
      for (int r0 = beg + rg; r0 < end; r0 += U * RG) {
        int idx[U];
#pragma unroll
        for (int u = 0; u < U; ++u) idx[u] = ph[min(r0 + u * RG, end - 1)];
        float xv[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) load8_f32(Xh + (int64_t)idx[u] * D + pc * 8, xv[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (r0 + u * RG < end) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += (double)xv[u][e];
          }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) part[rg][pc * 8 + e] = acc[e];
      __syncthreads();
      if (tid < D) {
        double sum = 0.0;
#pragma unroll
        for (int q = 0; q < RG; ++q) sum += part[q][tid];
        c = (float)(sum / (double)n);
        cj[tid] = c;
      }
    }
  }
  if (!euclid) return;
  if (n == 0 && tid < D) c = cj[tid];
  double term = 0.0;
  if (tid < D) {
    const int64_t gi = ((int64_t)h * C + j) * D + tid;
    float gv = c;
    if (bf16) {
      gv = bf16_bits_to_f32(f32_to_bf16_bits(gv));
      static_cast<uint16_t*>(g_out)[gi] = (uint16_t)(__float_as_uint(gv) >> 16);
    } else {
      static_cast<float*>(g_out)[gi] = gv;
    }
    term = (double)gv * (double)gv;
  }
  term = wave_sum_f64(term);
  if (lane_id() == 0) red[tid / kWave] = term;
  __syncthreads();
  if (tid == 0) b_out[(int64_t)h * C + j] = (float)(((red[0] + red[1]) + red[2]) + red[3]);
}

// QRKC consumed form for 32 centroids per block: y_j = M c_j (fp64 sums of fp64 products of the
// fp32 values; M staged in LDS as fp32 and read along columns, which M's symmetry makes equal to
// rows), g_j = fp32(y_j) (then bf16), b_j = fp32(c_j . y_j). Register tiles: thread t computes
// y_ja for the 4 centroids j = 4 (t / 32) + 0..3 and the D / 32 dims a = (t % 32) + 32 i, so per b
// it reads D / 32 values of M and 4 of c (the latter shared by the 32 threads of a half-wave).
template <int D>
__global__ __launch_bounds__(256) void consume_qrkc(const float* __restrict__ cent, int C, const float* __restrict__ M,
                                                    void* g_out, float* __restrict__ b_out, int bf16) {
  constexpr int JB = 32;      // centroids per block
  constexpr int AT = D / 32;  // dims per thread
  extern __shared__ float cq_lds[];
  float* ms = cq_lds;           // [D][D]
  float* cs = cq_lds + D * D;   // [JB][D]
  const int h = blockIdx.y;
  const int j0 = blockIdx.x * JB;
  // all staging loads of a thread are issued before their LDS stores
  f32x4_t mv4[D * D / 4 / 256], cv4[JB * D / 4 / 256];
#pragma unroll
  for (int k = 0; k < D * D / 4 / 256; ++k)
    mv4[k] = *reinterpret_cast<const f32x4_t*>(M + (int64_t)h * D * D + (threadIdx.x + k * 256) * 4);
#pragma unroll
  for (int k = 0; k < JB * D / 4 / 256; ++k) {
    const int e = (threadIdx.x + k * 256) * 4;
    cv4[k] = *reinterpret_cast<const f32x4_t*>(cent + ((int64_t)h * C + min(j0 + e / D, C - 1)) * D + e % D);
  }
#pragma unroll
  for (int k = 0; k < D * D / 4 / 256; ++k) *reinterpret_cast<f32x4_t*>(ms + (threadIdx.x + k * 256) * 4) = mv4[k];
#pragma unroll
  for (int k = 0; k < JB * D / 4 / 256; ++k) {
    const int e = (threadIdx.x + k * 256) * 4;
    f32x4_t v = cv4[k];
    if (j0 + e / D >= C) v = f32x4_t{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4_t*>(cs + e) = v;
  }
  __syncthreads();
  const int ai = threadIdx.x % 32;
  const int jg = threadIdx.x / 32;  // centroids 4 jg .. 4 jg + 3
  double acc[4][AT];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < AT; ++i) acc[q][i] = 0.0;
  for (int b = 0; b < D; ++b) {
    double m[AT], c[4];
#pragma unroll
    for (int i = 0; i < AT; ++i) m[i] = (double)ms[b * D + ai + 32 * i];  // M[b][a] == M[a][b]
#pragma unroll
    for (int q = 0; q < 4; ++q) c[q] = (double)cs[(4 * jg + q) * D + b];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < AT; ++i) acc[q][i] = __builtin_fma(m[i], c[q], acc[q][i]);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int jl = 4 * jg + q;
    const int j = j0 + jl;
    double term = 0.0;
#pragma unroll
    for (int i = 0; i < AT; ++i) {
      const int a = ai + 32 * i;
      term += (double)cs[jl * D + a] * acc[q][i];
      if (j < C) {
        const int64_t gi = ((int64_t)h * C + j) * D + a;
        const float gv = (float)acc[q][i];
        if (bf16)
          static_cast<uint16_t*>(g_out)[gi] = (uint16_t)f32_to_bf16_bits(gv);
        else
          static_cast<float*>(g_out)[gi] = gv;
      }
    }
    // the 32 threads of this half-wave hold the dims of centroid j
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) term += __shfl_xor(term, o, kWave);
    if (ai == 0 && j < C) b_out[(int64_t)h * C + j] = (float)term;
  }
}

// ------------------------------------------------------------------------------------------------
// Assignment
// ------------------------------------------------------------------------------------------------

constexpr int kAsgChunk = 128;  // centroids staged in LDS at a time

// Argmax keys. A lane holds 16 scores of one point per 32-centroid tile (slots 0..15, increasing
// centroid index). Its key replaces the 4 low mantissa bits of the fp32 score by 15 - slot, so one
// float max over keys finds the best score and, among scores equal in their top 20 bits, the
// lowest slot (for non-negative scores; equal negative scores go to the highest slot). Dropping
// 4 bits perturbs a comparison by less than 2^-19 of the scores' magnitude.
__device__ __forceinline__ float asg_key(float s, uint32_t code) {
  return __uint_as_float((__float_as_uint(s) & ~15u) | code);
}
__device__ __forceinline__ float asg_trunc(float k) { return __uint_as_float(__float_as_uint(k) & ~15u); }
// v_max3_f32 (keys are finite, never NaN)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// bf16 data. Each wave owns PT*32 points held as MFMA B operands; centroid tiles of 32 rows are
// the A operands. The accumulator starts at -b_j/2, so it holds x.g_j - b_j/2 and the label is the
// argmax. Per tile the lane's 16 keys are reduced with v_max3; the running best moves to a later
// tile only when that tile's best is larger in its top 20 bits, so equal scores keep the lower
// centroid index across tiles. Registers are capped for three waves per SIMD, so that one wave's
// MFMAs run while the others compare.
// Rows: the M points phase + p * stride, p < M (every row: stride 1, phase 0, M = N); the labels of
// the other rows are left as they are (subset updates).
template <int D, int PT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void assign_bf16(const uint16_t* __restrict__ X, int64_t N, int C,
                                                   const uint16_t* __restrict__ G, const float* __restrict__ b,
                                                   int32_t* __restrict__ labels, int64_t M, int stride,
                                                   int phase) {
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
    const int64_t row = phase + p * stride;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (p < M) v = *reinterpret_cast<const u32x4_t*>(Xh + row * D + kk * 16 + hl * 8);
      xb[pt][kk] = v;
    }
  }
  float best[PT];   // key of the best score so far
  float bestt[PT];  // its top 20 bits
  int btile[PT];    // its tile
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) {
    best[pt] = -FLT_MAX;
    bestt[pt] = -FLT_MAX;
    btile[pt] = 0;
  }
  // Centroid chunks of 128 rows pass through LDS; the next chunk is fetched into registers while
  // the current one is in use (loads clamped to row C - 1, padding rows zeroed on the LDS store).
  constexpr int PPT = kAsgChunk * (D / 8) / 256;  // 16-byte pieces per thread and chunk
  u32x4_t pre[PPT];
  float preb;
  auto fetch = [&](int cn) {
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
      const int e = threadIdx.x + q * 256;
      const int row = min(cn + e / (D / 8), C - 1);
      pre[q] = *reinterpret_cast<const u32x4_t*>(Gh + (int64_t)row * D + (e % (D / 8)) * 8);
    }
    preb = bh[min(cn + (int)(threadIdx.x % kAsgChunk), C - 1)];
  };
  fetch(0);
  for (int c0 = 0; c0 < C; c0 += kAsgChunk) {
    // stage centroids [c0, c0 + 128) and -b/2 (padding rows: zero centroid, score -FLT_MAX)
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
      const int e = threadIdx.x + q * 256;
      const int r = e / (D / 8);
      u32x4_t v = pre[q];
      if (c0 + r >= C) v = u32x4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(&gl[r * STR + (e % (D / 8)) * 8]) = v;
    }
    if (threadIdx.x < kAsgChunk) hb[threadIdx.x] = (c0 + (int)threadIdx.x < C) ? -0.5f * preb : -FLT_MAX;
    __syncthreads();
    if (c0 + kAsgChunk < C) fetch(c0 + kAsgChunk);
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
      const int tile = c0 / 32 + ct;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        float t = max3f(asg_key(acc[pt][0], 15u), asg_key(acc[pt][1], 14u), asg_key(acc[pt][2], 13u));
#pragma unroll
        for (int i = 3; i < 15; i += 2)
          t = max3f(t, asg_key(acc[pt][i], 15u - i), asg_key(acc[pt][i + 1], 14u - i));
        t = max3f(t, asg_key(acc[pt][15], 0u), asg_key(acc[pt][15], 0u));
        const float tt = asg_trunc(t);
        if (tt > bestt[pt]) {
          best[pt] = t;
          bestt[pt] = tt;
          btile[pt] = tile;
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) {
    const int slot = 15 - (int)(__float_as_uint(best[pt]) & 15u);
    int bi = btile[pt] * 32 + (slot / 4) * 8 + hl * 4 + slot % 4;
    // the other half-wave holds the other 16 centroids of every tile for the same point
    const float ob = __shfl_xor(bestt[pt], 32, kWave);
    const int oi = __shfl_xor(bi, 32, kWave);
    if (ob > bestt[pt] || (ob == bestt[pt] && oi < bi)) bi = oi;
    const int64_t p = p_base + pt * 32 + l % 32;
    if (hl == 0 && p < M) labels[(int64_t)h * N + phase + p * stride] = bi;
  }
}

// fp32 data: one thread per point, fp64 dot products against fp32 centroids staged in LDS.
template <int D>
__global__ __launch_bounds__(256) void assign_f32(const float* __restrict__ X, int64_t N, int C,
                                                  const float* __restrict__ G, const float* __restrict__ b,
                                                  int32_t* __restrict__ labels, int64_t M, int stride, int phase) {
  constexpr int CH = 32;
  __shared__ float gl[CH * D];
  __shared__ float bl[CH];
  const int h = blockIdx.y;
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = phase + (p < M ? p : 0) * stride;
  const float* x = X + ((int64_t)h * N + row) * D;
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
  if (p < M) labels[(int64_t)h * N + row] = bi;
}

// ------------------------------------------------------------------------------------------------
// Fused Euclidean Lloyd step (bf16 data, at most 128 clusters): the assignment and the per-cluster
// sums of the members in one pass over the points
// ------------------------------------------------------------------------------------------------

constexpr int kFuseT = 128;        // points per tile
constexpr int kFuseThreads = 512;  // eight waves

// Work-group (g, h) takes the tiles [g nt / P, (g + 1) nt / P) of head h (nt tiles of 128 points,
// P work-groups per head), staged in LDS in two buffers (rows XOR-swizzled by 16-byte chunk,
// chunk_swz; the loads of a tile are issued two tiles ahead). Per tile:
//  A. the assignment exactly as assign_bf16 computes it (same MFMAs, accumulators started at
//     -b_j/2, the same packed-key argmax): wave w takes the 32 points 32 (w % 4) .. and the
//     clusters 64 (w / 4) .. + 63; the two cluster halves of a point are merged in LDS (larger top
//     20 bits of the score, ties to the lower index, as the sequential scan over tiles gives);
//  B. the member sums S[c][d] += sum_p [label_p == c] x_p[d]: 32x32x16 MFMAs of a 0/1 matrix and
//     the points (transposing LDS reads, eight consecutive points of one dimension per lane for both
//     factors). The 0/1 factor comes from a per-tile membership bit mask of every cluster (set by
//     LDS atomics when the labels are merged): eight bits of it select one 16-byte entry of a
//     256-entry table of bf16 0/1 patterns; wave w owns the clusters 32 (w / 2) .. + 31 and the
//     dimensions (D / 2) (w % 2) .. ; each tile's fp32 sums (at most 128 terms) are added into
//     fp64 accumulators in tile order, so the sums do not depend on scheduling.
// Outputs: the labels, and per work-group the fp64 sums [C][D] and the member counts [C].
template <int D>
__global__ __launch_bounds__(kFuseThreads) void lloyd_fused(const uint16_t* __restrict__ X, int64_t N, int C,
                                                            const uint16_t* __restrict__ G,
                                                            const float* __restrict__ b,
                                                            int32_t* __restrict__ labels, double* __restrict__ psum,
                                                            int32_t* __restrict__ pcnt, int P) {
  constexpr int KS = D / 16;               // 16-dimension MFMA steps of the assignment
  constexpr int STR = D + 8;               // padded centroid row (bf16 elements)
  constexpr int CPR = D / 8;               // 16-byte chunks per point row
  constexpr int DTW = D / 64;              // 32-dimension tiles per wave in the sums
  constexpr int LOADS = kFuseT * CPR / kFuseThreads;  // 16-byte loads per thread and tile
  __shared__ __attribute__((aligned(16))) uint16_t xt[2][kFuseT * D];
  __shared__ __attribute__((aligned(16))) uint16_t gl[kFuseT * STR];
  __shared__ float hb[kFuseT];
  __shared__ float hbt[2][kFuseT];  // per cluster half: best top-20-bit score of each point
  __shared__ int hbi[2][kFuseT];    // and its cluster
  __shared__ __attribute__((aligned(16))) uint32_t mbits[kFuseT][kFuseT / 32];  // [cluster][point / 32]
  __shared__ __attribute__((aligned(16))) u32x4_t ohlut[256];  // bit i of e -> element i is bf16 1.0
  static_assert(kFuseT * kFuseT / 32 == kFuseThreads, "one membership word per thread");
  __shared__ int cnt[kFuseT];
  const int h = blockIdx.y;
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int hl = l / 32;
  const int g16 = l / 16, i16 = l % 16;
  const int64_t nt = (N + kFuseT - 1) / kFuseT;
  const int64_t tb = (int64_t)g * nt / P, te = (int64_t)(g + 1) * nt / P;
  const uint16_t* Xh = X + (int64_t)h * N * D;

  // centroids (rows past C: zero, score -FLT_MAX) and counts
  for (int e = tid; e < kFuseT * (D / 8); e += kFuseThreads) {
    const int r = e / (D / 8), c8 = e % (D / 8);
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (r < C) v = *reinterpret_cast<const u32x4_t*>(G + ((int64_t)h * C + r) * D + c8 * 8);
    *reinterpret_cast<u32x4_t*>(&gl[r * STR + c8 * 8]) = v;
  }
  for (int r = tid; r < kFuseT; r += kFuseThreads) {
    hb[r] = r < C ? -0.5f * b[(int64_t)h * C + r] : -FLT_MAX;
    cnt[r] = 0;
  }
  for (int e = tid; e < 256; e += kFuseThreads) {
    u32x4_t v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = ((e >> (2 * j)) & 1 ? 0x3F80u : 0u) | ((e >> (2 * j + 1)) & 1 ? 0x3F800000u : 0u);
    ohlut[e] = v;
  }

  // staging of tile t: pieces e = tid + 512 q: point row e / CPR, chunk e % CPR (rows past N: zero)
  auto gload = [&](u32x4_t(&pre)[LOADS], int64_t t) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
      const int e = tid + q * kFuseThreads;
      const int64_t row = min(t * kFuseT + e / CPR, N - 1);
      pre[q] = *reinterpret_cast<const u32x4_t*>(Xh + row * D + (e % CPR) * 8);
    }
  };
  auto sstore = [&](const u32x4_t(&pre)[LOADS], int buf, int64_t t) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
      const int e = tid + q * kFuseThreads;
      const int r = e / CPR, c = e % CPR;
      u32x4_t v = pre[q];
      if (t * kFuseT + r >= N) v = u32x4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(&xt[buf][r * D + (c ^ chunk_swz<CPR>(r)) * 8]) = v;
    }
  };

  // phase A: this lane's point (rows permuted so that each 16-lane group reads distinct swizzles)
  const int pw = w & 3, ch = w >> 2;
  const int r32 = l % 32;
  const int prow = pw * 32 + ((r32 / 4) % 2) * 16 + (r32 / 8) * 4 + r32 % 4;
  const int pswz = chunk_swz<CPR>(prow);
  // phase B: transposing-read offsets (bf16 elements) of dimension tile dt, sub-tile st, half kh,
  // rows z
  const int cw = w >> 1, dt0 = (w & 1) * DTW;
  int tofs[DTW][4][2][2];
#pragma unroll
  for (int x = 0; x < DTW; ++x) {
    const int D0 = (dt0 + x) * 32 + 16 * (g16 & 1);
    const int cc = (D0 + 4 * (i16 % 4)) / 8;
    const int half = (i16 % 4) & 1;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int z = 0; z < 2; ++z) {
          const int R = st * 32 + 16 * (g16 >> 1) + 8 * kh + i16 / 4 + 4 * z;
          tofs[x][st][kh][z] = R * D + (cc ^ chunk_swz<CPR>(R)) * 8 + half * 4;
        }
  }
  f32x16_t sacc[DTW];
  double s64[DTW][16];
#pragma unroll
  for (int x = 0; x < DTW; ++x)
#pragma unroll
    for (int i = 0; i < 16; ++i) s64[x][i] = 0.0;

  auto tile = [&](u32x4_t(&pre)[LOADS], int buf, int64_t t) __attribute__((always_inline)) {
    // tile t into buffer buf (read two tiles ago, before the previous tile's last barrier)
    sstore(pre, buf, t);
    __syncthreads();
    if (t + 2 < te) gload(pre, t + 2);
    (&mbits[0][0])[tid] = 0u;  // the previous tile's masks were read before the barrier above
    // ---- A: scores of this lane's point against the clusters 64 ch .. + 63
    float best = -FLT_MAX, bestt = -FLT_MAX;
    int btile = 2 * ch;
#pragma unroll
    for (int cti = 0; cti < 2; ++cti) {
      const int ct = 2 * ch + cti;
      f32x16_t acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = hb[ct * 32 + (i / 4) * 8 + hl * 4 + i % 4];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&gl[(ct * 32 + l % 32) * STR + kk * 16 + hl * 8]);
        const u32x4_t xb = *reinterpret_cast<const u32x4_t*>(&xt[buf][prow * D + ((2 * kk + hl) ^ pswz) * 8]);
        acc = mfma32(a, xb, acc);
      }
      float tk = max3f(asg_key(acc[0], 15u), asg_key(acc[1], 14u), asg_key(acc[2], 13u));
#pragma unroll
      for (int i = 3; i < 15; i += 2) tk = max3f(tk, asg_key(acc[i], 15u - i), asg_key(acc[i + 1], 14u - i));
      tk = max3f(tk, asg_key(acc[15], 0u), asg_key(acc[15], 0u));
      const float tt = asg_trunc(tk);
      if (tt > bestt) {
        best = tk;
        bestt = tt;
        btile = ct;
      }
    }
    {
      const int slot = 15 - (int)(__float_as_uint(best) & 15u);
      int bi = btile * 32 + (slot / 4) * 8 + hl * 4 + slot % 4;
      const float ob = __shfl_xor(bestt, 32, kWave);
      const int oi = __shfl_xor(bi, 32, kWave);
      if (ob > bestt || (ob == bestt && oi < bi)) bi = oi;
      if (hl == 0) {
        hbt[ch][prow] = fmaxf(bestt, ob);
        hbi[ch][prow] = bi;
      }
    }
    __syncthreads();
    // merge the cluster halves (the second only when strictly better: ties keep the lower index)
    if (tid < kFuseT) {
      const int64_t p = t * kFuseT + tid;
      int lb = hbt[1][tid] > hbt[0][tid] ? hbi[1][tid] : hbi[0][tid];
      if (p < N) {
        labels[(int64_t)h * N + p] = lb;
        atomicAdd(&cnt[lb], 1);
        atomicOr(&mbits[lb][tid / 32], 1u << (tid % 32));
      }
    }
    __syncthreads();
    // ---- B: member sums of this tile
#pragma unroll
    for (int x = 0; x < DTW; ++x)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[x][i] = 0.f;
    const PARK_LDS uint16_t* xs = (const PARK_LDS uint16_t*)&xt[buf][0];
    // membership of this lane's cluster in the tile: bit i of word st = point 32 st + i
    const u32x4_t mw = *reinterpret_cast<const u32x4_t*>(&mbits[cw * 32 + l % 32][0]);
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        // the 0/1 factor of the points 32 st + 16 hl + 8 kh .. + 7 (two points per word)
        const u32x4_t oh = ohlut[(mw[st] >> (16 * hl + 8 * kh)) & 0xFFu];
#pragma unroll
        for (int x = 0; x < DTW; ++x) {
          const s16x4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PARK_LDS s16x4_t*)(xs + tofs[x][st][kh][0]));
          const s16x4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PARK_LDS s16x4_t*)(xs + tofs[x][st][kh][1]));
          const u32x2_t u0 = __builtin_bit_cast(u32x2_t, r0), u1 = __builtin_bit_cast(u32x2_t, r1);
          sacc[x] = mfma32(oh, u32x4_t{u0[0], u0[1], u1[0], u1[1]}, sacc[x]);
        }
      }
#pragma unroll
    for (int x = 0; x < DTW; ++x)
#pragma unroll
      for (int i = 0; i < 16; ++i) s64[x][i] += (double)sacc[x][i];
  };

  u32x4_t pa[LOADS], pb[LOADS];
  if (tb < te) gload(pa, tb);
  if (tb + 1 < te) gload(pb, tb + 1);
  for (int64_t t = tb; t < te; t += 2) {
    tile(pa, 0, t);
    if (t + 1 < te) tile(pb, 1, t + 1);
  }
  __syncthreads();  // counts complete
  // element i of lane l in sums tile (cw, dt): cluster cw * 32 + (i / 4) * 8 + (l / 32) * 4 + i % 4,
  // dimension dt * 32 + l % 32
  double* ps = psum + ((int64_t)h * P + g) * C * D;
#pragma unroll
  for (int x = 0; x < DTW; ++x)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = cw * 32 + (i / 4) * 8 + (l / 32) * 4 + i % 4;
      if (c < C) ps[(int64_t)c * D + (dt0 + x) * 32 + l % 32] = s64[x][i];
    }
  for (int c = tid; c < C; c += kFuseThreads) pcnt[((int64_t)h * P + g) * C + c] = cnt[c];
}

// Per (cluster j, head): the member mean from the work-groups' sums (added in work-group order);
// empty clusters keep their centroid.
__global__ __launch_bounds__(128) void lloyd_fused_means(const double* __restrict__ psum,
                                                         const int32_t* __restrict__ pcnt, int C, int D, int P,
                                                         float* __restrict__ cent) {
  const int j = blockIdx.x, h = blockIdx.y;
  int n = 0;
  for (int g = 0; g < P; ++g) n += pcnt[((int64_t)h * P + g) * C + j];
  if (n == 0) return;
  for (int d = threadIdx.x; d < D; d += 128) {
    double s = 0.0;
    for (int g = 0; g < P; ++g) s += psum[(((int64_t)h * P + g) * C + j) * D + d];
    cent[((int64_t)h * C + j) * D + d] = (float)(s / (double)n);
  }
}

// Labels outside [0, C) (a caller's stale buffer) become cluster 0, so that the sort and update
// of a subset step never index outside their tables.
__global__ void clamp_labels(int32_t* __restrict__ labels, int64_t n, int C) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    const int v = labels[i];
    if (v < 0 || v >= C) labels[i] = 0;
  }
}

// ------------------------------------------------------------------------------------------------
// Stable counting sort: per-chunk histograms -> per-head scan -> ordered scatter
// ------------------------------------------------------------------------------------------------

__global__ __launch_bounds__(64) void sort_hist(const int32_t* __restrict__ labels, int64_t N, int C, int nchunk,
                                                int32_t* __restrict__ table) {
  __shared__ int cnt[kMaxClusters];
  constexpr int R = kSortChunk / 64;
  const int h = blockIdx.y;
  const int ch = blockIdx.x;
  const int64_t t0 = (int64_t)ch * kSortChunk + lane_id();
  const int32_t* lh = labels + (int64_t)h * N;
  int lab[R];  // all loads issued before the first use
#pragma unroll
  for (int r = 0; r < R; ++r) lab[r] = lh[min(t0 + r * 64, N - 1)];
  for (int c = threadIdx.x; c < C; c += 64) cnt[c] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (t0 + r * 64 < N) atomicAdd(&cnt[lab[r]], 1);
  __syncthreads();
  int32_t* out = table + ((int64_t)h * nchunk + ch) * C;
  for (int c = threadIdx.x; c < C; c += 64) out[c] = cnt[c];
}

// Per (head, cluster c): table[chunk][c] <- tokens of cluster c in the chunks before `chunk`
// (exclusive prefix over chunks, 16 loads in flight per thread); tot[c] <- all tokens of cluster c.
__global__ __launch_bounds__(64) void sort_scan_chunks(int32_t* __restrict__ table, int nchunk, int C,
                                                       int32_t* __restrict__ tot) {
  constexpr int B = 16;
  const int h = blockIdx.y;
  const int c = blockIdx.x * 64 + threadIdx.x;
  if (c >= C) return;
  int32_t* th = table + (int64_t)h * nchunk * C + c;
  int run = 0;
  for (int k0 = 0; k0 < nchunk; k0 += B) {
    int v[B];
#pragma unroll
    for (int q = 0; q < B; ++q) v[q] = th[(int64_t)min(k0 + q, nchunk - 1) * C];
#pragma unroll
    for (int q = 0; q < B; ++q) {
      if (k0 + q < nchunk) {
        th[(int64_t)(k0 + q) * C] = run;
        run += v[q];
      }
    }
  }
  tot[(int64_t)h * (C + 1) + c] = run;
}

// Per head: offsets[c] <- tokens with label < c (in place over the cluster totals), offsets[C] = N.
__global__ __launch_bounds__(1024) void sort_scan_offsets(int32_t* __restrict__ offsets, int C) {
  __shared__ int scratch[17];
  const int h = blockIdx.x;
  int32_t* oh = offsets + (int64_t)h * (C + 1);
  const int per = (C + 1023) / 1024;
  const int c_beg = threadIdx.x * per;
  int v[(kMaxClusters + 1023) / 1024];
  int local = 0;
#pragma unroll
  for (int k = 0; k < (kMaxClusters + 1023) / 1024; ++k) {
    v[k] = (k < per && c_beg + k < C) ? oh[c_beg + k] : 0;
    local += v[k];
  }
  int total;
  int run = block_exclusive_scan(local, scratch, &total);
#pragma unroll
  for (int k = 0; k < (kMaxClusters + 1023) / 1024; ++k) {
    if (k < per && c_beg + k < C) {
      oh[c_beg + k] = run;
      run += v[k];
    }
  }
  if (threadIdx.x == 0) oh[C] = total;
}

// One wave per chunk: tokens are placed in order, 64 at a time. A lane's peers (lanes with the same
// label) come from one ballot per label bit; its rank among them is the number of lower peer lanes,
// which keeps the original order inside each cluster, and the lowest peer advances the cluster's
// cursor. A single wave's LDS accesses complete in program order, so no barrier is needed between
// reading and advancing the cursors. Cursors start at offsets[c] + table[chunk][c].
__global__ __launch_bounds__(64) void sort_scatter(const int32_t* __restrict__ labels, int64_t N, int C,
                                                   int nchunk, const int32_t* __restrict__ table,
                                                   const int32_t* __restrict__ offsets, int32_t* __restrict__ perm) {
  __shared__ int cursor[kMaxClusters];
  constexpr int R = kSortChunk / 64;
  const int h = blockIdx.y;
  const int ch = blockIdx.x;
  const int l = lane_id();
  const int32_t* lh = labels + (int64_t)h * N;
  const int64_t t0 = (int64_t)ch * kSortChunk + l;
  int labs[R];  // all loads issued before the first use
#pragma unroll
  for (int r = 0; r < R; ++r) labs[r] = lh[min(t0 + r * 64, N - 1)];
  const int32_t* base = table + ((int64_t)h * nchunk + ch) * C;
  const int32_t* oh = offsets + (int64_t)h * (C + 1);
  for (int c0 = 0; c0 < C; c0 += 8 * 64) {  // 8 clusters per lane in flight
    int v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = min(c0 + k * 64 + l, C - 1);
      v[k] = base[c] + oh[c];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (c0 + k * 64 + l < C) cursor[c0 + k * 64 + l] = v[k];
  }
  __syncthreads();
  int32_t* ph = perm + (int64_t)h * N;
  const uint64_t lt_mask = (l == 0) ? 0ull : (~0ull >> (64 - l));
  constexpr int kLabelBits = 11;  // labels < kMaxClusters = 2^11
  static_assert((1 << kLabelBits) >= kMaxClusters, "label bits");
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t t = t0 + r * 64;
    const bool valid = t < N;
    const int lab = labs[r];
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int k = 0; k < kLabelBits; ++k) {
      const bool bit = (lab >> k) & 1;
      const uint64_t ones = __ballot(bit);
      peers &= bit ? ones : ~ones;
    }
    if (valid) {
      const int c0 = cursor[lab];
      const int pos = c0 + __popcll(peers & lt_mask);
      ph[pos] = (int32_t)t;
      if ((peers & lt_mask) == 0) cursor[lab] = c0 + __popcll(peers);
    }
  }
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------------------

std::atomic<int> g_force_seed_timeout{0};

// Single-workgroup seeding (any dtype): candidate norms, then one workgroup per (head, side).
static hipError_t launch_kpp_single(const Dims& s, const KppArgs* sides, int nsides, uint64_t seed, hipStream_t st) {
  KppSide ks[2];
  int smax = 0;
  for (int q = 0; q < nsides; ++q) {
    const KppArgs& a = sides[q];
    const int S = kpp_candidates(s.N, a.C);
    smax = S > smax ? S : smax;
    ks[q] = KppSide{a.x, a.xx, a.metric ? a.y : nullptr, a.cent, a.C, S, a.side};
  }
  if (nsides == 1) ks[1] = ks[0];
  const dim3 grid((unsigned)s.H, (unsigned)nsides);
  const size_t lds = (size_t)smax * sizeof(double);
#define PARK_SEED(T, D) kpp_seed<T, D><<<grid, kKppThreads, lds, st>>>(ks[0], ks[1], s.N, seed);
  if (s.bf16) {
    if (s.D == 128) {
      PARK_SEED(uint16_t, 128)
    } else {
      PARK_SEED(uint16_t, 64)
    }
  } else {
    if (s.D == 128) {
      PARK_SEED(float, 128)
    } else {
      PARK_SEED(float, 64)
    }
  }
#undef PARK_SEED
  return hipGetLastError();
}

// Parts per side for the cooperative seeding within `budget` workgroups per head; false if the
// candidates cannot be held on chip with that budget.
static bool plan_parts(const Dims& s, const KppArgs* sides, int nsides, int budget, int nt, int* G) {
  const int lmax = (140 * 1024) / (int)(s.D * 2);  // LDS-resident rows per part
  const int cap = nt + lmax;
  int used = 0;
  double work[2];
  for (int q = 0; q < nsides; ++q) {
    const int S = kpp_candidates(s.N, sides[q].C);
    G[q] = (int)ceil_div(S, cap);
    if (G[q] > kCoopMaxParts) return false;
    used += G[q];
    work[q] = (double)sides[q].C * S;
  }
  if (used > budget) return false;
  // spare workgroups go where the per-part work is largest
  while (used < budget) {
    int best = -1;
    double bw = 0.0;
    for (int q = 0; q < nsides; ++q) {
      const int S = kpp_candidates(s.N, sides[q].C);
      if (G[q] >= kCoopMaxParts || ceil_div(S, G[q] + 1) < 256) continue;
      const double wq = work[q] / G[q];
      if (wq > bw) {
        bw = wq;
        best = q;
      }
    }
    if (best < 0) break;
    ++G[best];
    ++used;
  }
  return true;
}

// One cooperative launch over heads h0 .. h0 + Hb - 1. The failure flag of a launch sits after its
// heads' step flags (for a leading batch: on the first flag of the next batch, which that batch's
// own launch clears before it runs).
static hipError_t launch_kpp_coop(const Dims& s, const KppArgs* sides, int nsides, const int* G, int nt,
                                  uint64_t seed, int* status, hipStream_t st, int h0 = 0, int Hb = -1) {
  if (Hb < 0) Hb = (int)s.H;
  CoopSide cs[2];
  size_t lds = 0;
  int64_t total = 0;
  for (int q = 0; q < nsides; ++q) {
    const KppArgs& a = sides[q];
    const int S = kpp_candidates(s.N, a.C);
    const int SP = (int)ceil_div(S, G[q]);
    uint64_t* psum = reinterpret_cast<uint64_t*>(a.psum) + (int64_t)h0 * a.C * kCoopMaxParts * 2;
    int* sync = a.sync + (int64_t)h0 * a.C * 3;
    cs[q] = CoopSide{static_cast<const uint16_t*>(a.x) + (int64_t)h0 * s.N * s.D, a.xx + (int64_t)h0 * S,
                     a.metric ? a.y + (int64_t)h0 * S * s.D : nullptr, a.cent + (int64_t)h0 * a.C * s.D, psum,
                     sync, a.C, S, a.side, G[q], SP};
    const size_t l = (size_t)(SP > nt ? SP - nt : 0) * (size_t)s.D * 2;
    lds = l > lds ? l : lds;
    total += (int64_t)Hb * G[q];
    const int64_t nsync = (int64_t)Hb * a.C * 3 + 1;
    fill_i32<<<(unsigned)ceil_div(nsync, 256), 256, 0, st>>>(sync, nsync, 0);
    const int64_t nslot = (int64_t)Hb * a.C * kCoopMaxParts * 2 * 2;  // as int32 words
    fill_i32<<<(unsigned)ceil_div(nslot, 256), 256, 0, st>>>(reinterpret_cast<int*>(psum), nslot, 0);
    // failure-handling hook: a raised flag makes every wait of the launch give up at once
    if (g_force_seed_timeout.load(std::memory_order_relaxed))
      fill_i32<<<1, 256, 0, st>>>(sync + (int64_t)Hb * a.C * 3, 1, 1);
  }
  if (nsides == 1) {
    cs[1] = cs[0];
    cs[1].G = 0;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int H = Hb;
  int64_t N = s.N;
  void* args[] = {&cs[0], &cs[1], &H, &h0, &N, &seed, &status};
  const void* fn = nt == kCoopThreads
                       ? (s.D == 128 ? (const void*)kpp_coop<128, kCoopThreads> : (const void*)kpp_coop<64, kCoopThreads>)
                       : (s.D == 128 ? (const void*)kpp_coop<128, kCoopThreadsWide>
                                     : (const void*)kpp_coop<64, kCoopThreadsWide>);
  (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  return hipLaunchCooperativeKernel(fn, dim3((unsigned)total), dim3((unsigned)nt), args, (unsigned)lds, st);
}

// Sides whose candidates need more 512-thread parts per head than one launch over all heads can
// hold run in batches of heads, 2 to 4 launches per side, each with the whole chip for its heads
// (the 1024-thread parts are kept for what still does not fit). True when every side launched.
static bool batched_kpp(const Dims& s, const KppArgs* sides, int nsides, int cus, uint64_t seed, int* status,
                        hipStream_t st) {
  int nb[2] = {0, 0}, G[2][1];
  for (int q = 0; q < nsides; ++q) {
    for (int B = 1; B <= 4 && !nb[q]; ++B) {
      const int hb = (int)ceil_div(s.H, B);
      if (cus / hb > 0 && plan_parts(s, sides + q, 1, cus / hb, kCoopThreads, G[q])) nb[q] = B;
    }
    if (!nb[q]) return false;
  }
  for (int q = 0; q < nsides; ++q) {
    const int hb = (int)ceil_div(s.H, nb[q]);
    for (int h0 = 0; h0 < (int)s.H; h0 += hb) {
      if (launch_kpp_coop(s, sides + q, 1, G[q], kCoopThreads, seed, status, st, h0,
                          (int)std::min<int64_t>(hb, s.H - h0)) != hipSuccess) {
        (void)hipGetLastError();
        return false;
      }
    }
  }
  return true;
}

hipError_t launch_kpp(const Dims& s, const KppArgs* sides, int nsides, uint64_t seed, int* status, hipStream_t st) {
  // candidate norms (and metric products) for every side
  for (int q = 0; q < nsides; ++q) {
    const KppArgs& a = sides[q];
    const int S = kpp_candidates(s.N, a.C);
    const dim3 g1((unsigned)ceil_div(S, 64), (unsigned)s.H);
    const size_t lds_t = (size_t)(68 * s.D + s.D * s.D) * sizeof(float);
#define PARK_PREP(T, D)                                                                                     \
  if (a.metric)                                                                                             \
    kpp_prep_tiled<T, D><<<g1, 256, lds_t, st>>>(static_cast<const T*>(a.x), s.N, S, a.metric, a.xx, a.y); \
  else                                                                                                      \
    kpp_prep<T, D><<<g1, 256, 0, st>>>(static_cast<const T*>(a.x), s.N, S, a.xx);
    if (s.bf16) {
      const dim3 g2((unsigned)ceil_div(S, 256), (unsigned)s.H);
      if (s.D == 128) {
        if (a.metric)
          kpp_prep_mfma<128><<<g2, 512, 0, st>>>(static_cast<const uint16_t*>(a.x), s.N, S, a.metric, a.xx, a.y);
        else
          kpp_prep<uint16_t, 128><<<g1, 256, 0, st>>>(static_cast<const uint16_t*>(a.x), s.N, S, a.xx);
      } else {
        if (a.metric)
          kpp_prep_mfma<64><<<g2, 512, 0, st>>>(static_cast<const uint16_t*>(a.x), s.N, S, a.metric, a.xx, a.y);
        else
          kpp_prep<uint16_t, 64><<<g1, 256, 0, st>>>(static_cast<const uint16_t*>(a.x), s.N, S, a.xx);
      }
    } else {
      if (s.D == 128) {
        PARK_PREP(float, 128)
      } else {
        PARK_PREP(float, 64)
      }
    }
#undef PARK_PREP
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (s.bf16) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                hipSuccess && cus > 0) {
      const int budget = cus / (int)s.H;
      int G[2];
      // in order: both sides in one launch with 512-thread parts; one launch per side with
      // 512-thread parts; per side, 512-thread parts over batches of heads; both sides with
      // 1024-thread parts; per side the narrowest parts that fit
      if (budget > 0 && plan_parts(s, sides, nsides, budget, kCoopThreads, G)) {
        if (launch_kpp_coop(s, sides, nsides, G, kCoopThreads, seed, status, st) == hipSuccess) return hipSuccess;
        (void)hipGetLastError();
      } else if (budget > 0 && nsides == 2 && plan_parts(s, sides, 1, budget, kCoopThreads, G) &&
                 plan_parts(s, sides + 1, 1, budget, kCoopThreads, G + 1)) {
        if (launch_kpp_coop(s, sides, 1, G, kCoopThreads, seed, status, st) == hipSuccess &&
            launch_kpp_coop(s, sides + 1, 1, G + 1, kCoopThreads, seed, status, st) == hipSuccess)
          return hipSuccess;
        (void)hipGetLastError();
      } else if (batched_kpp(s, sides, nsides, cus, seed, status, st)) {
        return hipSuccess;
      } else if (budget > 0 && plan_parts(s, sides, nsides, budget, kCoopThreadsWide, G)) {
        if (launch_kpp_coop(s, sides, nsides, G, kCoopThreadsWide, seed, status, st) == hipSuccess) return hipSuccess;
        (void)hipGetLastError();
      } else if (budget > 0) {
        int nt[2] = {0, 0};
        for (int q = 0; q < nsides; ++q)
          for (int w : {kCoopThreads, kCoopThreadsWide})
            if (!nt[q] && plan_parts(s, sides + q, 1, budget, w, G + q)) nt[q] = w;
        if (nt[0] && (nsides == 1 || nt[1])) {
          bool ok = true;
          for (int q = 0; q < nsides && ok; ++q)
            ok = launch_kpp_coop(s, sides + q, 1, G + q, nt[q], seed, status, st) == hipSuccess;
          if (ok) return hipSuccess;
          (void)hipGetLastError();
        }
      }
    }
  }
  return launch_kpp_single(s, sides, nsides, seed, st);
}

hipError_t launch_update(const Dims& s, const void* x, int C, const int32_t* perm, const int32_t* offsets, float* cent,
                         int do_update, const float* metric, void* g, float* b, hipStream_t st) {
  const dim3 grid((unsigned)C, (unsigned)s.H);
  const int euclid = metric == nullptr;
  if (do_update || euclid) {
#define PARK_MEAN(T, D)                                                                                    \
  centroid_mean<T, D><<<grid, 256, 0, st>>>(static_cast<const T*>(x), s.N, C, perm, offsets, cent, do_update, \
                                            euclid, g, b, s.bf16);
    if (s.bf16) {
      if (s.D == 128) {
        PARK_MEAN(uint16_t, 128)
      } else {
        PARK_MEAN(uint16_t, 64)
      }
    } else {
      if (s.D == 128) {
        PARK_MEAN(float, 128)
      } else {
        PARK_MEAN(float, 64)
      }
    }
#undef PARK_MEAN
  }
  if (!euclid) {
    const dim3 g2((unsigned)ceil_div(C, 32), (unsigned)s.H);
    const size_t lds = (size_t)s.D * s.D * sizeof(float) + (size_t)32 * s.D * sizeof(float);
    if (s.D == 128)
      consume_qrkc<128><<<g2, 256, lds, st>>>(cent, C, metric, g, b, s.bf16);
    else
      consume_qrkc<64><<<g2, 256, lds, st>>>(cent, C, metric, g, b, s.bf16);
  }
  return hipGetLastError();
}

hipError_t launch_assign(const Dims& s, const void* x, int C, const void* g, const float* b, int32_t* labels,
                         hipStream_t st, int stride, int phase) {
  const int64_t M = phase < s.N ? ceil_div(s.N - phase, stride) : 0;  // rows phase + p * stride < N
  if (M == 0) return hipGetLastError();
  if (s.bf16) {
    constexpr int PT = 2;
    const dim3 grid((unsigned)ceil_div(M, 4 * 32 * PT), (unsigned)s.H);
    if (s.D == 128)
      assign_bf16<128, PT><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x), s.N, C,
                                                 static_cast<const uint16_t*>(g), b, labels, M, stride, phase);
    else
      assign_bf16<64, PT><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x), s.N, C,
                                                static_cast<const uint16_t*>(g), b, labels, M, stride, phase);
  } else {
    const dim3 grid((unsigned)ceil_div(M, 256), (unsigned)s.H);
    if (s.D == 128)
      assign_f32<128><<<grid, 256, 0, st>>>(static_cast<const float*>(x), s.N, C, static_cast<const float*>(g), b,
                                            labels, M, stride, phase);
    else
      assign_f32<64><<<grid, 256, 0, st>>>(static_cast<const float*>(x), s.N, C, static_cast<const float*>(g), b,
                                           labels, M, stride, phase);
  }
  return hipGetLastError();
}

int fused_parts(const Dims& s, int C) {
  if (!s.bf16 || (s.D != 128 && s.D != 64) || C > kFuseT || C < 1) return 0;
  const int64_t nt = ceil_div(s.N, kFuseT);
  int64_t P = kFuseCUs / s.H;
  if (P < 1) P = 1;
  if (P > kFuseMaxParts) P = kFuseMaxParts;
  if (P > nt) P = nt;
  return (int)P;
}

hipError_t launch_lloyd_fused(const Dims& s, const void* x, int C, const void* g, const float* b, int32_t* labels,
                              double* psum, int32_t* pcnt, float* cent, hipStream_t st) {
  const int P = fused_parts(s, C);
  if (P == 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)P, (unsigned)s.H);
  if (s.D == 128)
    lloyd_fused<128><<<grid, kFuseThreads, 0, st>>>(static_cast<const uint16_t*>(x), s.N, C,
                                                    static_cast<const uint16_t*>(g), b, labels, psum, pcnt, P);
  else
    lloyd_fused<64><<<grid, kFuseThreads, 0, st>>>(static_cast<const uint16_t*>(x), s.N, C,
                                                   static_cast<const uint16_t*>(g), b, labels, psum, pcnt, P);
  lloyd_fused_means<<<dim3((unsigned)C, (unsigned)s.H), 128, 0, st>>>(psum, pcnt, C, (int)s.D, P, cent);
  return hipGetLastError();
}

hipError_t launch_clamp_labels(const Dims& s, int C, int32_t* labels, hipStream_t st) {
  const int64_t n = s.H * s.N;
  clamp_labels<<<(unsigned)ceil_div(n, 256), 256, 0, st>>>(labels, n, C);
  return hipGetLastError();
}

size_t sort_table_ints(const Dims& s, int C) { return (size_t)(s.H * ceil_div(s.N, kSortChunk) * C); }

hipError_t launch_sort(const Dims& s, int C, const int32_t* labels, int32_t* table, int32_t* perm,
                       int32_t* offsets, hipStream_t st) {
  const int nchunk = (int)ceil_div(s.N, kSortChunk);
  const dim3 grid((unsigned)nchunk, (unsigned)s.H);
  sort_hist<<<grid, 64, 0, st>>>(labels, s.N, C, nchunk, table);
  sort_scan_chunks<<<dim3((unsigned)ceil_div(C, 64), (unsigned)s.H), 64, 0, st>>>(table, nchunk, C, offsets);
  sort_scan_offsets<<<(unsigned)s.H, 1024, 0, st>>>(offsets, C);
  sort_scatter<<<grid, 64, 0, st>>>(labels, s.N, C, nchunk, table, offsets, perm);
  return hipGetLastError();
}

}  // namespace park
