// Cluster-contiguous row gather and its inverse scatter (the "Clustered" token ordering of the PARK
// page, Tables 1 and 10). One thread moves one 16-byte piece of a row; consecutive threads move
// consecutive pieces, so each row is read and written as whole cache lines.
#include "park_common.h"
#include "park_internal.h"

namespace park {

namespace {

template <int BYTES_PER_ROW>
__global__ __launch_bounds__(256) void permute_rows(const uint8_t* __restrict__ x, const int32_t* __restrict__ perm,
                                                    int64_t N, uint8_t* __restrict__ out, int inverse) {
  constexpr int PIECES = BYTES_PER_ROW / 16;
  const int h = blockIdx.y;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= N * PIECES) return;
  const int64_t p = e / PIECES;
  const int pc = (int)(e % PIECES);
  const int64_t q = perm[(int64_t)h * N + p];
  const int64_t src = inverse ? p : q;
  const int64_t dst = inverse ? q : p;
  const uint8_t* xs = x + ((int64_t)h * N + src) * BYTES_PER_ROW + pc * 16;
  uint8_t* od = out + ((int64_t)h * N + dst) * BYTES_PER_ROW + pc * 16;
  *reinterpret_cast<u32x4_t*>(od) = *reinterpret_cast<const u32x4_t*>(xs);
}

}  // namespace

hipError_t launch_permute(const Dims& s, const void* x, const int32_t* perm, void* out, int inverse, hipStream_t st) {
  const int bpr = (int)(s.D * (s.bf16 ? 2 : 4));
  const int64_t pieces = s.N * (bpr / 16);
  const dim3 grid((unsigned)ceil_div(pieces, 256), (unsigned)s.H);
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  uint8_t* ob = static_cast<uint8_t*>(out);
  switch (bpr) {
    case 128:
      permute_rows<128><<<grid, 256, 0, st>>>(xb, perm, s.N, ob, inverse);
      break;
    case 256:
      permute_rows<256><<<grid, 256, 0, st>>>(xb, perm, s.N, ob, inverse);
      break;
    default:
      permute_rows<512><<<grid, 256, 0, st>>>(xb, perm, s.N, ob, inverse);
      break;
  }
  return hipGetLastError();
}

}  // namespace park
