// Layout helpers: per-(batch, KV head) transposed copies of K or V so that a
// 64-key block of K^T / V^T is D contiguous 128-byte rows (keys fastest).
// The attention kernels contract over keys on the matrix cores (O^T += V^T P^T,
// dQ^T += K^T dS^T), which needs 8 keys contiguous per lane; with the
// transposed copy every tile is a plain 16-byte-granular copy.
//
// Key order inside each 32-key group: the P^T / dS^T operand comes straight
// out of the score tile's accumulator layout, where lane group g (0..3) holds
// keys 4g..4g+3 and 16+4g..16+4g+3.  The copy stores exactly those 8 keys at
// positions 8g..8g+7, so one 16-byte read gives a lane its whole operand.
#include "sas_kernels.h"

namespace sas {

namespace {

// src [B,T,H,D] -> dst [B,H,D,Tp] (Tp = 64 * ceil(T/64), tail zero-filled),
// keys permuted inside each 32-key group as described above.
// One workgroup = one 64-token block of one (b, h): reads 64 rows of D
// coalesced, writes D rows of 64 keys coalesced, through LDS.
template <int D>
__global__ __launch_bounds__(256) void transpose_tokens_kernel(const uint16_t* __restrict__ src,
                                                               uint16_t* __restrict__ dst, int T,
                                                               int H, int Tp) {
  constexpr int P = 64 + 2;          // LDS pitch (keys) of the transposed tile
  __shared__ uint16_t tile[D * P];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  for (int u = tid; u < 64 * (D / 8); u += 256) {
    const int r = u / (D / 8), ch = u - r * (D / 8);
    const int tok = j * 64 + r;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (tok < T)
      v = *reinterpret_cast<const uint4*>(src + ((static_cast<size_t>(b) * T + tok) * H + h) * D + ch * 8);
    const uint16_t* e = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[(ch * 8 + i) * P + r] = e[i];
  }
  __syncthreads();
  uint16_t* out = dst + (static_cast<size_t>(b) * H + h) * D * static_cast<size_t>(Tp) + j * 64;
  for (int u = tid; u < D * 32; u += 256) {
    const int d = u / 32, kp = u - d * 32;
    // output positions 2kp, 2kp+1 = group kg, lane group g, slot i (even)
    const int kg = kp >> 4, g = (kp >> 2) & 3, i = (kp & 3) * 2;
    const int key = kg * 32 + (i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4));
    const uint32_t w = static_cast<uint32_t>(tile[d * P + key]) |
                       (static_cast<uint32_t>(tile[d * P + key + 1]) << 16);
    *reinterpret_cast<uint32_t*>(out + static_cast<size_t>(d) * Tp + 2 * kp) = w;
  }
}

}  // namespace

hipError_t launch_transpose_tokens(const uint16_t* src, uint16_t* dst, int B, int T, int H, int D,
                                   hipStream_t st) {
  const int NB = (T + 63) / 64;
  const dim3 grid(NB, H, B);
  if (D == 128)
    hipLaunchKernelGGL((transpose_tokens_kernel<128>), grid, dim3(256), 0, st, src, dst, T, H, NB * 64);
  else if (D == 64)
    hipLaunchKernelGGL((transpose_tokens_kernel<64>), grid, dim3(256), 0, st, src, dst, T, H, NB * 64);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sas
