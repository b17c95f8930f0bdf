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

// max |src| over one 64-token block of one (b, h): amax[b, h, j].
template <int D>
__global__ __launch_bounds__(256) void block_amax_kernel(const uint16_t* __restrict__ src,
                                                         float* __restrict__ amax, int T, int H) {
  __shared__ float red[4];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  float m = 0.f;
  for (int u = tid; u < 64 * (D / 8); u += 256) {
    const int r = u / (D / 8), ch = u - r * (D / 8);
    const int tok = j * 64 + r;
    if (tok < T) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + ((static_cast<size_t>(b) * T + tok) * H + h) * D + ch * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        m = fmaxf(m, fmaxf(fabsf(__uint_as_float(w[i] << 16)), fabsf(__uint_as_float(w[i] & 0xffff0000u))));
    }
  }
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0)
    amax[(static_cast<size_t>(b) * H + h) * gridDim.x + j] =
        fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// As transpose_tokens_kernel, writing fp16 values of src * 2^-e with the
// head's exponent e (from the per-block maxima), so every value is finite in
// fp16 and the scaling is exact.
template <int D>
__global__ __launch_bounds__(256) void transpose_tokens_f16_kernel(
    const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, const float* __restrict__ amax,
    float* __restrict__ scale_out, int T, int H, int Tp) {
  constexpr int P = 64 + 2;
  __shared__ uint16_t tile[D * P];
  __shared__ float red[4];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int NB = gridDim.x;
  const int tid = threadIdx.x;
  // head maximum -> exponent e >= 0 with max * 2^-e <= 32768
  float m = 0.f;
  for (int i = tid; i < NB; i += 256) m = fmaxf(m, amax[(static_cast<size_t>(b) * H + h) * NB + i]);
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int e = 0;
  if (m > 32768.f) {
    int ex;
    frexpf(m / 32768.f, &ex);          // m / 32768 in [2^(ex-1), 2^ex)
    e = ex;
  }
  const float down = ldexpf(1.f, -e);
  if (j == 0 && tid == 0) scale_out[static_cast<size_t>(b) * H + h] = ldexpf(1.f, e);
  for (int u = tid; u < 64 * (D / 8); u += 256) {
    const int r = u / (D / 8), ch = u - r * (D / 8);
    const int tok = j * 64 + r;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (tok < T)
      v = *reinterpret_cast<const uint4*>(src + ((static_cast<size_t>(b) * T + tok) * H + h) * D + ch * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t hp = pack_h2(__uint_as_float(w[i] << 16) * down,
                                  __uint_as_float(w[i] & 0xffff0000u) * down);
      tile[(ch * 8 + 2 * i) * P + r] = static_cast<uint16_t>(hp & 0xffffu);
      tile[(ch * 8 + 2 * i + 1) * P + r] = static_cast<uint16_t>(hp >> 16);
    }
  }
  __syncthreads();
  uint16_t* out = dst + (static_cast<size_t>(b) * H + h) * D * static_cast<size_t>(Tp) + j * 64;
  for (int u = tid; u < D * 32; u += 256) {
    const int d = u / 32, kp = u - d * 32;
    const int kg = kp >> 4, g = (kp >> 2) & 3, i = (kp & 3) * 2;
    const int key = kg * 32 + (i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4));
    const uint32_t w = static_cast<uint32_t>(tile[d * P + key]) |
                       (static_cast<uint32_t>(tile[d * P + key + 1]) << 16);
    *reinterpret_cast<uint32_t*>(out + static_cast<size_t>(d) * Tp + 2 * kp) = w;
  }
}

}  // namespace

hipError_t launch_transpose_tokens_f16(const uint16_t* src, uint16_t* dst, float* amax,
                                       float* scale_out, int B, int T, int H, int D,
                                       hipStream_t st) {
  const int NB = (T + 63) / 64;
  const dim3 grid(NB, H, B);
  if (D == 128) {
    hipLaunchKernelGGL((block_amax_kernel<128>), grid, dim3(256), 0, st, src, amax, T, H);
    hipLaunchKernelGGL((transpose_tokens_f16_kernel<128>), grid, dim3(256), 0, st, src, dst, amax,
                       scale_out, T, H, NB * 64);
  } else if (D == 64) {
    hipLaunchKernelGGL((block_amax_kernel<64>), grid, dim3(256), 0, st, src, amax, T, H);
    hipLaunchKernelGGL((transpose_tokens_f16_kernel<64>), grid, dim3(256), 0, st, src, dst, amax,
                       scale_out, T, H, NB * 64);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

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
