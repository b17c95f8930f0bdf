// Decode-time gate key of a sequence's current block (model card,
// checkpoint configuration: block pooling max + min + average, K norm and
// gate RoPE; the current block c is represented by the causal prefix pool of
// its tokens 64c .. t).  A serving loop calls it after writing the new token
// at position L - 1 of the KV cache, so the gate-key cache entry of block c
// is refreshed before the decode step scores it.
//
// One workgroup of 128 threads per (sequence b, KV head kappa):
//   p = [max; min; mean] over rows 64c .. L-1 of the cache (thread per
//       channel, rows in order: the same values as the prefill pooling);
//   z = p Wk[kappa] (fp32 products of the bf16 weights, in order of f);
//   y = z / sqrt(mean(z^2) + eps) * w_kn;  kg = RoPE_{64c}(y), angles in fp64;
// written to the gate-key cache entry of block c (contiguous [B,Hkv,NBmax,dg]
// or the block's page [P,Hkv,dg]), fp32 or bf16 (round to nearest even).
#include "sas_kernels.h"

namespace sas {

namespace {

template <int D>
__global__ __launch_bounds__(128) void decode_gate_key_kernel(DecodeKeyParams p) {
  __shared__ float pv[3 * D];
  __shared__ float ys[128];
  __shared__ float red[2];
  const int unit = blockIdx.x, b = unit / p.Hkv, kv = unit - b * p.Hkv;
  const int tid = threadIdx.x, dg = p.dg;
  const int L = p.ctx_len[b];
  if (!(L >= 1 && L <= p.Lmax)) return;              // uniform: nothing to refresh
  const int t = L - 1, c = t / 64, n = t - 64 * c + 1;
  // rows 64c .. t of the current block: contiguous cache rows, or its page
  const uint16_t* rows;
  if (p.btab) {
    const int pg = p.btab[static_cast<size_t>(b) * p.NBmax + c];
    if (pg < 0 || pg >= p.num_pages) return;         // no page: nothing to refresh
    rows = p.k + (static_cast<size_t>(pg) * p.Hkv + kv) * 64 * D;
  } else {
    rows = p.k + ((static_cast<size_t>(b) * p.Hkv + kv) * p.Lmax + 64 * c) * D;
  }
  for (int d = tid; d < D; d += 128) {
    float mx = -INFINITY, mn = INFINITY, sm = 0.f;
    for (int r = 0; r < n; ++r) {
      const float x = bf2f(rows[static_cast<size_t>(r) * D + d]);
      mx = fmaxf(mx, x);
      mn = fminf(mn, x);
      sm += x;
    }
    pv[d] = mx;
    pv[D + d] = mn;
    pv[2 * D + d] = sm / static_cast<float>(n);
  }
  __syncthreads();
  const int e = tid;
  float z = 0.f;
  if (e < dg) {
    const uint16_t* w = p.wk + static_cast<size_t>(kv) * 3 * D * dg + e;
    for (int f = 0; f < 3 * D; ++f) z = fmaf(pv[f], bf2f(w[static_cast<size_t>(f) * dg]), z);
  }
  float sq = wave_sum(e < dg ? z * z : 0.f);
  if ((tid & 63) == 0) red[tid >> 6] = sq;
  __syncthreads();
  const float r = 1.f / sqrtf((red[0] + red[1]) / static_cast<float>(dg) + p.eps);
  if (e < dg) ys[e] = z * r * p.w_kn[e];
  __syncthreads();
  if (e >= dg) return;
  const int half = dg / 2, i = e < half ? e : e - half;
  const double ang = static_cast<double>(64 * c) * pow(p.theta, -2.0 * i / dg);
  double sd, cd;
  sincos(ang, &sd, &cd);
  const float cs = static_cast<float>(cd), sn = static_cast<float>(sd);
  const float out = e < half ? ys[e] * cs - ys[e + half] * sn : ys[e] * cs + ys[e - half] * sn;
  size_t row;
  if (p.btab) {
    const int pg = p.btab[static_cast<size_t>(b) * p.NBmax + c];
    row = static_cast<size_t>(pg) * p.Hkv + kv;
  } else {
    row = static_cast<size_t>(unit) * p.NBmax + c;
  }
  if (p.kg_bf16)
    reinterpret_cast<uint16_t*>(p.kg)[row * dg + e] = f2bf(out);
  else
    reinterpret_cast<float*>(p.kg)[row * dg + e] = out;
}

}  // namespace

hipError_t launch_decode_gate_key(const DecodeKeyParams& p, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.B) * p.Hkv);
  if (p.D == 128)
    hipLaunchKernelGGL((decode_gate_key_kernel<128>), grid, dim3(128), 0, st, p);
  else if (p.D == 64)
    hipLaunchKernelGGL((decode_gate_key_kernel<64>), grid, dim3(128), 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sas
