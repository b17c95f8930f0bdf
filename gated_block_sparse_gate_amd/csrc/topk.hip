// Candidate softmax and Top-K block selection (abstract: normalised softmax
// gates calibrate history against the always-retained current block; README
// item (a): discrete Top-K selection).
//
// For token t of block c and KV head kappa:
//   s_j = q_gate[t] . k_gate[64j+63] / sqrt(dg)   (complete historical blocks j < c)
//   s_c = q_gate[t] . k_gate[t] / sqrt(dg)        (current block, causal prefix key)
//   gate_lse = logsumexp_{j<=c} s_j,  log g_j = s_j - gate_lse
//   selection = min(K, c) largest s_j over j < c, equal scores -> lower j,
//   written in ascending order, then c; padding -1 / -inf.
//
// One workgroup = 16 consecutive tokens of one (batch, KV head); all 16 share
// the same block c, so the historical block keys form one fp32 tile product
// (LDS tiled, plain fp32 FMA: index parity needs fp32-accurate scores).
// Selection: exact K-th largest order key by a 32-step bitwise search with
// wave-wide counts, then equal keys taken in ascending block order.
#include "sas_kernels.h"

namespace sas {

namespace {

constexpr int kTokPerWG = 16;

template <int DG>
__global__ __launch_bounds__(256) void topk_kernel(TopkParams p) {
  constexpr int KCH = 64;            // block keys per LDS chunk
  constexpr int KPITCH = DG + 4;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* qs = smem;                            // [16][DG]
  float* ks = qs + kTokPerWG * DG;             // [64][KPITCH]
  float* sc = ks + KCH * KPITCH;               // [16][NBP]
  const int NBP = ((p.NB + 3) / 4) * 4;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int kv = blockIdx.y, b = blockIdx.z;
  const int t0 = blockIdx.x * kTokPerWG;
  const int c = t0 / 64;
  const int ntok = min(kTokPerWG, p.T - t0);
  const float inv_sqrt_dg = 1.0f / sqrtf(static_cast<float>(DG));

  for (int e = tid; e < kTokPerWG * DG; e += 256) {
    const int tl = e / DG, d = e - tl * DG;
    qs[e] = (tl < ntok)
                ? p.q_gate[((static_cast<size_t>(b) * p.T + t0 + tl) * p.Hkv + kv) * DG + d]
                : 0.f;
  }

  // historical scores: thread -> (token tl = tid/16, keys 4*kq .. 4*kq+3)
  const int tl_s = tid >> 4, kq = tid & 15;
  for (int j0 = 0; j0 < c; j0 += KCH) {
    __syncthreads();
    for (int e = tid; e < KCH * (DG / 4); e += 256) {
      const int jj = e / (DG / 4), d4 = e - jj * (DG / 4);
      const int j = j0 + jj;
      float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < c)
        val = *reinterpret_cast<const float4*>(
            p.k_gate + ((static_cast<size_t>(b) * p.T + j * 64 + 63) * p.Hkv + kv) * DG + d4 * 4);
      *reinterpret_cast<float4*>(&ks[jj * KPITCH + d4 * 4]) = val;
    }
    __syncthreads();
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const float* qrow = &qs[tl_s * DG];
#pragma unroll 4
    for (int d = 0; d < DG; d += 4) {
      const float4 qv = *reinterpret_cast<const float4*>(qrow + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 kvv = *reinterpret_cast<const float4*>(&ks[(kq * 4 + e) * KPITCH + d]);
        acc[e] = fmaf(qv.x, kvv.x, acc[e]);
        acc[e] = fmaf(qv.y, kvv.y, acc[e]);
        acc[e] = fmaf(qv.z, kvv.z, acc[e]);
        acc[e] = fmaf(qv.w, kvv.w, acc[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = j0 + kq * 4 + e;
      if (j < c) sc[tl_s * NBP + j] = acc[e] * inv_sqrt_dg;
    }
  }
  __syncthreads();
  // current-block score with the token's own prefix key
  {
    const int part = tid & 15;
    float acc = 0.f;
    if (tl_s < ntok) {
      const float* kg = p.k_gate + ((static_cast<size_t>(b) * p.T + t0 + tl_s) * p.Hkv + kv) * DG;
      for (int d = part; d < DG; d += 16) acc = fmaf(qs[tl_s * DG + d], kg[d], acc);
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    acc += __shfl_xor(acc, 4, 64);
    acc += __shfl_xor(acc, 8, 64);
    if (part == 0) sc[tl_s * NBP + c] = acc * inv_sqrt_dg;
  }
  __syncthreads();

  // per token row: logsumexp, selection, ascending compaction
  const int K = p.K, S = p.S;
  const int ncand = c + 1;
  const int E = (ncand + 63) / 64;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int tl = wv; tl < ntok; tl += 4) {
    const float* row = &sc[tl * NBP];
    float mx = -INFINITY;
    for (int e = 0; e < E; ++e) {
      const int j = lane + 64 * e;
      if (j < ncand) mx = fmaxf(mx, row[j]);
    }
    mx = wave_max(mx);
    float se = 0.f;
    for (int e = 0; e < E; ++e) {
      const int j = lane + 64 * e;
      if (j < ncand) se += expf(row[j] - mx);
    }
    se = wave_sum(se);
    const float lse = mx + logf(se);
    const size_t rowid = (static_cast<size_t>(b) * p.T + t0 + tl) * p.Hkv + kv;

    const int nsel = min(K, c);
    // order keys of the historical candidates, held in registers
    constexpr int EMAX = kMaxNB / 64;
    uint32_t kreg[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      const int j = lane + 64 * e;
      kreg[e] = (e < E && j < c) ? order_key(row[j]) : 0u;
    }
    uint32_t thr = 0;
    int need_eq = 0;
    const bool all = (c <= K);
    if (!all) {
      // largest thr with count(key >= thr) >= K  ->  thr = K-th largest key;
      // counts by ballot + scalar popcount (no cross-lane data movement)
      // kreg is 0 outside the historical candidates, and every candidate
      // threshold is >= 1, so no validity test is needed in the counts
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
          if (e < E) cnt += wave_count(kreg[e] >= cand);
        if (cnt >= K) thr = cand;
      }
      int gt = 0;
#pragma unroll
      for (int e = 0; e < EMAX; ++e)
        if (e < E) gt += wave_count(kreg[e] > thr);
      need_eq = K - gt;
    }
    int base = 0, eq_seen = 0;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (e >= E) break;
      const int j = lane + 64 * e;
      const bool hist = j < c;
      const bool gt = hist && !all && kreg[e] > thr;
      const bool eq = hist && !all && kreg[e] == thr;
      const uint64_t em = ballot64(eq);
      const bool s_in =
          hist && (all || gt || (eq && (eq_seen + __popcll(em & lt_mask)) < need_eq));
      eq_seen += __popcll(em);
      const uint64_t sm = ballot64(s_in);
      if (s_in) {
        const int pos = base + __popcll(sm & lt_mask);
        p.idx[rowid * S + pos] = j;
        p.logg[rowid * S + pos] = row[j] - lse;
      }
      base += __popcll(sm);
    }
    if (lane == 0) {
      p.idx[rowid * S + nsel] = c;
      p.logg[rowid * S + nsel] = row[c] - lse;
      p.gate_lse[rowid] = lse;
    }
    for (int s2 = nsel + 1 + lane; s2 < S; s2 += 64) {
      p.idx[rowid * S + s2] = -1;
      p.logg[rowid * S + s2] = -INFINITY;
    }
    if (p.gate_probs) {
      for (int j = lane; j < p.NB; j += 64)
        p.gate_probs[rowid * p.NB + j] = (j <= c) ? expf(row[j] - lse) : 0.f;
    }
  }
}

}  // namespace

size_t topk_smem_bytes(int NB, int dg) {
  const int NBP = ((NB + 3) / 4) * 4;
  return sizeof(float) * (static_cast<size_t>(kTokPerWG) * dg + 64 * (dg + 4) +
                          static_cast<size_t>(kTokPerWG) * NBP);
}

hipError_t launch_topk(const TopkParams& p, hipStream_t st) {
  const dim3 grid((p.T + kTokPerWG - 1) / kTokPerWG, p.Hkv, p.B);
  const size_t sm = topk_smem_bytes(p.NB, p.dg);
  switch (p.dg) {
    case 128:
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_kernel<128>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sm));
      hipLaunchKernelGGL((topk_kernel<128>), grid, dim3(256), sm, st, p);
      break;
    case 64:
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_kernel<64>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sm));
      hipLaunchKernelGGL((topk_kernel<64>), grid, dim3(256), sm, st, p);
      break;
    case 32:
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_kernel<32>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sm));
      hipLaunchKernelGGL((topk_kernel<32>), grid, dim3(256), sm, st, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sas
