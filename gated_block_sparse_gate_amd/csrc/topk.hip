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
// (fp32 MFMA: index parity needs fp32-accurate scores).
// Selection: exact K-th largest order key by bitwise searches with wave-wide
// counts (over the keys above the K-th largest lane maximum when they fit one
// per lane), then equal keys taken in ascending block order.
#include <type_traits>

#include "sas_kernels.h"

namespace sas {

namespace {

constexpr int kTokPerWG = 16;

template <int DG>
__global__ __launch_bounds__(256) void topk_kernel(TopkParams p) {
  constexpr int KCH = 64;            // block keys per chunk (16 per wave)
  constexpr int KP = DG + 4;         // LDS pitch (floats) of a staged key
  constexpr int NS = DG / 16;        // 16-wide d groups
  constexpr int KU = KCH * DG / 4 / 256;   // float4 per thread per chunk
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ uint32_t gath[4][64];             // per wave: keys above the lane-maximum bound
  float* ks = smem;                            // [64][KP]
  float* sc = ks + KCH * KP;                   // [16][NBP]
  const int NBP = ((p.NB + 3) / 4) * 4;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int kv = blockIdx.y, b = blockIdx.z;
  const int t0 = blockIdx.x * kTokPerWG;
  const int c = t0 / 64;
  const int ntok = min(kTokPerWG, p.T - t0);
  const float inv_sqrt_dg = 1.0f / sqrtf(static_cast<float>(DG));

  // historical scores S^T[key, token] = K Q^T on fp32 MFMA 16x16x4; the k
  // index of MFMA step (s, i) is d = 16 s + 4 (lane / 16) + i, the same for
  // both operands.  Query operand (token = lane % 16) in registers.
  float qb[NS][4];
  {
    const float* qrow =
        p.q_gate + ((static_cast<size_t>(b) * p.T + t0 + min(l16, ntok - 1)) * p.Hkv + kv) * DG;
#pragma unroll
    for (int sg = 0; sg < NS; ++sg) {
      const float4 v = *reinterpret_cast<const float4*>(qrow + 16 * sg + 4 * g4);
      qb[sg][0] = v.x; qb[sg][1] = v.y; qb[sg][2] = v.z; qb[sg][3] = v.w;
    }
  }
  // block keys k_gate[64 j + 63], staged per 64-key chunk through registers
  // (the next chunk's loads are in flight while the current one is used)
  float4 kst[KU];
  auto kload = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < KU; ++x) {
      const int u = tid + 256 * x;
      const int r = u / (DG / 4), f = u - r * (DG / 4);
      const int j = j0 + r;
      kst[x] = (j < c) ? *reinterpret_cast<const float4*>(
                             p.k_gate + ((static_cast<size_t>(b) * p.T + 64 * j + 63) * p.Hkv + kv) * DG + 4 * f)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  if (c > 0) kload(0);
  for (int j0 = 0; j0 < c; j0 += KCH) {
    __syncthreads();
#pragma unroll
    for (int x = 0; x < KU; ++x) {
      const int u = tid + 256 * x;
      const int r = u / (DG / 4), f = u - r * (DG / 4);
      *reinterpret_cast<float4*>(&ks[r * KP + 4 * f]) = kst[x];
    }
    __syncthreads();
    if (j0 + KCH < c) kload(j0 + KCH);
    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
    const float* krow = &ks[(16 * wv + l16) * KP + 4 * g4];
#pragma unroll
    for (int sg = 0; sg < NS; ++sg) {
      const float4 a = *reinterpret_cast<const float4*>(krow + 16 * sg);
      acc = mfma16x16x4f32(a.x, qb[sg][0], acc);
      acc = mfma16x16x4f32(a.y, qb[sg][1], acc);
      acc = mfma16x16x4f32(a.z, qb[sg][2], acc);
      acc = mfma16x16x4f32(a.w, qb[sg][3], acc);
    }
    const int jb = j0 + 16 * wv + 4 * g4;     // keys jb .. jb+3 of token l16
    if (l16 < ntok) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (jb + i < c) sc[l16 * NBP + jb + i] = acc[i] * inv_sqrt_dg;
    }
  }
  __syncthreads();
  // current-block score with the token's own prefix key
  {
    const int tl_s = tid >> 4, part = tid & 15;
    float acc = 0.f;
    if (tl_s < ntok) {
      const size_t rw = (static_cast<size_t>(b) * p.T + t0 + tl_s) * p.Hkv + kv;
      const float* kg = p.k_gate + rw * DG;
      const float* qg = p.q_gate + rw * DG;
      for (int d = part; d < DG; d += 16) acc = fmaf(qg[d], kg[d], acc);
    }
    acc += dpp_mov<0xB1>(acc);
    acc += dpp_mov<0x4E>(acc);
    acc += dpp_mov<0x141>(acc);
    acc += dpp_mov<0x140>(acc);
    if (part == 0 && tl_s < ntok) sc[tl_s * NBP + c] = acc * inv_sqrt_dg;
  }
  __syncthreads();

  // per token row (one wave per row): log-sum-exp, selection, ascending
  // compaction.  All rows of the workgroup share c, so the register count of
  // the order keys is chosen once per workgroup (no per-step branches).
  const int K = p.K, S = p.S;
  const int ncand = c + 1;
  const int E = (ncand + 63) / 64;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int nsel = min(K, c);
  const bool all = (c <= K);
  auto rows = [&](auto emc) __attribute__((always_inline)) {
    constexpr int EM = decltype(emc)::value;
    for (int tl = wv; tl < ntok; tl += 4) {
      const float* row = &sc[tl * NBP];
      float sv[EM];
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        const int j = lane + 64 * e;
        sv[e] = (j < ncand) ? row[j] : -INFINITY;
      }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < EM; ++e) mx = fmaxf(mx, sv[e]);
      mx = wave_max(mx);
      float se = 0.f;
#pragma unroll
      for (int e = 0; e < EM; ++e) se += expf(sv[e] - mx);
      se = wave_sum(se);
      const float lse = mx + logf(se);
      const size_t rowid = (static_cast<size_t>(b) * p.T + t0 + tl) * p.Hkv + kv;
      // order keys of the historical candidates; 0 elsewhere, which no
      // candidate threshold (always >= 1) reaches
      uint32_t kreg[EM];
#pragma unroll
      for (int e = 0; e < EM; ++e) kreg[e] = (lane + 64 * e < c) ? order_key(sv[e]) : 0u;
      uint32_t thr = 0;
      int need_eq = 0;
      if (!all) {
        // thr = the largest t with #(keys >= t) >= K, by a bitwise search.
        // The K-th largest lane maximum t0 bounds it from below (the K
        // largest lane maxima are K keys at or above t0; at least K lanes hold
        // a candidate since c > K and K < 64), so when the keys >= t0 fit one
        // per lane the search runs over them alone (same counts for every
        // t >= t0).
        uint32_t lmax = 0;
#pragma unroll
        for (int e = 0; e < EM; ++e) lmax = max(lmax, kreg[e]);
        uint32_t t0k = 0;
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t cand = t0k | (1u << bit);
          if (wave_count(lmax >= cand) >= K) t0k = cand;
        }
        int n0 = 0;
#pragma unroll
        for (int e = 0; e < EM; ++e) n0 += wave_count(kreg[e] >= t0k);
        if (n0 <= 64) {
          int nb = 0;
#pragma unroll
          for (int e = 0; e < EM; ++e) {
            const bool in = kreg[e] >= t0k;
            const uint64_t m = ballot64(in);
            if (in) gath[wv][nb + __popcll(m & lt_mask)] = kreg[e];
            nb += __popcll(m);
          }
          // the wave's LDS accesses complete in order
          const uint32_t v = lane < n0 ? gath[wv][lane] : 0u;
          for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = thr | (1u << bit);
            if (wave_count(v >= cand) >= K) thr = cand;
          }
        } else {
          for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = thr | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int e = 0; e < EM; ++e) cnt += wave_count(kreg[e] >= cand);
            if (cnt >= K) thr = cand;
          }
        }
        int gt = 0;
#pragma unroll
        for (int e = 0; e < EM; ++e) gt += wave_count(kreg[e] > thr);
        need_eq = K - gt;
      }
      int base = 0, eq_seen = 0;
#pragma unroll
      for (int e = 0; e < EM; ++e) {
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
          p.logg[rowid * S + pos] = sv[e] - lse;
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
  };
  if (E <= 1) rows(std::integral_constant<int, 1>{});
  else if (E <= 2) rows(std::integral_constant<int, 2>{});
  else if (E <= 4) rows(std::integral_constant<int, 4>{});
  else if (E <= 8) rows(std::integral_constant<int, 8>{});
  else rows(std::integral_constant<int, kMaxNB / 64>{});
}

}  // namespace

size_t topk_smem_bytes(int NB, int dg) {
  const int NBP = ((NB + 3) / 4) * 4;
  return sizeof(float) * (64 * (dg + 4) + static_cast<size_t>(kTokPerWG) * NBP);
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
