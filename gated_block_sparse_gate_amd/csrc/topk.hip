// Candidate softmax and Top-K block selection (abstract: normalised softmax
// gates calibrate history against the always-retained current block; README
// item (a): discrete Top-K selection).
//
// For token t of block c and selection head sg (KV head kappa = sg / kdiv):
//   s_j = q_gate[t,sg] . k_gate[64j+63,kappa] / sqrt(dg)   (historical blocks j < c)
//   s_c = q_gate[t,sg] . k_gate[t,kappa] / sqrt(dg)        (current block, prefix key)
//   gate_lse = logsumexp_{j<=c} s_j,  log g_j = s_j - gate_lse
//   selection = min(K, c) largest s_j over j < c, equal scores -> lower j,
//   written in ascending order, then c; padding -1 / -inf.
//
// One workgroup = 16 consecutive tokens of one (batch, selection head: a KV
// head, or a query head when every query head has its own gate, scoring the
// gate keys of its KV head); all 16 share the same block c, so the
// historical block keys form one fp32 tile product (fp32 MFMA: index parity
// needs fp32-accurate scores), its block-key operand read from memory (L2:
// the keys of one head are shared by all its workgroups) straight into
// registers.  The scores go through LDS to one wave per token row.
// Selection: exact K-th largest order key by bitwise searches with wave-wide
// counts (over the keys above the K-th largest lane maximum when they fit one
// per lane), then equal keys taken in ascending block order.
#include <type_traits>

#include "sas_kernels.h"

namespace sas {

namespace {

constexpr int kTokPerWG = 16;
// floats per score row: room for every candidate, odd so that the 16 rows
// start on different LDS banks
__host__ __device__ inline int topk_score_pitch(int NB) { return NB | 1; }

template <int DG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void topk_kernel(TopkParams p) {
  constexpr int NS = DG / 16;        // 16-wide d groups
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ uint32_t gath[4][64];             // per wave: keys above the lane-maximum bound
  __shared__ int selj[4][64];                  // per wave: selected blocks in output order
  __shared__ float sell[4][64];                // and their log-gates
  float* sc = smem;                            // [16][NBP] scores (odd pitch: no bank conflicts)
  const int NBP = topk_score_pitch(p.NB);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int sg = blockIdx.y, b = blockIdx.z;   // selection head
  const int kv = sg / p.kdiv;                    // its KV head (gate keys)
  const int t0 = (gridDim.x - 1 - blockIdx.x) * kTokPerWG;   // late (long) rows first
  const int c = t0 / 64;
  const int ntok = min(kTokPerWG, p.T - t0);
  const float inv_sqrt_dg = 1.0f / sqrtf(static_cast<float>(DG));

  // current-block score operands (the token's query and its own prefix key,
  // DG / 16 consecutive dims per thread) are requested first, so that their
  // memory latency overlaps the historical scores
  constexpr int CPT = DG / 16;
  const int tl_s = tid >> 4, part = tid & 15;
  float cq[CPT], ck[CPT];
  {
    const size_t tok = static_cast<size_t>(b) * p.T + t0 + min(tl_s, ntok - 1);
    const float* kg = p.k_gate + (tok * p.Hkv + kv) * DG + part * CPT;
    const float* qg = p.q_gate + (tok * p.Hs + sg) * DG + part * CPT;
    if constexpr (CPT % 4 == 0) {
#pragma unroll
      for (int i = 0; i < CPT; i += 4) {
        const float4 a4 = *reinterpret_cast<const float4*>(qg + i);
        const float4 b4 = *reinterpret_cast<const float4*>(kg + i);
        cq[i] = a4.x; cq[i + 1] = a4.y; cq[i + 2] = a4.z; cq[i + 3] = a4.w;
        ck[i] = b4.x; ck[i + 1] = b4.y; ck[i + 2] = b4.z; ck[i + 3] = b4.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        cq[i] = qg[i];
        ck[i] = kg[i];
      }
    }
  }
  // historical scores S^T[key, token] = K Q^T on fp32 MFMA 16x16x4; the k
  // index of MFMA step (s, i) is d = 16 s + 4 (lane / 16) + i, the same for
  // both operands.  Query operand (token = lane % 16) in registers; wave w
  // takes keys 16 w .. 16 w + 15 of each 64-key chunk, its block-key operand
  // (key = lane % 16) loaded from memory straight into registers, the next
  // chunk's while the current one is used.
  float qb[NS][4];
  {
    const float* qrow =
        p.q_gate + ((static_cast<size_t>(b) * p.T + t0 + min(l16, ntok - 1)) * p.Hs + sg) * DG;
#pragma unroll
    for (int dq = 0; dq < NS; ++dq) {
      const float4 v = *reinterpret_cast<const float4*>(qrow + 16 * dq + 4 * g4);
      qb[dq][0] = v.x; qb[dq][1] = v.y; qb[dq][2] = v.z; qb[dq][3] = v.w;
    }
  }
  float4 ka[NS], kn[NS];
  auto kload = [&](int j0, float4* dst) __attribute__((always_inline)) {
    const int j = j0 + 16 * wv + l16;
    const float* krow =
        p.k_gate + ((static_cast<size_t>(b) * p.T + 64 * min(j, c - 1) + 63) * p.Hkv + kv) * DG + 4 * g4;
#pragma unroll
    for (int dq = 0; dq < NS; ++dq) dst[dq] = *reinterpret_cast<const float4*>(krow + 16 * dq);
  };
  if (c > 0) kload(0, ka);
  for (int j0 = 0; j0 < c; j0 += 64) {
    if (j0 + 64 < c) kload(j0 + 64, kn);
    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dq = 0; dq < NS; ++dq) {
      acc = mfma16x16x4f32(ka[dq].x, qb[dq][0], acc);
      acc = mfma16x16x4f32(ka[dq].y, qb[dq][1], acc);
      acc = mfma16x16x4f32(ka[dq].z, qb[dq][2], acc);
      acc = mfma16x16x4f32(ka[dq].w, qb[dq][3], acc);
    }
    const int jb = j0 + 16 * wv + 4 * g4;     // keys jb .. jb+3 of token l16
    if (l16 < ntok) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (jb + i < c) sc[l16 * NBP + jb + i] = acc[i] * inv_sqrt_dg;
    }
#pragma unroll
    for (int dq = 0; dq < NS; ++dq) ka[dq] = kn[dq];
  }
  __syncthreads();
  // current-block score with the token's own prefix key
  {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) acc = fmaf(cq[i], ck[i], acc);
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
      mx = wave_max_dpp(mx);
      float se = 0.f;
#pragma unroll
      for (int e = 0; e < EM; ++e) se += fast_exp2((sv[e] - mx) * kLog2e);
      se = wave_sum_dpp(se);
      const float lse = mx + __builtin_amdgcn_logf(se) * kLn2;
      const size_t rowid = (static_cast<size_t>(b) * p.T + t0 + tl) * p.Hs + sg;
      // order keys of the historical candidates; 0 elsewhere, which no
      // candidate threshold (always >= 1) reaches
      uint32_t kreg[EM];
#pragma unroll
      for (int e = 0; e < EM; ++e) kreg[e] = (lane + 64 * e < c) ? order_key(sv[e]) : 0u;
      uint32_t thr = 0;
      int n_ge = 0;                 // keys at or above thr
      if (!all) {
        // thr = the largest t with #(keys >= t) >= K, by a bitwise search.
        // The K-th largest lane maximum bounds it from below (the K largest
        // lane maxima are K keys at or above it; at least K lanes hold a
        // candidate since c > K and K < 64), and so does t0, that maximum
        // with its low 16 bits cleared; when the keys >= t0 fit one per lane
        // the search runs over them alone (same counts for every t >= t0).
        uint32_t lmax = 0;
#pragma unroll
        for (int e = 0; e < EM; ++e) lmax = max(lmax, kreg[e]);
        // (its top 16 bits suffice for a bound: any t with K keys at or
        // above it and few enough above it to gather will do)
        uint32_t t0k = 0;
        for (int bit = 31; bit >= 16; --bit) {
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
          // every key >= thr (>= t0k) is among the gathered ones
          n_ge = wave_count(v >= thr);
        } else {
          for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = thr | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int e = 0; e < EM; ++e) cnt += wave_count(kreg[e] >= cand);
            if (cnt >= K) thr = cand;
          }
#pragma unroll
          for (int e = 0; e < EM; ++e) n_ge += wave_count(kreg[e] >= thr);
        }
      }
      // selected historical blocks in ascending order into the wave's LDS
      // slots, then one contiguous store of the row
      int base = 0;
      if (all || n_ge == K) {
        // every key at or above the threshold is taken (no tie crosses it)
#pragma unroll
        for (int e = 0; e < EM; ++e) {
          const int j = lane + 64 * e;
          const bool s_in = j < c && (all || kreg[e] >= thr);
          const uint64_t sm = ballot64(s_in);
          if (s_in) {
            const int pos = base + __popcll(sm & lt_mask);
            selj[wv][pos] = j;
            sell[wv][pos] = sv[e] - lse;
          }
          base += __popcll(sm);
        }
      } else {
        // equal keys at the threshold: the lower block indices first
        int gt = 0;
#pragma unroll
        for (int e = 0; e < EM; ++e) gt += wave_count(kreg[e] > thr);
        const int need_eq = K - gt;
        int eq_seen = 0;
#pragma unroll
        for (int e = 0; e < EM; ++e) {
          const int j = lane + 64 * e;
          const bool hist = j < c;
          const bool eq = hist && kreg[e] == thr;
          const uint64_t em = ballot64(eq);
          const bool s_in =
              hist && (kreg[e] > thr || (eq && (eq_seen + __popcll(em & lt_mask)) < need_eq));
          eq_seen += __popcll(em);
          const uint64_t sm = ballot64(s_in);
          if (s_in) {
            const int pos = base + __popcll(sm & lt_mask);
            selj[wv][pos] = j;
            sell[wv][pos] = sv[e] - lse;
          }
          base += __popcll(sm);
        }
      }
      // (base == nsel) the current block, then the padding
      for (int s2 = lane; s2 < S; s2 += 64) {
        int jo = -1;
        float lo = -INFINITY;
        if (s2 < nsel) {
          jo = selj[wv][s2];
          lo = sell[wv][s2];
        } else if (s2 == nsel) {
          jo = c;
          lo = row[c] - lse;
        }
        p.idx[rowid * S + s2] = jo;
        p.logg[rowid * S + s2] = lo;
      }
      if (lane == 0) p.gate_lse[rowid] = lse;
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
  (void)dg;
  return sizeof(float) * static_cast<size_t>(kTokPerWG) * topk_score_pitch(NB);
}

hipError_t launch_topk(const TopkParams& p, hipStream_t st) {
  const dim3 grid((p.T + kTokPerWG - 1) / kTokPerWG, p.Hs, p.B);
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
