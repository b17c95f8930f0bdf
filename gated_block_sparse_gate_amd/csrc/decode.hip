// Budgeted single-token decode (model card: 2,048-token sparse decode budget
// by default, 1,024 and 4,096 also supported; usage guide pitfall 3: the
// budget limits the tokens each query attends, not the cache).
//
// Unit = (sequence b, KV head kappa), L = ctx_len[b], c = (L-1)/64:
//   score : s_j = q_gate . kg_cache[j] / sqrt(dg), j = 0..c (chunks of 128
//           candidates per workgroup);
//   top-k : log-sum-exp; the min(K, c) best historical blocks (ties ->
//           lower j) + block c (one wave per unit).
//   attend: the G query heads attend to the selected blocks' keys tau < L
//           with log g added (apply_gate = 1), split over NSPLIT workgroups
//           of 2 slots whose K/V blocks (16 KiB each per tensor, contiguous
//           in the head-major cache) are all loaded before any arithmetic.
//   merge: one workgroup per unit merges the per-split (max, sum, o)
//           partials.
#include <type_traits>

#include "sas_kernels.h"

namespace sas {

namespace {

constexpr int kSlotsPerSplit = 2;

// Score step: workgroup = (unit, chunk of 128 candidate blocks), 256
// threads, 8 lanes per candidate; all of the chunk's gate-key loads are issued
// before any arithmetic.  s_j = q_gate . kg_cache[j] / sqrt(dg) for j <= c
// goes to the workspace.
template <int DG>
__global__ __launch_bounds__(256) void decode_score_kernel(DecodeParams p) {
  constexpr int LPC = 8;                 // lanes per candidate
  constexpr int F4 = DG / 4 / LPC;       // float4 per lane per candidate
  constexpr int NPASS = 4;               // 4 x 32 candidates per workgroup
  const int tid = threadIdx.x;
  const int unit = blockIdx.x, chunk = blockIdx.y;
  const int b = unit / p.Hkv;
  const int L = p.ctx_len[b];
  if (!(L >= 1 && L <= p.Lmax)) return;
  const int ncand = (L - 1) / 64 + 1;
  const int j0 = chunk * 32 * NPASS;
  if (j0 >= ncand) return;
  const int sub = tid & (LPC - 1), cl = tid / LPC;    // 32 candidates per pass
  const float* kgb = p.kg_cache + static_cast<size_t>(unit) * p.NBmax * DG;
  const float* qgp = p.q_gate + static_cast<size_t>(unit) * DG;
  float4 qv[F4], kvv[NPASS][F4];
#pragma unroll
  for (int pss = 0; pss < NPASS; ++pss) {
    const int j = j0 + pss * 32 + cl;
#pragma unroll
    for (int f = 0; f < F4; ++f)
      kvv[pss][f] = (j < ncand) ? *reinterpret_cast<const float4*>(
                                      kgb + static_cast<size_t>(j) * DG + (f * LPC + sub) * 4)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int f = 0; f < F4; ++f) qv[f] = *reinterpret_cast<const float4*>(qgp + (f * LPC + sub) * 4);
  const float inv_sqrt_dg = 1.0f / sqrtf(static_cast<float>(DG));
  float* sco = p.ws_score + static_cast<size_t>(unit) * p.NBmax;
#pragma unroll
  for (int pss = 0; pss < NPASS; ++pss) {
    float a = 0.f;
#pragma unroll
    for (int f = 0; f < F4; ++f) {
      a = fmaf(qv[f].x, kvv[pss][f].x, a);
      a = fmaf(qv[f].y, kvv[pss][f].y, a);
      a = fmaf(qv[f].z, kvv[pss][f].z, a);
      a = fmaf(qv[f].w, kvv[pss][f].w, a);
    }
    // the candidate's 8 lanes: xor 1, xor 2, then the 8-lane mirror
    a += dpp_mov<0xB1>(a);
    a += dpp_mov<0x4E>(a);
    a += dpp_mov<0x141>(a);
    const int j = j0 + pss * 32 + cl;
    if (sub == 0 && j < ncand) sco[j] = a * inv_sqrt_dg;
  }
}

// Selection step: one wave per unit (4 units per workgroup).  Log-sum-exp
// over the c + 1 scores, then the min(K, c) largest historical scores by a
// 32-step bitwise search on order keys with ballot counts (ties -> lower
// block), ascending, then block c; pads -1 / -inf.
template <bool LONG>
__global__ __launch_bounds__(256) void decode_topk_kernel(DecodeParams p) {
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= p.B * p.Hkv) return;
  const int b = unit / p.Hkv;
  const int L = p.ctx_len[b];
  const bool ok = (L >= 1 && L <= p.Lmax);
  const int S = p.S, K = p.K;
  int32_t* wid = p.ws_idx + static_cast<size_t>(unit) * S;
  float* wlg = p.ws_logg + static_cast<size_t>(unit) * S;
  int32_t* oid = p.idx_out ? p.idx_out + static_cast<size_t>(unit) * S : nullptr;
  float* olg = p.logg_out ? p.logg_out + static_cast<size_t>(unit) * S : nullptr;
  auto put = [&](int pos, int j, float v) {
    wid[pos] = j;
    wlg[pos] = v;
    if (oid) oid[pos] = j;
    if (olg) olg[pos] = v;
  };
  if (!ok) {
    for (int s2 = lane; s2 < S; s2 += 64) put(s2, -1, -INFINITY);
    return;
  }
  const float* sc = p.ws_score + static_cast<size_t>(unit) * p.NBmax;
  const int c = (L - 1) / 64;
  const int ncand = c + 1;
  const int E = (ncand + 63) / 64;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const bool all = (c <= K);
  const int nsel = min(K, c);
  float lse = 0.f;
  // scores in registers (EMAX per lane, all loads issued at once), or
  // (REG = false, contexts beyond 1,024 blocks) re-read at every use
  auto select = [&](auto emc, auto regc) __attribute__((always_inline)) {
    constexpr int EMAX = decltype(emc)::value;
    constexpr bool REG = decltype(regc)::value;
    float sv[REG ? EMAX : 1];
    if constexpr (REG) {
      // unconditional loads at clamped addresses (no branch between them, so
      // they are all in flight together), then masked
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        const int j = lane + 64 * e;
        const float v = sc[min(j, ncand - 1)];
        sv[e] = (j < ncand) ? v : -INFINITY;
      }
    }
    auto score = [&](int e) -> float {
      if constexpr (REG) return sv[e];
      const int j = lane + 64 * e;
      return j < ncand ? sc[j] : -INFINITY;
    };
    // trip count EMAX (unrolled, guarded) in registers, E (rolled) otherwise
    constexpr int NE = REG ? EMAX : 0;
    const int ne = REG ? NE : E;
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < ne; ++e)
      if (e < E) mx = fmaxf(mx, score(e));
    mx = wave_max(mx);
    float se = 0.f;
#pragma unroll
    for (int e = 0; e < ne; ++e)
      if (e < E) se += expf(score(e) - mx);
    se = wave_sum(se);
    lse = mx + logf(se);
    // order keys of the historical candidates; 0 for everything else, which
    // no candidate threshold (always >= 1) reaches
    uint32_t kreg[REG ? EMAX : 1];
    if constexpr (REG) {
#pragma unroll
      for (int e = 0; e < EMAX; ++e) kreg[e] = (lane + 64 * e < c) ? order_key(sv[e]) : 0u;
    }
    auto key = [&](int e) -> uint32_t {
      if constexpr (REG) return kreg[e];
      return (lane + 64 * e < c) ? order_key(score(e)) : 0u;
    };
    uint32_t thr = 0;
    int need_eq = 0;
    if (!all) {
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < ne; ++e) cnt += wave_count(key(e) >= cand);
        if (cnt >= K) thr = cand;
      }
      int gt = 0;
#pragma unroll
      for (int e = 0; e < ne; ++e) gt += wave_count(key(e) > thr);
      need_eq = K - gt;
    }
    int base = 0, eq_seen = 0;
#pragma unroll
    for (int e = 0; e < ne; ++e) {
      if (e < E) {
        const int j = lane + 64 * e;
        const bool hist = j < c;
        const uint32_t kk = key(e);
        const bool gt = hist && !all && kk > thr;
        const bool eq = hist && !all && kk == thr;
        const uint64_t em = ballot64(eq);
        const bool s_in =
            hist && (all || gt || (eq && (eq_seen + __popcll(em & lt_mask)) < need_eq));
        eq_seen += __popcll(em);
        const uint64_t sm = ballot64(s_in);
        if (s_in) put(base + __popcll(sm & lt_mask), j, score(e) - lse);
        base += __popcll(sm);
      }
    }
  };
  if constexpr (!LONG)
    select(std::integral_constant<int, kMaxNB / 64>{}, std::true_type{});
  else
    select(std::integral_constant<int, kMaxDecodeNB / 64>{}, std::false_type{});
  if (lane == 0) put(nsel, c, sc[c] - lse);
  for (int s2 = nsel + 1 + lane; s2 < S; s2 += 64) put(s2, -1, -INFINITY);
}

// Sum over aligned groups of N consecutive lanes inside 16-lane rows
// (N = 8 or 16): quad butterflies, then the 8- and 16-lane mirrors.
template <int N>
__device__ __forceinline__ float lane_group_sum(float x) {
  x += dpp_mov<0xB1>(x);                  // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);                  // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);                 // row_half_mirror
  if (N == 16) x += dpp_mov<0x140>(x);    // row_mirror
  return x;
}

// o[h] = sum_split o_split exp2(m_split - M) / sum_split l_split exp2(m_split - M)
// over the unit's splits (one workgroup of 256 threads).  The per-split
// weights are formed once per (split, head) in LDS.
template <int D, int G>
__device__ __forceinline__ void merge_splits(const DecodeParams& p, int unit, int b, int kv,
                                             bool ok) {
  __shared__ float wsp[kMaxS][G];
  __shared__ float inv_l[G];
  const int tid = threadIdx.x;
  const float* base = p.ws_part + static_cast<size_t>(unit) * p.nsplit * G * (D + 2);
  if (tid < G) {
    const int h = tid;
    float M = -INFINITY;
    for (int sp = 0; sp < p.nsplit; ++sp) M = fmaxf(M, base[(sp * G + h) * (D + 2) + D]);
    float l = 0.f;
    for (int sp = 0; sp < p.nsplit; ++sp) {
      const float m = base[(sp * G + h) * (D + 2) + D];
      const float w = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
      wsp[sp][h] = w;
      l += base[(sp * G + h) * (D + 2) + D + 1] * w;
    }
    inv_l[h] = (ok && l > 0.f) ? 1.f / l : __builtin_nanf("");
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += 256) {
    const int h = e / D, d = e - h * D;
    float o = 0.f;
    for (int sp = 0; sp < p.nsplit; ++sp) o = fmaf(base[(sp * G + h) * (D + 2) + d], wsp[sp][h], o);
    p.o[(static_cast<size_t>(b) * p.Hq + kv * G + h) * D + d] = f2bf(o * inv_l[h]);
  }
}

// Workgroup = (unit, split of kSlotsPerSplit selected blocks), 256 threads.
// Thread t owns 16-byte chunk ch = t % (D/8) of rows rg + (256/(D/8)) x of
// each block, so one block of K (and of V) is one coalesced 16 KiB read per
// tensor; every K/V load of the split is issued before any arithmetic, which
// keeps 64 KiB per workgroup in flight.  Scores: per-thread 8-element partial
// dots, reduced over the row's lanes with DPP; softmax state and the output
// partials are per wave (online over the split's blocks), merged across the
// wave's row groups with lane permutes and across the 4 waves in LDS once.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeParams p) {
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;          // rows per pass of the workgroup
  constexpr int RPT = 64 / RPP;           // rows per thread per block
  constexpr int SPW = kSlotsPerSplit;
  __shared__ float red_m[4][G], red_l[4][G];
  __shared__ __attribute__((aligned(16))) float red_o[4][G][D];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ch = tid % CPR, rg = tid / CPR;
  const int unit = blockIdx.x, split = blockIdx.y;
  const int b = unit / p.Hkv, kv = unit - b * p.Hkv;
  const int L = p.ctx_len[b];
  const bool ok = (L >= 1 && L <= p.Lmax);
  const int s0 = split * SPW;
  float* part = p.ws_part + (static_cast<size_t>(unit) * p.nsplit + split) * G * (D + 2);

  int jsl[SPW];
  float lgl[SPW];
#pragma unroll
  for (int sl = 0; sl < SPW; ++sl) {
    const int s = s0 + sl;
    const int j = (ok && s < p.S) ? p.ws_idx[static_cast<size_t>(unit) * p.S + s] : -1;
    jsl[sl] = (j >= 0 && 64 * j < L) ? j : -1;
    lgl[sl] = (jsl[sl] >= 0 && p.apply_gate)
                  ? p.ws_logg[static_cast<size_t>(unit) * p.S + s] * kLog2e : 0.f;
  }
  const size_t ubase = (static_cast<size_t>(b) * p.Hkv + kv) * p.Lmax * D + ch * 8;
  uint4 kr[SPW][RPT], vr[SPW][RPT];
#pragma unroll
  for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
    for (int x = 0; x < RPT; ++x) {
      const int tok = 64 * jsl[sl] + rg + RPP * x;
      const bool in = jsl[sl] >= 0 && tok < L;
      kr[sl][x] = in ? ld16(p.k_cache + ubase + static_cast<size_t>(tok) * D) : make_uint4(0, 0, 0, 0);
      vr[sl][x] = in ? ld16(p.v_cache + ubase + static_cast<size_t>(tok) * D) : make_uint4(0, 0, 0, 0);
    }
  uint4 qr[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qr[h] = ld16(p.q + (static_cast<size_t>(b) * p.Hq + kv * G + h) * D + ch * 8);

  float m_run[G], l_run[G], oacc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) oacc[h][e] = 0.f;
  }
  const float sl2 = p.scale_log2;
#pragma unroll
  for (int sl = 0; sl < SPW; ++sl) {
    if (jsl[sl] < 0) continue;                       // uniform over the workgroup
    // scores: 8-element partial dots with v_dot2_f32_bf16 (exact bf16
    // products, fp32 accumulation), then summed over the row's lanes
    float sc[RPT][G];
#pragma unroll
    for (int x = 0; x < RPT; ++x) {
      const uint32_t kw[4] = {kr[sl][x].x, kr[sl][x].y, kr[sl][x].z, kr[sl][x].w};
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint32_t qw[4] = {qr[h].x, qr[h].y, qr[h].z, qr[h].w};
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) a = dot2_bf16(qw[i], kw[i], a);
        sc[x][h] = lane_group_sum<CPR>(a);
      }
      const int tok = 64 * jsl[sl] + rg + RPP * x;
#pragma unroll
      for (int h = 0; h < G; ++h)
        sc[x][h] = (tok < L) ? fmaf(sc[x][h], sl2, lgl[sl]) : -INFINITY;
    }
    // online softmax per head (state shared by the wave)
    float pv[RPT][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = sc[0][h];
#pragma unroll
      for (int x = 1; x < RPT; ++x) mx = fmaxf(mx, sc[x][h]);
      if (CPR == 8) mx = fmaxf(mx, dpp_mov<0x140>(mx));   // the two row groups of a 16-lane row
      mx = row4_max(mx);
      // a wave may hold no visible key of a partial current block: keep its
      // state at -inf without forming -inf - -inf
      const float m_new = fmaxf(m_run[h], mx);
      const float msafe = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[h] - msafe);   // 0 while m_run is -inf
      float ps = 0.f;
#pragma unroll
      for (int x = 0; x < RPT; ++x) {
        pv[x][h] = fast_exp2(sc[x][h] - msafe);
        ps += pv[x][h];
      }
      l_run[h] = l_run[h] * alpha + ps;
#pragma unroll
      for (int e = 0; e < 8; ++e) oacc[h][e] *= alpha;
      m_run[h] = m_new;
    }
    // O += P V: each V row chunk converted once, used by every head
#pragma unroll
    for (int x = 0; x < RPT; ++x) {
      const uint32_t vw[4] = {vr[sl][x].x, vr[sl][x].y, vr[sl][x].z, vr[sl][x].w};
      float vf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vf[2 * i] = __uint_as_float(vw[i] << 16);
        vf[2 * i + 1] = __uint_as_float(vw[i] & 0xffff0000u);
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[h][e] = fmaf(pv[x][h], vf[e], oacc[h][e]);
    }
  }
  // wave totals: sum over the wave's row groups (lanes with equal ch)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float l = l_run[h];
    if (CPR == 8) l += dpp_mov<0x140>(l);
    l = row4_sum(l);
    if (lane == 0) {
      red_m[wv][h] = m_run[h];
      red_l[wv][h] = l;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float o = oacc[h][e];
      if (CPR == 8) o += dpp_mov<0x128>(o);          // row_ror:8 pairs lanes i, i+8
      o = row4_sum(o);
      if (lane < CPR) red_o[wv][h][ch * 8 + e] = o;
    }
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += 256) {
    const int h = e / D, d = e - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w][h]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = red_m[w][h];
      if (mw == -INFINITY) continue;
      const float f = fast_exp2(mw - M);
      o += red_o[w][h][d] * f;
      l += red_l[w][h] * f;
    }
    part[h * (D + 2) + d] = o;
    if (d == 0) {
      part[h * (D + 2) + D] = M;
      part[h * (D + 2) + D + 1] = l;
    }
  }
}

// One workgroup per unit merges the unit's split partials.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
  const int unit = blockIdx.x;
  const int b = unit / p.Hkv, kv = unit - b * p.Hkv;
  const int L = p.ctx_len[b];
  merge_splits<D, G>(p, unit, b, kv, L >= 1 && L <= p.Lmax);
}

}  // namespace

int decode_nsplit(int S) { return (S + kSlotsPerSplit - 1) / kSlotsPerSplit; }

hipError_t launch_decode(const DecodeParams& p, hipStream_t st) {
  const unsigned units = static_cast<unsigned>(p.B) * p.Hkv;
  const dim3 sgrid(units, (p.NBmax + 127) / 128);
  switch (p.dg) {
    case 128: hipLaunchKernelGGL((decode_score_kernel<128>), sgrid, dim3(256), 0, st, p); break;
    case 64: hipLaunchKernelGGL((decode_score_kernel<64>), sgrid, dim3(256), 0, st, p); break;
    case 32: hipLaunchKernelGGL((decode_score_kernel<32>), sgrid, dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  if (p.NBmax <= kMaxNB)
    hipLaunchKernelGGL((decode_topk_kernel<false>), dim3((units + 3) / 4), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((decode_topk_kernel<true>), dim3((units + 3) / 4), dim3(256), 0, st, p);
  const dim3 agrid(units, p.nsplit);
  if (p.D == 128) {
    switch (p.G) {
      case 1:
        hipLaunchKernelGGL((decode_attn_kernel<128, 1>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<128, 1>), dim3(units), dim3(256), 0, st, p);
        break;
      case 2:
        hipLaunchKernelGGL((decode_attn_kernel<128, 2>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<128, 2>), dim3(units), dim3(256), 0, st, p);
        break;
      case 3:
        hipLaunchKernelGGL((decode_attn_kernel<128, 3>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<128, 3>), dim3(units), dim3(256), 0, st, p);
        break;
      case 4:
        hipLaunchKernelGGL((decode_attn_kernel<128, 4>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<128, 4>), dim3(units), dim3(256), 0, st, p);
        break;
      case 5:
        hipLaunchKernelGGL((decode_attn_kernel<128, 5>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<128, 5>), dim3(units), dim3(256), 0, st, p);
        break;
      case 6:
        hipLaunchKernelGGL((decode_attn_kernel<128, 6>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<128, 6>), dim3(units), dim3(256), 0, st, p);
        break;
      case 7:
        hipLaunchKernelGGL((decode_attn_kernel<128, 7>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<128, 7>), dim3(units), dim3(256), 0, st, p);
        break;
      case 8:
        hipLaunchKernelGGL((decode_attn_kernel<128, 8>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<128, 8>), dim3(units), dim3(256), 0, st, p);
        break;
      default: return hipErrorInvalidValue;
    }
  } else if (p.D == 64) {
    switch (p.G) {
      case 1:
        hipLaunchKernelGGL((decode_attn_kernel<64, 1>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<64, 1>), dim3(units), dim3(256), 0, st, p);
        break;
      case 2:
        hipLaunchKernelGGL((decode_attn_kernel<64, 2>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<64, 2>), dim3(units), dim3(256), 0, st, p);
        break;
      case 3:
        hipLaunchKernelGGL((decode_attn_kernel<64, 3>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<64, 3>), dim3(units), dim3(256), 0, st, p);
        break;
      case 4:
        hipLaunchKernelGGL((decode_attn_kernel<64, 4>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<64, 4>), dim3(units), dim3(256), 0, st, p);
        break;
      case 5:
        hipLaunchKernelGGL((decode_attn_kernel<64, 5>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<64, 5>), dim3(units), dim3(256), 0, st, p);
        break;
      case 6:
        hipLaunchKernelGGL((decode_attn_kernel<64, 6>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<64, 6>), dim3(units), dim3(256), 0, st, p);
        break;
      case 7:
        hipLaunchKernelGGL((decode_attn_kernel<64, 7>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<64, 7>), dim3(units), dim3(256), 0, st, p);
        break;
      case 8:
        hipLaunchKernelGGL((decode_attn_kernel<64, 8>), agrid, dim3(256), 0, st, p);
        hipLaunchKernelGGL((decode_merge_kernel<64, 8>), dim3(units), dim3(256), 0, st, p);
        break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sas
