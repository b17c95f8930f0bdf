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
//           of 4 slots whose K/V blocks (16 KiB each per tensor, contiguous
//           in the head-major cache) are all loaded before any arithmetic;
//           scores and P V on MFMA.
//   merge: one workgroup per unit merges the per-split (max, sum, o)
//           partials.
#include <type_traits>

#include "sas_kernels.h"

namespace sas {

namespace {

constexpr int kSlotsPerSplit = 4;

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
  constexpr int RF = decode_part_floats(G, D);
  const int tid = threadIdx.x;
  const float* base = p.ws_part + static_cast<size_t>(unit) * p.nsplit * RF;
  if (tid < G) {
    const int h = tid;
    float M = -INFINITY;
    for (int sp = 0; sp < p.nsplit; ++sp) M = fmaxf(M, base[sp * RF + G * D + h]);
    float l = 0.f;
    for (int sp = 0; sp < p.nsplit; ++sp) {
      const float m = base[sp * RF + G * D + h];
      const float w = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
      wsp[sp][h] = w;
      l += base[sp * RF + G * D + 16 + h] * w;
    }
    inv_l[h] = (ok && l > 0.f) ? 1.f / l : __builtin_nanf("");
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += 256) {
    const int h = e / D;
    float o = 0.f;
    for (int sp = 0; sp < p.nsplit; ++sp) o = fmaf(base[sp * RF + e], wsp[sp][h], o);
    p.o[(static_cast<size_t>(b) * p.Hq + kv * G) * D + e] = f2bf(o * inv_l[h]);
  }
}

// Workgroup = (unit, split of four selected blocks), 256 threads, in two
// passes of two blocks; in a pass, wave w takes keys 16w .. 16w + 15 of each
// of the two blocks (32 keys), so the scores and P V of a wave are single
// MFMA tiles with the G heads padded to 16 columns:
//   S^T[key][h] = K Q^T      A = the wave's 16 keys of one block, loaded from
//                            HBM straight into the operand layout (16 bytes
//                            per lane, 64 contiguous bytes per key and load);
//   O^T[d][h]  += V^T P^T    A = V^T from LDS with transposing reads, B = the
//                            bf16 softmax weights as they sit in S's
//                            accumulator lanes (k slot 8g + i <-> key 4g + i
//                            of the pass's first block for i < 4, of its
//                            second block for i >= 4, on both operands).
// Every K and V load of the workgroup (128 KiB) is issued before any
// arithmetic: the first pass's V rows go HBM -> LDS by DMA into a per-wave
// region, the second pass's wait in registers and take their place once the
// first pass has read them (no workgroup barrier).  The softmax state is
// carried online across the passes.  Keys at or beyond the context length
// read as zeros (K: buffer range) or as the last valid row (V, with weight
// 0); a slot without a block reads no K and zeroes its V operand.  The
// per-wave (max, sum, O) are merged across the 4 waves in LDS, each wave's in
// place of its own V rows, into one partial per split, written in whole
// 128-byte lines.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeParams p) {
  static_assert(kSlotsPerSplit == 4, "two passes of two 16-key tiles per wave");
  static_assert(G >= 1 && G <= 16, "heads per KV head");
  constexpr int NKS = D / 32;             // k steps of S
  constexpr int NDT = D / 16;             // d tiles of O
  constexpr int ROWB = 2 * D;             // bytes per key row
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;           // rows per 1 KiB wave load
  constexpr int NVT = 16 / RPI;           // wave loads per 16-row tile
  constexpr int G4 = (G + 3) / 4 * 4;     // keeps o 16-byte aligned
  // a wave's (max, sum, O) replace its own V rows once it has read them
  struct WaveRed {
    float m[G4], l[G4];
    float o[G][D];
  };
  static_assert(sizeof(WaveRed) <= 32 * ROWB, "wave partial fits the wave's V rows");
  __shared__ __attribute__((aligned(16))) unsigned char vs[4 * 32 * ROWB];   // [wave][32 rows][ROWB], chunk-swizzled

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int unit = blockIdx.x, split = blockIdx.y;
  const int b = unit / p.Hkv, kv = unit - b * p.Hkv;
  const int L = p.ctx_len[b];
  const bool ok = (L >= 1 && L <= p.Lmax);
  const int s0 = split * 4;
  float* part = p.ws_part + (static_cast<size_t>(unit) * p.nsplit + split) * decode_part_floats(G, D);

  int jsl[4];
  float lgl[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int s = s0 + t;
    const int j = (ok && s < p.S) ? p.ws_idx[static_cast<size_t>(unit) * p.S + s] : -1;
    jsl[t] = (j >= 0 && 64 * j < L) ? j : -1;
    lgl[t] = (jsl[t] >= 0 && p.apply_gate)
                 ? p.ws_logg[static_cast<size_t>(unit) * p.S + s] * kLog2e : 0.f;
  }
  // Q^T operand: column h = r (zero for r >= G)
  uint4 qb[NKS];
  {
    const int h = min(r, G - 1);
    const uint16_t* qp = p.q + (static_cast<size_t>(b) * p.Hq + kv * G + h) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint4 v = ld16(qp + 32 * ks);
      qb[ks] = (r < G) ? v : make_uint4(0, 0, 0, 0);
    }
  }
  const size_t ubase = (static_cast<size_t>(b) * p.Hkv + kv) * p.Lmax * D;
  // K: keys >= L lie beyond the resource and read as zeros
  const unsigned krec = ok ? static_cast<unsigned>(L) * ROWB : 0u;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.k_cache + ubase), 0, krec, kBufferWord3);
  uint4 ka[4][NKS];
  // V: wave row 16 u + i (u = t % 2) = key 16 w + i of slot t's block; rows
  // of a slot without a block repeat block 0 and are zeroed on reading, which
  // keeps the loads branch-free
  unsigned char* vw = vs + w * 32 * ROWB;
  uint4 vr[2][NVT];
  auto vsrc = [&](int t, int n) {
    const int rho = 16 * (t & 1) + RPI * n + lane / CPR;
    const int c = (lane % CPR) ^ lds_swz<ROWB>(rho);
    const int tok = max(min(64 * max(jsl[t], 0) + 16 * w + (rho & 15), L - 1), 0);
    return p.v_cache + ubase + static_cast<size_t>(tok) * D + c * 8;
  };
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const unsigned row = static_cast<unsigned>(64 * jsl[t] + 16 * w + r);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      ka[t][ks] = buffer_ld16(krs, jsl[t] >= 0 ? row * ROWB + 64 * ks + 16 * g : krec);
#pragma unroll
    for (int n = 0; n < NVT; ++n) {
      if (t < 2)
        load_lds16(vsrc(t, n), vw + (16 * t + RPI * n) * ROWB);
      else
        vr[t - 2][n] = ld16(vsrc(t, n));
    }
  }
  __builtin_amdgcn_sched_barrier(0);               // every load issued before the MFMAs
  const float sl2 = p.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  floatx4 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  // transposing reads: lane s of group g addresses row 4g + s/4 (of each
  // tile), columns 16 dt + 4 (s % 4) .. +3 and receives column 16 dt + s
  const int rho0 = 4 * g + (r >> 2);
  const int cb = (r & 3) >> 1, hb = 8 * (r & 1);
#pragma unroll
  for (int ps = 0; ps < 2; ++ps) {
    const int t0 = 2 * ps;
    // S^T tiles: lane holds head r, keys 4g .. 4g + 3 of each tile
    floatx4 sacc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sacc[u] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) sacc[u] = mfma16x16x32(ka[t0 + u][ks], qb[ks], sacc[u]);
    }
    float sv[2][4];
    float mx = m_run;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 64 * jsl[t0 + u] + 16 * w + 4 * g + i;
        sv[u][i] = (jsl[t0 + u] >= 0 && tok < L) ? fmaf(sacc[u][i], sl2, lgl[t0 + u]) : -INFINITY;
        mx = fmaxf(mx, sv[u][i]);
      }
    mx = row4_max(mx);
    // a wave may see no valid key: keep its state at -inf, weights 0
    const float msafe = (mx == -INFINITY) ? 0.f : mx;
    const float alpha = fast_exp2(m_run - msafe);   // 0 while m_run is -inf
    float ls = 0.f, pw[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pw[u][i] = fast_exp2(sv[u][i] - msafe);
        ls += pw[u][i];
      }
    l_run = l_run * alpha + row4_sum(ls);
    m_run = mx;
    const uint4 pb = make_uint4(pack_bf2(pw[0][0], pw[0][1]), pack_bf2(pw[0][2], pw[0][3]),
                                pack_bf2(pw[1][0], pw[1][1]), pack_bf2(pw[1][2], pw[1][3]));
    if (ps == 0) {
      wait_vmem_all();
    } else {
      // the second pass's rows replace the first's (this wave's LDS accesses
      // complete in order, after its reads of them)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int n = 0; n < NVT; ++n) st16(vw + (16 * u + RPI * n) * ROWB + 16 * lane, vr[u][n]);
    }
    // O^T tiles: lane holds head r, d = 16 dt + 4g .. +3
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint2 v0 = lds_read_tr16(vw + rho0 * ROWB + (((2 * dt + cb) ^ lds_swz<ROWB>(rho0)) << 4) + hb);
      uint2 v1 = lds_read_tr16(vw + (rho0 + 16) * ROWB +
                               (((2 * dt + cb) ^ lds_swz<ROWB>(rho0 + 16)) << 4) + hb);
      if (jsl[t0] < 0) v0 = make_uint2(0, 0);
      if (jsl[t0 + 1] < 0) v1 = make_uint2(0, 0);
      oacc[dt] = mfma16x16x32(make_uint4(v0.x, v0.y, v1.x, v1.y), pb, oacc[dt] * alpha);
    }
  }
  // the wave's LDS accesses complete in order: its reads of its V rows are
  // done before these stores reach them
  WaveRed& mine = *reinterpret_cast<WaveRed*>(vw);
  if (r < G) {
    if (g == 0) {
      mine.m[r] = m_run;
      mine.l[r] = l_run;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<floatx4*>(&mine.o[r][16 * dt + 4 * g]) = oacc[dt];
  }
  __syncthreads();
  // the split's partial, written in whole 128-byte lines
  auto wred = [&](int q) -> const WaveRed& { return *reinterpret_cast<const WaveRed*>(vs + q * 32 * ROWB); };
  for (int e = tid; e < G * D; e += 256) {
    const int h = e / D, d = e - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) M = fmaxf(M, wred(q).m[h]);
    float o = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float mq = wred(q).m[h];
      if (mq != -INFINITY) o += wred(q).o[h][d] * fast_exp2(mq - M);
    }
    part[e] = o;
  }
  if (tid < 32) {
    const int h = tid & 15;
    float M = -INFINITY, l = 0.f;
    if (h < G) {
#pragma unroll
      for (int q = 0; q < 4; ++q) M = fmaxf(M, wred(q).m[h]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float mq = wred(q).m[h];
        if (mq != -INFINITY) l += wred(q).l[h] * fast_exp2(mq - M);
      }
    }
    part[G * D + tid] = tid < 16 ? M : l;
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
