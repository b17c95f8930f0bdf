// Budgeted single-token decode (model card: 2,048-token sparse decode budget
// by default, 1,024 and 4,096 also supported; usage guide pitfall 3: the
// budget limits the tokens each query attends, not the cache).
//
// Unit = (sequence b, selection head sg), L = ctx_len[b], c = (L-1)/64; the
// selection head is a KV head kappa whose gate its G query heads share, or
// (one gate per query head) a single query head of KV head kappa = sg / kdiv:
//   score : s_j = q_gate[sg] . kg_cache[kappa, j] / sqrt(dg), j = 0..c
//           (chunks of 128 candidates per workgroup; gate keys fp32 or bf16);
//   top-k : log-sum-exp; the min(K, c) best historical blocks (ties ->
//           lower j) + block c (one wave per unit).
//   attend: the unit's query heads attend to the selected blocks' keys tau < L
//           with log g added (apply_gate = 1); a workgroup walks its unit's
//           selected blocks (16 KiB each per tensor, contiguous in the
//           head-major cache) two at a time, software-pipelined, with scores
//           and P V on MFMA.  With fewer units than the chip needs, each
//           unit's slots are split over NSPLIT workgroups and
//   merge: one workgroup per unit merges the per-split (max, sum, o)
//           partials.
#include <algorithm>
#include <type_traits>

#include "sas_kernels.h"

namespace sas {

namespace {

// workgroups the attention step aims for: two per compute unit (each holds
// 64 KiB of loads in flight while it computes)
constexpr int kDecodeWorkgroups = 512;

// Score step: workgroup = (unit, chunk of 128 candidate blocks), 256
// threads, 8 lanes per candidate; all of the chunk's gate-key loads are issued
// before any arithmetic.  s_j = q_gate . kg_cache[j] / sqrt(dg) for j <= c
// goes to the workspace.
template <int DG, bool BF>
__global__ __launch_bounds__(256) void decode_score_kernel(DecodeParams p) {
  constexpr int LPC = 8;                 // lanes per candidate
  constexpr int F4 = DG / 4 / LPC;       // float4 per lane per candidate
  constexpr int NPASS = 4;               // 4 x 32 candidates per workgroup
  const int tid = threadIdx.x;
  const int unit = blockIdx.x, chunk = blockIdx.y;
  const int b = unit / p.Hs;
  const int L = p.ctx_len[b];
  if (!(L >= 1 && L <= p.Lmax)) return;
  const int ncand = (L - 1) / 64 + 1;
  const int j0 = chunk * 32 * NPASS;
  if (j0 >= ncand) return;
  const int sub = tid & (LPC - 1), cl = tid / LPC;    // 32 candidates per pass
  const int kv = (unit - b * p.Hs) / p.kdiv;          // KV head of the unit's gate keys
  const float* qgp = p.q_gate + static_cast<size_t>(unit) * DG;
  // element index of candidate j's gate key: row j of the unit's cache, or
  // (paged) the key of the block's page; -1 past the candidates or for a page
  // outside the pool (reads as zeros)
  auto key_row = [&](int j) -> long {
    if (j >= ncand) return -1;
    if (!p.btab) return ((static_cast<long>(b) * p.Hkv + kv) * p.NBmax + j) * DG;
    const int pg = p.btab[static_cast<size_t>(b) * p.NBmax + j];
    return (pg >= 0 && pg < p.num_pages) ? (static_cast<long>(pg) * p.Hkv + kv) * DG : -1;
  };
  // 4 consecutive key elements (fp32, or bf16 widened exactly)
  auto load4 = [&](long e) -> float4 {
    if constexpr (BF) {
      const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p.kg_cache) + e);
      return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                         __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
    } else {
      return *reinterpret_cast<const float4*>(p.kg_cache + e);
    }
  };
  float4 qv[F4], kvv[NPASS][F4];
#pragma unroll
  for (int pss = 0; pss < NPASS; ++pss) {
    const long kr = key_row(j0 + pss * 32 + cl);
#pragma unroll
    for (int f = 0; f < F4; ++f)
      kvv[pss][f] = kr >= 0 ? load4(kr + (f * LPC + sub) * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
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
// over the c + 1 scores, then the min(K, c) largest historical scores by
// bitwise searches on order keys with ballot counts (ties -> lower block),
// ascending, then block c; pads -1 / -inf.
template <bool LONG>
__global__ __launch_bounds__(256) void decode_topk_kernel(DecodeParams p) {
  __shared__ uint32_t gath[4][64];
  __shared__ int selj[4][64];                  // per wave: selected blocks in output order
  __shared__ float sell[4][64];                // and their log-gates
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int unit = blockIdx.x * 4 + wv;
  if (unit >= p.B * p.Hs) return;
  const int b = unit / p.Hs;
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
    // loops over the lane's slots e: unrolled over the EMAX register slots
    // (each_cand: only e < E; each_slot: all, the keys past E being 0), a
    // rolled loop of E trips otherwise
    auto each_cand = [&](auto&& f) __attribute__((always_inline)) {
      if constexpr (REG) {
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
          if (e < E) f(e);
      } else {
        for (int e = 0; e < E; ++e) f(e);
      }
    };
    auto each_slot = [&](auto&& f) __attribute__((always_inline)) {
      if constexpr (REG) {
#pragma unroll
        for (int e = 0; e < EMAX; ++e) f(e);
      } else {
        for (int e = 0; e < E; ++e) f(e);
      }
    };
    float mx = -INFINITY;
    each_cand([&](int e) { mx = fmaxf(mx, score(e)); });
    mx = wave_max(mx);
    float se = 0.f;
    each_cand([&](int e) { se += fast_exp2((score(e) - mx) * kLog2e); });
    se = wave_sum(se);
    lse = mx + __builtin_amdgcn_logf(se) * kLn2;
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
    int n_ge = 0;                 // keys at or above thr
    if (!all) {
      // thr = the largest t with #(keys >= t) >= K, by a bitwise search.
      // The K-th largest lane maximum bounds it from below (the K largest
      // lane maxima are K keys at or above it; at least K lanes hold a
      // candidate since c > K and K < 64), and so does t0, that maximum with
      // its low 16 bits cleared; when the keys >= t0 fit one per lane the
      // search runs over them alone (same counts for every t >= t0).
      uint32_t lmax = 0;
      each_slot([&](int e) { lmax = max(lmax, key(e)); });
      uint32_t t0 = 0;
      for (int bit = 31; bit >= 16; --bit) {
        const uint32_t cand = t0 | (1u << bit);
        if (wave_count(lmax >= cand) >= K) t0 = cand;
      }
      int n0 = 0;
      each_slot([&](int e) { n0 += wave_count(key(e) >= t0); });
      if (n0 <= 64) {
        int nb = 0;
        each_slot([&](int e) {
          const uint32_t kk = key(e);
          const bool in = kk >= t0;
          const uint64_t m = ballot64(in);
          if (in) gath[wv][nb + __popcll(m & lt_mask)] = kk;
          nb += __popcll(m);
        });
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
          each_slot([&](int e) { cnt += wave_count(key(e) >= cand); });
          if (cnt >= K) thr = cand;
        }
      }
      n_ge = 0;
      each_slot([&](int e) { n_ge += wave_count(key(e) >= thr); });
    }
    // selected historical blocks in ascending order into the wave's LDS
    // slots (read back for one contiguous store of the unit's row)
    int base = 0;
    if (all || n_ge == K) {
      // every key at or above the threshold is taken (no tie crosses it)
      each_cand([&](int e) {
        const int j = lane + 64 * e;
        const bool s_in = j < c && (all || key(e) >= thr);
        const uint64_t sm = ballot64(s_in);
        if (s_in) {
          const int pos = base + __popcll(sm & lt_mask);
          selj[wv][pos] = j;
          sell[wv][pos] = score(e) - lse;
        }
        base += __popcll(sm);
      });
    } else {
      // equal keys at the threshold: the lower block indices first
      int gt = 0;
      each_slot([&](int e) { gt += wave_count(key(e) > thr); });
      const int need_eq = K - gt;
      int eq_seen = 0;
      each_cand([&](int e) {
        const int j = lane + 64 * e;
        const bool hist = j < c;
        const uint32_t kk = key(e);
        const bool eq = hist && kk == thr;
        const uint64_t em = ballot64(eq);
        const bool s_in = hist && (kk > thr || (eq && (eq_seen + __popcll(em & lt_mask)) < need_eq));
        eq_seen += __popcll(em);
        const uint64_t sm = ballot64(s_in);
        if (s_in) {
          const int pos = base + __popcll(sm & lt_mask);
          selj[wv][pos] = j;
          sell[wv][pos] = score(e) - lse;
        }
        base += __popcll(sm);
      });
    }
  };
  if constexpr (!LONG)
    select(std::integral_constant<int, kMaxNB / 64>{}, std::true_type{});
  else
    select(std::integral_constant<int, kMaxDecodeNB / 64>{}, std::false_type{});
  // the wave's LDS accesses are performed in order: its slots are complete
  for (int s2 = lane; s2 < S; s2 += 64) {
    if (s2 < nsel) put(s2, selj[wv][s2], sell[wv][s2]);
    else if (s2 == nsel) put(s2, c, sc[c] - lse);
    else put(s2, -1, -INFINITY);
  }
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
__device__ __forceinline__ void merge_splits(const DecodeParams& p, int unit, int b, int sg,
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
    p.o[(static_cast<size_t>(b) * p.Hq + sg * G) * D + e] = f2bf(o * inv_l[h]);
  }
}

// Workgroup = (unit, split of spw selected blocks), 256 threads, walking the
// split in passes of two blocks; in a pass, wave w takes keys 16w .. 16w + 15
// of each of the two blocks (32 keys), so the scores and P V of a wave are
// single MFMA tiles with the G heads padded to 16 columns:
//   S^T[key][h] = K Q^T      A = the wave's 16 keys of one block, loaded from
//                            HBM straight into the operand layout (16 bytes
//                            per lane, 64 contiguous bytes per key and load);
//   O^T[d][h]  += V^T P^T    A = V^T from LDS with transposing reads, B = the
//                            bf16 softmax weights as they sit in S's
//                            accumulator lanes (k slot 8g + i <-> key 4g + i
//                            of the pass's first block for i < 4, of its
//                            second block for i >= 4, on both operands).
// The walk is software-pipelined over two register buffers: the next pass's
// K and V loads (64 KiB per workgroup) are in flight while the current pass
// computes; its V rows go through a per-wave LDS region (no workgroup
// barrier).  The softmax state is carried online across the passes.  Each
// block is read through a buffer resource over its rows below the context
// length (rows 64 j.. of the contiguous cache, or the block's page of a paged
// cache), so keys at or beyond it, slots without a block, pages outside the
// pool and passes past the split's end read zeros and make no memory
// request.  The per-wave (max, sum, O) are
// merged across the 4 waves in LDS, each wave's in place of its own V rows;
// with one split per unit the workgroup writes the normalised output,
// otherwise one partial per split (whole 128-byte lines) for the merge.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeParams p) {
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
  struct PassBuf {
    uint4 k[2][NKS];
    uint4 v[2][NVT];
  };

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int unit = blockIdx.x, split = blockIdx.y;
  const int b = unit / p.Hs, sg = unit - b * p.Hs, kv = sg / p.kdiv;
  const int L = p.ctx_len[b];
  const bool ok = (L >= 1 && L <= p.Lmax);
  const int spw = p.spw, npass = spw / 2;
  const int s0 = split * spw;

  // slot table: lane i < spw holds slot s0 + i (block, log2-domain gate
  // bias, and for a paged cache the block's page, -1 outside the pool)
  int jv = -1, pgv = -1;
  float lv = 0.f;
  if (lane < spw) {
    const int s = s0 + lane;
    const int j = (ok && s < p.S) ? p.ws_idx[static_cast<size_t>(unit) * p.S + s] : -1;
    jv = (j >= 0 && 64 * j < L) ? j : -1;
    lv = (jv >= 0 && p.apply_gate) ? p.ws_logg[static_cast<size_t>(unit) * p.S + s] * kLog2e : 0.f;
    if (p.btab && jv >= 0) {
      const int pg = p.btab[static_cast<size_t>(b) * p.NBmax + jv];
      pgv = (pg >= 0 && pg < p.num_pages) ? pg : -1;
    }
  }
  auto slot_j = [&](int t) { return t < spw ? __builtin_amdgcn_readlane(jv, t) : -1; };
  auto slot_lg = [&](int t) {
    return t < spw ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), t)) : 0.f;
  };

  // Q^T operand: column h = r (zero for r >= G)
  uint4 qb[NKS];
  {
    const int h = min(r, G - 1);
    const uint16_t* qp = p.q + (static_cast<size_t>(b) * p.Hq + sg * G + h) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint4 v = ld16(qp + 32 * ks);
      qb[ks] = (r < G) ? v : make_uint4(0, 0, 0, 0);
    }
  }
  // slot t's block of K (or V) as a buffer resource over its rows below the
  // context length: contiguous cache rows 64 j.., or the block's page; no
  // rows for a slot without a block or a page outside the pool
  const size_t ubase = (static_cast<size_t>(b) * p.Hkv + kv) * p.Lmax * D;
  auto block_rsrc = [&](const uint16_t* cache, int t) {
    const int j = slot_j(t);
    size_t off;
    int rows;
    if (p.btab) {
      const int pg = t < spw ? __builtin_amdgcn_readlane(pgv, t) : -1;
      off = (static_cast<size_t>(max(pg, 0)) * p.Hkv + kv) * 64 * D;
      rows = (j >= 0 && pg >= 0) ? min(64, L - 64 * j) : 0;
    } else {
      off = ubase + static_cast<size_t>(max(j, 0)) * 64 * D;
      rows = j >= 0 ? min(64, L - 64 * j) : 0;
    }
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(cache + off), 0, rows * ROWB,
                                             kBufferWord3);
  };
  // V rows of a pass: wave row 16 u + i = key 16 w + i of block u, lane's
  // 16-byte chunk stored at its swizzled place
  const int vrow = lane / CPR;
  auto issue = [&](PassBuf& pb, int ps) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const __amdgpu_buffer_rsrc_t krs = block_rsrc(p.k_cache, 2 * ps + u);
      const __amdgpu_buffer_rsrc_t vrs = block_rsrc(p.v_cache, 2 * ps + u);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        pb.k[u][ks] = buffer_ld16(krs, (16 * w + r) * ROWB + 64 * ks + 16 * g);
#pragma unroll
      for (int n = 0; n < NVT; ++n) {
        const int rho = 16 * u + RPI * n + vrow;
        const int c = (lane % CPR) ^ lds_swz<ROWB>(rho);
        pb.v[u][n] = buffer_ld16(vrs, (16 * w + RPI * n + vrow) * ROWB + 16 * c);
      }
    }
  };
  unsigned char* vw = vs + w * 32 * ROWB;
  const float sl2 = p.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  floatx4 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  // transposing reads: lane s of group g addresses row 4g + s/4 (of each
  // tile), columns 16 dt + 4 (s % 4) .. +3 and receives column 16 dt + s
  const int rho0 = 4 * g + (r >> 2);
  const int cb = (r & 3) >> 1, hb = 8 * (r & 1);
  auto attend = [&](const PassBuf& pb, int ps) {
    int jt[2];
    float lg[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      jt[u] = slot_j(2 * ps + u);
      lg[u] = slot_lg(2 * ps + u);
    }
    // S^T tiles: lane holds head r, keys 4g .. 4g + 3 of each tile
    floatx4 sacc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sacc[u] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) sacc[u] = mfma16x16x32(pb.k[u][ks], qb[ks], sacc[u]);
    }
    float sv[2][4];
    float mx = m_run;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 64 * jt[u] + 16 * w + 4 * g + i;
        sv[u][i] = (jt[u] >= 0 && tok < L) ? fmaf(sacc[u][i], sl2, lg[u]) : -INFINITY;
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
    const uint4 pbf = make_uint4(pack_bf2(pw[0][0], pw[0][1]), pack_bf2(pw[0][2], pw[0][3]),
                                 pack_bf2(pw[1][0], pw[1][1]), pack_bf2(pw[1][2], pw[1][3]));
    // this pass's rows replace the previous pass's (the wave's LDS accesses
    // complete in order, after its reads of them)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int n = 0; n < NVT; ++n) st16(vw + (16 * u + RPI * n) * ROWB + 16 * lane, pb.v[u][n]);
    // O^T tiles: lane holds head r, d = 16 dt + 4g .. +3
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint2 v0 = lds_read_tr16(vw + rho0 * ROWB + (((2 * dt + cb) ^ lds_swz<ROWB>(rho0)) << 4) + hb);
      const uint2 v1 = lds_read_tr16(vw + (rho0 + 16) * ROWB +
                                     (((2 * dt + cb) ^ lds_swz<ROWB>(rho0 + 16)) << 4) + hb);
      oacc[dt] = mfma16x16x32(make_uint4(v0.x, v0.y, v1.x, v1.y), pbf, oacc[dt] * alpha);
    }
  };
  PassBuf bufa, bufb;
  issue(bufa, 0);
  for (int ps = 0; ps < npass; ps += 2) {
    issue(bufb, ps + 1);          // past the end: no memory request
    attend(bufa, ps);
    issue(bufa, ps + 2);
    if (ps + 1 < npass) attend(bufb, ps + 1);
  }
  wait_vmem_all();
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
  auto wred = [&](int q) -> const WaveRed& { return *reinterpret_cast<const WaveRed*>(vs + q * 32 * ROWB); };
  auto head_ml = [&](int h, float& M, float& l) {
    M = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) M = fmaxf(M, wred(q).m[h]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float mq = wred(q).m[h];
      if (mq != -INFINITY) l += wred(q).l[h] * fast_exp2(mq - M);
    }
  };
  if (p.nsplit == 1) {
    // the unit's output, normalised (NaN for an invalid context length)
    for (int e = tid; e < G * D; e += 256) {
      const int h = e / D, d = e - h * D;
      float M, l;
      head_ml(h, M, l);
      float o = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float mq = wred(q).m[h];
        if (mq != -INFINITY) o += wred(q).o[h][d] * fast_exp2(mq - M);
      }
      const float inv_l = (ok && l > 0.f) ? 1.f / l : __builtin_nanf("");
      p.o[(static_cast<size_t>(b) * p.Hq + sg * G) * D + e] = f2bf(o * inv_l);
    }
    return;
  }
  // the split's partial, written in whole 128-byte lines
  float* part = p.ws_part + (static_cast<size_t>(unit) * p.nsplit + split) * decode_part_floats(G, D);
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
    if (h < G) head_ml(h, M, l);
    part[G * D + tid] = tid < 16 ? M : l;
  }
}

// One workgroup per unit merges the unit's split partials.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
  const int unit = blockIdx.x;
  const int b = unit / p.Hs, sg = unit - b * p.Hs;
  const int L = p.ctx_len[b];
  merge_splits<D, G>(p, unit, b, sg, L >= 1 && L <= p.Lmax);
}

}  // namespace

void decode_split(int S, int units, int* nsplit, int* spw) {
  // about kDecodeWorkgroups workgroups over the chip; a split walks an even
  // number of slots (passes of two blocks)
  const int pairs = (S + 1) / 2;
  const int want = (kDecodeWorkgroups + units - 1) / units;
  const int ns = std::max(1, std::min(pairs, want));
  const int ppw = (pairs + ns - 1) / ns;
  *spw = 2 * ppw;
  *nsplit = (pairs + ppw - 1) / ppw;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t st) {
  const unsigned units = static_cast<unsigned>(p.B) * p.Hs;
  const dim3 sgrid(units, (p.NBmax + 127) / 128);
  auto score = [&](auto dgc) {
    constexpr int DG = decltype(dgc)::value;
    if (p.kg_bf16)
      hipLaunchKernelGGL((decode_score_kernel<DG, true>), sgrid, dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((decode_score_kernel<DG, false>), sgrid, dim3(256), 0, st, p);
  };
  switch (p.dg) {
    case 128: score(std::integral_constant<int, 128>{}); break;
    case 64: score(std::integral_constant<int, 64>{}); break;
    case 32: score(std::integral_constant<int, 32>{}); break;
    default: return hipErrorInvalidValue;
  }
  if (p.NBmax <= kMaxNB)
    hipLaunchKernelGGL((decode_topk_kernel<false>), dim3((units + 3) / 4), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((decode_topk_kernel<true>), dim3((units + 3) / 4), dim3(256), 0, st, p);
  const dim3 agrid(units, p.nsplit);
  auto attend = [&](auto dc, auto gc) {
    constexpr int D = decltype(dc)::value, G = decltype(gc)::value;
    hipLaunchKernelGGL((decode_attn_kernel<D, G>), agrid, dim3(256), 0, st, p);
    if (p.nsplit > 1)
      hipLaunchKernelGGL((decode_merge_kernel<D, G>), dim3(units), dim3(256), 0, st, p);
  };
  auto by_g = [&](auto dc) -> bool {
    switch (p.G) {
      case 1: attend(dc, std::integral_constant<int, 1>{}); return true;
      case 2: attend(dc, std::integral_constant<int, 2>{}); return true;
      case 3: attend(dc, std::integral_constant<int, 3>{}); return true;
      case 4: attend(dc, std::integral_constant<int, 4>{}); return true;
      case 5: attend(dc, std::integral_constant<int, 5>{}); return true;
      case 6: attend(dc, std::integral_constant<int, 6>{}); return true;
      case 7: attend(dc, std::integral_constant<int, 7>{}); return true;
      case 8: attend(dc, std::integral_constant<int, 8>{}); return true;
      default: return false;
    }
  };
  bool launched = false;
  if (p.D == 128) launched = by_g(std::integral_constant<int, 128>{});
  else if (p.D == 64) launched = by_g(std::integral_constant<int, 64>{});
  if (!launched) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sas
