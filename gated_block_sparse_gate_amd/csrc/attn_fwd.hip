// Gated sparse attention forward (SAS abstract: log gate inside the attention
// softmax; README item (b): a continuous gate on every selected block).
//
// o[t,h] = softmax_tau( scale * q[t,h].k[tau] + logg[t, slot(block(tau))] ) . v
// over the keys of the blocks selected for (t, kappa = h/G), tau <= t.
//
// Schedule (query-group stationary):
//   one workgroup = (batch b, selection head sg, a group of TPW <= 64
//   consecutive tokens): NCW compute waves, each owning one row tile of 16
//   rows = TPT tokens x Gs heads (the Gs query heads that share sg's
//   selection: the G heads of a KV head, or one head when every query head
//   has its own gate), plus two stager waves.  The stagers copy the K tile and
//   the V^T tile (from a transposed copy of V made once per call, keys in
//   operand order) of every block in the union of the group's selections, in
//   the order walk_order.hip makes for the group, into LDS ring slots
//   with asynchronous global -> LDS copies (16-byte chunks XOR-swizzled per
//   row, so that the MFMA operand reads are conflict-free).  A compute wave visits only the blocks its tile
//   needs: S^T = K Q^T and O^T += V^T P^T on MFMA 16x16x32, with rows outside
//   the selection masked out.  Online-softmax state stays in registers (one
//   query row per lane column); the running reference maximum is moved only
//   when a row's new maximum exceeds it by more than 2^kLazyLog2, so the
//   output rescale is rare.  K and V^T travel in two rings of LDS slots, with the
//   dQ kernel's protocol each (progress words of the compute waves, fill
//   counters of the stager, no workgroup barrier; see attn_bwd.hip): a wave
//   releases a block's K slot right after its S^T reads, so the K stager
//   waits only on the waves' score steps and runs ahead of the P.V steps.
#include "sas_kernels.h"

namespace sas {

namespace {

constexpr float kLazyLog2 = 8.f;   // weights stay below 2^8 between rescales
constexpr int kFwdStagers = 2;     // stager 0 copies K tiles, stager 1 V^T tiles
constexpr int kFwdInflight = 1;    // blocks in flight per stager (< ring depth): each is published as soon as it lands
constexpr int kFwdRingK = 4;       // ring depths (K tiles, V^T tiles): 128 KiB of LDS at D = 128
constexpr int kFwdRingV = 4;

// HILO (the fp32 output is requested, for the backward's Delta): V^T is the
// bf16 copy and P enters PV as bf16 hi + lo parts (exact to ~2^-16).
// Otherwise V^T is the scaled fp16 copy and P enters once, in fp16.
template <int D, bool HILO, int RK, int RV>
__global__ __launch_bounds__(1024) void sparse_fwd_kernel(FwdParams a, int ncw, int tpw) {
  constexpr int KROWB = D * 2;              // bytes per K row
  constexpr int KB = 64 * KROWB;            // K tile bytes
  constexpr int VB = D * 128;               // V^T tile bytes (D rows x 64 keys)
  constexpr int RMAX = RK > RV ? RK : RV;
  constexpr int KU = KB / 16;               // 16-byte units per tile
  constexpr int MPS = KU / 64;              // copies per stager per block
  constexpr int KCPR = KROWB / 16;          // 16-byte chunks per K row
  constexpr int NKS = D / 32;
  constexpr int NDT = D / 16;
  static_assert(KB == VB && KU % 64 == 0, "one tile per stager");
  static_assert(RK > kFwdInflight && RV > kFwdInflight, "ring depth");

  __shared__ __attribute__((aligned(16))) uint8_t ring[RK * KB + RV * VB];   // K ring, then V^T ring
  __shared__ uint32_t bits[64 * kMaxNBW];     // per-token selection bitmaps [64][NBW]
  __shared__ uint8_t pcnt[64 * kMaxNBW];      // popcount prefix per word
  __shared__ uint16_t ulist[kMaxNB];          // union blocks in staging order
  __shared__ float lgs[64 * kMaxS];           // log2 gates by selection rank [64][S]
  __shared__ uint32_t actw[14 * kMaxNBW];     // per compute wave: which union blocks it needs
  __shared__ int prog[kFwdStagers][16];        // per ring: each compute wave's next block
  __shared__ unsigned fill_cnt[kFwdStagers][RMAX];
  __shared__ int s_nU;

  const int tid = threadIdx.x;
  const int NT = blockDim.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int NBW = (a.NB + 31) >> 5;
  const int S = a.S;
  const int Tp = a.NB * 64;

  const int ngrp = (a.T + tpw - 1) / tpw;
  const int bid = blockIdx.x;
  const int sg = bid % a.Hs;             // selection head
  const int kv = sg / a.kdiv;            // its KV head
  const int rest = bid / a.Hs;
  const int grp = ngrp - 1 - (rest % ngrp);   // late (long) groups first
  const int b = rest / ngrp;
  const int t0 = grp * tpw;
  const int ntok = min(tpw, a.T - t0);

  // ---- selection bitmaps of the group's tokens, their union, log-gates by rank
  for (int i = tid; i < 64 * NBW; i += NT) bits[i] = 0u;
  if (tid < kFwdStagers * 16) prog[tid >> 4][tid & 15] = 0;
  if (tid < kFwdStagers * RMAX) fill_cnt[tid / RMAX][tid % RMAX] = 0u;
  __syncthreads();
  const size_t rowbase = (static_cast<size_t>(b) * a.T + t0) * a.Hs + sg;
  for (int e = tid; e < ntok * S; e += NT) {
    const int tl = e / S, s = e - tl * S;
    const int j = a.idx[(rowbase + static_cast<size_t>(tl) * a.Hs) * S + s];
    if (j >= 0 && j <= (t0 + tl) / 64) atomicOr(&bits[tl * NBW + (j >> 5)], 1u << (j & 31));
  }
  __syncthreads();
  if (tid < 64) {
    int run = 0;
    for (int w = 0; w < NBW; ++w) {
      pcnt[tid * NBW + w] = static_cast<uint8_t>(run);
      run += __popc(bits[tid * NBW + w]);
    }
  }
  __syncthreads();
  for (int e = tid; e < ntok * S; e += NT) {
    const int tl = e / S, s = e - tl * S;
    const size_t off = (rowbase + static_cast<size_t>(tl) * a.Hs) * S + s;
    const int j = a.idx[off];
    if (j >= 0 && j <= (t0 + tl) / 64) {
      const uint32_t wbits = bits[tl * NBW + (j >> 5)];
      const int rank = pcnt[tl * NBW + (j >> 5)] + __popc(wbits & ((1u << (j & 31)) - 1u));
      if (rank < S) lgs[tl * S + rank] = a.logg[off] * kLog2e;
    }
  }
  // the union of the group's selections in the staging order that spreads
  // each compute wave's blocks over the ring windows (walk_order.hip)
  {
    const uint16_t* ord =
        a.order + ((static_cast<size_t>(b) * a.Hs + sg) * ngrp + grp) * static_cast<size_t>(a.ost);
    const int n = min(static_cast<int>(ord[0]), a.NB);    // in range whatever it holds
    for (int i = tid; i < n; i += NT) ulist[i] = static_cast<uint16_t>(min(static_cast<int>(ord[1 + i]), a.NB - 1));
    if (tid == 0) s_nU = n;
  }
  wait_vmem_all();
  __syncthreads();
  const int nU = __builtin_amdgcn_readfirstlane(s_nU);

  if (wv >= ncw) {
    // ================================================================ stager
    // LDS unit p (16 bytes) of a K slot holds chunk (p % KCPR) ^ lds_swz(r)
    // of K row r = p / KCPR; unit p of a V^T slot holds chunk (p % 8) ^
    // tr_swz(d) of V^T row d = p / 8; lane i of copy m fetches unit 64 m + i
    // of its stager's tile.
    // the copies are what the compute waves wait on: issue them first
    __builtin_amdgcn_s_setprio(3);
    const int stg = wv - ncw;           // the ring it fills (0: K, 1: V^T)
    const int* sprog = prog[stg];
    unsigned* sfill = fill_cnt[stg];
    const int Rs = stg == 0 ? RK : RV;   // its ring's depth
    auto slot_of = [&](int n) __attribute__((always_inline)) { return stg == 0 ? n % RK : n % RV; };
    const uint16_t* kbase = a.k + (static_cast<size_t>(b) * a.T * a.Hkv + kv) * D;
    const uint16_t* vtbase =
        a.vt + (static_cast<size_t>(b) * a.Hkv + kv) * D * static_cast<size_t>(Tp);
    const int tokstride = a.Hkv * D;       // offsets inside one batch's K fit 32 bits
    int grow[MPS], goff[MPS];
#pragma unroll
    for (int m = 0; m < MPS; ++m) {
      const int pu = m * 64 + lane;
      if (stg == 0) {
        grow[m] = pu / KCPR;
        goff[m] = ((pu % KCPR) ^ lds_swz<KROWB>(grow[m])) * 8;
      } else {
        const int d = pu >> 3;
        grow[m] = 0;
        goff[m] = d * Tp + ((pu & 7) ^ tr_swz(d)) * 8;       // < 2^31 (D * Tp)
      }
    }
    auto min_prog = [&]() __attribute__((always_inline)) {
      asm volatile("" ::: "memory");
      int v = l16 < ncw ? sprog[l16] : 0x7fffffff;
      asm volatile("" ::: "memory");
      v = min(v, __float_as_int(dpp_mov<0xB1>(__int_as_float(v))));
      v = min(v, __float_as_int(dpp_mov<0x4E>(__int_as_float(v))));
      v = min(v, __float_as_int(dpp_mov<0x141>(__int_as_float(v))));
      v = min(v, __float_as_int(dpp_mov<0x140>(__int_as_float(v))));
      return __builtin_amdgcn_readfirstlane(v);
    };
    int oldest = 0;                  // oldest block copied but not published
    bool failed = false;
    for (int n = 0; n < nU && !failed; ++n) {
      if (min_prog() < n - Rs + 1) {
        // publish everything in flight, then wait for the slot
        wait_vmem_all();
        asm volatile("" ::: "memory");
        for (; oldest < n; ++oldest) ring_bump(&sfill[slot_of(oldest)], lane);
        for (int it = 0; min_prog() < n - Rs + 1; ++it) {
          if (it == kSpinLimit) {
            failed = true;
            break;
          }
          __builtin_amdgcn_s_sleep(kStagerNap);
        }
        if (failed) break;
      }
      const int j = ulist[n];
      uint8_t* dst = stg == 0 ? ring + slot_of(n) * KB : ring + RK * KB + slot_of(n) * VB;
      if (stg == 0) {
#pragma unroll
        for (int m = 0; m < MPS; ++m)
          load_lds16(kbase + (min(j * 64 + grow[m], a.T - 1) * tokstride + goff[m]), dst + m * 1024);
      } else {
#pragma unroll
        for (int m = 0; m < MPS; ++m) load_lds16(vtbase + (goff[m] + j * 64), dst + m * 1024);
      }
      if (n - oldest + 1 == kFwdInflight) {
        // the oldest block's copies are older than the (kFwdInflight - 1)
        // newer blocks' copies: wait for them, then publish it
        constexpr int kNewer = (kFwdInflight - 1) * MPS;
        static_assert(kNewer < 64, "vmcnt immediate");
        __builtin_amdgcn_s_waitcnt(0x0f70 | (kNewer & 15) | ((kNewer >> 4) << 14));
        asm volatile("" ::: "memory");
        ring_bump(&sfill[slot_of(oldest)], lane);
        ++oldest;
      }
    }
    wait_vmem_all();       // no copy may still be landing when the workgroup ends
    asm volatile("" ::: "memory");
    if (failed) {
      ring_fault(lane);
    } else {
      for (; oldest < nU; ++oldest) ring_bump(&sfill[slot_of(oldest)], lane);
    }
    return;
  }

  // ================================================================ compute
  // row r = l16 of the wave's tile -> token r / G, head r % G
  const int G = a.Gs, TPT = a.TPT;       // query heads per token row group
  const int tile = wv;
  const int tl = min(tile * TPT + l16 / G, 63);
  const int hh = l16 - (l16 / G) * G;
  const bool valid = (l16 < TPT * G) && (tile * TPT + l16 / G < ntok);
  uint4 qa[NKS];
  floatx4 oacc[NDT];
  float m_run = -INFINITY, l_run = 0.f;
  {
    const uint16_t* qrow =
        a.q + ((static_cast<size_t>(b) * a.T + t0 + tl) * a.Hq + sg * G + hh) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qa[ks] = valid ? *reinterpret_cast<const uint4*>(qrow + ks * 32 + g4 * 8)
                     : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // activity of the tile for every union block: bit v of actw[wv] = some
  // token of the tile selected block ulist[v]
  for (int v0 = 0; v0 < nU; v0 += 64) {
    const int v = v0 + lane;
    bool any = false;
    if (v < nU) {
      const int j = ulist[v];
      for (int k = 0; k < TPT; ++k) {
        const int tk = tile * TPT + k;
        if (tk < ntok) any = any || ((bits[tk * NBW + (j >> 5)] >> (j & 31)) & 1u);
      }
    }
    const uint64_t m = ballot64(any);
    if (lane == 0) {
      actw[wv * NBW + (v0 >> 5)] = static_cast<uint32_t>(m);
      if ((v0 >> 5) + 1 < NBW) actw[wv * NBW + (v0 >> 5) + 1] = static_cast<uint32_t>(m >> 32);
    }
  }
  auto next_active = [&](int v) __attribute__((always_inline)) {
    while (v < nU) {
      const uint32_t w = __builtin_amdgcn_readfirstlane(actw[wv * NBW + (v >> 5)]) >> (v & 31);
      if (w) return min(v + static_cast<int>(__builtin_ctz(w)), nU);
      v = (v | 31) + 1;
    }
    return nU;
  };

  // per-lane LDS read offsets of the MFMA operands (immediate offsets add
  // the 16-key / 16-d tile steps)
  int kofs[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    kofs[ks] = l16 * KROWB + (((ks * 4 + g4) ^ lds_swz<KROWB>(l16)) << 4);
  int vofs[2];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) vofs[k2] = l16 * 128 + (((k2 * 4 + g4) ^ tr_swz(l16)) << 4);

  const float sl2 = a.scale_log2;
  const int cfirst = t0 / 64;            // earliest current block of the group's tokens
  // wait until ring r's slot holds block u; false if the wait gave up
  auto wait_slot = [&](int r, int u) __attribute__((always_inline)) {
    const int Rr = r == 0 ? RK : RV;
    const unsigned need = static_cast<unsigned>(u / Rr + 1);
    for (int it = 0; ring_count(&fill_cnt[r][u % Rr]) < need; ++it) {
      if (it == kSpinLimit) return false;
      __builtin_amdgcn_s_sleep(kComputeNap);
    }
    return true;
  };
  // the block of union position u, whether this lane's row selected it, and
  // the row's log2 gate for it (looked up one visit ahead, so that the LDS
  // round trips overlap the current visit's MFMA work)
  struct Visit {
    int j;
    bool sel;
    float lgv;
  };
  auto look = [&](int u) __attribute__((always_inline)) {
    Visit r{0, false, 0.f};
    if (u < nU) {
      r.j = ulist[u];
      const uint32_t jbit = 1u << (r.j & 31);
      const int jw = r.j >> 5;
      const uint32_t w = bits[tl * NBW + jw];
      r.sel = valid && (w & jbit);
      if (r.sel) r.lgv = lgs[tl * S + pcnt[tl * NBW + jw] + __popc(w & (jbit - 1u))];
    }
    return r;
  };
  int v = next_active(0);
  asm volatile("" ::: "memory");
  if (lane == 0) {                       // done with every block before its first needed one
    prog[0][wv] = v;
    prog[1][wv] = v;
  }
  Visit cur = look(v);
  bool failed = false;
  while (v < nU) {
    if (!wait_slot(0, v)) {
      failed = true;
      break;
    }
    const uint8_t* stk = ring + (v % RK) * KB;
    const uint8_t* stv = ring + RK * KB + (v % RV) * VB;
    const int j = cur.j;
    const bool sel = cur.sel;
    const bool maybe_cur = j >= cfirst;  // the current block of some token of the group
    const float lgv = cur.lgv;
    // S^T[key, row] = K[key,:] . Q[row,:]
    floatx4 sacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      sacc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint4 ka = *reinterpret_cast<const uint4*>(stk + mt * 16 * KROWB + kofs[ks]);
        sacc[mt] = mfma16x16x32(ka, qa[ks], sacc[mt]);
      }
    }
    const int vnext = next_active(v + 1);
    asm volatile("" ::: "memory");
    if (lane == 0) prog[0][wv] = vnext;  // after this wave's last K read of the slot
    asm volatile("" ::: "memory");
    const Visit nxt = look(vnext);
    // maximum of this lane's raw scores over the keys its row may see (the
    // row's 64 keys are spread over the 4 lanes g4 of the row); in the
    // current block the row sees keys 0 .. t - 64 j
    const int lim = t0 + tl - j * 64 - g4 * 4;
    float mr = -INFINITY;
    if (maybe_cur) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (mt * 16 + i <= lim) mr = fmaxf(mr, sacc[mt][i]);
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        mr = fmaxf(mr, fmaxf(fmaxf(sacc[mt][0], sacc[mt][1]), fmaxf(sacc[mt][2], sacc[mt][3])));
    }
    // A row's reference moves only if its maximum passes it by 2^kLazyLog2,
    // i.e. if one of its lanes does; only then are the 4 lanes' maxima
    // combined (rare), so the common path needs no cross-lane step.
    const float cand_l = sel ? mr * sl2 + lgv : -INFINITY;
    if (ballot64(cand_l > m_run + kLazyLog2)) {
      const float cand = row4_max(cand_l);
      const bool up = cand > m_run + kLazyLog2;
      const float alpha = up ? fast_exp2(m_run - cand) : 1.f;
      m_run = up ? cand : m_run;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
    }
    const float bias = sel ? lgv - m_run : -INFINITY;
    float x[4][4];
    if (maybe_cur) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(fmaf(sacc[mt][i], sl2, bias));
          x[mt][i] = (mt * 16 + i <= lim) ? e : 0.f;
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[mt][i] = fast_exp2(fmaf(sacc[mt][i], sl2, bias));
    }
    // pairwise sum (short dependency chain)
    float ps[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) ps[mt] = (x[mt][0] + x[mt][1]) + (x[mt][2] + x[mt][3]);
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    uint4 pb[2], pl[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      if (HILO) {
        split_bf2(x[2 * k2][0], x[2 * k2][1], pb[k2].x, pl[k2].x);
        split_bf2(x[2 * k2][2], x[2 * k2][3], pb[k2].y, pl[k2].y);
        split_bf2(x[2 * k2 + 1][0], x[2 * k2 + 1][1], pb[k2].z, pl[k2].z);
        split_bf2(x[2 * k2 + 1][2], x[2 * k2 + 1][3], pb[k2].w, pl[k2].w);
      } else {
        // fp16 (P <= 2^kLazyLog2, 11-bit significand) against the fp16 V^T
        pb[k2].x = pack_h2(x[2 * k2][0], x[2 * k2][1]);
        pb[k2].y = pack_h2(x[2 * k2][2], x[2 * k2][3]);
        pb[k2].z = pack_h2(x[2 * k2 + 1][0], x[2 * k2 + 1][1]);
        pb[k2].w = pack_h2(x[2 * k2 + 1][2], x[2 * k2 + 1][3]);
      }
    }
    if (!wait_slot(1, v)) {
      failed = true;
      break;
    }
    // O^T[d, row] += V^T[d, keys] . P^T[keys, row]; inside a 32-key step the
    // lane's 8 keys are {4g..4g+3, 16+4g..16+4g+3}, stored contiguously in
    // the transposed copy.
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const uint4 va = *reinterpret_cast<const uint4*>(stv + dt * 2048 + vofs[k2]);
        if (HILO) {
          oacc[dt] = mfma16x16x32(va, pb[k2], oacc[dt]);
          oacc[dt] = mfma16x16x32(va, pl[k2], oacc[dt]);
        } else {
          oacc[dt] = mfma16x16x32h(va, pb[k2], oacc[dt]);
        }
      }
    }
    v = vnext;
    cur = nxt;
    asm volatile("" ::: "memory");
    if (lane == 0) prog[1][wv] = v;      // after this wave's last V^T read of the slot
    asm volatile("" ::: "memory");
  }
  if (failed) {
    ring_fault(lane);
    l_run = NAN;
    asm volatile("" ::: "memory");
    if (lane == 0) {                     // let the stagers finish
      prog[0][wv] = nU;
      prog[1][wv] = nU;
    }
  }

  // ---- epilogue
  const float vsc = HILO ? 1.f : a.vscale[static_cast<size_t>(b) * a.Hkv + kv];
  if (valid) {
    const float lsum = row4_sum(l_run);
    const size_t row = (static_cast<size_t>(b) * a.T + t0 + tl) * a.Hq + sg * G + hh;
    const float inv = (lsum > 0.f) ? vsc / lsum : 0.f;   // vsc undoes the V^T scaling
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint2 pk;
      pk.x = pack_bf2(oacc[dt][0] * inv, oacc[dt][1] * inv);
      pk.y = pack_bf2(oacc[dt][2] * inv, oacc[dt][3] * inv);
      *reinterpret_cast<uint2*>(a.o + row * D + dt * 16 + g4 * 4) = pk;
      if (a.o32)
        *reinterpret_cast<float4*>(a.o32 + row * D + dt * 16 + g4 * 4) =
            make_float4(oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv,
                        oacc[dt][3] * inv);
    }
    if (g4 == 0) a.lse[row] = (lsum > 0.f) ? (m_run + log2f(lsum)) * kLn2 : -INFINITY;
  }
}

// Tokens per workgroup: 14 compute waves of TPT tokens each, at most 64;
// static LDS: the K and V^T rings plus the selection data.
template <int D, bool HILO>
hipError_t launch_fwd_dh(const FwdParams& p, hipStream_t st) {
  const int tpw = walk_tpw(p.TPT);
  const int ncw = walk_ncw(p.TPT);
  const unsigned ngrp = (p.T + tpw - 1) / tpw;
  const dim3 grid(static_cast<unsigned>(p.B) * p.Hs * ngrp);
  hipLaunchKernelGGL((sparse_fwd_kernel<D, HILO, kFwdRingK, kFwdRingV>), grid, dim3((ncw + kFwdStagers) * 64), 0, st,
                     p, ncw, tpw);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_d(const FwdParams& p, hipStream_t st) {
  return p.o32 ? launch_fwd_dh<D, true>(p, st) : launch_fwd_dh<D, false>(p, st);
}

}  // namespace

hipError_t launch_sparse_fwd(const FwdParams& p, hipStream_t st) {
  timing_mark(0, st);
  WalkOrderParams wo{p.idx, p.order, p.B, p.T, p.Hs, p.S, p.NB, p.TPT, p.ost};
  hipError_t e = launch_walk_order(wo, st);
  if (e != hipSuccess) return e;
  // V^T: bf16 for the hi/lo product (fp32 output requested), else scaled fp16
  e = p.o32 ? launch_transpose_tokens(p.v, p.vt, p.B, p.T, p.Hkv, p.D, st)
                       : launch_transpose_tokens_f16(p.v, p.vt, p.vamax, p.vscale, p.B, p.T,
                                                     p.Hkv, p.D, st);
  if (e != hipSuccess) return e;
  timing_mark(1, st);
  e = p.D == 128 ? launch_fwd_d<128>(p, st) : p.D == 64 ? launch_fwd_d<64>(p, st)
                                                         : hipErrorInvalidValue;
  timing_mark(2, st);
  return e;
}

hipError_t take_ring_fault_fwd(unsigned* out) {
  unsigned v = 0;
  hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_ring_fault), sizeof(v));
  if (e == hipSuccess && v != 0) {
    const unsigned zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_ring_fault), &zero, sizeof(zero));
  }
  *out |= v;
  return e;
}

}  // namespace sas
