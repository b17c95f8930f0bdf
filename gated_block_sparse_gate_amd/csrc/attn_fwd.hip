// Gated sparse attention forward (SAS abstract: log gate inside the attention
// softmax; README item (b): a continuous gate on every selected block).
//
// o[t,h] = softmax_tau( scale * q[t,h].k[tau] + logg[t, slot(block(tau))] ) . v
// over the keys of the blocks selected for (t, kappa = h/G), tau <= t.
//
// Schedule (query-block stationary):
//   one workgroup = (batch b, KV head kappa, query block c) = 64 tokens x G heads.
//   The workgroup walks the union of the blocks its 64 tokens selected, in
//   ascending order.  Each block's K tile and V^T tile (from a transposed copy
//   of V made once per call, keys in operand order) is staged once into
//   double-buffered LDS (plain 16-byte copies, chunks XOR-swizzled per row so
//   the MFMA operand reads are conflict-free); the next block's loads are in
//   flight in registers while the current one is computed, with one
//   workgroup barrier per block.  A wave owns TW row tiles of 16 rows =
//   floor(16/G) tokens x G heads; a tile in which no token selected the block
//   skips it, otherwise S^T = K Q^T and O^T += V^T P^T run on bf16 MFMA
//   16x16x32 with rows outside the selection masked out.  Online-softmax
//   state stays in registers (one query row per lane column); the running
//   reference maximum is moved only when a row's new maximum exceeds it by
//   more than 2^kLazyLog2, so the output rescale is rare.
#include "sas_kernels.h"

namespace sas {

namespace {

constexpr float kLazyLog2 = 8.f;   // weights stay below 2^8 between rescales

// HILO (the fp32 output is requested, for the backward's Delta): V^T is the
// bf16 copy and P enters PV as bf16 hi + lo parts (exact to ~2^-16).
// Otherwise V^T is the scaled fp16 copy and P enters once, in fp16.
template <int D, int NW, int TW, bool HILO, int R>
__global__ __launch_bounds__(NW * 64) void sparse_fwd_kernel(FwdParams a) {
  constexpr int NT = NW * 64;
  constexpr int KROWB = D * 2;              // bytes per K row
  constexpr int KB = 64 * KROWB;            // K tile bytes
  constexpr int VB = D * 128;               // V^T tile bytes (D rows x 64 keys)
  constexpr int STAGE = KB + VB;
  constexpr int KU = KB / 16;               // 16-byte K units per tile
  constexpr int UPT = STAGE / 16 / NT;      // 16-byte units per thread per block
  constexpr int KCPR = KROWB / 16;          // 16-byte chunks per K row
  constexpr int NKS = D / 32;
  constexpr int NDT = D / 16;
  static_assert(STAGE % (16 * NT) == 0, "unit split");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int NBW = (a.NB + 31) >> 5;
  const int S = a.S;
  const WalkLds L = walk_lds(R, STAGE, a.NB, S, NW, false);
  uint8_t* const ring = smem + L.ring;                      // slot sl at ring + sl * STAGE
  uint32_t* const bits = reinterpret_cast<uint32_t*>(smem + L.bits);   // [64][NBW]
  uint8_t* const pcnt = smem + L.pcnt;                      // [64][NBW]
  uint32_t* const ubits = reinterpret_cast<uint32_t*>(smem + L.ubits);
  uint16_t* const ulist = reinterpret_cast<uint16_t*>(smem + L.ulist);
  float* const lgs = reinterpret_cast<float*>(smem + L.lgs);          // [64][S]
  unsigned* const fill_cnt = reinterpret_cast<unsigned*>(smem + L.cnt);
  unsigned* const done_cnt = fill_cnt + R;
  int* const s_nU = reinterpret_cast<int*>(smem + L.nu);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  const int NQB = (a.T + 63) / 64;
  const int bid = blockIdx.x;
  const int kv = bid % a.Hkv;
  const int rest = bid / a.Hkv;
  const int c = NQB - 1 - (rest % NQB);
  const int b = rest / NQB;
  const int t0 = c * 64;
  const int ntok = min(64, a.T - t0);
  const int Tp = a.NB * 64;

  // ---- selection bitmaps of the 64 tokens, their union, log-gates by rank
  for (int i = tid; i < 64 * NBW; i += NT) bits[i] = 0u;
  if (tid < NBW) ubits[tid] = 0u;
  if (tid < 2 * R) fill_cnt[tid] = 0u;          // fill and done counters
  __syncthreads();
  const size_t rowbase = (static_cast<size_t>(b) * a.T + t0) * a.Hkv + kv;
  for (int e = tid; e < ntok * S; e += NT) {
    const int tl = e / S, s = e - tl * S;
    const int j = a.idx[(rowbase + static_cast<size_t>(tl) * a.Hkv) * S + s];
    if (j >= 0 && j <= c) {
      atomicOr(&bits[tl * NBW + (j >> 5)], 1u << (j & 31));
      atomicOr(&ubits[j >> 5], 1u << (j & 31));
    }
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
    const size_t off = (rowbase + static_cast<size_t>(tl) * a.Hkv) * S + s;
    const int j = a.idx[off];
    if (j >= 0 && j <= c) {
      const uint32_t wbits = bits[tl * NBW + (j >> 5)];
      const int rank = pcnt[tl * NBW + (j >> 5)] + __popc(wbits & ((1u << (j & 31)) - 1u));
      if (rank < S) lgs[tl * S + rank] = a.logg[off] * kLog2e;
    }
  }
  if (wv == 0) {
    int base = 0;
    for (int w0 = 0; w0 < NBW; w0 += 64) {
      const uint32_t word = (w0 + lane < NBW) ? ubits[w0 + lane] : 0u;
      const int cnt = __popc(word);
      const int incl = wave_incl_scan(cnt);
      int pos = base + incl - cnt;
      uint32_t wb = word;
      while (wb) {
        const int bp = __ffs(wb) - 1;
        wb &= wb - 1;
        ulist[pos++] = static_cast<uint16_t>((w0 + lane) * 32 + bp);
      }
      base += __shfl(incl, 63, 64);
    }
    if (lane == 0) *s_nU = base;
  }

  // ---- per-tile query rows: row r = l16 -> token r/G, head r%G
  const int G = a.G, TPT = a.TPT;
  int tl_row[TW];
  bool valid[TW];
  uint4 qa[TW][NKS];
  floatx4 oacc[TW][NDT];
  float m_run[TW], l_run[TW];
#pragma unroll
  for (int ti = 0; ti < TW; ++ti) {
    const int tile = wv + NW * ti;
    const int tl = tile * TPT + l16 / G;
    const int hh = l16 - (l16 / G) * G;
    valid[ti] = (tile < a.ntiles) && (l16 < TPT * G) && (tl < ntok);
    tl_row[ti] = valid[ti] ? tl : 0;
    const uint16_t* qrow =
        a.q + ((static_cast<size_t>(b) * a.T + t0 + tl_row[ti]) * a.Hq + kv * G + hh) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qa[ti][ks] = valid[ti] ? *reinterpret_cast<const uint4*>(qrow + ks * 32 + g4 * 8)
                             : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[ti][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    m_run[ti] = -INFINITY;
    l_run[ti] = 0.f;
  }
  wait_vmem_all();
  __syncthreads();
  const int nU = __builtin_amdgcn_readfirstlane(*s_nU);

  // ---- block staging: the thread's 16-byte units tid + NT*x of a block go
  // global -> registers -> its LDS ring slot (chunks XOR-swizzled per row)
  const uint16_t* kbase = a.k + (static_cast<size_t>(b) * a.T * a.Hkv + kv) * D;
  const uint16_t* vtbase =
      a.vt + (static_cast<size_t>(b) * a.Hkv + kv) * D * static_cast<size_t>(Tp);
  uint4 stg[UPT];
  auto gload = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
      const int u = tid + NT * x;
      if (u < KU) {
        const int r = u / KCPR, ch = u - r * KCPR;
        const int tok = min(j * 64 + r, a.T - 1);
        stg[x] = ld16(kbase + (tok * a.Hkv * D + ch * 8));   // < 2^31 within a batch
      } else {
        const int v = u - KU;
        const int d = v >> 3, kc = v & 7;
        stg[x] = ld16(vtbase + static_cast<size_t>(d) * Tp + j * 64 + kc * 8);
      }
    }
  };
  // LDS store offsets of this thread's units (loop-invariant): 16-byte-chunk
  // XOR swizzles for K rows (lds_swz) and V^T rows (tr_swz).
  int soff[UPT];
#pragma unroll
  for (int x = 0; x < UPT; ++x) {
    const int u = tid + NT * x;
    if (u < KU) {
      const int r = u / KCPR, ch = u - r * KCPR;
      soff[x] = r * KROWB + ((ch ^ lds_swz<KROWB>(r)) << 4);
    } else {
      const int v = u - KU;
      const int d = v >> 3, kc = v & 7;
      soff[x] = KB + d * 128 + ((kc ^ tr_swz(d)) << 4);
    }
  }
  // The wave's share of block `nxt` sits in stg; it is written to its slot as
  // soon as every wave is done with the slot's previous block, and the share
  // of the following block is fetched right after.
  int nxt = 0;
  if (nU > 0) gload(ulist[0]);
  auto try_write = [&]() __attribute__((always_inline)) {
    if (nxt < nU) {
      const int sl = nxt % R;
      if (ring_count(&done_cnt[sl]) >= static_cast<unsigned>(NW * (nxt / R))) {
        uint8_t* dst = ring + sl * STAGE;
#pragma unroll
        for (int x = 0; x < UPT; ++x) st16(dst + soff[x], stg[x]);
        ring_bump(&fill_cnt[sl], lane);
        ++nxt;
        if (nxt < nU) gload(ulist[nxt]);
      }
    }
  };

  // per-lane LDS read offsets of the MFMA operands (immediate offsets add
  // the 16-key / 16-d tile steps)
  int kofs[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    kofs[ks] = l16 * KROWB + (((ks * 4 + g4) ^ lds_swz<KROWB>(l16)) << 4);
  int vofs[2];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) vofs[k2] = KB + l16 * 128 + (((k2 * 4 + g4) ^ tr_swz(l16)) << 4);

  const float sl2 = a.scale_log2;
  bool failed = false;
  for (int u = 0; u < nU; ++u) {
    const int sl = u % R;
    try_write();
    const unsigned need = static_cast<unsigned>(NW * (u / R + 1));
    for (int it = 0; ring_count(&fill_cnt[sl]) < need; ++it) {
      if (it == kSpinLimit) {
        failed = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      try_write();
    }
    if (failed) {
      ring_fault(lane);
      break;
    }
    const uint8_t* st = ring + sl * STAGE;
    const int j = ulist[u];
    const uint32_t jbit = 1u << (j & 31);
    const int jw = j >> 5;
    const bool cur = (j == c);
    bool sel[TW];
    bool act[TW];
#pragma unroll
    for (int ti = 0; ti < TW; ++ti) {
      sel[ti] = valid[ti] && (bits[tl_row[ti] * NBW + jw] & jbit);
      act[ti] = ballot64(sel[ti]) != 0;
    }
#pragma unroll
    for (int ti = 0; ti < TW; ++ti) {
      if (!act[ti]) continue;
      const int tl = tl_row[ti];
      float lgv = 0.f;
      if (sel[ti]) {
        const int rank = pcnt[tl * NBW + jw] + __popc(bits[tl * NBW + jw] & (jbit - 1u));
        lgv = lgs[tl * S + rank];
      }
      // S^T[key, row] = K[key,:] . Q[row,:]
      floatx4 sacc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        sacc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const uint4 ka = *reinterpret_cast<const uint4*>(st + mt * 16 * KROWB + kofs[ks]);
          sacc[mt] = mfma16x16x32(ka, qa[ti][ks], sacc[mt]);
        }
      }
      // maximum of this lane's raw scores over the keys its row may see (the
      // row's 64 keys are spread over the 4 lanes g4 of the row)
      const int lim = t0 + tl - j * 64 - g4 * 4;     // current block: key offset limit
      float mr = -INFINITY;
      if (cur) {
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
      const float cand_l = sel[ti] ? mr * sl2 + lgv : -INFINITY;
      if (ballot64(cand_l > m_run[ti] + kLazyLog2)) {
        const float cand = row4_max(cand_l);
        const bool up = cand > m_run[ti] + kLazyLog2;
        const float alpha = up ? fast_exp2(m_run[ti] - cand) : 1.f;
        m_run[ti] = up ? cand : m_run[ti];
        l_run[ti] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[ti][dt] *= alpha;
      }
      const float bias = sel[ti] ? lgv - m_run[ti] : -INFINITY;
      float x[4][4];
      if (cur) {
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
      const float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
      l_run[ti] += psum;
      // a block's compute is long: hand over this wave's next share now, so
      // that the other waves do not wait for its end
      try_write();
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
      // O^T[d, row] += V^T[d, keys] . P^T[keys, row]; inside a 32-key step the
      // lane's 8 keys are {4g..4g+3, 16+4g..16+4g+3}, stored contiguously in
      // the transposed copy.
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const uint4 va = *reinterpret_cast<const uint4*>(st + dt * 2048 + vofs[k2]);
          if (HILO) {
            oacc[ti][dt] = mfma16x16x32(va, pb[k2], oacc[ti][dt]);
            oacc[ti][dt] = mfma16x16x32(va, pl[k2], oacc[ti][dt]);
          } else {
            oacc[ti][dt] = mfma16x16x32h(va, pb[k2], oacc[ti][dt]);
          }
        }
      }
    }
    ring_bump(&done_cnt[sl], lane);
  }
  if (failed) {
#pragma unroll
    for (int ti = 0; ti < TW; ++ti) l_run[ti] = NAN;
  }

  // ---- epilogue
  const float vsc = HILO ? 1.f : a.vscale[static_cast<size_t>(b) * a.Hkv + kv];
#pragma unroll
  for (int ti = 0; ti < TW; ++ti) {
    if (!valid[ti]) continue;
    const float lsum = row4_sum(l_run[ti]);
    const int tl = tl_row[ti];
    const int hh = l16 - (l16 / G) * G;
    const size_t row = (static_cast<size_t>(b) * a.T + t0 + tl) * a.Hq + kv * G + hh;
    const float inv = (lsum > 0.f) ? vsc / lsum : 0.f;   // vsc undoes the V^T scaling
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint2 pk;
      pk.x = pack_bf2(oacc[ti][dt][0] * inv, oacc[ti][dt][1] * inv);
      pk.y = pack_bf2(oacc[ti][dt][2] * inv, oacc[ti][dt][3] * inv);
      *reinterpret_cast<uint2*>(a.o + row * D + dt * 16 + g4 * 4) = pk;
      if (a.o32)
        *reinterpret_cast<float4*>(a.o32 + row * D + dt * 16 + g4 * 4) =
            make_float4(oacc[ti][dt][0] * inv, oacc[ti][dt][1] * inv, oacc[ti][dt][2] * inv,
                        oacc[ti][dt][3] * inv);
    }
    if (g4 == 0)
      a.lse[row] = (lsum > 0.f) ? (m_run[ti] + log2f(lsum)) * kLn2 : -INFINITY;
  }
}

// Launch with the deepest LDS ring (4 or 3 slots) whose layout fits.
template <int D, int NW, int TW, bool HILO>
hipError_t launch_fwd_ring(const FwdParams& p, dim3 grid, hipStream_t st) {
  constexpr int STAGE = 256 * D;     // K tile + V^T tile
  const WalkLds L4 = walk_lds(4, STAGE, p.NB, p.S, NW, false);
  const WalkLds L3 = walk_lds(3, STAGE, p.NB, p.S, NW, false);
  if (L4.total <= kLdsBytes) {
    auto k = sparse_fwd_kernel<D, NW, TW, HILO, 4>;
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize, L4.total);
    hipLaunchKernelGGL(k, grid, dim3(NW * 64), L4.total, st, p);
  } else if (L3.total <= kLdsBytes) {
    auto k = sparse_fwd_kernel<D, NW, TW, HILO, 3>;
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize, L3.total);
    hipLaunchKernelGGL(k, grid, dim3(NW * 64), L3.total, st, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, bool HILO>
hipError_t launch_fwd_dh(const FwdParams& p, hipStream_t st) {
  const int NQB = (p.T + 63) / 64;
  const dim3 grid(static_cast<unsigned>(p.B) * p.Hkv * NQB);
  // up to 16 row tiles: one tile per wave, 16 waves (4 per SIMD hide the
  // latency of the per-tile MFMA -> softmax -> MFMA chain); more tiles
  // (G >= 5): 8 waves with TW tiles each.
  if (p.ntiles <= 16) return launch_fwd_ring<D, 16, 1, HILO>(p, grid, st);
  switch ((p.ntiles + 7) / 8) {
    case 3: return launch_fwd_ring<D, 8, 3, HILO>(p, grid, st);
    case 4: return launch_fwd_ring<D, 8, 4, HILO>(p, grid, st);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_fwd_d(const FwdParams& p, hipStream_t st) {
  return p.o32 ? launch_fwd_dh<D, true>(p, st) : launch_fwd_dh<D, false>(p, st);
}

}  // namespace

hipError_t launch_sparse_fwd(const FwdParams& p, hipStream_t st) {
  timing_mark(0, st);
  // V^T: bf16 for the hi/lo product (fp32 output requested), else scaled fp16
  hipError_t e = p.o32 ? launch_transpose_tokens(p.v, p.vt, p.B, p.T, p.Hkv, p.D, st)
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
