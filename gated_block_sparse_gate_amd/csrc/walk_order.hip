// Staging order of the query-group walks (forward and dQ).
//
// Both kernels stage the blocks in the union of a token group's selections
// through an LDS ring of a few slots shared by 14 compute waves; a slot is
// refilled only when every wave is past the block it holds.  In ascending
// block order a wave often needs several blocks of one ring window while
// others need none, and the whole workgroup then waits for it.  The order
// made here spreads each wave's blocks over the sequence of windows.  Any
// order gives the same attention (the online softmax and the dQ sum take the
// blocks in any order); a fixed one keeps the results deterministic.
//
// One wave per token group (b, selection head, group of tpw tokens, the
// grouping of the walks):
//  1. per compute tile w (TPT consecutive tokens), the bitmap of the blocks
//     some token of the tile selected; their union, in ascending order, with
//     mask[p] = the set of tiles that need union block p;
//  2. placement: the candidates are the first 64 union blocks not yet placed
//     (one per lane); a candidate ranks by the load of its busiest tile in
//     the window of the last kWin - 1 placed blocks, then by the number of
//     tiles that need it (more first), then by position.  Each step places
//     the best candidate and then, ranked on the same window, the best one
//     whose tiles are disjoint from the first's (its rank is unchanged by
//     the first), so the serial chain has half as many steps; the next
//     unplaced blocks take their lanes.
// Output per group (stride ost uint16): [nU, block of position 0, ...].
#include "sas_kernels.h"

namespace sas {

namespace {

constexpr int kWin = 4;     // ring window the placement balances (the forward's ring depth)

// minimum over the wave: within each 16-lane row by DPP, then the four rows
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, __float_as_uint(dpp_mov<0xB1>(__uint_as_float(v))));    // quad_perm [1,0,3,2]
  v = min(v, __float_as_uint(dpp_mov<0x4E>(__uint_as_float(v))));    // quad_perm [2,3,0,1]
  v = min(v, __float_as_uint(dpp_mov<0x141>(__uint_as_float(v))));   // row_half_mirror
  v = min(v, __float_as_uint(dpp_mov<0x140>(__uint_as_float(v))));   // row_mirror
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return min(min(r0, r1), min(r2, r3));
}

__global__ __launch_bounds__(64) void walk_order_kernel(WalkOrderParams a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const int lane = threadIdx.x;
  const int NBW = (a.NB + 31) >> 5;
  uint32_t* tb = smem;                                                 // [ncw][NBW]
  uint16_t* mask = reinterpret_cast<uint16_t*>(smem + 14 * NBW);       // [NB]
  uint16_t* asc = mask + a.NB;                                         // [NB]
  uint16_t* ord = asc + a.NB;                                          // [NB] placed positions

  const int tpw = walk_tpw(a.TPT), ncw = walk_ncw(a.TPT);
  const int ngrp = (a.T + tpw - 1) / tpw;
  const int g = blockIdx.x;                     // (b * Hs + sg) * ngrp + grp
  const int grp = g % ngrp;
  const int sg = (g / ngrp) % a.Hs;
  const int b = g / (ngrp * a.Hs);
  const int t0 = grp * tpw;
  const int ntok = min(tpw, a.T - t0);

  for (int i = lane; i < ncw * NBW; i += 64) tb[i] = 0u;
  __syncthreads();
  const size_t rowbase = (static_cast<size_t>(b) * a.T + t0) * a.Hs + sg;
  for (int e = lane; e < ntok * a.S; e += 64) {
    const int tl = e / a.S, s = e - tl * a.S;
    const int j = a.idx[(rowbase + static_cast<size_t>(tl) * a.Hs) * a.S + s];
    if (j >= 0 && j <= (t0 + tl) / 64) atomicOr(&tb[(tl / a.TPT) * NBW + (j >> 5)], 1u << (j & 31));
  }
  __syncthreads();

  // union positions and tile masks, one bitmap word per lane
  int nU = 0;
  for (int w0 = 0; w0 < NBW; w0 += 64) {
    const int wd = w0 + lane;
    uint32_t tw[14];
    uint32_t u = 0u;
#pragma unroll
    for (int w = 0; w < 14; ++w) {
      tw[w] = (w < ncw && wd < NBW) ? tb[w * NBW + wd] : 0u;
      u |= tw[w];
    }
    const int cnt = __popc(u);
    const int incl = wave_incl_scan(cnt);
    int pos = nU + incl - cnt;
    while (u) {
      const int bit = __ffs(u) - 1;
      u &= u - 1;
      uint32_t m = 0u;
#pragma unroll
      for (int w = 0; w < 14; ++w) m |= ((tw[w] >> bit) & 1u) << w;
      mask[pos] = static_cast<uint16_t>(m);
      asc[pos] = static_cast<uint16_t>(wd * 32 + bit);
      ++pos;
    }
    nU += __shfl(incl, 63, 64);
  }
  nU = __builtin_amdgcn_readfirstlane(nU);
  __syncthreads();

  // placement.  Lane l holds a candidate: its position cp, tile mask cm and
  // base key kb = (64 - tiles needing it) << 16 | cp; a step's key adds the
  // window load ml << 22, so the smallest key is the least loaded, then the
  // most needed, then the earliest candidate.  No candidate: kb above every
  // key.  sb holds the masks of the 64-position chunk of the stream that nxt
  // (the next unplaced position) is in; ordv collects the current 64-entry
  // chunk of placements.  Each step places the best candidate and then, on
  // the same window, the best one whose tiles are disjoint from its tiles.
  constexpr uint32_t kNone = 0xFF000000u;
  uint32_t cp = lane < nU ? lane : 0xFFFFu;
  uint32_t cm = lane < nU ? mask[lane] : 0u;
  uint32_t kb = lane < nU ? (((64u - __popc(cm)) << 16) | lane) : kNone;
  int nxt = min(64, nU);
  uint32_t sb = (nxt + lane < nU) ? mask[nxt + lane] : 0u;
  uint32_t ordv = 0u;
  uint32_t c0 = 0u, c1 = 0u;                    // per-tile window load, bit-sliced (0..3)
  uint32_t h0 = 0u, h1 = 0u, h2 = 0u;           // masks of the last three placed blocks
  static_assert(kWin == 4, "three-deep history");
  int n = 0;
  // record position p (mask m, held by lane wl) as placement n; its lane
  // takes the next unplaced position; the window moves on by one block
  auto commit = [&](uint32_t p, uint32_t m, int wl) __attribute__((always_inline)) {
    ordv = (lane == (n & 63)) ? p : ordv;
    if ((n & 63) == 63) ord[(n & ~63) + lane] = static_cast<uint16_t>(ordv);
    ++n;
    uint32_t ncp = 0xFFFFu, ncm = 0u, nkb = kNone;
    if (nxt < nU) {
      ncm = __builtin_amdgcn_readlane(sb, nxt & 63);
      ncp = static_cast<uint32_t>(nxt);
      nkb = ((64u - __popc(ncm)) << 16) | ncp;
      ++nxt;
      if ((nxt & 63) == 0) sb = (nxt + lane < nU) ? mask[nxt + lane] : 0u;
    }
    const bool win = lane == wl;
    cp = win ? ncp : cp;
    cm = win ? ncm : cm;
    kb = win ? nkb : kb;
    // drop the block placed kWin - 1 steps ago, add this one
    const uint32_t borrow = ~c0 & h2;
    c0 ^= h2;
    c1 ^= borrow;
    const uint32_t carry = c0 & m;
    c0 ^= m;
    c1 ^= carry;
    h2 = h1;
    h1 = h0;
    h0 = m;
  };
  while (n < nU) {
    // window load of the candidate's busiest tile, in bits 22..23 of the key
    const uint32_t b1 = min(cm & c0, 1u), b2 = min(cm & c1, 1u), b3 = min(cm & c0 & c1, 1u);
    const uint32_t key = kb + (max(max(b1, b2 << 1), b3 * 3u) << 22);
    const uint32_t k1 = wave_min_u32(key);
    const uint32_t p1 = k1 & 0xFFFFu;
    const int w1 = static_cast<int>(__builtin_ctzll(ballot64(cp == p1)));   // one lane
    const uint32_t m1 = __builtin_amdgcn_readlane(cm, w1);
    const uint32_t k2 = wave_min_u32((cp != p1 && (cm & m1) == 0u) ? key : 0xFFFFFFFFu);
    commit(p1, m1, w1);
    if (k2 < kNone) {
      const uint32_t p2 = k2 & 0xFFFFu;
      const int w2 = static_cast<int>(__builtin_ctzll(ballot64(cp == p2)));
      commit(p2, __builtin_amdgcn_readlane(cm, w2), w2);
    }
  }
  if ((nU & 63) != 0 && lane < (nU & 63)) ord[(nU & ~63) + lane] = static_cast<uint16_t>(ordv);
  __syncthreads();
  uint16_t* out = a.order + static_cast<size_t>(g) * a.ost;
  if (lane == 0) out[0] = static_cast<uint16_t>(nU);
  for (int n = lane; n < nU; n += 64) out[1 + n] = asc[ord[n]];
}

}  // namespace

size_t walk_order_smem_bytes(int NB) {
  const int NBW = (NB + 31) >> 5;
  return sizeof(uint32_t) * 14 * NBW + sizeof(uint16_t) * 3 * NB;
}

hipError_t launch_walk_order(const WalkOrderParams& p, hipStream_t st) {
  const int tpw = walk_tpw(p.TPT);
  const unsigned ngrp = (p.T + tpw - 1) / tpw;
  const dim3 grid(static_cast<unsigned>(p.B) * p.Hs * ngrp);
  hipLaunchKernelGGL(walk_order_kernel, grid, dim3(64), walk_order_smem_bytes(p.NB), st, p);
  return hipGetLastError();
}

}  // namespace sas
