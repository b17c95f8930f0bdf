// Staging order of one token group (see walk_order.hip), as an inline device
// function so that other kernels can run it beside their own work.
#pragma once
#include "sas_kernels.h"

namespace sas {

namespace walk {

constexpr int kWin = 4;     // ring window the placement balances (the forward's ring depth)
constexpr int kPick = 2;    // placements per step
constexpr int kLook = 64;   // candidates: the first kLook unplaced blocks
static_assert(kLook >= 1 && kLook <= 64, "one candidate per lane");

// v = min(v, v of another lane) by a DPP move; lanes outside row_mask (or
// reading outside the wave) take the minimum's identity
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_min(uint32_t v) {
  const uint32_t t = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(-1, static_cast<int>(v), CTRL, ROWS, 0xF, false));
  return min(v, t);
}
// minimum over the wave: within each 16-lane row, then rows 0 -> 1 and
// 2 -> 3 by row broadcast 15, then rows 0..1 -> 2..3 by row broadcast 31;
// lane 63 ends up with the whole wave's minimum
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = dpp_min<0xB1>(v);           // quad_perm [1,0,3,2]
  v = dpp_min<0x4E>(v);           // quad_perm [2,3,0,1]
  v = dpp_min<0x141>(v);          // row_half_mirror
  v = dpp_min<0x140>(v);          // row_mirror
  v = dpp_min<0x142, 0xA>(v);     // row_bcast:15
  v = dpp_min<0x143, 0xC>(v);     // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

}  // namespace walk

// Group g by one wave (lane = its lane) with smem = walk_order_smem_bytes(NB)
// of LDS.  Every wave of a workgroup that calls it must call it (the same four
// barriers); live = false runs the barriers only.
__device__ inline void walk_order_group(const WalkOrderParams& a, int g, bool live, int lane,
                                 uint32_t* smem) {
  using namespace walk;
  const int NBW = (a.NB + 31) >> 5;
  uint32_t* tb = smem;                                                 // [ncw][NBW]
  uint16_t* mask = reinterpret_cast<uint16_t*>(smem + 14 * NBW);       // [NB]
  uint16_t* asc = mask + a.NB;                                         // [NB]
  uint16_t* ord = asc + a.NB;                                          // [NB] placed positions

  const int tpw = walk_tpw(a.TPT), ncw = walk_ncw(a.TPT);
  const int ngrp = (a.T + tpw - 1) / tpw;
  // g = (b * Hs + sg) * ngrp + grp
  const int grp = g % ngrp;
  const int sg = (g / ngrp) % a.Hs;
  const int b = g / (ngrp * a.Hs);
  const int t0 = grp * tpw;
  const int ntok = live ? min(tpw, a.T - t0) : 0;

  for (int i = lane; i < ncw * NBW; i += 64) tb[i] = 0u;
  __syncthreads();
  const size_t rowbase = (static_cast<size_t>(b) * a.T + t0) * a.Hs + sg;
  for (int e = lane; e < ntok * a.S; e += 64) {
    const int tl = e / a.S, s = e - tl * a.S;
    const int j = a.idx[(rowbase + static_cast<size_t>(tl) * a.Hs) * a.S + s];
    if (j >= 0 && j <= (t0 + tl) / 64) atomicOr(&tb[(tl / a.TPT) * NBW + (j >> 5)], 1u << (j & 31));
  }
  __syncthreads();

  // union positions and tile masks, one block per lane: bit w of block j's
  // mask is bit j of tile w's bitmap
  int nU = 0;
  for (int j0 = 0; live && j0 < a.NB; j0 += 64) {
    const int j = j0 + lane;
    uint32_t m = 0u;
    if (j < a.NB) {
      const uint32_t* col = tb + (j >> 5);
      for (int w = 0; w < ncw; ++w) m |= ((col[w * NBW] >> (j & 31)) & 1u) << w;
    }
    const uint64_t in = ballot64(m != 0u);
    if (m != 0u) {
      const int pos = nU + static_cast<int>(__popcll(in & ((1ull << lane) - 1ull)));
      mask[pos] = static_cast<uint16_t>(m);
      asc[pos] = static_cast<uint16_t>(j);
    }
    nU += static_cast<int>(__popcll(in));
  }
  nU = __builtin_amdgcn_readfirstlane(nU);
  __syncthreads();

  // placement.  Lane l holds a candidate: its tile mask cm and base key
  // kb = (64 - tiles needing it) << 16 | position << 6 | l; a step's key adds
  // the window load ml << 22, so the smallest key is the least loaded, then
  // the most needed, then the earliest candidate, and its low bits name the
  // lane.  No candidate: kb above every key.  sb holds the masks of the
  // 64-position chunk of the stream that nxt (the next unplaced position) is
  // in; ordv collects the current 64-entry chunk of placements.  Each step
  // ranks the candidates on the current window and places up to kPick of
  // them: the best, then the best whose tiles are disjoint from the tiles
  // already picked, and so on.
  constexpr uint32_t kNone = 0xFF000000u;
  const bool cand0 = lane < min(kLook, nU);
  uint32_t cm = cand0 ? mask[lane] : 0u;
  uint32_t kb = cand0 ? (((64u - __popc(cm)) << 16) | (lane << 6) | lane) : kNone;
  int nxt = min(kLook, nU);
  uint32_t sb = ((nxt & ~63) + lane < nU) ? mask[(nxt & ~63) + lane] : 0u;
  uint32_t ordv = 0u;
  uint32_t c0 = 0u, c1 = 0u;                    // per-tile window load, bit-sliced (0..3)
  uint32_t h0 = 0u, h1 = 0u, h2 = 0u;           // masks of the last three placed blocks
  static_assert(kWin == 4, "three-deep history");
  int n = 0;
  // record the candidate of key k (mask m) as placement n; its lane takes the
  // next unplaced position; the window moves on by one block
  auto commit = [&](uint32_t k, uint32_t m) __attribute__((always_inline)) {
    const int wl = static_cast<int>(k & 63u);
    ordv = (lane == (n & 63)) ? ((k >> 6) & 1023u) : ordv;
    if ((n & 63) == 63) ord[(n & ~63) + lane] = static_cast<uint16_t>(ordv);
    ++n;
    uint32_t ncm = 0u, nkb = kNone;
    if (nxt < nU) {
      ncm = __builtin_amdgcn_readlane(sb, nxt & 63);
      nkb = ((64u - __popc(ncm)) << 16) | (static_cast<uint32_t>(nxt) << 6) | static_cast<uint32_t>(wl);
      ++nxt;
      if ((nxt & 63) == 0) sb = (nxt + lane < nU) ? mask[nxt + lane] : 0u;
    }
    const bool win = lane == wl;
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
    // up to kPick picks on this window, each the best candidate whose tiles
    // are disjoint from the tiles of the picks before it
    uint32_t pk[kPick], pm[kPick];
    uint32_t used = 0u;
#pragma unroll
    for (int i = 0; i < kPick; ++i) {
      pk[i] = wave_min_u32((cm & used) == 0u ? key : 0xFFFFFFFFu);
      pm[i] = pk[i] < kNone ? __builtin_amdgcn_readlane(cm, static_cast<int>(pk[i] & 63u)) : 0u;
      used |= pm[i];
    }
#pragma unroll
    for (int i = 0; i < kPick; ++i)
      if (pk[i] < kNone) commit(pk[i], pm[i]);
  }
  if ((nU & 63) != 0 && lane < (nU & 63)) ord[(nU & ~63) + lane] = static_cast<uint16_t>(ordv);
  __syncthreads();
  if (!live) return;
  uint16_t* out = a.order + static_cast<size_t>(g) * a.ost;
  if (lane == 0) out[0] = static_cast<uint16_t>(nU);
  for (int n = lane; n < nU; n += 64) out[1 + n] = asc[ord[n]];
}

}  // namespace sas
