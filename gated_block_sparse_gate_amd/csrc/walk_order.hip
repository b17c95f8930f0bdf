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
//  2. placement: the candidates are the first kLook union blocks not yet
//     placed (one per lane); a candidate ranks by the load of its busiest tile in
//     the window of the last kWin - 1 placed blocks, then by the number of
//     tiles that need it (more first), then by position.  Each step ranks
//     the candidates once and places up to kPick of them: the best, then the
//     best whose tiles are disjoint from all tiles picked so far, and so on
//     (a disjoint pick's load is not changed by the picks before it), so the
//     serial chain has 1 / kPick as many steps; the next unplaced blocks
//     take the picked candidates' lanes.
// Output per group (stride ost uint16): [nU, block of position 0, ...].
#include "walk_order.h"

namespace sas {

namespace {

__global__ __launch_bounds__(64) void walk_order_kernel(WalkOrderParams a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  walk_order_group(a, blockIdx.x, true, threadIdx.x, smem);
}

}  // namespace

size_t walk_order_smem_bytes(int NB) {
  const int NBW = (NB + 31) >> 5;
  // tile bitmaps, then masks, blocks and placements; a multiple of 16 bytes,
  // so that several waves' regions can follow one another
  return (sizeof(uint32_t) * 14 * NBW + sizeof(uint16_t) * 3 * NB + 15) & ~static_cast<size_t>(15);
}

hipError_t launch_walk_order(const WalkOrderParams& p, hipStream_t st) {
  const int tpw = walk_tpw(p.TPT);
  const unsigned ngrp = (p.T + tpw - 1) / tpw;
  const dim3 grid(static_cast<unsigned>(p.B) * p.Hs * ngrp);
  hipLaunchKernelGGL(walk_order_kernel, grid, dim3(64), walk_order_smem_bytes(p.NB), st, p);
  return hipGetLastError();
}

}  // namespace sas
