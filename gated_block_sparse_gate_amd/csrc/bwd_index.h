// Index arithmetic of the dQ kernel's dS-row loads, shared by the kernel and
// by a host-side replay (tests/native/dq_index_check.hip) that walks every
// workgroup, tile, lane and slot of the test shapes on the CPU.
#pragma once
#include <hip/hip_runtime.h>

namespace sas {

// Tokens per workgroup of the query-block walks (forward and dQ): 14 compute
// waves of TPT tokens each, at most 64.
__host__ __device__ inline int walk_tpw(int TPT) { return 14 * TPT < 64 ? 14 * TPT : 64; }
__host__ __device__ inline int walk_ncw(int TPT) { return (walk_tpw(TPT) + TPT - 1) / TPT; }

// Row held by lane l16 of compute tile `tile`: token tl of the group (clamped
// to the 64 per-token LDS rows) and head hh; live = the row exists (the lane
// is inside the tile's TPT * G rows and its token inside the group's ntok).
struct WalkRow {
  int tl, hh;
  bool live;
};
__host__ __device__ inline WalkRow walk_row(int tile, int l16, int TPT, int G, int ntok) {
  WalkRow r;
  const int t = tile * TPT + l16 / G;
  r.tl = t < 63 ? t : 63;
  r.hh = l16 - (l16 / G) * G;
  r.live = (l16 < TPT * G) && (t < ntok);
  return r;
}

// Bytes of a token group's dS rows of one KV head, from its first row to the
// end of its last token's rows ([token][kappa][slot][head] x 256 bytes).
__host__ __device__ inline unsigned dq_ds_bytes(int ntok, int HSG, int S, int G) {
  return static_cast<unsigned>(((ntok - 1) * HSG + S) * G) * 256u;
}

// Offset of lane group g4's 16-byte piece of the dS row (token tl, slot sl,
// head hh) relative to the group's first row, when `take` (the lane's row
// exists and selected the block); otherwise the end of the group's rows, so a
// buffer load there returns zeros without a memory request.  The kernel reads
// the pieces at +0, +64, +128, +192 (hi, lo halves).
__host__ __device__ inline unsigned dq_ds_offset(bool take, int tl, int HSG, int sl, int G, int hh,
                                                 int g4, unsigned end) {
  return take ? static_cast<unsigned>(((tl * HSG + sl) * G + hh) * 256 + 16 * g4) : end;
}

}  // namespace sas
