// Host-side replay of the dQ kernel's dS-row addressing (bwd_index.h, the
// same functions the kernel calls) over every workgroup, compute tile, lane
// and slot of the given shapes.  Checks, without a GPU:
//   * every lane's token index stays inside the 64 per-token LDS rows;
//   * a lane with a row loads inside its group's dS rows (all four 16-byte
//     pieces), for a token inside the sequence;
//   * a lane without a row (past a tile's rows or past the group's last
//     token, as in the last group of a ragged length) gets exactly the
//     group's end offset, where the buffer load returns zeros;
//   * every group's rows end inside the dS workspace.
// Usage: dq_index_check B T Hq Hkv K [B T Hq Hkv K ...]; exit 0 when all hold.
#include <cstdio>
#include <cstdlib>

#include "bwd_index.h"

static int check_shape(int B, int T, int Hq, int Hkv, int K) {
  using namespace sas;
  const int G = Hq / Hkv, S = K + 1, TPT = 16 / G;
  const int tpw = walk_tpw(TPT), ncw = walk_ncw(TPT);
  const int ngrp = (T + tpw - 1) / tpw;
  const int HSG = Hkv * S;
  const unsigned long long total = 256ull * B * T * Hq * S;   // dS workspace bytes
  long long loads = 0, ends = 0;
  for (int b = 0; b < B; ++b)
    for (int kv = 0; kv < Hkv; ++kv)
      for (int grp = 0; grp < ngrp; ++grp) {
        const int t0 = grp * tpw;
        const int ntok = T - t0 < tpw ? T - t0 : tpw;
        const unsigned long long rowbase = (static_cast<unsigned long long>(b) * T + t0) * Hkv + kv;
        const unsigned long long base = rowbase * S * G * 256ull;
        const unsigned end = dq_ds_bytes(ntok, HSG, S, G);
        if (base + end > total) {
          std::printf("FAIL B%d T%d kv%d grp%d: rows end at %llu > workspace %llu\n", B, T, kv,
                      grp, base + end, total);
          return 1;
        }
        for (int tile = 0; tile < ncw; ++tile)
          for (int lane = 0; lane < 64; ++lane) {
            const int l16 = lane & 15, g4 = lane >> 4;
            const WalkRow r = walk_row(tile, l16, TPT, G, ntok);
            if (r.tl < 0 || r.tl > 63) {
              std::printf("FAIL T%d grp%d tile%d lane%d: token row %d outside LDS\n", T, grp, tile,
                          lane, r.tl);
              return 1;
            }
            for (int sl = 0; sl < S; ++sl) {
              const unsigned off = dq_ds_offset(r.live, r.tl, HSG, sl, G, r.hh, g4, end);
              if (r.live) {
                if (t0 + r.tl >= T || off + 192u + 16u > end) {
                  std::printf("FAIL T%d grp%d tile%d lane%d slot%d: offset %u (+208) past %u\n",
                              T, grp, tile, lane, sl, off, end);
                  return 1;
                }
                ++loads;
              } else {
                if (off != end) {
                  std::printf("FAIL T%d grp%d tile%d lane%d slot%d: rowless lane offset %u != %u\n",
                              T, grp, tile, lane, sl, off, end);
                  return 1;
                }
                ++ends;
              }
            }
          }
      }
  std::printf("ok B=%d T=%d Hq=%d Hkv=%d K=%d: %lld row loads in range, %lld rowless lanes at the end\n",
              B, T, Hq, Hkv, K, loads, ends);
  return 0;
}

int main(int argc, char** argv) {
  if (argc < 6 || (argc - 1) % 5) {
    std::printf("usage: %s B T Hq Hkv K [...]\n", argv[0]);
    return 2;
  }
  int bad = 0;
  for (int i = 1; i + 4 < argc; i += 5)
    bad |= check_shape(std::atoi(argv[i]), std::atoi(argv[i + 1]), std::atoi(argv[i + 2]),
                       std::atoi(argv[i + 3]), std::atoi(argv[i + 4]));
  return bad;
}
