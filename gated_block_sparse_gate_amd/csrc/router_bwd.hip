// Router backward (GitHub README intro (b): the continuous gate on every
// selected block gives the LM loss a gradient path to the selector; model
// card "Checkpoint configuration": Qproj, max + min + average key pooling,
// Q/K normalisation, gate RoPE).
//
// Input: dlogg = dL/d log g per selected slot, as the gated attention
// backward produces it, with the selection held fixed.  log g = s - lse(s)
// over the candidate blocks 0..c of the row, so in general
//   ds_j = dlogg_j [j selected] - g_j * (sum of the row's dlogg).
// The row's normaliser lse is one constant added to all of the row's
// attention logits, so the attention softmax cancels it and the attention's
// dlogg sums to zero over the row: ds = dlogg on the selected blocks, 0
// elsewhere, which is what is computed here.  Then, with
// s_j = q_gate[t] . key_j / sqrt(dg) (key_j = k_gate[64j+63] for a historical
// block, k_gate[t] for the current one):
//   1. per row: dq_gate and the current-block part of dk_gate;
//   2. per historical block: the block key's gradient, summed over the rows
//      that selected it (dense tiles of the selection on MFMA);
//   3. query side: inverse RoPE, RMSNorm backward, dx = dy Wq^T;
//   4. key side: inverse RoPE, RMSNorm backward, dp = dz Wk^T, and the
//      pooling backward (max and min pass their gradient to the first row of
//      the prefix that attains them, the mean to every row of the prefix);
//   5. weight gradients as sums over token chunks, reduced in a fixed order.
// Everything is deterministic.  Products and sums are fp32; the projections
// are recomputed exactly as the forward router computes them.
#include "sas_kernels.h"

namespace sas {

namespace {

// 8 consecutive fp32 values -> MFMA operand words of their bf16 hi and lo
// parts (v = hi + lo to ~2^-16), in memory order
__device__ __forceinline__ void split8(const float* src, uint4& hi, uint4& lo) {
  const float4 a = *reinterpret_cast<const float4*>(src);
  const float4 b = *reinterpret_cast<const float4*>(src + 4);
  split_bf2(a.x, a.y, hi.x, lo.x);
  split_bf2(a.z, a.w, hi.y, lo.y);
  split_bf2(b.x, b.y, hi.z, lo.z);
  split_bf2(b.z, b.w, hi.w, lo.w);
}

// ---------------------------------------------------------------- 1. rows
// One wave per row (b, t, kappa); lane l owns gate dims 2l, 2l + 1.
template <int DG>
__global__ __launch_bounds__(256) void gbwd_rows_kernel(GateBwdParams p) {
  const int lane = threadIdx.x & 63;
  const long nrows = static_cast<long>(p.B) * p.T * p.Hkv;
  const long row = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;
  const long bt = row / p.Hkv;
  const int kv = static_cast<int>(row - bt * p.Hkv);
  const int t = static_cast<int>(bt % p.T);
  const long b = bt / p.T;
  const int c = t / 64;
  const bool on = 2 * lane < DG;
  const int dd = on ? 2 * lane : 0;
  float2 acc = make_float2(0.f, 0.f);
  float dcur = 0.f;
  // the row's slots on lanes 0..S-1 (S <= 64); valid slots in slot order,
  // their keys gathered 8 at a time
  int jl = -1;
  float dll = 0.f;
  if (lane < p.S) {
    jl = p.idx[row * p.S + lane];
    dll = p.dlogg[row * p.S + lane];
  }
  uint64_t m = ballot64(jl >= 0 && jl <= c);
  while (m) {
    float w[8];
    float2 kk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      w[u] = 0.f;
      kk[u] = make_float2(0.f, 0.f);
      if (m) {
        const int src = __builtin_ctzll(m);
        m &= m - 1;
        const int j = __shfl(jl, src, 64);
        w[u] = __shfl(dll, src, 64);
        if (j == c) dcur += w[u];
        const long krow = (j == c) ? row : ((b * p.T + 64L * j + 63) * p.Hkv + kv);
        kk[u] = *reinterpret_cast<const float2*>(p.k_gate + krow * DG + dd);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc.x = fmaf(w[u], kk[u].x, acc.x);
      acc.y = fmaf(w[u], kk[u].y, acc.y);
    }
  }
  if (!on) return;
  const float2 qq = *reinterpret_cast<const float2*>(p.q_gate + row * DG + dd);
  *reinterpret_cast<float2*>(p.dqg + row * DG + dd) =
      make_float2(acc.x * p.inv_sqrt_dg, acc.y * p.inv_sqrt_dg);
  *reinterpret_cast<float2*>(p.dkg + row * DG + dd) =
      make_float2(dcur * qq.x * p.inv_sqrt_dg, dcur * qq.y * p.inv_sqrt_dg);
}

// ---------------------------------------------------------------- 2. block keys
// The key of historical block j (token 64j+63) receives dlogg * q_gate from
// every row that selected it: per KV head, dK_blk [NB x dg] = DS^T Q_gate
// with DS [T x NB] holding dlogg at the selected historical slots.  Dense
// per tile: workgroup = (64-block tile j0.., chunk of query blocks,
// b * Hkv + kappa); per query block c of the chunk it builds the DS^T tile
// [64 j x 64 tokens] and the Q_gate tile [64 tokens x dg] in LDS as bf16 hi
// and lo parts and adds their product (hi.hi + hi.lo + lo.hi) on MFMA; the
// chunk partials are added in order by a second kernel.
constexpr int kKeyTile = 64;
constexpr int kKeyChunk = kGateBwdKeyChunk;         // query blocks per workgroup

template <int DG>
__global__ __launch_bounds__(256) void gbwd_blockkey_kernel(GateBwdParams p) {
  constexpr int NT = DG / 16;
  constexpr int SP = 64 + 8;                        // DS^T row pitch (bf16)
  constexpr int QP = DG + 8;                        // Q tile row pitch (bf16)
  __shared__ __attribute__((aligned(16))) uint16_t dsh[64 * SP], dsl[64 * SP];
  __shared__ __attribute__((aligned(16))) uint16_t qh[64 * QP], ql[64 * QP];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int j0 = blockIdx.x * kKeyTile, cc = blockIdx.y, bk = blockIdx.z;
  const int kv = bk % p.Hkv;
  const long b = bk / p.Hkv;
  const int c0 = cc * kKeyChunk, c1 = min(p.NB, c0 + kKeyChunk);
  if (c1 - 1 <= j0) return;                         // no block of the tile is history here
  floatx4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  // B operand (Q tile) k order: tokens 8 g4 + {0..3}, then 8 g4 + 4 + {0..3}
  const int trow = 8 * g4 + (l16 >> 2);
  const int tcol = 4 * (l16 & 3);
  for (int c = max(c0, j0 + 1); c < c1; ++c) {
    const int ntok = min(64, p.T - 64 * c);
    __syncthreads();                                // previous block's reads are done
    for (int u = tid; u < 64 * SP / 8; u += 256) {
      st16(&dsh[u * 8], make_uint4(0, 0, 0, 0));
      st16(&dsl[u * 8], make_uint4(0, 0, 0, 0));
    }
    for (int u = tid; u < 64 * (DG / 8); u += 256) {
      const int tl = u / (DG / 8), ch = u - tl * (DG / 8);
      uint4 hi = make_uint4(0, 0, 0, 0), lo = hi;
      if (tl < ntok)
        split8(p.q_gate + ((b * p.T + 64L * c + tl) * p.Hkv + kv) * DG + ch * 8, hi, lo);
      st16(&qh[tl * QP + ch * 8], hi);
      st16(&ql[tl * QP + ch * 8], lo);
    }
    __syncthreads();                                // zeroed DS^T before the scatter
    for (int u = tid; u < ntok * p.S; u += 256) {
      const int tl = u / p.S, s = u - tl * p.S;
      const long row = (b * p.T + 64L * c + tl) * p.Hkv + kv;
      const int j = p.idx[row * p.S + s];
      if (j >= j0 && j < j0 + kKeyTile && j < c) {
        const float dl = p.dlogg[row * p.S + s];
        const uint32_t h = pack_bf2(dl, 0.f) & 0xffffu;
        const float lo = dl - __uint_as_float(h << 16);
        dsh[(j - j0) * SP + tl] = static_cast<uint16_t>(h);
        dsl[(j - j0) * SP + tl] = static_cast<uint16_t>(pack_bf2(lo, 0.f) & 0xffffu);
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {                // 64 tokens = 2 steps of 32
      const uint4 ah = ld16(&dsh[(wv * 16 + l16) * SP + ks * 32 + g4 * 8]);
      const uint4 al = ld16(&dsl[(wv * 16 + l16) * SP + ks * 32 + g4 * 8]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int o0 = (ks * 32 + trow) * QP + nt * 16 + tcol;
        const uint2 h0 = lds_read_tr16(&qh[o0]), h1 = lds_read_tr16(&qh[o0 + 4 * QP]);
        const uint2 q0 = lds_read_tr16(&ql[o0]), q1 = lds_read_tr16(&ql[o0 + 4 * QP]);
        const uint4 bh = make_uint4(h0.x, h0.y, h1.x, h1.y);
        const uint4 bl = make_uint4(q0.x, q0.y, q1.x, q1.y);
        acc[nt] = mfma16x16x32(ah, bh, acc[nt]);
        acc[nt] = mfma16x16x32(ah, bl, acc[nt]);
        acc[nt] = mfma16x16x32(al, bh, acc[nt]);
      }
    }
  }
  const int nj = min(kKeyTile, p.NB - j0);
  float* out = p.bk_part + ((static_cast<size_t>(bk) * gridDim.y + cc) * p.NB + j0) * DG;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jj = wv * 16 + g4 * 4 + i;
      if (jj < nj) out[jj * DG + nt * 16 + l16] = acc[nt][i];
    }
}

// dkg[64j+63] += (sum of the chunk partials of j's tile) / sqrt(dg), over
// the chunks whose workgroup ran, in order
template <int DG>
__global__ __launch_bounds__(256) void gbwd_blockkey_sum_kernel(GateBwdParams p, int nchunk) {
  const long e = blockIdx.x * 256L + threadIdx.x;
  const long tot = static_cast<long>(p.B) * p.Hkv * p.NB * DG;
  if (e >= tot) return;
  const int d = static_cast<int>(e % DG);
  const long r = e / DG;
  const int j = static_cast<int>(r % p.NB);
  const int bk = static_cast<int>(r / p.NB);
  if (64L * j + 63 >= p.T) return;
  const int kv = bk % p.Hkv;
  const long b = bk / p.Hkv;
  const int j0 = (j / kKeyTile) * kKeyTile;
  float s = 0.f;
  const float* src = p.bk_part + (static_cast<size_t>(bk) * nchunk * p.NB + j) * DG + d;
  for (int c = 0; c < nchunk; ++c) {
    const int c1 = min(p.NB, (c + 1) * kKeyChunk);
    if (c1 - 1 > j0) s += src[static_cast<size_t>(c) * p.NB * DG];
  }
  float* dst = p.dkg + ((b * p.T + 64L * j + 63) * p.Hkv + kv) * DG + d;
  *dst += s * p.inv_sqrt_dg;
}

// RMSNorm backward and inverse RoPE for 4 rows held in MFMA C layout:
// acc[nt][i] = pre-norm value of row 4 g4 + i, column 16 nt + l16; g[nt][i]
// = dL/d(output) on entry, dL/d(pre-norm) on exit.  Adds dL/dw * (row valid)
// into wsum[n] for the lane's columns.
template <int DG>
__device__ __forceinline__ void norm_rope_bwd(const floatx4 (&acc)[DG / 16],
                                              floatx4 (&g)[DG / 16], const float* w,
                                              float eps, const float2* rope,
                                              const int (&pos)[4], const bool (&ok)[4],
                                              float (&wsum)[DG / 16], int l16) {
  constexpr int NT = DG / 16, HALF = DG / 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // inverse rotation (the transpose of the forward's)
#pragma unroll
    for (int nt = 0; nt < NT / 2; ++nt) {
      const int n = nt * 16 + l16;
      const float2 cs = rope[static_cast<size_t>(pos[i]) * HALF + n];
      const float a = g[nt][i], bq = g[nt + NT / 2][i];
      g[nt][i] = a * cs.x + bq * cs.y;
      g[nt + NT / 2][i] = bq * cs.x - a * cs.y;
    }
    float ss = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) ss += acc[nt][i] * acc[nt][i];
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    ss += __shfl_xor(ss, 4, 64);
    ss += __shfl_xor(ss, 8, 64);
    const float rs = 1.0f / sqrtf(ss * (1.0f / DG) + eps);
    float uy = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = nt * 16 + l16;
      const float dn = g[nt][i];
      if (ok[i]) wsum[nt] = fmaf(dn, acc[nt][i] * rs, wsum[nt]);
      const float u = dn * w[n];
      g[nt][i] = u;
      uy = fmaf(u, acc[nt][i], uy);
    }
    uy += __shfl_xor(uy, 1, 64);
    uy += __shfl_xor(uy, 2, 64);
    uy += __shfl_xor(uy, 4, 64);
    uy += __shfl_xor(uy, 8, 64);
    const float cf = rs * rs * rs * uy * (1.0f / DG);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) g[nt][i] = rs * g[nt][i] - cf * acc[nt][i];
  }
}

// Per-workgroup column sums of the norm-weight gradient: wsum of every lane
// (columns 16 nt + l16), summed over g4 and the 4 waves in a fixed order.
template <int DG>
__device__ __forceinline__ void store_wn_partial(float (&wsum)[DG / 16], float* red, float* out,
                                                 int wv, int lane) {
  constexpr int NT = DG / 16;
  const int l16 = lane & 15;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float v = wsum[nt];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (lane < 16) red[wv * DG + nt * 16 + l16] = v;
  }
  __syncthreads();
  for (int n = threadIdx.x; n < DG; n += blockDim.x)
    out[n] = (red[n] + red[DG + n]) + (red[2 * DG + n] + red[3 * DG + n]);
}

// ---------------------------------------------------------------- 3. query side
// Tiling of the forward's gate query: wave = 32 token rows, workgroup = 128.
// dy = RMSNorm/RoPE backward of dq_gate; dq[row, f] = sum_n dy[row, n] Wq[f, n].
template <int DG>
__global__ __launch_bounds__(256) void gbwd_query_kernel(GateBwdParams p) {
  constexpr int NT = DG / 16;
  __shared__ __attribute__((aligned(16))) float dyl[4][32][DG + 4];
  __shared__ float red[4 * DG];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int kv = blockIdx.y;
  const int F = p.G * p.D;
  const long nrows = static_cast<long>(p.B) * p.T;
  const long r0 = static_cast<long>(blockIdx.x) * 128 + wv * 32;

  floatx4 acc[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* xr[2];
  bool okr[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const long r = r0 + mt * 16 + l16;
    okr[mt] = r < nrows;
    xr[mt] = p.q + ((okr[mt] ? r : 0) * p.Hq + static_cast<long>(kv) * p.G) * p.D;
  }
  const uint16_t* wt = p.wqT + static_cast<size_t>(kv) * DG * F;
  for (int f = 0; f < F; f += 32) {
    uint4 av[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      av[mt] = okr[mt] ? *reinterpret_cast<const uint4*>(xr[mt] + f + g4 * 8)
                       : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint4 bv = *reinterpret_cast<const uint4*>(wt + (nt * 16 + l16) * F + f + g4 * 8);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = mfma16x16x32(av[mt], bv, acc[mt][nt]);
    }
  }

  float wsum[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) wsum[nt] = 0.f;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    floatx4 g[NT];
    int pos[4];
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long r = r0 + mt * 16 + g4 * 4 + i;
      ok[i] = r < nrows;
      pos[i] = ok[i] ? static_cast<int>(r % p.T) : 0;
      const float* src = p.dqg + ((ok[i] ? r : 0) * p.Hkv + kv) * DG;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) g[nt][i] = ok[i] ? src[nt * 16 + l16] : 0.f;
    }
    norm_rope_bwd<DG>(acc[mt], g, p.w_qn, p.eps, p.rope, pos, ok, wsum, l16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long r = r0 + mt * 16 + g4 * 4 + i;
      float* dst = p.dy + ((ok[i] ? r : 0) * p.Hkv + kv) * DG;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        dyl[wv][mt * 16 + g4 * 4 + i][nt * 16 + l16] = g[nt][i];
        if (ok[i]) dst[nt * 16 + l16] = g[nt][i];
      }
    }
  }
  store_wn_partial<DG>(wsum, red, p.wn_part + (static_cast<size_t>(kv) * gridDim.x + blockIdx.x) * DG,
                       wv, lane);

  // dq[row, f] = sum_n dy[row, n] Wq[f, n]: bf16 MFMA with dy as hi + lo
  // parts against the bf16 weights (8 f tiles at a time)
  uint4 ah[2][DG / 32], al[2][DG / 32];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < DG / 32; ++ks)
      split8(&dyl[wv][mt * 16 + l16][ks * 32 + g4 * 8], ah[mt][ks], al[mt][ks]);
  const uint16_t* wqk = p.wq + static_cast<size_t>(kv) * F * DG;
  for (int f0 = 0; f0 < F; f0 += 128) {
    floatx4 o[2][8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ft = 0; ft < 8; ++ft) o[mt][ft] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ft = 0; ft < 8; ++ft) {
      if (f0 + ft * 16 >= F) break;                 // F = G * D is a multiple of 64
      const uint16_t* wrow = wqk + static_cast<size_t>(f0 + ft * 16 + l16) * DG + g4 * 8;
#pragma unroll
      for (int ks = 0; ks < DG / 32; ++ks) {
        const uint4 bw = *reinterpret_cast<const uint4*>(wrow + ks * 32);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          o[mt][ft] = mfma16x16x32(ah[mt][ks], bw, o[mt][ft]);
          o[mt][ft] = mfma16x16x32(al[mt][ks], bw, o[mt][ft]);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long r = r0 + mt * 16 + g4 * 4 + i;
        if (r >= nrows) continue;
        float* dst = p.dq + (r * p.Hq + static_cast<long>(kv) * p.G) * p.D + f0 + l16;
#pragma unroll
        for (int ft = 0; ft < 8; ++ft)
          if (f0 + ft * 16 < F) dst[ft * 16] = o[mt][ft][i];
      }
  }
}

// ---------------------------------------------------------------- 4. key side
// One workgroup = one 64-token block of one (b, kappa); wave w owns tokens
// 16w .. 16w + 15 in the projections.
template <int D, int DG>
__global__ __launch_bounds__(256) void gbwd_key_kernel(GateBwdParams p) {
  constexpr int NT = DG / 16;
  constexpr int KP = D + 8;
  constexpr int ZP = DG + 4;
  constexpr int DP = D + 4;
  // phase 1: key rows and prefix pools (bf16); phase 2 reuses the space
  constexpr int P1 = 3 * 64 * KP * 2;
  constexpr int P2 = 2 * 64 * DP * 4;
  __shared__ __attribute__((aligned(16))) uint8_t big[P1 > P2 ? P1 : P2];
  __shared__ __attribute__((aligned(16))) float zt[64][ZP];   // dz, then suffix sums
  __shared__ uint8_t amx[64][D], amn[64][D];
  __shared__ float wsum4[4][DG];
  __shared__ float red[4 * DG];
  uint16_t* kb = reinterpret_cast<uint16_t*>(big);
  uint16_t* pmx = kb + 64 * KP;
  uint16_t* pmn = pmx + 64 * KP;
  float* dpb = reinterpret_cast<float*>(big);                  // [64][DP] dp (max or min part)
  float* dkb = dpb + 64 * DP;                                  // [64][DP] dk accumulators

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int c = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int t0 = c * 64;
  const int ntok = min(64, p.T - t0);
  const size_t rowbase = (static_cast<size_t>(b) * p.T + t0) * p.Hkv + kv;   // row of token t0

  for (int u = tid; u < 64 * (D / 8); u += 256) {
    const int row = u / (D / 8), ch = u - row * (D / 8);
    uint4 val = make_uint4(0, 0, 0, 0);
    if (row < ntok)
      val = *reinterpret_cast<const uint4*>(p.k + (rowbase + static_cast<size_t>(row) * p.Hkv) * D +
                                            ch * 8);
    *reinterpret_cast<uint4*>(&kb[row * KP + ch * 8]) = val;
  }
  __syncthreads();
  // prefix max (threads 0..D-1) and min (D..2D-1) per channel, with the first
  // row attaining each
  if (tid < 2 * D) {
    const bool ismax = tid < D;
    const int ch = ismax ? tid : tid - D;
    uint16_t* pool = ismax ? pmx : pmn;
    uint8_t(*arg)[D] = ismax ? amx : amn;
    float best = 0.f;
    uint16_t bb = 0;
    int ai = 0;
    for (int r = 0; r < 64; ++r) {
      const uint16_t h = kb[r * KP + ch];
      const float v = bf2f(h);
      if (r < ntok && (r == 0 || (ismax ? v > best : v < best))) {
        best = v;
        bb = h;
        ai = r;
      }
      pool[r * KP + ch] = r < ntok ? bb : 0;
      arg[r][ch] = static_cast<uint8_t>(ai);
    }
  }
  __syncthreads();
  // pools to the workspace (for the weight gradient)
  for (int u = tid; u < ntok * (D / 8); u += 256) {
    const int row = u / (D / 8), ch = u - row * (D / 8);
    uint16_t* dst = p.pmm + (rowbase + static_cast<size_t>(row) * p.Hkv) * (2 * D) + ch * 8;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(&pmx[row * KP + ch * 8]);
    *reinterpret_cast<uint4*>(dst + D) = *reinterpret_cast<const uint4*>(&pmn[row * KP + ch * 8]);
  }

  // z = [max; min] . Wk[0:2D] + prefix mean of k . Wk[2D:3D] (as the forward)
  const uint16_t* wt = p.wkT + static_cast<size_t>(kv) * DG * (3 * D);
  const int arow = wv * 16 + l16;
  floatx4 amm[NT], ak[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    amm[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    ak[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  for (int f = 0; f < 2 * D; f += 32) {
    const uint16_t* src = (f < D) ? &pmx[arow * KP + f] : &pmn[arow * KP + f - D];
    const uint4 av = *reinterpret_cast<const uint4*>(src + g4 * 8);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint4 bv =
          *reinterpret_cast<const uint4*>(wt + (nt * 16 + l16) * (3 * D) + f + g4 * 8);
      amm[nt] = mfma16x16x32(av, bv, amm[nt]);
    }
  }
  for (int f = 0; f < D; f += 32) {
    const uint4 av = *reinterpret_cast<const uint4*>(&kb[arow * KP + f + g4 * 8]);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint4 bv =
          *reinterpret_cast<const uint4*>(wt + (nt * 16 + l16) * (3 * D) + 2 * D + f + g4 * 8);
      ak[nt] = mfma16x16x32(av, bv, ak[nt]);
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    floatx4 v = ak[nt];
    v[1] += v[0];
    v[2] += v[1];
    v[3] += v[2];
    const float tot = v[3];
    float s = tot;
    float t = __shfl_up(s, 16, 64);
    if (g4 >= 1) s += t;
    t = __shfl_up(s, 32, 64);
    if (g4 >= 2) s += t;
    const float excl = s - tot;
    v[0] += excl;
    v[1] += excl;
    v[2] += excl;
    v[3] += excl;
    ak[nt] = v;
    if (g4 == 3) wsum4[wv][nt * 16 + l16] = s;
  }
  __syncthreads();            // wsum4 complete; kb / pools no longer read after this
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float off = 0.f;
    for (int w2 = 0; w2 < wv; ++w2) off += wsum4[w2][nt * 16 + l16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = wv * 16 + g4 * 4 + i;
      amm[nt][i] += (ak[nt][i] + off) / static_cast<float>(tl + 1);
    }
  }

  // dz from dk_gate
  float wsum[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) wsum[nt] = 0.f;
  {
    floatx4 g[NT];
    int pos[4];
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = wv * 16 + g4 * 4 + i;
      ok[i] = tl < ntok;
      pos[i] = t0;
      const float* src = p.dkg + (rowbase + static_cast<size_t>(ok[i] ? tl : 0) * p.Hkv) * DG;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) g[nt][i] = ok[i] ? src[nt * 16 + l16] : 0.f;
    }
    norm_rope_bwd<DG>(amm, g, p.w_kn, p.eps, p.rope, pos, ok, wsum, l16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = wv * 16 + g4 * 4 + i;
      float* dst = p.dz + (rowbase + static_cast<size_t>(ok[i] ? tl : 0) * p.Hkv) * DG;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        zt[tl][nt * 16 + l16] = ok[i] ? g[nt][i] : 0.f;
        if (ok[i]) dst[nt * 16 + l16] = g[nt][i];
      }
    }
  }
  store_wn_partial<DG>(wsum, red,
                       p.wn_part + (static_cast<size_t>(p.nq_part) +
                                    (static_cast<size_t>(b) * p.Hkv + kv) * gridDim.x + c) * DG,
                       wv, lane);     // (its barrier also publishes zt)

  // dp = dz . Wk^T for the max part, then the min part: wave w rows 16w..
  // (16x16x4 fp32 MFMA), scattered per channel to the first row attaining it
  for (int u = tid; u < 64 * D; u += 256) dkb[(u / D) * DP + u % D] = 0.f;
  // dz rows of the wave as bf16 hi + lo MFMA operands (against bf16 Wk)
  constexpr int DT = D / 16;
  const uint16_t* wkk = p.wk + static_cast<size_t>(kv) * (3 * D) * DG;
  uint4 zh[DG / 32], zl[DG / 32];
#pragma unroll
  for (int ks = 0; ks < DG / 32; ++ks) split8(&zt[wv * 16 + l16][ks * 32 + g4 * 8], zh[ks], zl[ks]);
#pragma unroll 1
  for (int part = 0; part < 2; ++part) {
    {
      floatx4 o[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint16_t* wrow = wkk + static_cast<size_t>(part * D + dt * 16 + l16) * DG + g4 * 8;
#pragma unroll
        for (int ks = 0; ks < DG / 32; ++ks) {
          const uint4 bw = *reinterpret_cast<const uint4*>(wrow + ks * 32);
          o[dt] = mfma16x16x32(zh[ks], bw, o[dt]);
          o[dt] = mfma16x16x32(zl[ks], bw, o[dt]);
        }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dpb[(wv * 16 + g4 * 4 + i) * DP + dt * 16 + l16] = o[dt][i];
    }
    __syncthreads();
    if (tid < D) {
      uint8_t(*arg)[D] = part == 0 ? amx : amn;
      for (int r = 0; r < ntok; ++r) dkb[arg[r][tid] * DP + tid] += dpb[r * DP + tid];
    }
    __syncthreads();
  }
  // suffix sums of dz / n over the block (n = t - 64c + 1): the mean pool
  // passes dz_t / n_t to every row r <= t
  if (tid < DG) {
    float run = 0.f;
    for (int r = ntok - 1; r >= 0; --r) {
      run += zt[r][tid] / static_cast<float>(r + 1);
      zt[r][tid] = run;
      p.dzs[(rowbase + static_cast<size_t>(r) * p.Hkv) * DG + tid] = run;
    }
  }
  __syncthreads();
  // mean part: dk[r] += dzs[r] . Wk[2D:3D]^T; then store dk rows
  {
#pragma unroll
    for (int ks = 0; ks < DG / 32; ++ks)
      split8(&zt[wv * 16 + l16][ks * 32 + g4 * 8], zh[ks], zl[ks]);
    floatx4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint16_t* wrow = wkk + static_cast<size_t>(2 * D + dt * 16 + l16) * DG + g4 * 8;
#pragma unroll
      for (int ks = 0; ks < DG / 32; ++ks) {
        const uint4 bw = *reinterpret_cast<const uint4*>(wrow + ks * 32);
        o[dt] = mfma16x16x32(zh[ks], bw, o[dt]);
        o[dt] = mfma16x16x32(zl[ks], bw, o[dt]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = wv * 16 + g4 * 4 + i;
      if (tl >= ntok) continue;
      float* dst = p.dk + (rowbase + static_cast<size_t>(tl) * p.Hkv) * D + l16;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dst[dt * 16] = dkb[tl * DP + dt * 16 + l16] + o[dt][i];
    }
  }
}

// ---------------------------------------------------------------- 5. weights
// part[chunk][kappa][f][n] = sum over the chunk's token rows of A[row][f] *
// Bm[row][n]; A bf16 (row stride a_rs, kappa stride a_ks), Bm fp32 [rows,
// Hkv, dg].  Workgroup: 64 f x dg, wave w: f tile w.  Per 32-row step the
// workgroup stages A and Bm (as bf16 hi and lo parts) row-major in LDS and
// the waves read both operands with transposing LDS reads, so that the rows
// are the contraction index of a bf16 MFMA.
template <int DG>
__global__ __launch_bounds__(256) void gbwd_wsum_kernel(const uint16_t* A, long a_rs, long a_ks,
                                                        const float* Bm, float* part, int F,
                                                        int f_off, int Ftot, long nrows,
                                                        int Hkv) {
  constexpr int NT = DG / 16;
  constexpr int AP = 64 + 8, BP = DG + 8;           // row pitches (bf16)
  __shared__ __attribute__((aligned(16))) uint16_t As[32 * AP];
  __shared__ __attribute__((aligned(16))) uint16_t Bh[32 * BP];
  __shared__ __attribute__((aligned(16))) uint16_t Bl[32 * BP];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int fw = blockIdx.x * 64;                   // F is a multiple of 64
  const int chunk = blockIdx.y, kv = blockIdx.z;
  const long r0 = static_cast<long>(chunk) * kGateBwdChunk;
  const long r1 = min(nrows, r0 + kGateBwdChunk);
  floatx4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  // operand k order (shared by both): rows 4 g4 + {0..3}, then 16 + 4 g4 + {0..3}
  const int trow = 4 * g4 + (l16 >> 2);
  const int tcol = 4 * (l16 & 3);
  for (long r = r0; r < r1; r += 32) {
    __syncthreads();                                // the previous step's reads are done
    {
      const int row = tid >> 3, ch = tid & 7;
      const long rr = r + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (rr < r1) v = ld16(A + kv * a_ks + rr * a_rs + fw + ch * 8);
      st16(&As[row * AP + ch * 8], v);
    }
    for (int u = tid; u < 32 * (DG / 8); u += 256) {
      const int row = u / (DG / 8), ch = u - row * (DG / 8);
      const long rr = r + row;
      uint4 hi = make_uint4(0, 0, 0, 0), lo = hi;
      if (rr < r1) split8(Bm + (rr * Hkv + kv) * DG + ch * 8, hi, lo);
      st16(&Bh[row * BP + ch * 8], hi);
      st16(&Bl[row * BP + ch * 8], lo);
    }
    __syncthreads();
    const uint2 a0 = lds_read_tr16(&As[trow * AP + wv * 16 + tcol]);
    const uint2 a1 = lds_read_tr16(&As[(trow + 16) * AP + wv * 16 + tcol]);
    const uint4 av = make_uint4(a0.x, a0.y, a1.x, a1.y);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint2 h0 = lds_read_tr16(&Bh[trow * BP + nt * 16 + tcol]);
      const uint2 h1 = lds_read_tr16(&Bh[(trow + 16) * BP + nt * 16 + tcol]);
      const uint2 q0 = lds_read_tr16(&Bl[trow * BP + nt * 16 + tcol]);
      const uint2 q1 = lds_read_tr16(&Bl[(trow + 16) * BP + nt * 16 + tcol]);
      acc[nt] = mfma16x16x32(av, make_uint4(h0.x, h0.y, h1.x, h1.y), acc[nt]);
      acc[nt] = mfma16x16x32(av, make_uint4(q0.x, q0.y, q1.x, q1.y), acc[nt]);
    }
  }
  float* dst = part + ((static_cast<size_t>(chunk) * Hkv + kv) * Ftot + f_off + fw + wv * 16) * DG;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(g4 * 4 + i) * DG + nt * 16 + l16] = acc[nt][i];
}

// out[e] = sum over c < n of part[c * stride + e], in order
__global__ void gbwd_reduce_kernel(const float* part, float* out, long stride, int n, long count) {
  for (long e = blockIdx.x * static_cast<long>(blockDim.x) + threadIdx.x; e < count;
       e += static_cast<long>(gridDim.x) * blockDim.x) {
    float s = 0.f;
#pragma unroll 8
    for (int c = 0; c < n; ++c) s += part[c * stride + e];
    out[e] = s;
  }
}

// out[col] = sum over the n rows of part[row * ncol + col]: one workgroup per
// column, thread i adds rows i, i + 256, ..., then a fixed pairwise tree
__global__ __launch_bounds__(256) void gbwd_colsum_kernel(const float* part, float* out, int n,
                                                         int ncol) {
  __shared__ float red[256];
  const int col = blockIdx.x, tid = threadIdx.x;
  float s = 0.f;
  for (int r = tid; r < n; r += 256) s += part[static_cast<size_t>(r) * ncol + col];
  red[tid] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) out[col] = red[0];
}

template <int D, int DG>
hipError_t launch_gate_bwd_t(const GateBwdParams& p, hipStream_t st) {
  const long nrows = static_cast<long>(p.B) * p.T;
  const long nrk = nrows * p.Hkv;
  hipLaunchKernelGGL((gbwd_rows_kernel<DG>), dim3(static_cast<unsigned>((nrk + 3) / 4)), dim3(256),
                     0, st, p);
  const int ntc = (p.NB + kKeyChunk - 1) / kKeyChunk;
  hipLaunchKernelGGL((gbwd_blockkey_kernel<DG>), dim3((p.NB + kKeyTile - 1) / kKeyTile, ntc,
                                                      p.B * p.Hkv),
                     dim3(256), 0, st, p);
  const long nbk = static_cast<long>(p.B) * p.Hkv * p.NB * DG;
  hipLaunchKernelGGL((gbwd_blockkey_sum_kernel<DG>), dim3(static_cast<unsigned>((nbk + 255) / 256)),
                     dim3(256), 0, st, p, ntc);
  hipLaunchKernelGGL((gbwd_query_kernel<DG>), dim3(static_cast<unsigned>((nrows + 127) / 128), p.Hkv),
                     dim3(256), 0, st, p);
  hipLaunchKernelGGL((gbwd_key_kernel<D, DG>), dim3(p.NB, p.Hkv, p.B), dim3(256), 0, st, p);
  const int F = p.G * p.D;
  const dim3 gq((F + 63) / 64, p.nchunk, p.Hkv), gk((D + 63) / 64, p.nchunk, p.Hkv);
  // dWq: A = q (row stride Hq * D, kappa stride G * D), Bm = dy
  hipLaunchKernelGGL((gbwd_wsum_kernel<DG>), gq, dim3(256), 0, st, p.q,
                     static_cast<long>(p.Hq) * D, static_cast<long>(p.G) * D, p.dy, p.wq_part, F,
                     0, F, nrows, p.Hkv);
  // dWk: [max | min] pools with dz, then k with the suffix sums dzs
  hipLaunchKernelGGL((gbwd_wsum_kernel<DG>), gk, dim3(256), 0, st, p.pmm,
                     static_cast<long>(p.Hkv) * 2 * D, 2L * D, p.dz, p.wk_part, D, 0, 3 * D, nrows,
                     p.Hkv);
  hipLaunchKernelGGL((gbwd_wsum_kernel<DG>), gk, dim3(256), 0, st, p.pmm + D,
                     static_cast<long>(p.Hkv) * 2 * D, 2L * D, p.dz, p.wk_part, D, D, 3 * D, nrows,
                     p.Hkv);
  hipLaunchKernelGGL((gbwd_wsum_kernel<DG>), gk, dim3(256), 0, st, p.k,
                     static_cast<long>(p.Hkv) * D, static_cast<long>(D), p.dzs, p.wk_part, D,
                     2 * D, 3 * D, nrows, p.Hkv);
  const long nwq = static_cast<long>(p.Hkv) * F * DG, nwk = static_cast<long>(p.Hkv) * 3 * D * DG;
  hipLaunchKernelGGL(gbwd_reduce_kernel, dim3(static_cast<unsigned>(min(2048L, (nwq + 255) / 256))),
                     dim3(256), 0, st, p.wq_part, p.dwq, nwq, p.nchunk, nwq);
  hipLaunchKernelGGL(gbwd_reduce_kernel, dim3(static_cast<unsigned>(min(2048L, (nwk + 255) / 256))),
                     dim3(256), 0, st, p.wk_part, p.dwk, nwk, p.nchunk, nwk);
  hipLaunchKernelGGL(gbwd_colsum_kernel, dim3(DG), dim3(256), 0, st, p.wn_part, p.dw_qn,
                     p.nq_part, DG);
  hipLaunchKernelGGL(gbwd_colsum_kernel, dim3(DG), dim3(256), 0, st,
                     p.wn_part + static_cast<size_t>(p.nq_part) * DG, p.dw_kn, p.nk_part, DG);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_bwd(const GateBwdParams& p, hipStream_t st) {
  if (p.D == 128) {
    if (p.dg == 128) return launch_gate_bwd_t<128, 128>(p, st);
    if (p.dg == 64) return launch_gate_bwd_t<128, 64>(p, st);
    if (p.dg == 32) return launch_gate_bwd_t<128, 32>(p, st);
  } else if (p.D == 64) {
    if (p.dg == 128) return launch_gate_bwd_t<64, 128>(p, st);
    if (p.dg == 64) return launch_gate_bwd_t<64, 64>(p, st);
    if (p.dg == 32) return launch_gate_bwd_t<64, 32>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace sas
