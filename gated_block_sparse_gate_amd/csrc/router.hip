// Gate router (model card "Checkpoint configuration": Qproj, key block pooling
// max + min + average, Q/K normalisation, gate RoPE; abstract: lightweight
// selector that scores context blocks).
//
//   q_gate[t] = RoPE_t( RMSNorm( concat_i q[t, sg*Gs+i] . Wq[sg] ) * w_qn )
//     per selection head sg: Gs = G query heads of KV head sg (one gate per KV
//     head), or Gs = 1, query head sg alone (one gate per query head)
//   k_gate[t] = RoPE_{64c}( RMSNorm( [max; min; mean]_{64c..t} k . Wk[kappa] ) * w_kn )
//
// Both projections run on bf16 MFMA with fp32 accumulation.  The inputs and
// weights are bf16, so every product is exact in fp32.  The max and min pools
// are themselves bf16 values; the mean pool is not, so its projection uses
// linearity: mean_tau(k_tau) . Wk_mean = mean_tau(k_tau . Wk_mean), i.e. each
// token's key is projected exactly and the prefix mean is taken in fp32.
#include "sas_kernels.h"

namespace sas {

namespace {

// (cos, sin) of pos * theta^(-2i/dg), argument built and reduced in double:
// each thread keeps one frequency i (the thread count is a multiple of dg / 2)
// and walks positions; the angle is reduced by a two-part 2 pi before sincos.
__global__ void rope_table_kernel(float2* tab, int T, int dg, double theta) {
  const int half = dg / 2;
  const int nthr = gridDim.x * blockDim.x;
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int i = gid % half;
  const double inv_freq = pow(theta, -2.0 * i / dg);
  constexpr double kTwoPiHi = 6.283185307179586;        // 2 pi rounded to double
  constexpr double kTwoPiLo = 2.4492935982947064e-16;   // 2 pi - kTwoPiHi
  for (int t = gid / half; t < T; t += nthr / half) {
    const double ang = static_cast<double>(t) * inv_freq;
    const double k = rint(ang * (1.0 / kTwoPiHi));
    const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang));
    double s, c;
    sincos(r, &s, &c);
    tab[static_cast<size_t>(t) * half + i] = make_float2(static_cast<float>(c), static_cast<float>(s));
  }
}

// out[h][n][f] = in[h][f][n]
__global__ void transpose_w_kernel(const uint16_t* in, uint16_t* out, int H, int F, int N) {
  const long tot = static_cast<long>(H) * F * N;
  for (long e = blockIdx.x * static_cast<long>(blockDim.x) + threadIdx.x; e < tot;
       e += static_cast<long>(gridDim.x) * blockDim.x) {
    const long h = e / (static_cast<long>(F) * N);
    const long r = e - h * F * N;
    const long f = r / N, n = r - f * N;
    out[(h * N + n) * F + f] = in[e];
  }
}

// RMSNorm over the DG columns of four rows held in MFMA C layout, then
// rotate-half RoPE, then store.  acc[nt][i]: row 4*g4+i, column 16*nt+l16.
template <int DG>
__device__ __forceinline__ void norm_rope_store(floatx4 (&acc)[DG / 16], const float* w,
                                                float eps, const float2* rope,
                                                const int (&pos)[4], float* const (&out)[4],
                                                int l16) {
  constexpr int NT = DG / 16, HALF = DG / 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float ss = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) ss += acc[nt][i] * acc[nt][i];
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    ss += __shfl_xor(ss, 4, 64);
    ss += __shfl_xor(ss, 8, 64);
    const float rs = 1.0f / sqrtf(ss * (1.0f / DG) + eps);
    if (out[i] == nullptr) continue;
#pragma unroll
    for (int nt = 0; nt < NT / 2; ++nt) {
      const int n = nt * 16 + l16;
      const float y1 = acc[nt][i] * rs * w[n];
      const float y2 = acc[nt + NT / 2][i] * rs * w[n + HALF];
      const float2 cs = rope[static_cast<size_t>(pos[i]) * HALF + n];
      out[i][n] = y1 * cs.x - y2 * cs.y;
      out[i][n + HALF] = y2 * cs.x + y1 * cs.y;
    }
  }
}

// One workgroup = 128 token rows of one selection head, wave w owning rows
// 32 w .. 32 w + 31 (two 16-row tiles) x all DG gate columns.  The weights
// are staged through LDS 64 inputs at a time, shared by the four waves
// (asynchronous global -> LDS copies, double-buffered; 128-byte rows whose
// 16-byte chunks are XOR-swizzled by (row >> 1) & 7, so that 16 lanes reading
// one chunk of 16 consecutive rows hit distinct banks), and each wave's query
// operands for the next stage load while the current one runs: 32 contiguous
// bytes of a row per lane, so each row's 128-byte line is read whole.
template <int DG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void gate_query_kernel(RouterParams p) {
  constexpr int NT = DG / 16;
  constexpr int MT = 2;
  constexpr int WROWB = 128;                     // bytes per staged weight row (64 inputs)
  constexpr int YP = DG + 16;          // floats per staged output row (the four row
                                       // groups of a store fall on distinct banks)
  constexpr int WLSB = 2 * DG * WROWB, YRB = 4 * 16 * YP * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[WLSB > YRB ? WLSB : YRB];
  uint8_t (*wls)[DG * WROWB] = reinterpret_cast<uint8_t (*)[DG * WROWB]>(lds_raw);
  // the output rows reuse the weight stage's LDS after the loop's last barrier
  float* const yrows = reinterpret_cast<float*>(lds_raw);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int sg = blockIdx.y;
  const int F = p.Gs * p.D;
  const long nrows = static_cast<long>(p.B) * p.T;
  const long r0 = static_cast<long>(blockIdx.x) * (64 * MT) + wv * 16 * MT;

  floatx4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* xr[MT];
  bool ok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const long r = r0 + mt * 16 + l16;
    ok[mt] = r < nrows;
    xr[mt] = p.q + ((ok[mt] ? r : 0) * p.Hq + static_cast<long>(sg) * p.Gs) * p.D;
  }
  const uint16_t* wt = p.wqT + static_cast<size_t>(sg) * DG * F;
  // weight inputs f .. f + 63 of all DG rows into buffer buf: copy m moves
  // units 64 m .. 64 m + 63 (unit u = row u / 8, slot u % 8 holding chunk
  // (u % 8) ^ swizzle)
  auto wstage = [&](int f, int buf) __attribute__((always_inline)) {
    for (int m = wv; m < DG * WROWB / 1024; m += 4) {
      const int u = m * 64 + lane, n = u >> 3;
      load_lds16(wt + static_cast<size_t>(n) * F + f + (((u & 7) ^ ((n >> 1) & 7)) << 3),
                 &wls[buf][m * 1024]);
    }
  };
  // inputs f + 16 (lane / 16) .. + 15 of each tile row: 32 contiguous bytes
  // per lane, whole 128-byte lines per row and instruction pair; MFMA half
  // h takes the inputs f + 16 (lane / 16) + 8 h .. + 7 on both operands
  auto qload = [&](int f, uint4 (&a)[MT][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        a[mt][h] = ok[mt] ? ld16(xr[mt] + f + g4 * 16 + 8 * h) : make_uint4(0, 0, 0, 0);
  };
  uint4 av[MT][2];
  wstage(0, 0);
  qload(0, av);
  wait_vmem_all();
  __syncthreads();
  for (int f = 0, it = 0; f < F; f += 64, ++it) {
    const int buf = it & 1;
    const bool more = f + 64 < F;
    uint4 an[MT][2];
    if (more) {
      wstage(f + 64, buf ^ 1);     // the copies first, then this wave's query loads
      qload(f + 64, an);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = nt * 16 + l16;
        const uint4 bv = ld16(&wls[buf][n * WROWB + (((2 * g4 + h) ^ ((n >> 1) & 7)) << 4)]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][nt] = mfma16x16x32(av[mt][h], bv, acc[mt][nt]);
      }
    if (more) {
      // all but the 2 MT query loads: the next stage's weights have landed
      static_assert(2 * MT < 16, "vmcnt immediate");
      __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * MT));
      asm volatile("" ::: "memory");
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        av[mt][0] = an[mt][0];
        av[mt][1] = an[mt][1];
      }
    }
    __syncthreads();
  }
  // each 16-row tile: RMSNorm and RoPE into the wave's LDS rows, then whole
  // rows out as 16-byte stores (the wave's LDS accesses are performed in
  // order, so its rows are complete when it reads them back, and the next
  // tile's writes come after these reads)
  float* const yb = yrows + wv * 16 * YP;
  constexpr int CH = DG / 4;             // 16-byte chunks per row
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int pos[4];
    float* yrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long r = r0 + mt * 16 + g4 * 4 + i;
      pos[i] = r < nrows ? static_cast<int>(r % p.T) : 0;
      yrow[i] = yb + (g4 * 4 + i) * YP;
    }
    norm_rope_store<DG>(acc[mt], p.w_qn, p.eps, p.rope, pos, yrow, l16);
    for (int e = lane; e < 16 * CH; e += 64) {
      const int rl = e / CH, ch = e - rl * CH;
      const long r = r0 + mt * 16 + rl;
      if (r < nrows)
        *reinterpret_cast<float4*>(p.q_gate + (r * p.Hs + sg) * DG + 4 * ch) =
            *reinterpret_cast<const float4*>(yb + rl * YP + 4 * ch);
    }
  }
}

// One workgroup = one 64-token block of one (batch, KV head).  Wave w owns a
// slice of the DG output columns for the block's rows (all 64 rows and DG / 4
// columns when DG >= 64; at DG = 32 two waves per column tile, 32 rows each),
// with that slice of the projection weights loaded once into registers as the
// MFMA B operands, requested before the block is pooled so that they land
// meanwhile; no weight staging and no barrier between the projection steps.
// The RMSNorm sums and the RoPE pairs (columns n and n + DG / 2 sit in
// different waves) go through LDS, and the rows leave as contiguous stores.
template <int D, int DG>
__global__ __launch_bounds__(256) void gate_key_kernel(RouterParams p) {
  constexpr int KP = D + 8;
  constexpr int NPAIR = D / 2;
  constexpr int NSEG = 256 / NPAIR;     // token segments for the prefix scan
  constexpr int SEGL = 64 / NSEG;
  constexpr int NTT = DG / 16;          // column tiles
  constexpr int WC = NTT >= 4 ? 4 : NTT;   // waves across the columns
  constexpr int WR = 4 / WC;               // waves across the rows
  constexpr int NTW = NTT / WC;            // column tiles per wave
  constexpr int MTW = 4 / WR;              // 16-row tiles per wave
  constexpr int NSTEP = 3 * D / 32;        // projection steps (max, min, mean sections)
  constexpr int KBUF = 3 * 64 * KP * 2;    // bytes of the key rows and the two prefix pools
  constexpr int YBUF = 64 * DG * 4;        // bytes of the normalised rows (reuse the same LDS)
  static_assert(WC * NTW == NTT && WR * MTW == 4, "wave tiling");
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[KBUF > YBUF ? KBUF : YBUF];
  __shared__ float segmx[NSEG * D];
  __shared__ float segmn[NSEG * D];
  __shared__ float csum[4][DG];          // per wave: its rows' mean-section column totals
  __shared__ float ssum[WC][64];         // per column group: each row's sum of squares
  uint16_t* const kb = reinterpret_cast<uint16_t*>(kbuf);
  uint16_t* const pmx = kb + 64 * KP;
  uint16_t* const pmn = kb + 2 * 64 * KP;
  float* const ybuf = reinterpret_cast<float*>(kbuf);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int c = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int t0 = c * 64;
  const int ntok = min(64, p.T - t0);
  const int cg = wv % WC, rg = wv / WC;   // the wave's column group and row group

  // the wave's weight slice, B operand of step s and column tile nt: column
  // n = 16 (cg NTW + nt) + lane % 16, inputs 32 s + 8 (lane / 16) .. + 7
  uint4 bw[NSTEP][NTW];
  {
    const uint16_t* wt = p.wkT + static_cast<size_t>(kv) * DG * (3 * D) + 8 * g4;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const uint16_t* wr = wt + static_cast<size_t>(16 * (cg * NTW + nt) + l16) * (3 * D);
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) bw[st][nt] = ld16(wr + 32 * st);
    }
  }

  for (int u = tid; u < 64 * (D / 8); u += 256) {
    const int row = u / (D / 8), ch = u - row * (D / 8);
    uint4 val = make_uint4(0, 0, 0, 0);
    if (row < ntok)
      val = *reinterpret_cast<const uint4*>(
          p.k + ((static_cast<size_t>(b) * p.T + t0 + row) * p.Hkv + kv) * D + ch * 8);
    *reinterpret_cast<uint4*>(&kb[row * KP + ch * 8]) = val;
  }
  __syncthreads();

  // prefix max / min over tokens, channel-wise (exact: bf16 values kept as is)
  {
    const int cp = tid % NPAIR, seg = tid / NPAIR;
    float mx0 = -INFINITY, mx1 = -INFINITY, mn0 = INFINITY, mn1 = INFINITY;
    uint16_t bmx0 = 0, bmx1 = 0, bmn0 = 0, bmn1 = 0;
    for (int r = seg * SEGL; r < seg * SEGL + SEGL; ++r) {
      const uint32_t w2 = *reinterpret_cast<const uint32_t*>(&kb[r * KP + 2 * cp]);
      const uint16_t h0 = static_cast<uint16_t>(w2 & 0xffffu), h1 = static_cast<uint16_t>(w2 >> 16);
      const float f0 = bf2f(h0), f1 = bf2f(h1);
      if (f0 > mx0 || r == seg * SEGL) { mx0 = f0; bmx0 = h0; }
      if (f1 > mx1 || r == seg * SEGL) { mx1 = f1; bmx1 = h1; }
      if (f0 < mn0 || r == seg * SEGL) { mn0 = f0; bmn0 = h0; }
      if (f1 < mn1 || r == seg * SEGL) { mn1 = f1; bmn1 = h1; }
      *reinterpret_cast<uint32_t*>(&pmx[r * KP + 2 * cp]) = bmx0 | (static_cast<uint32_t>(bmx1) << 16);
      *reinterpret_cast<uint32_t*>(&pmn[r * KP + 2 * cp]) = bmn0 | (static_cast<uint32_t>(bmn1) << 16);
    }
    segmx[seg * D + 2 * cp] = mx0;
    segmx[seg * D + 2 * cp + 1] = mx1;
    segmn[seg * D + 2 * cp] = mn0;
    segmn[seg * D + 2 * cp + 1] = mn1;
    __syncthreads();
    if (seg > 0) {
      float cx0 = -INFINITY, cx1 = -INFINITY, cn0 = INFINITY, cn1 = INFINITY;
      for (int s2 = 0; s2 < seg; ++s2) {
        cx0 = fmaxf(cx0, segmx[s2 * D + 2 * cp]);
        cx1 = fmaxf(cx1, segmx[s2 * D + 2 * cp + 1]);
        cn0 = fminf(cn0, segmn[s2 * D + 2 * cp]);
        cn1 = fminf(cn1, segmn[s2 * D + 2 * cp + 1]);
      }
      for (int r = seg * SEGL; r < seg * SEGL + SEGL; ++r) {
        uint32_t* px = reinterpret_cast<uint32_t*>(&pmx[r * KP + 2 * cp]);
        uint32_t* pn = reinterpret_cast<uint32_t*>(&pmn[r * KP + 2 * cp]);
        uint32_t vx = *px, vn = *pn;
        uint16_t x0 = vx & 0xffffu, x1 = vx >> 16, n0 = vn & 0xffffu, n1 = vn >> 16;
        if (cx0 > bf2f(x0)) x0 = f2bf(cx0);
        if (cx1 > bf2f(x1)) x1 = f2bf(cx1);
        if (cn0 < bf2f(n0)) n0 = f2bf(cn0);
        if (cn1 < bf2f(n1)) n1 = f2bf(cn1);
        *px = x0 | (static_cast<uint32_t>(x1) << 16);
        *pn = n0 | (static_cast<uint32_t>(n1) << 16);
      }
    }
  }
  __syncthreads();

  // [max; min] and mean-section projections of the wave's rows and columns;
  // C layout: element i of tile (mt, nt) is row 16 (rg MTW + mt) + 4 (lane /
  // 16) + i of the block, column 16 (cg NTW + nt) + lane % 16
  floatx4 amm[MTW][NTW], ak[MTW][NTW];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      amm[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
      ak[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    const int f = 32 * st;
    const uint16_t* src = (f < D) ? pmx + f : (f < 2 * D) ? pmn + (f - D) : kb + (f - 2 * D);
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
      const uint4 av = ld16(src + (16 * (rg * MTW + mt) + l16) * KP + 8 * g4);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        if (f < 2 * D)
          amm[mt][nt] = mfma16x16x32(av, bw[st][nt], amm[mt][nt]);
        else
          ak[mt][nt] = mfma16x16x32(av, bw[st][nt], ak[mt][nt]);
      }
    }
  }

  // prefix sum over the block's rows of the per-token mean-section
  // projections: inside a lane, across the four lane groups, across the
  // wave's row tiles, then across the row groups (WR > 1)
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    float carry = 0.f;
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
      floatx4 v = ak[mt][nt];
      v[1] += v[0];
      v[2] += v[1];
      v[3] += v[2];
      float sg = v[3];
      float t = __shfl_up(sg, 16, 64);
      if (g4 >= 1) sg += t;
      t = __shfl_up(sg, 32, 64);
      if (g4 >= 2) sg += t;
      const float excl = carry + sg - v[3];
      v[0] += excl;
      v[1] += excl;
      v[2] += excl;
      v[3] += excl;
      ak[mt][nt] = v;
      carry += __shfl(sg, 48 + l16, 64);    // the tile's total (lane group 3)
    }
    if (g4 == 0) csum[wv][16 * (cg * NTW + nt) + l16] = carry;
  }
  __syncthreads();
  float ss_part[MTW][4];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) ss_part[mt][i] = 0.f;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int col = 16 * (cg * NTW + nt) + l16;
    float off = 0.f;
    for (int r2 = 0; r2 < rg; ++r2) off += csum[r2 * WC + cg][col];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tl = 16 * (rg * MTW + mt) + 4 * g4 + i;
        const float y = amm[mt][nt][i] + (ak[mt][nt][i] + off) / static_cast<float>(tl + 1);
        amm[mt][nt][i] = y;
        ss_part[mt][i] += y * y;
      }
  }
  // each row's sum of squares over the wave's columns (16 lanes of a row
  // group), then over the column groups through LDS
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float r = row16_sum(ss_part[mt][i]);
      if (l16 == 0) ssum[cg][16 * (rg * MTW + mt) + 4 * g4 + i] = r;
    }
  __syncthreads();                       // (also: every read of the pooled rows is done)
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = 16 * (rg * MTW + mt) + 4 * g4 + i;
      float ss = 0.f;
#pragma unroll
      for (int g = 0; g < WC; ++g) ss += ssum[g][tl];
      const float rs = 1.0f / sqrtf(ss * (1.0f / DG) + p.eps);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int col = 16 * (cg * NTW + nt) + l16;
        ybuf[tl * DG + col] = amm[mt][nt][i] * rs * p.w_kn[col];
      }
    }
  __syncthreads();
  // rotate-half RoPE at the block start 64 c; four threads per row, each
  // DG / 8 consecutive pairs (n, n + DG / 2)
  {
    constexpr int HALF = DG / 2, PPT = DG / 8;
    const int tl = tid >> 2, n0 = (tid & 3) * PPT;
    if (tl < ntok) {
      float* out = p.k_gate + ((static_cast<size_t>(b) * p.T + t0 + tl) * p.Hkv + kv) * DG;
      const float2* rope = p.rope + static_cast<size_t>(t0) * HALF;
#pragma unroll
      for (int q = 0; q < PPT; q += 4) {
        float4 o1, o2;
        float* a1 = &o1.x;
        float* a2 = &o2.x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = n0 + q + e;
          const float y1 = ybuf[tl * DG + n], y2 = ybuf[tl * DG + n + HALF];
          const float2 cs = rope[n];
          a1[e] = y1 * cs.x - y2 * cs.y;
          a2[e] = y2 * cs.x + y1 * cs.y;
        }
        *reinterpret_cast<float4*>(out + n0 + q) = o1;
        *reinterpret_cast<float4*>(out + n0 + q + HALF) = o2;
      }
    }
  }
}

template <int D, int DG>
hipError_t launch_router_t(const RouterParams& p, hipStream_t st) {
  const long nrows = static_cast<long>(p.B) * p.T;
  hipLaunchKernelGGL((gate_query_kernel<DG>), dim3((nrows + 127) / 128, p.Hs), dim3(256), 0,
                     st, p);
  const int NB = (p.T + 63) / 64;
  hipLaunchKernelGGL((gate_key_kernel<D, DG>), dim3(NB, p.Hkv, p.B), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_transpose_w(const uint16_t* in, uint16_t* out, int H, int F, int N,
                              hipStream_t st) {
  const long n = static_cast<long>(H) * F * N;
  hipLaunchKernelGGL(transpose_w_kernel, dim3(static_cast<unsigned>(min(2048L, (n + 255) / 256))),
                     dim3(256), 0, st, in, out, H, F, N);
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* tab, int T, int dg, double theta, hipStream_t st) {
  // 256 threads per workgroup: a multiple of dg / 2 (16, 32 or 64)
  const long nr = static_cast<long>(T) * (dg / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>(min(1024L, (nr + 255) / 256))),
                     dim3(256), 0, st, tab, T, dg, theta);
  return hipGetLastError();
}

hipError_t launch_router(const RouterParams& p0, const uint16_t* wq, const uint16_t* wk,
                         uint16_t* wqT, uint16_t* wkT, float2* rope, double theta,
                         hipStream_t st) {
  RouterParams p = p0;
  p.wqT = wqT;
  p.wkT = wkT;
  p.rope = rope;
  const long nr = static_cast<long>(p.T) * (p.dg / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>(min(1024L, (nr + 255) / 256))),
                     dim3(256), 0, st, rope, p.T, p.dg, theta);
  const long nq = static_cast<long>(p.Hs) * p.Gs * p.D * p.dg;
  const long nk = static_cast<long>(p.Hkv) * 3 * p.D * p.dg;
  hipLaunchKernelGGL(transpose_w_kernel, dim3(static_cast<unsigned>(min(2048L, (nq + 255) / 256))),
                     dim3(256), 0, st, wq, wqT, p.Hs, p.Gs * p.D, p.dg);
  hipLaunchKernelGGL(transpose_w_kernel, dim3(static_cast<unsigned>(min(2048L, (nk + 255) / 256))),
                     dim3(256), 0, st, wk, wkT, p.Hkv, 3 * p.D, p.dg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.D == 128) {
    if (p.dg == 128) return launch_router_t<128, 128>(p, st);
    if (p.dg == 64) return launch_router_t<128, 64>(p, st);
    if (p.dg == 32) return launch_router_t<128, 32>(p, st);
  } else if (p.D == 64) {
    if (p.dg == 128) return launch_router_t<64, 128>(p, st);
    if (p.dg == 64) return launch_router_t<64, 64>(p, st);
    if (p.dg == 32) return launch_router_t<64, 32>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace sas
