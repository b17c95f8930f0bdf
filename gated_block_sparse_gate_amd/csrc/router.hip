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

// (cos, sin) of pos * theta^(-2i/dg), argument built and reduced in double.
__global__ void rope_table_kernel(float2* tab, int T, int dg, double theta) {
  const int half = dg / 2;
  const long n = static_cast<long>(T) * half;
  for (long e = blockIdx.x * static_cast<long>(blockDim.x) + threadIdx.x; e < n;
       e += static_cast<long>(gridDim.x) * blockDim.x) {
    const int t = static_cast<int>(e / half);
    const int i = static_cast<int>(e - static_cast<long>(t) * half);
    const double inv_freq = pow(theta, -2.0 * i / dg);
    const double ang = static_cast<double>(t) * inv_freq;
    double s, c;
    sincos(ang, &s, &c);
    tab[e] = make_float2(static_cast<float>(c), static_cast<float>(s));
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
// 32 w .. 32 w + 31 (two 16-row tiles) x all DG gate columns.  The weight
// columns are staged through LDS in 32-wide steps shared by the four waves
// (asynchronous global -> LDS copies, double-buffered; 64-byte rows whose
// 16-byte chunks are XOR-swizzled by (row >> 2) & 3, so that 16 lanes reading
// one chunk of 16 consecutive rows hit distinct banks), and each wave's query
// operands for the next step load while the current step runs.
template <int DG>
__global__ __launch_bounds__(256) void gate_query_kernel(RouterParams p) {
  constexpr int NT = DG / 16;
  constexpr int MT = 2;
  constexpr int WROWB = 64;                      // bytes per staged weight row
  __shared__ __attribute__((aligned(16))) uint8_t wls[2][DG * WROWB];
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
  // weight columns f .. f + 31 of all DG rows into buffer buf: copy m moves
  // units 64 m .. 64 m + 63 (unit u = row u / 4, slot u % 4 holding chunk
  // (u % 4) ^ swizzle)
  auto wstage = [&](int f, int buf) __attribute__((always_inline)) {
    for (int m = wv; m < DG / 16; m += 4) {
      const int u = m * 64 + lane, n = u >> 2;
      load_lds16(wt + static_cast<size_t>(n) * F + f + (((u & 3) ^ ((n >> 2) & 3)) << 3),
                 &wls[buf][m * 1024]);
    }
  };
  auto qload = [&](int f, uint4 (&a)[MT]) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      a[mt] = ok[mt] ? ld16(xr[mt] + f + g4 * 8) : make_uint4(0, 0, 0, 0);
  };
  uint4 av[MT];
  wstage(0, 0);
  qload(0, av);
  wait_vmem_all();
  __syncthreads();
  for (int f = 0, it = 0; f < F; f += 32, ++it) {
    const int buf = it & 1;
    const bool more = f + 32 < F;
    uint4 an[MT];
    if (more) {
      wstage(f + 32, buf ^ 1);     // the copies first, then this wave's query loads
      qload(f + 32, an);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = nt * 16 + l16;
      const uint4 bv = ld16(&wls[buf][n * WROWB + ((g4 ^ ((n >> 2) & 3)) << 4)]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt][nt] = mfma16x16x32(av[mt], bv, acc[mt][nt]);
    }
    if (more) {
      // all but the MT query loads: the next step's weights have landed
      static_assert(MT < 16, "vmcnt immediate");
      __builtin_amdgcn_s_waitcnt(0x0f70 | MT);
      asm volatile("" ::: "memory");
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) av[mt] = an[mt];
    }
    __syncthreads();
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int pos[4];
    float* out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long r = r0 + mt * 16 + g4 * 4 + i;
      const bool v = r < nrows;
      pos[i] = v ? static_cast<int>(r % p.T) : 0;
      out[i] = v ? p.q_gate + (r * p.Hs + sg) * DG : nullptr;
    }
    norm_rope_store<DG>(acc[mt], p.w_qn, p.eps, p.rope, pos, out, l16);
  }
}

// One workgroup = one 64-token block of one (batch, KV head); wave w owns
// tokens 16w .. 16w+15.
template <int D, int DG>
__global__ __launch_bounds__(256) void gate_key_kernel(RouterParams p) {
  constexpr int NT = DG / 16;
  constexpr int KP = D + 8;
  constexpr int NPAIR = D / 2;
  constexpr int NSEG = 256 / NPAIR;     // token segments for the prefix scan
  constexpr int SEGL = 64 / NSEG;
  __shared__ __attribute__((aligned(16))) uint16_t kb[64 * KP];
  __shared__ __attribute__((aligned(16))) uint16_t pmx[64 * KP];
  __shared__ __attribute__((aligned(16))) uint16_t pmn[64 * KP];
  __shared__ float segmx[NSEG * D];
  __shared__ float segmn[NSEG * D];
  __shared__ float wsum[4][DG];
  // weight columns of 32-wide steps, double-buffered (as in gate_query_kernel)
  constexpr int WROWB = 64;
  __shared__ __attribute__((aligned(16))) uint8_t wls[2][DG * WROWB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int c = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int t0 = c * 64;
  const int ntok = min(64, p.T - t0);

  const uint16_t* wt = p.wkT + static_cast<size_t>(kv) * DG * (3 * D);
  auto wstage = [&](int f, int buf) __attribute__((always_inline)) {
    for (int m = wv; m < DG / 16; m += 4) {
      const int u = m * 64 + lane, n = u >> 2;
      load_lds16(wt + static_cast<size_t>(n) * (3 * D) + f + (((u & 3) ^ ((n >> 2) & 3)) << 3),
                 &wls[buf][m * 1024]);
    }
  };
  wstage(0, 0);                 // lands while the block is pooled

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

  const int arow = wv * 16 + l16;
  floatx4 amm[NT], ak[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    amm[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    ak[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  // inputs f .. f + 31 of the 3D (max, min, mean sections) against the
  // staged weight columns; the next step's weights land meanwhile
  wait_vmem_all();
  __syncthreads();
  for (int f = 0, it = 0; f < 3 * D; f += 32, ++it) {
    const int buf = it & 1;
    const bool more = f + 32 < 3 * D;
    if (more) wstage(f + 32, buf ^ 1);
    const uint16_t* src = (f < D) ? &pmx[arow * KP + f]
                                  : (f < 2 * D) ? &pmn[arow * KP + f - D] : &kb[arow * KP + f - 2 * D];
    const uint4 av = ld16(src + g4 * 8);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = nt * 16 + l16;
      const uint4 bv = ld16(&wls[buf][n * WROWB + ((g4 ^ ((n >> 2) & 3)) << 4)]);
      if (f < 2 * D)
        amm[nt] = mfma16x16x32(av, bv, amm[nt]);
      else
        ak[nt] = mfma16x16x32(av, bv, ak[nt]);
    }
    if (more) wait_vmem_all();
    __syncthreads();
  }

  // prefix sum of the per-token mean-section projections over the block
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
    if (g4 == 3) wsum[wv][nt * 16 + l16] = s;
  }
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float off = 0.f;
    for (int w2 = 0; w2 < wv; ++w2) off += wsum[w2][nt * 16 + l16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = wv * 16 + g4 * 4 + i;
      amm[nt][i] += (ak[nt][i] + off) / static_cast<float>(tl + 1);
    }
  }
  int pos[4];
  float* out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tl = wv * 16 + g4 * 4 + i;
    pos[i] = t0;
    out[i] = (tl < ntok)
                 ? p.k_gate + ((static_cast<size_t>(b) * p.T + t0 + tl) * p.Hkv + kv) * DG
                 : nullptr;
  }
  norm_rope_store<DG>(amm, p.w_kn, p.eps, p.rope, pos, out, l16);
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
  const long nr = static_cast<long>(T) * (dg / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>(min(4096L, (nr + 255) / 256))),
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
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>(min(4096L, (nr + 255) / 256))),
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
