// Budgeted single-token decode (model card: 2,048-token sparse decode budget
// by default, 1,024 and 4,096 also supported; usage guide pitfall 3: the
// budget limits the tokens each query attends, not the cache).
//
// Unit = (sequence b, KV head kappa), L = ctx_len[b], c = (L-1)/64:
//   score : s_j = q_gate . kg_cache[j] / sqrt(dg), j = 0..c; log-sum-exp; the
//           min(K, c) best historical blocks (ties -> lower j) + block c.
//   attend: the G query heads attend to the selected blocks' keys tau < L
//           with log g added (apply_gate = 1), split over NSPLIT workgroups
//           that each stream 4 slots' K/V blocks (16 KiB each, contiguous in
//           the head-major cache) with the next block's loads in flight.
//   combine: merge the per-split (max, sum, o) partials.
#include "sas_kernels.h"

namespace sas {

namespace {

constexpr int kSlotsPerSplit = 4;

template <int DG>
__global__ __launch_bounds__(512) void decode_select_kernel(DecodeParams p) {
  constexpr int LPC = 8;                 // lanes per candidate
  constexpr int F4 = DG / 4 / LPC;       // float4 per lane per candidate
  __shared__ float sc[4096];
  __shared__ float qg[DG];
  __shared__ float red[8];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int unit = blockIdx.x;
  const int b = unit / p.Hkv, kv = unit - b * p.Hkv;
  const int L = p.ctx_len[b];
  const bool ok = (L >= 1 && L <= p.Lmax);
  int32_t* wid = p.ws_idx + static_cast<size_t>(unit) * p.S;
  float* wlg = p.ws_logg + static_cast<size_t>(unit) * p.S;
  if (!ok) {
    for (int s = tid; s < p.S; s += 512) {
      wid[s] = -1;
      wlg[s] = -INFINITY;
      if (p.idx_out) p.idx_out[static_cast<size_t>(unit) * p.S + s] = -1;
      if (p.logg_out) p.logg_out[static_cast<size_t>(unit) * p.S + s] = -INFINITY;
    }
    return;
  }
  const int c = (L - 1) / 64;
  const int ncand = c + 1;
  if (tid < DG) qg[tid] = p.q_gate[static_cast<size_t>(unit) * DG + tid];
  __syncthreads();
  const float inv_sqrt_dg = 1.0f / sqrtf(static_cast<float>(DG));
  const float* kgb = p.kg_cache + static_cast<size_t>(unit) * p.NBmax * DG;
  // 8 lanes per candidate; 64 candidates per pass over the 8 waves
  const int sub = lane & (LPC - 1);
  const int cl = lane / LPC;                 // candidate slot inside the wave
  float4 qv[F4];
#pragma unroll
  for (int f = 0; f < F4; ++f) qv[f] = *reinterpret_cast<const float4*>(&qg[(f * LPC + sub) * 4]);
  for (int j0 = 0; j0 < ncand; j0 += 128) {
    float acc[2];
    float4 kvv[2][F4];
#pragma unroll
    for (int pss = 0; pss < 2; ++pss) {
      const int j = j0 + pss * 64 + wv * 8 + cl;
#pragma unroll
      for (int f = 0; f < F4; ++f)
        kvv[pss][f] = (j < ncand) ? *reinterpret_cast<const float4*>(
                                        kgb + static_cast<size_t>(j) * DG + (f * LPC + sub) * 4)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int pss = 0; pss < 2; ++pss) {
      float a = 0.f;
#pragma unroll
      for (int f = 0; f < F4; ++f) {
        a = fmaf(qv[f].x, kvv[pss][f].x, a);
        a = fmaf(qv[f].y, kvv[pss][f].y, a);
        a = fmaf(qv[f].z, kvv[pss][f].z, a);
        a = fmaf(qv[f].w, kvv[pss][f].w, a);
      }
      a += __shfl_xor(a, 1, 64);
      a += __shfl_xor(a, 2, 64);
      a += __shfl_xor(a, 4, 64);
      acc[pss] = a;
    }
#pragma unroll
    for (int pss = 0; pss < 2; ++pss) {
      const int j = j0 + pss * 64 + wv * 8 + cl;
      if (sub == 0 && j < ncand) sc[j] = acc[pss] * inv_sqrt_dg;
    }
  }
  __syncthreads();
  // log-sum-exp over all candidates (block-wide)
  float mx = -INFINITY;
  for (int j = tid; j < ncand; j += 512) mx = fmaxf(mx, sc[j]);
  mx = wave_max(mx);
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  mx = red[0];
  for (int w = 1; w < 8; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();
  float se = 0.f;
  for (int j = tid; j < ncand; j += 512) se += expf(sc[j] - mx);
  se = wave_sum(se);
  if (lane == 0) red[wv] = se;
  __syncthreads();
  if (wv != 0) return;
  se = 0.f;
  for (int w = 0; w < 8; ++w) se += red[w];
  const float lse = mx + logf(se);

  // selection by wave 0
  const int K = p.K, S = p.S;
  const int E = (ncand + 63) / 64;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const bool all = (c <= K);
  const int nsel = min(K, c);
  uint32_t thr = 0;
  int need_eq = 0;
  if (!all) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      int cnt = 0;
      for (int e = 0; e < E; ++e) {
        const int j = lane + 64 * e;
        cnt += wave_count(j < c && order_key(sc[j]) >= cand);
      }
      if (cnt >= K) thr = cand;
    }
    int gt = 0;
    for (int e = 0; e < E; ++e) {
      const int j = lane + 64 * e;
      gt += wave_count(j < c && order_key(sc[j]) > thr);
    }
    need_eq = K - gt;
  }
  int32_t* oid = p.idx_out ? p.idx_out + static_cast<size_t>(unit) * S : nullptr;
  float* olg = p.logg_out ? p.logg_out + static_cast<size_t>(unit) * S : nullptr;
  auto put = [&](int pos, int j, float v) {
    wid[pos] = j;
    wlg[pos] = v;
    if (oid) oid[pos] = j;
    if (olg) olg[pos] = v;
  };
  int base = 0, eq_seen = 0;
  for (int e = 0; e < E; ++e) {
    const int j = lane + 64 * e;
    const bool hist = j < c;
    bool gt = false, eq = false;
    if (hist && !all) {
      const uint32_t kk = order_key(sc[j]);
      gt = kk > thr;
      eq = kk == thr;
    }
    const uint64_t em = ballot64(eq);
    const bool s_in = hist && (all || gt || (eq && (eq_seen + __popcll(em & lt_mask)) < need_eq));
    eq_seen += __popcll(em);
    const uint64_t sm = ballot64(s_in);
    if (s_in) put(base + __popcll(sm & lt_mask), j, sc[j] - lse);
    base += __popcll(sm);
  }
  if (lane == 0) put(nsel, c, sc[c] - lse);
  for (int s2 = nsel + 1 + lane; s2 < S; s2 += 64) put(s2, -1, -INFINITY);
}

// Workgroup = (unit, split): 256 threads; G <= 8 query heads of the unit.
template <int D>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeParams p) {
  constexpr int KP = D + 8;
  constexpr int UN = 64 * (D / 8);          // 16-byte units per K (or V) block
  constexpr int UPT = UN / 256;             // per thread
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[64 * KP];
  __shared__ __attribute__((aligned(16))) float qs[8 * D];
  __shared__ float ps[8][64];
  __shared__ float sm_alpha[8];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int unit = blockIdx.x, split = blockIdx.y;
  const int b = unit / p.Hkv, kv = unit - b * p.Hkv;
  const int G = p.G;
  const int L = p.ctx_len[b];
  const bool ok = (L >= 1 && L <= p.Lmax);
  const int s0 = split * kSlotsPerSplit;
  const int s1 = min(p.S, s0 + kSlotsPerSplit);
  float* part = p.ws_part + (static_cast<size_t>(unit) * p.nsplit + split) * G * (D + 2);

  for (int e = tid; e < G * D; e += 256)
    qs[e] = bf2f(p.q[(static_cast<size_t>(b) * p.Hq + kv * G) * D + e]);

  // running softmax state: head hq = wv (+4) for the dot/softmax phase; the
  // output accumulators are (head, d-pair) per thread.
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  float oacc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};   // [head rep][d pair elem]

  const int32_t* wid = p.ws_idx + static_cast<size_t>(unit) * p.S;
  const float* wlg = p.ws_logg + static_cast<size_t>(unit) * p.S;
  const uint16_t* kbase = p.k_cache + (static_cast<size_t>(b) * p.Hkv + kv) * p.Lmax * D;
  const uint16_t* vbase = p.v_cache + (static_cast<size_t>(b) * p.Hkv + kv) * p.Lmax * D;

  uint4 kr[UPT], vr[UPT];
  auto gload = [&](int j) {
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
      const int u = tid + 256 * x;
      const int row = u / (D / 8), ch = u - row * (D / 8);
      const int tok = j * 64 + row;
      const bool in = (j >= 0) && ok && tok < L;
      kr[x] = in ? *reinterpret_cast<const uint4*>(kbase + static_cast<size_t>(tok) * D + ch * 8)
                 : make_uint4(0, 0, 0, 0);
      vr[x] = in ? *reinterpret_cast<const uint4*>(vbase + static_cast<size_t>(tok) * D + ch * 8)
                 : make_uint4(0, 0, 0, 0);
    }
  };
  int jn = (ok && s0 < s1) ? wid[s0] : -1;
  gload(jn);
  for (int s = s0; s < s1; ++s) {
    const int j = jn;
    const float lg = (j >= 0) ? (p.apply_gate ? wlg[s] * kLog2e : 0.f) : 0.f;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
      const int u = tid + 256 * x;
      const int row = u / (D / 8), ch = u - row * (D / 8);
      *reinterpret_cast<uint4*>(&Ks[row * KP + ch * 8]) = kr[x];
      *reinterpret_cast<uint4*>(&Vs[row * KP + ch * 8]) = vr[x];
    }
    __syncthreads();
    jn = (ok && s + 1 < s1) ? wid[s + 1] : -1;
    if (s + 1 < s1) gload(jn);
    if (j < 0) continue;
    // scores: thread (head = wv + 4r, key = lane)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int h = wv + 4 * r;
      if (h >= G) break;
      float a = 0.f;
      const uint16_t* krow = &Ks[lane * KP];
      const float* qh = &qs[h * D];
#pragma unroll 4
      for (int d = 0; d < D; d += 8) {
        const uint4 kk = *reinterpret_cast<const uint4*>(krow + d);
        const uint32_t w4[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a = fmaf(qh[d + 2 * i], __uint_as_float(w4[i] << 16), a);
          a = fmaf(qh[d + 2 * i + 1], __uint_as_float(w4[i] & 0xffff0000u), a);
        }
      }
      const int tok = j * 64 + lane;
      float x = (tok < L) ? a * p.scale_log2 + lg : -INFINITY;
      const float mx = wave_max(x);
      const float m_new = fmaxf(m_run[r], mx);
      const float msafe = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run[r] - msafe);
      const float pe = exp2f(x - msafe);
      l_run[r] = l_run[r] * alpha + wave_sum(pe);
      m_run[r] = m_new;
      ps[h][lane] = pe;
      if (lane == 0) sm_alpha[h] = alpha;
    }
    __syncthreads();
    // O[h][d] += sum_key P[h][key] V[key][d]: thread -> (head hh = tid / (D/2), d pair)
    for (int r = 0; r < 2; ++r) {
      const int idx = tid + 256 * r;
      const int hh = idx / (D / 2), dp = idx - hh * (D / 2);
      if (hh >= G) break;
      const float al = sm_alpha[hh];
      float o0 = oacc[r][0] * al, o1 = oacc[r][1] * al;
      for (int key = 0; key < 64; ++key) {
        const float pp = ps[hh][key];
        const uint32_t w2 = *reinterpret_cast<const uint32_t*>(&Vs[key * KP + 2 * dp]);
        o0 = fmaf(pp, __uint_as_float(w2 << 16), o0);
        o1 = fmaf(pp, __uint_as_float(w2 & 0xffff0000u), o1);
      }
      oacc[r][0] = o0;
      oacc[r][1] = o1;
    }
  }
  // write partials: (m, l) by lane 0 of the head's wave, o by the (head, d pair) threads
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int h = wv + 4 * r;
    if (h < G && lane == 0) {
      part[h * (D + 2) + D] = m_run[r];
      part[h * (D + 2) + D + 1] = l_run[r];
    }
  }
  for (int r = 0; r < 2; ++r) {
    const int idx = tid + 256 * r;
    const int hh = idx / (D / 2), dp = idx - hh * (D / 2);
    if (hh >= G) break;
    part[hh * (D + 2) + 2 * dp] = oacc[r][0];
    part[hh * (D + 2) + 2 * dp + 1] = oacc[r][1];
  }
}

template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  const int unit = blockIdx.x;
  const int b = unit / p.Hkv, kv = unit - b * p.Hkv;
  const int G = p.G;
  const int L = p.ctx_len[b];
  const bool ok = (L >= 1 && L <= p.Lmax);
  for (int e = threadIdx.x; e < G * D; e += 256) {
    const int h = e / D, d = e - h * D;
    float M = -INFINITY;
    for (int sp = 0; sp < p.nsplit; ++sp) {
      const float* part = p.ws_part + ((static_cast<size_t>(unit) * p.nsplit + sp) * G + h) * (D + 2);
      M = fmaxf(M, part[D]);
    }
    float Lsum = 0.f, O = 0.f;
    for (int sp = 0; sp < p.nsplit; ++sp) {
      const float* part = p.ws_part + ((static_cast<size_t>(unit) * p.nsplit + sp) * G + h) * (D + 2);
      const float m = part[D];
      if (m == -INFINITY) continue;
      const float w = exp2f(m - M);
      Lsum += part[D + 1] * w;
      O += part[d] * w;
    }
    const float res = (ok && Lsum > 0.f) ? O / Lsum : __builtin_nanf("");
    p.o[(static_cast<size_t>(b) * p.Hq + kv * G + h) * D + d] = f2bf(res);
  }
}

}  // namespace

int decode_nsplit(int S) { return (S + kSlotsPerSplit - 1) / kSlotsPerSplit; }

hipError_t launch_decode(const DecodeParams& p, hipStream_t st) {
  const unsigned units = static_cast<unsigned>(p.B) * p.Hkv;
  switch (p.dg) {
    case 128: hipLaunchKernelGGL((decode_select_kernel<128>), dim3(units), dim3(512), 0, st, p); break;
    case 64: hipLaunchKernelGGL((decode_select_kernel<64>), dim3(units), dim3(512), 0, st, p); break;
    case 32: hipLaunchKernelGGL((decode_select_kernel<32>), dim3(units), dim3(512), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  if (p.D == 128) {
    hipLaunchKernelGGL((decode_attn_kernel<128>), dim3(units, p.nsplit), dim3(256), 0, st, p);
    hipLaunchKernelGGL((decode_combine_kernel<128>), dim3(units), dim3(256), 0, st, p);
  } else if (p.D == 64) {
    hipLaunchKernelGGL((decode_attn_kernel<64>), dim3(units, p.nsplit), dim3(256), 0, st, p);
    hipLaunchKernelGGL((decode_combine_kernel<64>), dim3(units), dim3(256), 0, st, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sas
