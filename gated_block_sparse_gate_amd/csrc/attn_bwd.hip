// Gated sparse attention backward (README item (b) / abstract: the LM loss
// reaches the selector through the log gate inside the softmax).
//
//   Delta = rowsum(dO * O);  P = exp(scale q.k + logg - lse);  dS = P (dO.v - Delta)
//   dq = scale sum dS k;  dk = scale sum dS q;  dv = sum P dO;
//   dlogg[t, sg, slot] = sum over the Gs query heads of selection head sg
//   and the slot block's keys of dS (sg: a KV head's gate shared by its G
//   heads, Gs = G; or one query head's own gate, Gs = 1).
//
// Kernels (all deterministic, no floating-point atomics):
//   delta      : Delta per query row.
//   csr_*      : for every (b, selection head sg, key block j) the list of
//                (token, slot) that selected j, in ascending token order
//                (counting sort with per-(query block, key block) offsets).
//   dkdv       : KV-block stationary.  One workgroup per (b, kappa, j); wave w
//                owns keys 16w..16w+15 and keeps dK, dV for them in registers.
//                The rows that selected the block (the lists of every
//                selection head of kappa, one after the other) are streamed
//                as compacted 32-row tiles (two tiles of floor(16/Gs) entries
//                x Gs heads), so no MFMA row is wasted on a query that did not
//                select the block.
//   dq         : query-block stationary, same walk as the forward; also
//                produces dlogg (each (t, j) pair is visited exactly once).
#include "bwd_index.h"
#include "walk_order.h"

namespace sas {

namespace {

// Delta = rowsum(dO * o) of 16 rows per 256 threads (16 threads per row),
// rows of workgroup blk
template <int D>
__device__ __forceinline__ void delta_rows(const uint16_t* o, const float* o32,
                                           const uint16_t* dout, float* delta, long nrows,
                                           long blk) {
  constexpr int EPL = D / 16;
  const long gid = blk * 256 + threadIdx.x;
  const long row = gid >> 4;
  const int part = static_cast<int>(gid & 15);
  float acc = 0.f;
  if (row < nrows) {
    const uint16_t* pd = dout + row * D + part * EPL;
    if (o32) {
      const float* po = o32 + row * D + part * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc = fmaf(po[e], bf2f(pd[e]), acc);
    } else {
      const uint16_t* po = o + row * D + part * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc = fmaf(bf2f(po[e]), bf2f(pd[e]), acc);
    }
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  acc += __shfl_xor(acc, 4, 64);
  acc += __shfl_xor(acc, 8, 64);
  if (part == 0 && row < nrows) delta[row] = acc;
}

// Per (b, selection head sg, query block c): which of the 64 tokens selected
// each block j.
__device__ __forceinline__ void build_token_masks(const BwdParams& p, unsigned long long* mask,
                                                  int b, int sg, int c, int ntok) {
  const size_t rowbase = (static_cast<size_t>(b) * p.T + c * 64) * p.Hs + sg;
  for (int e = threadIdx.x; e < ntok * p.S; e += blockDim.x) {
    const int tl = e / p.S, s = e - tl * p.S;
    const int j = p.idx[(rowbase + static_cast<size_t>(tl) * p.Hs) * p.S + s];
    if (j >= 0 && j <= c) atomicOr(&mask[j], 1ull << tl);
  }
}

// CSR counts of query block (b, sg, c) = workgroup index bid: cnt2d[c][j] =
// how many of its tokens selected block j (mask: NB words of LDS).
__device__ __forceinline__ void csr_count_block(const BwdParams& p, unsigned long long* mask,
                                                int bid) {
  const int NQB = p.NB;
  const int sg = bid % p.Hs, rest = bid / p.Hs;
  const int c = rest % NQB, b = rest / NQB;
  const int ntok = min(64, p.T - c * 64);
  for (int j = threadIdx.x; j < p.NB; j += blockDim.x) mask[j] = 0ull;
  __syncthreads();
  build_token_masks(p, mask, b, sg, c, ntok);
  __syncthreads();
  int32_t* out = p.cnt2d + ((static_cast<size_t>(b) * p.Hs + sg) * NQB + c) * p.NB;
  for (int j = threadIdx.x; j < p.NB; j += blockDim.x) out[j] = __popcll(mask[j]);
}

// The backward's first launch: the dQ walk's staging order, the CSR counts
// and Delta side by side.  The order's workgroups (one token group per wave; a
// serial, latency-bound placement) come first, then the counts' (one query
// block each, short and latency-bound), and the Delta rows (bandwidth-bound)
// fill the slots beside them, so the three overlap.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p, WalkOrderParams wo,
                                                       int nord_blocks, int ngroups,
                                                       int wave_words, int ncnt_blocks,
                                                       long nrows) {
  extern __shared__ __attribute__((aligned(16))) uint32_t prep_smem[];
  const int bid = static_cast<int>(blockIdx.x);
  if (bid < nord_blocks) {
    const int w = threadIdx.x >> 6;
    const int g = bid * 4 + w;
    walk_order_group(wo, g, g < ngroups, threadIdx.x & 63, prep_smem + w * wave_words);
    return;
  }
  if (bid < nord_blocks + ncnt_blocks) {
    csr_count_block(p, reinterpret_cast<unsigned long long*>(prep_smem), bid - nord_blocks);
    return;
  }
  delta_rows<D>(p.o, p.o32, p.dout, p.delta, nrows,
                static_cast<long>(bid) - nord_blocks - ncnt_blocks);
}

// cnt2d[c][j] -> exclusive offset of query block c inside column j; column
// totals -> rowptr[j].  Workgroup = 16 columns x 16 segments of query blocks
// (thread: column tid % 16, segment tid / 16; 16 consecutive columns make a
// 64-byte row piece); segment sums, their exclusive scan through LDS, then
// the offsets.
__global__ __launch_bounds__(256) void csr_colscan_kernel(BwdParams p) {
  constexpr int NC = 16, NSG = 16;
  __shared__ int part[NSG][NC];
  const int cl = threadIdx.x % NC, sg = threadIdx.x / NC;
  const int j = blockIdx.x * NC + cl;
  const int bk = blockIdx.y;
  const int NQB = p.NB;
  const int seglen = (NQB + NSG - 1) / NSG;
  const int c0 = min(NQB, sg * seglen), c1 = min(NQB, c0 + seglen);
  int32_t* col = p.cnt2d + static_cast<size_t>(bk) * NQB * p.NB + j;
  int sum = 0;
  if (j < p.NB) {
#pragma unroll 8
    for (int c = c0; c < c1; ++c) sum += col[static_cast<size_t>(c) * p.NB];
  }
  part[sg][cl] = sum;
  __syncthreads();
  int off = 0;
  for (int s2 = 0; s2 < sg; ++s2) off += part[s2][cl];
  if (j < p.NB) {
    for (int c = c0; c < c1; ++c) {
      const int v = col[static_cast<size_t>(c) * p.NB];
      col[static_cast<size_t>(c) * p.NB] = off;
      off += v;
    }
    if (sg == NSG - 1) p.rowptr[static_cast<size_t>(bk) * (p.NB + 1) + j] = off;
  }
}

__global__ __launch_bounds__(1024) void csr_rowptr_kernel(BwdParams p) {
  __shared__ int wsums[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t* rp = p.rowptr + static_cast<size_t>(blockIdx.x) * (p.NB + 1);
  const int v = (tid < p.NB) ? rp[tid] : 0;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wsums[wv] = incl;
  __syncthreads();
  if (wv == 0) {
    const int s = (lane < 16) ? wsums[lane] : 0;
    const int si = wave_incl_scan(s);
    if (lane < 16) wsums[lane] = si - s;
  }
  __syncthreads();
  const int excl = incl - v + wsums[wv];
  if (tid < p.NB) rp[tid] = excl;
  if (tid == p.NB - 1) rp[p.NB] = excl + v;
}

__global__ __launch_bounds__(256) void csr_fill_kernel(BwdParams p) {
  __shared__ unsigned long long mask[kMaxNB];
  __shared__ int base[kMaxNB];
  const int NQB = p.NB;
  const int bid = blockIdx.x;
  const int sg = bid % p.Hs, rest = bid / p.Hs;
  const int c = rest % NQB, b = rest / NQB;
  const int ntok = min(64, p.T - c * 64);
  const size_t bk = static_cast<size_t>(b) * p.Hs + sg;
  for (int j = threadIdx.x; j <= c; j += 256) {
    mask[j] = 0ull;
    base[j] = p.rowptr[bk * (p.NB + 1) + j] + p.cnt2d[(bk * NQB + c) * p.NB + j];
  }
  __syncthreads();
  build_token_masks(p, mask, b, sg, c, ntok);
  __syncthreads();
  const size_t rowbase = (static_cast<size_t>(b) * p.T + c * 64) * p.Hs + sg;
  int32_t* ent = p.entries + bk * static_cast<size_t>(p.T) * p.S;
  for (int e = threadIdx.x; e < ntok * p.S; e += 256) {
    const int tl = e / p.S, s = e - tl * p.S;
    const int j = p.idx[(rowbase + static_cast<size_t>(tl) * p.Hs) * p.S + s];
    if (j >= 0 && j <= c) {
      const int pos = base[j] + __popcll(mask[j] & ((1ull << tl) - 1ull));
      ent[pos] = ((c * 64 + tl) << 6) | s;
    }
  }
}

// ---------------------------------------------------------------- dK, dV
// One workgroup = one KV block (b, kappa, j); wave w owns keys 16w..16w+15 and
// keeps their dK^T, dV^T in registers.  The rows of the queries that selected
// the block arrive as 32-row tile pairs, taken in descending token order: all
// workgroups start at the end of the sequence and sweep it at about the same
// rate, so the ones in flight on an XCD gather from nearby rows.  Software
// pipeline per tile pair `it`: the CSR entry is read 3 pairs ahead, the row
// metadata (lse, Delta, log g) 2 ahead, the Q / dO rows 1 ahead (registers),
// so the gathers overlap the MFMA work of the current pair.
template <int D>
__global__ __launch_bounds__(256) void dkdv_kernel(BwdParams p) {
  constexpr int NKS = D / 32, NDT = D / 16;
  constexpr int ROWB = D * 2;          // row-major tile row, 16-byte chunks swizzled
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int UNITS = 16 * CH;       // (chunk, row pair) units per tile pair
  constexpr int UPT = (UNITS + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint8_t Qs[2][32 * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t dOs[2][32 * ROWB];
  // row metadata of the tile pairs in flight (slot it % 4), read as 4-row
  // vectors: token (-1 = no row), log2-domain bias log g - lse, Delta, source
  // row, entry.  Pair it's slot is written during pair it - 2; its previous
  // contents (pair it - 4) were last read by that pair's dS stores during
  // pair it - 3, so the barrier that ends each pair orders every reuse.
  __shared__ __attribute__((aligned(16))) int m_t[4][32];
  __shared__ __attribute__((aligned(16))) float m_bias[4][32];
  __shared__ __attribute__((aligned(16))) float m_delta[4][32];
  __shared__ __attribute__((aligned(16))) int m_src[4][32];
  __shared__ __attribute__((aligned(16))) int m_ent[4][32];
  // dS of the tile pair, [32 rows][hi 64 | lo 64] bf16 in operand key order
  // (row pitch 272 bytes: rows 4 apart start on different banks), and each
  // wave's row sums of dS over its 16 keys; two of each, so that pair `it`
  // is written while pair it - 1 is stored
  constexpr int DSP = 272;
  __shared__ __attribute__((aligned(16))) uint8_t dsT[2][32 * DSP];
  __shared__ __attribute__((aligned(16))) float dsum[2][4][32];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int bid = blockIdx.x;
  const int kv = bid % p.Hkv, rest = bid / p.Hkv;
  const int j = rest % p.NB, b = rest / p.NB;
  // rows per CSR entry: the Gs query heads of the entry's selection head
  const int G = p.Gs, TPT = p.TPT, RT = p.TPT * G;

  const int key = j * 64 + wv * 16 + l16;
  const bool keyok = key < p.T;
  uint4 kb[NKS], vb[NKS];
  {
    const size_t off = ((static_cast<size_t>(b) * p.T + (keyok ? key : 0)) * p.Hkv + kv) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kb[ks] = keyok ? *reinterpret_cast<const uint4*>(p.k + off + ks * 32 + g4 * 8)
                     : make_uint4(0, 0, 0, 0);
      vb[ks] = keyok ? *reinterpret_cast<const uint4*>(p.v + off + ks * 32 + g4 * 8)
                     : make_uint4(0, 0, 0, 0);
    }
  }
  floatx4 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    dk[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    dv[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  // The selections that chose this block come from the kdiv selection heads
  // sg = kappa * kdiv + i of this KV head (one, with one gate per KV head):
  // their CSR lists for block j, concatenated in head order.
  __shared__ long long seg_base[8];     // first entry of head i's list for block j
  __shared__ int seg_cum[9];            // entries before head i's list
  if (tid == 0) {
    int cum = 0;
    for (int i = 0; i < p.kdiv; ++i) {
      const size_t bs = static_cast<size_t>(b) * p.Hs + kv * p.kdiv + i;
      const int e0 = p.rowptr[bs * (p.NB + 1) + j];
      seg_base[i] = static_cast<long long>(bs * static_cast<size_t>(p.T) * p.S + e0);
      seg_cum[i] = cum;
      cum += p.rowptr[bs * (p.NB + 1) + j + 1] - e0;
    }
    seg_cum[p.kdiv] = cum;
  }
  __syncthreads();
  // uniform over the workgroup: read from LDS, so made scalar explicitly (a
  // loop bound the compiler sees as per-lane turns every branch on it into
  // an exec-masked one)
  const int n = __builtin_amdgcn_readfirstlane(seg_cum[p.kdiv]);
  const int nit = (n + 2 * TPT - 1) / (2 * TPT);
  const size_t bs0 = static_cast<size_t>(b) * p.Hs + kv * p.kdiv;
  const int32_t* const ent0 =            // head i = 0's list (the only one when kdiv == 1)
      p.entries + bs0 * static_cast<size_t>(p.T) * p.S + p.rowptr[bs0 * (p.NB + 1) + j];
  const float sl2 = p.scale_log2;

  // ---- per-row metadata (threads 0..31, one row each)
  const int mr = tid & 31, mtt = mr >> 4, mrr = mr & 15;
  const int mhh = mrr - (mrr / G) * G;
  // list position of this row in tile pair `it`, and which selection head's
  // list (i, the head's index in the KV head's group) it falls in
  auto ent_pos = [&](int it) -> int { return (nit - 1 - it) * 2 * TPT + mtt * TPT + mrr / G; };
  auto seg_of = [&](int ti) -> int {
    int i = 0;
    while (i + 1 < p.kdiv && seg_cum[i + 1] <= ti) ++i;
    return i;
  };
  // raw CSR entry (token << 6 | slot) of this row in tile pair `it` (-1 past
  // the lists); it is checked and repacked only when used, an iteration
  // later, so the load is not waited for here
  auto load_ent = [&](int it) -> int {
    const int ti = ent_pos(it);
    if (mrr >= RT || ti >= n) return -1;
    if (p.kdiv == 1) return ent0[ti];
    const int i = seg_of(ti);
    return p.entries[seg_base[i] + (ti - seg_cum[i])];
  };
  float r_lse = -INFINITY, r_del = 0.f, r_lg = 0.f;
  int r_t = -1, r_src = -1, r_en = -1;
  // metadata of the row whose raw entry `en` load_ent(it) gave; the entry is
  // kept repacked as (token << 9) | (i << 6) | slot
  auto meta_issue = [&](int en, int it) {
    if (en >= 0) {
      const int tk = en >> 6, s = en & 63;
      if (tk < j * 64 || tk >= p.T || s >= p.S) en = -1;
      else en = (tk << 9) | ((p.kdiv == 1 ? 0 : seg_of(ent_pos(it))) << 6) | s;
    }
    r_t = -1; r_src = -1; r_en = en;
    if (en >= 0) {
      const int tk = en >> 9, s = en & 63;
      const int sg = kv * p.kdiv + ((en >> 6) & 7);
      const size_t qrow = (static_cast<size_t>(b) * p.T + tk) * p.Hq + sg * G + mhh;
      r_lse = p.lse[qrow];
      r_del = p.delta[qrow];
      r_lg = p.logg[((static_cast<size_t>(b) * p.T + tk) * p.Hs + sg) * p.S + s];
      r_t = tk;
      r_src = static_cast<int>(qrow);
    }
  };
  auto meta_store = [&](int slot) {
    const bool ok = r_t >= 0 && r_lse > -INFINITY;
    m_t[slot][mr] = ok ? r_t : -1;
    m_src[slot][mr] = ok ? r_src : -1;
    m_ent[slot][mr] = r_en;
    m_bias[slot][mr] = ok ? r_lg * kLog2e - r_lse * kLog2e : 0.f;
    m_delta[slot][mr] = ok ? r_del : 0.f;
  };

  // ---- Q / dO rows (all threads): unit = (chunk ch, row pair rp)
  uint4 rq[UPT][2], rd[UPT][2];
  auto rows_issue = [&](int slot) {
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
      const int u = tid + 256 * x;
      const int ch = u >> 4, rp = u & 15;
      const uint4 z = make_uint4(0, 0, 0, 0);
      const int2 sp = (u < UNITS) ? *reinterpret_cast<const int2*>(&m_src[slot][2 * rp])
                                  : make_int2(-1, -1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int src = h ? sp.y : sp.x;
        rq[x][h] = (src >= 0) ? ld16(p.q + static_cast<size_t>(src) * D + ch * 8) : z;
        rd[x][h] = (src >= 0) ? ld16(p.dout + static_cast<size_t>(src) * D + ch * 8) : z;
      }
    }
  };
  auto rows_store = [&](int buf) {
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
      const int u = tid + 256 * x;
      if (u >= UNITS) continue;
      const int ch = u >> 4, rp = u & 15;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 2 * rp + h;
        const int off = row * ROWB + ((ch ^ lds_swz<ROWB>(row)) << 4);
        st16(&Qs[buf][off], rq[x][h]);
        st16(&dOs[buf][off], rd[x][h]);
      }
    }
  };

  // ---- prologue: metadata of pairs 0, 1; rows of pair 0; entry of pair 2
  int en_n2 = -1, en_n3 = -1;
  if (tid < 32) {
    const int en0 = load_ent(0);
    const int en1 = (nit > 1) ? load_ent(1) : -1;
    meta_issue(en0, 0);
    meta_store(0);
    meta_issue(en1, 1);
    meta_store(1);
    en_n2 = (nit > 2) ? load_ent(2) : -1;
  }
  __syncthreads();
  if (nit > 0) {
    rows_issue(0);
    rows_store(0);
  }
  wait_vmem_all();
  __syncthreads();

  int qofs[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qofs[ks] = l16 * ROWB + (((ks * 4 + g4) ^ lds_swz<ROWB>(l16)) << 4);

  // Q^T / dO^T operands of dK^T = Q^T dS, dV^T = dO^T P for d tile dt: lane
  // (l16, g4) needs column 16 dt + l16 of rows 4 g4 + {0..3} and
  // 16 + 4 g4 + {0..3} (the operand order of P and dS).  A transposing read
  // (ds_read_b64_tr_b16) gives each lane of a 16-lane group one column of a
  // 4-row x 16-column block when source lane s addresses row base + s / 4,
  // columns 4 (s % 4) .. 4 (s % 4) + 3.  Rows 16 apart share their swizzle, so
  // (2 dt + h) ^ swz = 2 (dt ^ (swz >> 1)) + (h ^ (swz & 1)).
  const int trow = 4 * g4 + (l16 >> 2);
  const int tswz = lds_swz<ROWB>(trow);
  const int tbase = trow * ROWB + ((((l16 & 3) >> 1) ^ (tswz & 1)) << 4) + 8 * (l16 & 1);
  const int tx = tswz >> 1;

  // position of this lane's key (16 wv + l16) in the stored operand order
  const int kpos = 32 * (wv >> 1) + 8 * (l16 >> 2) + 4 * (wv & 1) + (l16 & 3);
  // dS rows of tile pair pp (LDS, complete after a barrier) -> global; d log g
  // of each (token, slot) = sum of its G heads' dS over the block's 64 keys
  // (each (token, slot) is in exactly one tile pair of one workgroup)
  auto store_ds = [&](int pp) __attribute__((always_inline)) {
    const int msp = pp & 3;
    // thread: 16-byte part `part` of rows r0 and r0 + 16 (same head)
    const int r0 = tid >> 4, part = tid & 15, hh = r0 % G;
    const int en0 = m_ent[msp][r0], en1 = m_ent[msp][r0 + 16];
    const uint8_t* dsp = dsT[pp & 1];
    const float(*dsu)[32] = dsum[pp & 1];
    const uint4 v0 = ld16(dsp + r0 * DSP + part * 16);
    const uint4 v1 = ld16(dsp + (r0 + 16) * DSP + part * 16);
    auto dst = [&](int en) {
      const int sg = kv * p.kdiv + ((en >> 6) & 7);
      return p.dsbuf +
             ((((static_cast<size_t>(b) * p.T + (en >> 9)) * p.Hs + sg) * p.S + (en & 63)) * G +
              hh) * 128 + part * 8;
    };
    if (en0 >= 0) st16(dst(en0), v0);
    if (en1 >= 0) st16(dst(en1), v1);
    // wave 1: d log g of one (token, slot) per lane, summed over the G heads
    // and the 4 waves' key quarters in a fixed order
    const int q = tid - 64;
    if (q >= 0 && q < 2 * TPT) {
      const int tt = q / TPT, rr = tt * 16 + (q - tt * TPT) * G;
      const int en = m_ent[msp][rr];
      float tot = 0.f;
      if ((G & 3) == 0) {
        for (int h = 0; h < G; h += 4) {
          const float4 a0 = *reinterpret_cast<const float4*>(&dsu[0][rr + h]);
          const float4 a1 = *reinterpret_cast<const float4*>(&dsu[1][rr + h]);
          const float4 a2 = *reinterpret_cast<const float4*>(&dsu[2][rr + h]);
          const float4 a3 = *reinterpret_cast<const float4*>(&dsu[3][rr + h]);
          tot += (a0.x + a1.x) + (a2.x + a3.x);
          tot += (a0.y + a1.y) + (a2.y + a3.y);
          tot += (a0.z + a1.z) + (a2.z + a3.z);
          tot += (a0.w + a1.w) + (a2.w + a3.w);
        }
      } else {
        for (int h = 0; h < G; ++h)
          tot += (dsu[0][rr + h] + dsu[1][rr + h]) + (dsu[2][rr + h] + dsu[3][rr + h]);
      }
      if (en >= 0)
        p.dlogg[((static_cast<size_t>(b) * p.T + (en >> 9)) * p.Hs + kv * p.kdiv +
                 ((en >> 6) & 7)) * p.S + (en & 63)] = tot;
    }
  };

  for (int it = 0; it < nit; ++it) {
    const int buf = it & 1, ms = it & 3;
    if (tid < 32) {
      if (it + 2 < nit) meta_issue(en_n2, it + 2);
      en_n3 = (it + 3 < nit) ? load_ent(it + 3) : -1;
    }
    if (it + 1 < nit) rows_issue((it + 1) & 3);
    if (it > 0) store_ds(it - 1);

    // S, dP for the two row tiles: [rows x 16 keys of this wave]
    floatx4 sacc[2], pacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
      pacc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint4 qa = *reinterpret_cast<const uint4*>(&Qs[buf][tt * 16 * ROWB + qofs[ks]]);
        const uint4 da = *reinterpret_cast<const uint4*>(&dOs[buf][tt * 16 * ROWB + qofs[ks]]);
        sacc[tt] = mfma16x16x32(qa, kb[ks], sacc[tt]);
        pacc[tt] = mfma16x16x32(da, vb[ks], pacc[tt]);
      }
    }
    float pv[2][4], ds[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int r = tt * 16 + g4 * 4;
      const int4 tv = *reinterpret_cast<const int4*>(&m_t[ms][r]);
      const float4 bv = *reinterpret_cast<const float4*>(&m_bias[ms][r]);
      const float4 dl = *reinterpret_cast<const float4*>(&m_delta[ms][r]);
      const int ta[4] = {tv.x, tv.y, tv.z, tv.w};
      const float ba[4] = {bv.x, bv.y, bv.z, bv.w}, da[4] = {dl.x, dl.y, dl.z, dl.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // masked entries (no query row, or a key past the token) are dropped
        // by the select, whatever the exponent gives for them
        const float e = fast_exp2(fmaf(sacc[tt][i], sl2, ba[i]));
        const float pp = (ta[i] >= 0 && key <= ta[i]) ? e : 0.f;
        pv[tt][i] = pp;
        ds[tt][i] = pp * (pacc[tt][i] - da[i]);
      }
    }
    // dS as bf16 hi + lo into tile `buf` (the other one holds pair it - 1,
    // being stored; this one was last read by the stores of pair it - 2,
    // during pair it - 1, before the barrier that ended it).  Lane (l16, g4) holds rows 4 g4 + i
    // (i = 0..3) of its key 16 wv + l16; the lanes of an even/odd key pair
    // (adjacent operand positions) swap halves so that each writes two rows
    // as 32-bit (two-key) words: the even lane rows 0, 1, the odd lane rows 2, 3.
    {
      const bool odd = l16 & 1;
      const int pe = kpos & ~1;                 // operand position of the even key
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        uint32_t h01, l01, h23, l23;           // (row 0 | row 1 << 16), ...
        split_bf2(ds[tt][0], ds[tt][1], h01, l01);
        split_bf2(ds[tt][2], ds[tt][3], h23, l23);
        const uint32_t rh = __float_as_uint(dpp_mov<0xB1>(__uint_as_float(odd ? h01 : h23)));
        const uint32_t rl = __float_as_uint(dpp_mov<0xB1>(__uint_as_float(odd ? l01 : l23)));
        const uint32_t ah = odd ? rh : h01, bh = odd ? h23 : rh;   // even key, odd key
        const uint32_t al = odd ? rl : l01, bl = odd ? l23 : rl;
        uint8_t* row0 = dsT[buf] + (tt * 16 + 4 * g4 + 2 * (l16 & 1)) * DSP + 2 * pe;
        *reinterpret_cast<uint32_t*>(row0) = __builtin_amdgcn_perm(bh, ah, 0x05040100u);
        *reinterpret_cast<uint32_t*>(row0 + 128) = __builtin_amdgcn_perm(bl, al, 0x05040100u);
        *reinterpret_cast<uint32_t*>(row0 + DSP) = __builtin_amdgcn_perm(bh, ah, 0x07060302u);
        *reinterpret_cast<uint32_t*>(row0 + DSP + 128) = __builtin_amdgcn_perm(bl, al, 0x07060302u);
        // row sums over the wave's 16 keys: halve the row set per exchange
        // (xor 1: even lanes keep rows 0, 1; xor 2: one row each), then add
        // the 4 lanes that hold the same row (rotations by 4 and 8)
        const float sa = dpp_mov<0xB1>(odd ? ds[tt][0] : ds[tt][2]);
        const float sb = dpp_mov<0xB1>(odd ? ds[tt][1] : ds[tt][3]);
        const float y0 = (odd ? ds[tt][2] : ds[tt][0]) + sa;
        const float y1 = (odd ? ds[tt][3] : ds[tt][1]) + sb;
        const bool hi2 = l16 & 2;
        float z = (hi2 ? y1 : y0) + dpp_mov<0x4E>(hi2 ? y0 : y1);
        z += dpp_mov<0x124>(z);                // row_ror:4
        z += dpp_mov<0x128>(z);                // row_ror:8
        // lane l16 < 4 now holds row 2 (l16 & 1) + (l16 >> 1) of its g4 group
        if (l16 < 4) dsum[buf][wv][tt * 16 + 4 * g4 + 2 * (l16 & 1) + (l16 >> 1)] = z;
      }
    }
    // P and dS enter the products as bf16 hi + lo parts (exact to ~2^-16)
    uint4 pb, pl, db, dl;
    split_bf2(pv[0][0], pv[0][1], pb.x, pl.x);
    split_bf2(pv[0][2], pv[0][3], pb.y, pl.y);
    split_bf2(pv[1][0], pv[1][1], pb.z, pl.z);
    split_bf2(pv[1][2], pv[1][3], pb.w, pl.w);
    split_bf2(ds[0][0], ds[0][1], db.x, dl.x);
    split_bf2(ds[0][2], ds[0][3], db.y, dl.y);
    split_bf2(ds[1][0], ds[1][1], db.z, dl.z);
    split_bf2(ds[1][2], ds[1][3], db.w, dl.w);
    // dV^T[d, key] += dO^T[d, rows] P[rows, key];  dK^T += Q^T dS
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int o = tbase + ((dt ^ tx) << 5);
      const uint2 dlo = lds_read_tr16(&dOs[buf][o]);
      const uint2 dhi = lds_read_tr16(&dOs[buf][o + 16 * ROWB]);
      const uint2 qlo = lds_read_tr16(&Qs[buf][o]);
      const uint2 qhi = lds_read_tr16(&Qs[buf][o + 16 * ROWB]);
      const uint4 dta = make_uint4(dlo.x, dlo.y, dhi.x, dhi.y);
      const uint4 qta = make_uint4(qlo.x, qlo.y, qhi.x, qhi.y);
      dv[dt] = mfma16x16x32(dta, pb, dv[dt]);
      dv[dt] = mfma16x16x32(dta, pl, dv[dt]);
      dk[dt] = mfma16x16x32(qta, db, dk[dt]);
      dk[dt] = mfma16x16x32(qta, dl, dk[dt]);
    }
    if (tid < 32 && it + 2 < nit) {
      meta_store((it + 2) & 3);
      en_n2 = en_n3;
    }
    if (it + 1 < nit) rows_store(buf ^ 1);
    // every load of this iteration has been used: with the counter empty at
    // the back edge, the next iteration's register reuse needs no wait after
    // its own new loads
    wait_vmem_all();
    __syncthreads();
  }
  if (nit > 0) store_ds(nit - 1);
  if (keyok) {
    const size_t off = ((static_cast<size_t>(b) * p.T + key) * p.Hkv + kv) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint2 pk;
      pk.x = pack_bf2(dk[dt][0] * p.scale, dk[dt][1] * p.scale);
      pk.y = pack_bf2(dk[dt][2] * p.scale, dk[dt][3] * p.scale);
      *reinterpret_cast<uint2*>(p.dk + off + dt * 16 + g4 * 4) = pk;
      pk.x = pack_bf2(dv[dt][0], dv[dt][1]);
      pk.y = pack_bf2(dv[dt][2], dv[dt][3]);
      *reinterpret_cast<uint2*>(p.dv + off + dt * 16 + g4 * 4) = pk;
    }
  }
}

// ---------------------------------------------------------------- dQ
// dQ[t, h] = scale * sum over the selected blocks j of dS[t, h, j, :] K_j,
// with dS as written by the dK/dV kernel (bf16 hi + lo parts, so the product
// is exact to ~2^-16).
//
// One workgroup = (b, kappa, a group of TPW <= 64 consecutive tokens): NCW
// compute waves, each owning one 16-row tile (TPT tokens x G heads), plus two
// stager waves.  The stagers copy the K tile of every block in the union of
// the group's selections, in the order walk_order.hip makes for the group,
// into a ring of R LDS slots with asynchronous global -> LDS copies (up to L
// blocks in flight each).  A compute wave visits only the blocks its tile
// needs: it waits for the block's slot to
// be filled, runs dQ^T += K^T dS^T on bf16 MFMA 16x16x32 (K^T read from the K
// rows with transposing LDS reads, dS rows loaded from memory, zero rows for
// tokens that did not select the block), and the dS rows of its next needed
// block start loading right after.
//
// Protocol (all counters in LDS, only growing; no workgroup barrier):
//  * prog[c]: compute wave c is done with every staged position below
//    prog[c] (it sets it to the position of its next needed block after
//    reading one, nU at the end);
//  * a stager copies its half of block n into slot n % R once
//    min_c prog[c] >= n - R + 1, and bumps fill[n % R] once the copies have
//    landed (s_waitcnt vmcnt); before it waits for a slot it publishes all
//    its copies in flight;
//  * a compute wave reads block v once fill[v % R] >= 2 * (v / R + 1).
// Stagers and compute waves run disjoint code, so the compute waves' LDS reads
// carry no compiler-inserted wait for the copies.
constexpr int kDqStagers = 2;
constexpr int kDqInflight = 3;      // blocks in flight per stager (< R)

template <int D, int R>
__global__ __launch_bounds__(1024) void dq_kernel(BwdParams a, int ncw, int tpw) {
  constexpr int KROWB = D * 2;              // bytes per K row
  constexpr int STAGE = 64 * KROWB;         // K tile
  constexpr int TU = STAGE / 16;            // 16-byte units per tile
  constexpr int UPS = TU / kDqStagers;      // units per stager per block
  constexpr int MPS = UPS / 64;             // copies per stager per block
  constexpr int KCPR = KROWB / 16;
  constexpr int NDT = D / 16;
  static_assert(UPS % 64 == 0 && R > kDqInflight, "stager split / ring depth");

  __shared__ __attribute__((aligned(16))) uint8_t ring[R * STAGE];
  __shared__ uint32_t bits[64 * kMaxNBW];     // per-token selection bitmaps [64][NBW]
  __shared__ uint8_t pcnt[64 * kMaxNBW];      // popcount prefix per word
  __shared__ uint16_t ulist[kMaxNB];          // union blocks in staging order
  __shared__ uint8_t slot_of[64 * kMaxS];     // slot numbers by selection rank [64][S]
  __shared__ uint32_t actw[14 * kMaxNBW];     // per compute wave: which union blocks it needs
  __shared__ int prog[16];
  __shared__ unsigned fill_cnt[R];
  __shared__ int s_nU;

  const int tid = threadIdx.x;
  const int NT = blockDim.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int NBW = (a.NB + 31) >> 5;
  const int S = a.S;

  const int ngrp = (a.T + tpw - 1) / tpw;
  const int bid = blockIdx.x;
  const int sg = bid % a.Hs;             // selection head
  const int kv = sg / a.kdiv;            // its KV head
  const int rest = bid / a.Hs;
  const int grp = ngrp - 1 - (rest % ngrp);   // late (long) groups first
  const int b = rest / ngrp;
  const int t0 = grp * tpw;
  const int ntok = min(tpw, a.T - t0);

  // ---- selection bitmaps of the group's tokens, their union, slots by rank
  for (int i = tid; i < 64 * NBW; i += NT) bits[i] = 0u;
  if (tid < 16) prog[tid] = 0;
  if (tid < R) fill_cnt[tid] = 0u;
  __syncthreads();
  const size_t rowbase = (static_cast<size_t>(b) * a.T + t0) * a.Hs + sg;
  for (int e = tid; e < ntok * S; e += NT) {
    const int tl = e / S, s = e - tl * S;
    const size_t off = (rowbase + static_cast<size_t>(tl) * a.Hs) * S + s;
    const int j = a.idx[off];
    if (j >= 0 && j <= (t0 + tl) / 64) {
      atomicOr(&bits[tl * NBW + (j >> 5)], 1u << (j & 31));
    } else {
      a.dlogg[off] = 0.f;     // padding / ignored slot (the others come from dK/dV)
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
    const size_t off = (rowbase + static_cast<size_t>(tl) * a.Hs) * S + s;
    const int j = a.idx[off];
    if (j >= 0 && j <= (t0 + tl) / 64) {
      const int rank = pcnt[tl * NBW + (j >> 5)] + __popc(bits[tl * NBW + (j >> 5)] & ((1u << (j & 31)) - 1u));
      if (rank < S) slot_of[tl * S + rank] = static_cast<uint8_t>(s);
    }
  }
  // the union of the group's selections in the staging order that spreads
  // each compute wave's blocks over the ring windows (walk_order.hip)
  {
    const uint16_t* ord =
        a.order + ((static_cast<size_t>(b) * a.Hs + sg) * ngrp + grp) * static_cast<size_t>(a.ost);
    const int n = min(static_cast<int>(ord[0]), a.NB);    // in range whatever it holds
    for (int i = tid; i < n; i += NT) ulist[i] = static_cast<uint16_t>(min(static_cast<int>(ord[1 + i]), a.NB - 1));
    if (tid == 0) s_nU = n;
  }
  wait_vmem_all();
  __syncthreads();
  const int nU = __builtin_amdgcn_readfirstlane(s_nU);
  const unsigned nstg = kDqStagers;

  if (wv >= ncw) {
    // ================================================================ stager
    const int stg = wv - ncw;                                // 0 or 1
    const uint16_t* kbase = a.k + (static_cast<size_t>(b) * a.T * a.Hkv + kv) * D;
    const int tokstride = a.Hkv * D;       // offsets inside one batch's K fit 32 bits
    int grow[MPS], gch[MPS];
#pragma unroll
    for (int m = 0; m < MPS; ++m) {
      const int pu = stg * UPS + m * 64 + lane;
      grow[m] = pu / KCPR;
      gch[m] = ((pu % KCPR) ^ lds_swz<KROWB>(grow[m])) * 8;
    }
    // smallest progress word of the compute waves (lanes < ncw <= 14 < 16)
    auto min_prog = [&]() __attribute__((always_inline)) {
      asm volatile("" ::: "memory");
      int v = l16 < ncw ? prog[l16] : 0x7fffffff;
      asm volatile("" ::: "memory");
      v = min(v, __float_as_int(dpp_mov<0xB1>(__int_as_float(v))));
      v = min(v, __float_as_int(dpp_mov<0x4E>(__int_as_float(v))));
      v = min(v, __float_as_int(dpp_mov<0x141>(__int_as_float(v))));
      v = min(v, __float_as_int(dpp_mov<0x140>(__int_as_float(v))));
      return __builtin_amdgcn_readfirstlane(v);
    };
    int oldest = 0;                  // oldest block copied but not published
    bool failed = false;
    for (int n = 0; n < nU && !failed; ++n) {
      if (min_prog() < n - R + 1) {
        // publish everything in flight, then wait for the slot
        wait_vmem_all();
        asm volatile("" ::: "memory");
        for (; oldest < n; ++oldest) ring_bump(&fill_cnt[oldest % R], lane);
        for (int it = 0; min_prog() < n - R + 1; ++it) {
          if (it == kSpinLimit) {
            failed = true;
            break;
          }
          __builtin_amdgcn_s_sleep(kStagerNap);
        }
        if (failed) break;
      }
      const int j = ulist[n];
      uint8_t* dst = ring + (n % R) * STAGE + stg * UPS * 16;
#pragma unroll
      for (int m = 0; m < MPS; ++m)
        load_lds16(kbase + (min(j * 64 + grow[m], a.T - 1) * tokstride + gch[m]), dst + m * 1024);
      if (n - oldest + 1 == kDqInflight) {
        // the oldest block's copies are older than the (kDqInflight - 1)
        // newer blocks' copies: wait for them, then publish it
        __builtin_amdgcn_s_waitcnt(0x0f70 | (((kDqInflight - 1) * MPS) & 15) |
                                   ((((kDqInflight - 1) * MPS) >> 4) << 14));
        asm volatile("" ::: "memory");
        ring_bump(&fill_cnt[oldest % R], lane);
        ++oldest;
      }
    }
    wait_vmem_all();       // no copy may still be landing when the workgroup ends
    asm volatile("" ::: "memory");
    if (failed) {
      ring_fault(lane);
    } else {
      for (; oldest < nU; ++oldest) ring_bump(&fill_cnt[oldest % R], lane);
    }
    return;
  }

  // ================================================================ compute
  const int G = a.Gs, TPT = a.TPT;       // query heads per token row group
  const int tile = wv;
  const WalkRow wrow = walk_row(tile, l16, TPT, G, ntok);
  const int tl_row = wrow.tl;
  const int hh = wrow.hh;
  bool valid = wrow.live;
  {
    const size_t qrow = (static_cast<size_t>(b) * a.T + t0 + tl_row) * a.Hq + sg * G + hh;
    valid = valid && (a.lse[qrow] > -INFINITY);
  }
  floatx4 dqa[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dqa[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // activity of the tile for every union block: bit v of actw[wv] = some
  // token of the tile selected block ulist[v]
  for (int v0 = 0; v0 < nU; v0 += 64) {
    const int v = v0 + lane;
    bool any = false;
    if (v < nU) {
      const int j = ulist[v];
      for (int k = 0; k < TPT; ++k) {
        const int tl = tile * TPT + k;
        if (tl < ntok) any = any || ((bits[tl * NBW + (j >> 5)] >> (j & 31)) & 1u);
      }
    }
    const uint64_t m = ballot64(any);
    if (lane == 0) {
      actw[wv * NBW + (v0 >> 5)] = static_cast<uint32_t>(m);
      if ((v0 >> 5) + 1 < NBW) actw[wv * NBW + (v0 >> 5) + 1] = static_cast<uint32_t>(m >> 32);
    }
  }
  auto next_active = [&](int v) __attribute__((always_inline)) {
    while (v < nU) {
      const uint32_t w = __builtin_amdgcn_readfirstlane(actw[wv * NBW + (v >> 5)]) >> (v & 31);
      if (w) return min(v + static_cast<int>(__builtin_ctz(w)), nU);
      v = (v | 31) + 1;
    }
    return nU;
  };

  // dS of (token tl, slot sl, head hh) at dsq + ((tl * Hs * S + sl) * G + hh) * 128
  const uint16_t* const dsq = a.dsbuf + rowbase * S * G * 128;
  const int HSG = a.Hs * S;
  // dS rows of the tile for union block v (two blocks in flight).  Every
  // lane issues its loads, so the loads of one block never wait behind the
  // other's; through a buffer over this group's dS rows, a lane whose row did
  // not select the block (or that has no row) reads at an offset past the
  // buffer, which returns zeros without a memory request.
  // bytes from this group's first row to the end of its last token's rows of kappa
  const unsigned dsbytes = dq_ds_bytes(ntok, HSG, S, G);
  const auto dsr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(dsq), 0,
                                                     static_cast<int>(dsbytes), kBufferWord3);
  struct DsRows { uint4 h[2], l[2]; };
  auto load_ds = [&](int v, DsRows& r) __attribute__((always_inline)) {
    unsigned off = dsbytes;
    if (v < nU) {
      const int j = ulist[v];
      const int jw = j >> 5;
      const uint32_t jbit = 1u << (j & 31);
      const bool take = valid && (bits[tl_row * NBW + jw] & jbit);
      int sl = 0;
      if (take) {
        const int rank = pcnt[tl_row * NBW + jw] + __popc(bits[tl_row * NBW + jw] & (jbit - 1u));
        sl = slot_of[tl_row * S + rank];
      }
      off = dq_ds_offset(take, tl_row, HSG, sl, G, hh, g4, dsbytes);
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      r.h[k2] = buffer_ld16(dsr, off + 64 * k2);
      r.l[k2] = buffer_ld16(dsr, off + 128 + 64 * k2);
    }
  };

  // K^T operand of dQ^T = K^T dS^T for d tile dt and 32-key step k2: lane
  // (l16, g4) needs K[key][16 dt + l16] for keys 32 k2 + 4 g4 + {0..3} and
  // 32 k2 + 16 + 4 g4 + {0..3} (the stored operand order of dS).  A
  // transposing read (ds_read_b64_tr_b16) gives each lane of a 16-lane group
  // one column of a 4-row x 16-column block when source lane s addresses row
  // base + s / 4, columns 4 (s % 4) .. 4 (s % 4) + 3.  The row's swizzle
  // depends only on the lane (the steps between reads are multiples of 16
  // rows); (2 dt + h) ^ swz = 2 (dt ^ (swz >> 1)) + (h ^ (swz & 1)).
  const int trow = 4 * g4 + (l16 >> 2);
  const int tswz = lds_swz<KROWB>(trow);
  const int tbase0 = trow * KROWB + ((((l16 & 3) >> 1) ^ (tswz & 1)) << 4) + 8 * (l16 & 1);
  const int tx = tswz >> 1;

  bool failed = false;
  // block v from ring slot v % R with its dS rows r
  auto process = [&](int v, const DsRows& r) __attribute__((always_inline)) {
    const int sl = v % R;
    const unsigned need = nstg * static_cast<unsigned>(v / R + 1);
    for (int it = 0; ring_count(&fill_cnt[sl]) < need; ++it) {
      if (it == kSpinLimit) {
        failed = true;
        return;
      }
      __builtin_amdgcn_s_sleep(kComputeNap);
    }
    const uint8_t* st = ring + sl * STAGE;
    int tbase = tbase0;
    asm volatile("" : "+v"(tbase));     // recomputed per block rather than kept live
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint8_t* tp = st + tbase + ((dt ^ tx) << 5);
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const uint2 lo = lds_read_tr16(tp + k2 * 32 * KROWB);
        const uint2 hi = lds_read_tr16(tp + (k2 * 32 + 16) * KROWB);
        const uint4 kta = make_uint4(lo.x, lo.y, hi.x, hi.y);
        dqa[dt] = mfma16x16x32(kta, r.h[k2], dqa[dt]);
        dqa[dt] = mfma16x16x32(kta, r.l[k2], dqa[dt]);
      }
    }
  };
  // two active blocks in flight: A holds v0's rows, B v1's
  DsRows ra, rb;
  int v0 = next_active(0);
  load_ds(v0, ra);
  int v1 = next_active(v0 + 1);
  load_ds(v1, rb);
  asm volatile("" ::: "memory");
  prog[wv] = v0;                // done with every block before its first needed one
  while (v0 < nU) {
    process(v0, ra);
    if (failed) break;
    asm volatile("" ::: "memory");
    if (lane == 0) prog[wv] = v1;     // after this wave's last read of v0's slot
    asm volatile("" ::: "memory");
    const int v2 = next_active(v1 + 1);
    load_ds(v2, ra);
    if (v1 >= nU) break;
    process(v1, rb);
    if (failed) break;
    asm volatile("" ::: "memory");
    if (lane == 0) prog[wv] = v2;
    asm volatile("" ::: "memory");
    const int v3 = next_active(v2 + 1);
    load_ds(v3, rb);
    v0 = v2;
    v1 = v3;
  }
  wait_vmem_all();              // the last prefetches are unused
  if (failed) {
    ring_fault(lane);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dqa[dt] = floatx4{NAN, NAN, NAN, NAN};
    // let the stagers finish: this wave needs nothing more
    asm volatile("" ::: "memory");
    if (lane == 0) prog[wv] = nU;
  }

  if (l16 < TPT * G && tile * TPT + l16 / G < ntok) {
    const size_t row = (static_cast<size_t>(b) * a.T + t0 + tl_row) * a.Hq + sg * G + hh;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint2 pk;
      pk.x = pack_bf2(dqa[dt][0] * a.scale, dqa[dt][1] * a.scale);
      pk.y = pack_bf2(dqa[dt][2] * a.scale, dqa[dt][3] * a.scale);
      *reinterpret_cast<uint2*>(a.dq + row * D + dt * 16 + g4 * 4) = pk;
    }
  }
}

// Tokens per workgroup: 14 compute waves of TPT tokens each, at most 64.
// Static LDS: ring of 8 K tiles (D = 128: 128 KiB) plus the selection data.
template <int D>
hipError_t launch_dq(const BwdParams& p, hipStream_t st) {
  const int tpw = walk_tpw(p.TPT);
  const int ncw = walk_ncw(p.TPT);
  const unsigned ngrp = (p.T + tpw - 1) / tpw;
  const dim3 grid(static_cast<unsigned>(p.B) * p.Hs * ngrp);
  hipLaunchKernelGGL((dq_kernel<D, 8>), grid, dim3((ncw + kDqStagers) * 64), 0, st, p, ncw, tpw);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t st) {
  const long nrows = static_cast<long>(p.B) * p.T * p.Hq;
  timing_mark(0, st);
  {
    const WalkOrderParams wo{p.idx, p.order, p.B, p.T, p.Hs, p.S, p.NB, p.TPT, p.ost};
    const int ngroups = static_cast<int>(walk_order_groups(p.B, p.T, p.Hs, p.TPT));
    const int nord = (ngroups + 3) / 4;
    const size_t wave_bytes = walk_order_smem_bytes(p.NB);
    const long ndelta = (nrows * 16 + 255) / 256;
    const int ncnt = p.B * p.Hs * p.NB;
    // four waves' staging-order scratch; the counts' NB mask words fit in it
    const size_t lds = std::max(4 * wave_bytes, sizeof(unsigned long long) * p.NB);
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3(static_cast<unsigned>(nord + ncnt + ndelta)),
                       dim3(256), lds, st, p, wo, nord, ngroups, static_cast<int>(wave_bytes / 4),
                       ncnt, nrows);
  }
  const int NQB = p.NB;
  const unsigned nblk = static_cast<unsigned>(p.B) * p.Hs * NQB;
  hipLaunchKernelGGL(csr_colscan_kernel, dim3((p.NB + 15) / 16, p.B * p.Hs), dim3(256), 0, st, p);
  hipLaunchKernelGGL(csr_rowptr_kernel, dim3(p.B * p.Hs), dim3(1024), 0, st, p);
  hipLaunchKernelGGL(csr_fill_kernel, dim3(nblk), dim3(256), 0, st, p);
  timing_mark(1, st);
  hipLaunchKernelGGL((dkdv_kernel<D>), dim3(static_cast<unsigned>(p.B) * p.Hkv * p.NB),
                     dim3(256), 0, st, p);
  timing_mark(2, st);
  const hipError_t e = launch_dq<D>(p, st);
  if (e != hipSuccess) return e;
  timing_mark(3, st);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_bwd(const BwdParams& p, hipStream_t st) {
  if (p.D == 128) return launch_bwd_d<128>(p, st);
  if (p.D == 64) return launch_bwd_d<64>(p, st);
  return hipErrorInvalidValue;
}

hipError_t take_ring_fault_bwd(unsigned* out) {
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
