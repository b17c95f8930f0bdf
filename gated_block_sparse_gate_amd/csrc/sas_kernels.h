// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bwd_index.h"
#include "sas_device.h"

namespace sas {

constexpr int kMaxNB = 1024;            // T <= 65536
constexpr int kMaxNBW = kMaxNB / 32;    // bitmap words per token
constexpr int kMaxS = 64;
constexpr int kMaxDecodeNB = 4096;      // decode: Lmax <= 262144               // topk <= 63

// Selection heads: the heads that each carry one gate and one selection.
// One gate per KV head: Hs = Hkv, Gs = G query heads per gate.  One gate per
// query head: Hs = Hq, Gs = 1.  Selection head sg attends KV head
// sg / kdiv (kdiv = Hs / Hkv) with query heads sg * Gs .. sg * Gs + Gs - 1.
struct RouterParams {
  const uint16_t* q;    // [B,T,Hq,D]
  const uint16_t* k;    // [B,T,Hkv,D]
  const uint16_t* wqT;  // [Hs,dg,Gs*D]  (transposed copy in the workspace)
  const uint16_t* wkT;  // [Hkv,dg,3*D]
  const float* w_qn;    // [dg]
  const float* w_kn;    // [dg]
  const float2* rope;   // [T, dg/2] (cos, sin)
  float* q_gate;        // [B,T,Hs,dg]
  float* k_gate;        // [B,T,Hkv,dg]
  int B, T, Hq, Hkv, D, dg, G;
  int Hs, Gs;
  float eps;
};

// Router backward: gradients of the router from dL/d log g per selected slot.
struct GateBwdParams {
  const uint16_t* q;      // [B,T,Hq,D]
  const uint16_t* k;      // [B,T,Hkv,D]
  const uint16_t* wq;     // [Hkv,G*D,dg]
  const uint16_t* wk;     // [Hkv,3*D,dg]
  const uint16_t* wqT;    // [Hkv,dg,G*D]  (transposed copy in the workspace)
  const uint16_t* wkT;    // [Hkv,dg,3*D]
  const float* w_qn;      // [dg]
  const float* w_kn;      // [dg]
  const float2* rope;     // [T, dg/2] (cos, sin)
  const float* q_gate;    // [B,T,Hkv,dg]
  const float* k_gate;    // [B,T,Hkv,dg]
  const int32_t* idx;     // [B,T,Hkv,S]
  const float* dlogg;     // [B,T,Hkv,S]
  float* dq;              // [B,T,Hq,D]    outputs
  float* dk;              // [B,T,Hkv,D]
  float* dwq;             // [Hkv,G*D,dg]
  float* dwk;             // [Hkv,3*D,dg]
  float* dw_qn;           // [dg]
  float* dw_kn;           // [dg]
  // workspace
  float* dqg;             // [B,T,Hkv,dg] dL/d q_gate
  float* dkg;             // [B,T,Hkv,dg] dL/d k_gate (per-token key)
  float* dy;              // [B,T,Hkv,dg] dL/d (x . Wq) before the norm
  float* dz;              // [B,T,Hkv,dg] dL/d (p . Wk) before the norm
  float* dzs;             // [B,T,Hkv,dg] suffix sums of dz / n over each block
  uint16_t* pmm;          // [B,T,Hkv,2D] prefix max | min pools (bf16 values)
  float* wq_part;         // [nchunk,Hkv,G*D,dg] per row-chunk partial sums
  float* wk_part;         // [nchunk,Hkv,3*D,dg]
  float* wn_part;         // [nq_part + nk_part, dg] per-workgroup norm-weight sums
  float* bk_part;         // [B*Hkv, ceil(NB / key chunk), NB, dg] block-key gradient per chunk
  int B, T, Hq, Hkv, D, dg, G, S, NB, nchunk, nq_part, nk_part;
  float eps, inv_sqrt_dg;
};

// rows per chunk of the weight-gradient reductions over tokens, and query
// blocks per chunk of the block-key gradient
constexpr int kGateBwdChunk = 1024;
constexpr int kGateBwdKeyChunk = 32;

struct TopkParams {
  const float* q_gate;  // [B,T,Hs,dg]
  const float* k_gate;  // [B,T,Hkv,dg]
  int32_t* idx;         // [B,T,Hs,S]
  float* logg;          // [B,T,Hs,S]
  float* gate_lse;      // [B,T,Hs]
  float* gate_probs;    // [B,T,Hs,NB] or null
  int B, T, Hkv, dg, K, S, NB;
  int Hs, kdiv;
};

// Dynamic LDS of the query-block walks (forward, dQ): R ring slots of `stage`
// bytes, the per-token selection bitmaps (NBW words per token) with their
// running popcounts, the union list, the log-gates (and, for dQ, slot numbers)
// by selection rank, the dQ head-sum scratch, and the ring counters.
struct WalkLds {
  int ring, bits, pcnt, ubits, ulist, lgs, slot, red, cnt, nu, total;
};
__host__ __device__ inline int align16(int x) { return (x + 15) & ~15; }
__host__ __device__ inline WalkLds walk_lds(int R, int stage, int NB, int S, int NW, bool dq) {
  const int NBW = (NB + 31) >> 5;
  WalkLds L;
  L.ring = 0;
  L.bits = R * stage;
  L.pcnt = align16(L.bits + 64 * NBW * 4);
  L.ubits = align16(L.pcnt + 64 * NBW);
  L.ulist = align16(L.ubits + NBW * 4);
  L.lgs = align16(L.ulist + NB * 2);
  L.slot = align16(L.lgs + 64 * S * 4);
  L.red = align16(L.slot + (dq ? 64 * S : 0));
  L.cnt = align16(L.red + (dq ? NW * 16 * 4 : 0));
  L.nu = L.cnt + 2 * R * 4;
  L.total = align16(L.nu + 4);
  return L;
}
constexpr int kLdsBytes = 160 * 1024;   // LDS per workgroup on gfx950

// Optional stage-boundary timing events (sas_set_timing_events).
void timing_mark(int i, hipStream_t st);

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  const float* logg;
  uint16_t* o;
  float* lse;
  float* o32;   // optional fp32 copy of o (null = skip)
  uint16_t* vt; // workspace: V^T [B,Hkv,D,64*NB] in fp16, scaled by 1/vscale
  float* vamax; // workspace: [B,Hkv,NB] max |v| per 64-token block
  float* vscale;// workspace: [B,Hkv] power of two restoring the V^T scaling
  uint16_t* order;        // workspace: staging order of each token group (walk_order)
  int ost;      // its per-group stride (uint16 entries)
  int B, T, Hq, Hkv, D, G, S, NB;
  int Hs, Gs, kdiv;   // selection heads (idx, logg [B,T,Hs,S]); rows per token = Gs
  int TPT;      // tokens per 16-row tile = floor(16 / Gs)
  int ntiles;   // tiles per 64-token query block = ceil(64 / TPT)
  float scale_log2;   // scale * log2(e)
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const float* o32;     // optional fp32 forward output (preferred for Delta)
  const uint16_t* dout;
  const float* lse;
  const int32_t* idx;
  const float* logg;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dlogg;
  // workspace
  float* delta;         // [B,T,Hq]
  int32_t* cnt2d;       // [B,Hs,NQB,NB]  per (query block, key block) counts -> offsets
  int32_t* rowptr;      // [B,Hs,NB+1]
  int32_t* entries;     // [B,Hs,T*S] packed (t << 6) | slot
  // [B,T,Hs,S,Gs][hi 64 | lo 64] bf16: dS of each selected (token, head, slot)
  // as bf16 hi + lo parts, the 64 keys of the block in MFMA operand order
  // (position 32 k2 + 8 g + e holds key 32 k2 + 4 g + e for e < 4, else
  // key 32 k2 + 16 + 4 g + e - 4)
  uint16_t* dsbuf;
  uint16_t* order;        // workspace: staging order of each dQ token group (walk_order)
  int ost;              // its per-group stride (uint16 entries)
  int B, T, Hq, Hkv, D, G, S, NB;
  int Hs, Gs, kdiv;     // selection heads (idx, logg, dlogg [B,T,Hs,S])
  int TPT, ntiles;      // tokens per 16-row tile = floor(16 / Gs)
  float scale, scale_log2;
};

struct DecodeParams {
  const uint16_t* q;        // [B,Hq,D]
  const float* q_gate;      // [B,Hs,dg]
  const uint16_t* k_cache;  // [B,Hkv,Lmax,D]
  const uint16_t* v_cache;
  const float* kg_cache;    // [B,Hkv,NBmax,dg]; paged: k/v [P,Hkv,64,D], kg [P,Hkv,dg]
  const int32_t* btab;      // paged: [B,NBmax] page of each block, else null
  int num_pages;
  const int32_t* ctx_len;   // [B]
  uint16_t* o;              // [B,Hq,D]
  int32_t* idx_out;         // [B,Hs,S] or null
  float* logg_out;          // [B,Hs,S] or null
  // workspace (one unit = one (sequence, selection head))
  int32_t* ws_idx;          // [B,Hs,S]
  float* ws_logg;           // [B,Hs,S]
  float* ws_part;           // [B,Hs,NSPLIT] records of decode_part_floats(Gs, D)
  float* ws_score;          // [B,Hs,NBmax] gate logits of the candidate blocks
  int B, Hq, Hkv, D, dg, G, K, S, Lmax, NBmax, apply_gate;
  int Hs, Gs, kdiv;         // units per sequence = selection heads; G = Gs query heads per unit
  int nsplit, spw;          // attention splits per unit, slots per split
  int kg_bf16;              // gate keys stored as bf16 (else fp32)
  float scale_log2;
};

hipError_t launch_router(const RouterParams& p, const uint16_t* wq, const uint16_t* wk,
                         uint16_t* wqT, uint16_t* wkT, float2* rope, double theta,
                         hipStream_t st);
hipError_t launch_topk(const TopkParams& p, hipStream_t st);
// out[h][n][f] = in[h][f][n] for bf16 weights
hipError_t launch_transpose_w(const uint16_t* in, uint16_t* out, int H, int F, int N,
                              hipStream_t st);
// (cos, sin) table of the gate RoPE, [T, dg/2]
hipError_t launch_rope_table(float2* tab, int T, int dg, double theta, hipStream_t st);
hipError_t launch_gate_bwd(const GateBwdParams& p, hipStream_t st);

hipError_t launch_sparse_fwd(const FwdParams& p, hipStream_t st);
// OR the ring-wait fault flag of the forward kernels into *out and clear it
hipError_t take_ring_fault_fwd(unsigned* out);
// src [B,T,H,D] -> dst [B,H,D,64*ceil(T/64)] (zero tail)
hipError_t launch_transpose_tokens(const uint16_t* src, uint16_t* dst, int B, int T, int H, int D,
                                   hipStream_t st);
// src [B,T,H,D] bf16 -> dst [B,H,D,64*ceil(T/64)] fp16 of src * 2^-e(b,h), with
// e(b,h) >= 0 the least exponent bringing max |src| of the head within
// 32768 (exact scaling); scale_out[b,h] = 2^e.  amax: [B,H,NB] workspace.
hipError_t launch_transpose_tokens_f16(const uint16_t* src, uint16_t* dst, float* amax,
                                       float* scale_out, int B, int T, int H, int D,
                                       hipStream_t st);
hipError_t launch_sparse_bwd(const BwdParams& p, hipStream_t st);
// OR the ring-wait fault flag of the backward kernels into *out and clear it
hipError_t take_ring_fault_bwd(unsigned* out);
hipError_t launch_decode(const DecodeParams& p, hipStream_t st);

struct DecodeKeyParams {
  const uint16_t* k;        // [B,Hkv,Lmax,D], or paged [P,Hkv,64,D]
  const int32_t* btab;      // paged: [B,NBmax], else null
  int num_pages;
  const uint16_t* wk;       // [Hkv,3D,dg] bf16
  const float* w_kn;        // [dg]
  const int32_t* ctx_len;   // [B]
  void* kg;                 // [B,Hkv,NBmax,dg] or paged [P,Hkv,dg]; fp32 or bf16
  int B, Hkv, D, dg, Lmax, NBmax, kg_bf16;
  double theta;
  float eps;
};
hipError_t launch_decode_gate_key(const DecodeKeyParams& p, hipStream_t st);

// decode attention splits per unit and (even) slots per split for S slots and
// units = B * Hkv (also sizes the workspace)
void decode_split(int S, int units, int* nsplit, int* spw);
// floats per decode split partial: o[G][D], then one 128-byte line holding the
// per-head running max (16 slots) and sum (16 slots); a multiple of 32 floats,
// so every partial starts on a 128-byte line and is written in whole lines
constexpr int decode_part_floats(int G, int D) { return G * D + 32; }

// Staging order of the union blocks of every token group of the query-group
// walks: group g = (b * Hs + sg) * ngrp + grp (tpw = walk_tpw(TPT) tokens per
// group) gets [nU, nU block indices] at order + g * ost.
struct WalkOrderParams {
  const int32_t* idx;   // [B,T,Hs,S]
  uint16_t* order;      // [B * Hs * ngrp][ost]
  int B, T, Hs, S, NB, TPT, ost;
};
hipError_t launch_walk_order(const WalkOrderParams& p, hipStream_t st);
size_t walk_order_smem_bytes(int NB);

// uint16 entries per group of the order buffer, and the groups of a call
inline int walk_order_stride(int NB) { return (NB + 1 + 7) & ~7; }
inline size_t walk_order_groups(int B, int T, int Hs, int TPT) {
  const int tpw = walk_tpw(TPT);
  return static_cast<size_t>(B) * Hs * ((T + tpw - 1) / tpw);
}

// dynamic LDS bytes of the Top-K kernel
size_t topk_smem_bytes(int NB, int dg);

}  // namespace sas
