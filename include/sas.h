/*
 * sas.h - C ABI of libsas: SAS gated block-sparse attention on MI355X (gfx950).
 *
 * SAS ("Simple Attention Sparsification via End-to-End Optimization of
 * Context Ranking", arXiv 2609.13141) lets a lightweight router score 64-token
 * KV blocks per query, keeps the Top-K historical blocks plus the always-kept
 * current block, and adds log(gate) of each selected block inside the
 * attention softmax, so the language-modelling loss reaches the router
 * (paper abstract; GitHub README, items (a) and (b)).  Router settings come
 * from the model card's "Checkpoint configuration" table: KV block 64, Top-K
 * 31, gate hidden 128, Qproj, key pooling max + min + average, Q/K
 * normalisation, gate RoPE.
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a device pointer to contiguous memory in the
 *     layout stated beside it, 16-byte aligned.  `bf16` tensors are passed as
 *     uint16_t bit patterns.  The caller owns every buffer.
 *   - `stream` is a hipStream_t (NULL = default stream).  Work is enqueued
 *     asynchronously; the library never synchronises the device.
 *   - The library allocates no device memory.  Calls that need scratch space
 *     take a caller-provided workspace `ws` of at least the size reported by
 *     sas_workspace_size() / sas_decode_workspace_size(); the one exception,
 *     sas_decode_noalloc, uses a fixed static scratch array of the library.
 *   - All arguments are validated before anything is launched.  On any error
 *     the call returns a non-zero sas_status, writes nothing and records a
 *     message readable through sas_last_error() (thread-local).
 *   - Index and selection data computed on the device (idx, ctx_len,
 *     block_table) are range-checked by the kernels: out-of-range entries are
 *     ignored, never dereferenced.
 *   - NaN/Inf inputs propagate to outputs; selections made from NaN scores
 *     are unspecified but always in range.
 *
 * Supported specialisations: block = 64; D in {64, 128}; dg in {32, 64, 128};
 * 1 <= G = Hq / Hkv <= 8 (Hq divisible by Hkv); 0 <= topk <= 63;
 * 1 <= T <= 65536; B >= 1.
 */
#ifndef SAS_H_
#define SAS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAS_VERSION 1

typedef enum {
  SAS_OK = 0,
  SAS_ERR_INVALID = 1,      /* null pointer, bad shape or value, misalignment */
  SAS_ERR_UNSUPPORTED = 2,  /* dimensions outside the compiled specialisations */
  SAS_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  SAS_ERR_HIP = 4           /* a HIP launch failed; see sas_last_error() */
} sas_status;

/*
 * sas_dims.flags / sas_decode_dims.flags.
 *
 * SAS_FLAG_GATE_PER_QUERY_HEAD: one gate per query head instead of one per KV
 * head (the README's "per query" selection read at head granularity; the
 * released checkpoints' parameter count fits both, since Hq x D x dg =
 * Hkv x G*D x dg).  Every query head h gets its own gate query
 * q_gate[b,t,h] = RoPE_t(RMSNorm(q[b,t,h] . wq[h]) * w_qn) with wq [Hq,D,dg],
 * scores the gate keys of its KV head h/G (k_gate stays [B,T,Hkv,dg]), and
 * has its own selection and log-gates.  The "selection heads" Hs are then Hq
 * (else Hkv): q_gate [B,T,Hs,dg]; idx, logg, dlogg [B,T,Hs,K+1]; gate_lse
 * [B,T,Hs]; gate_probs [B,T,Hs,NB]; decode q_gate [B,Hs,dg] and idx_out,
 * logg_out [B,Hs,K+1].  In the attention, query head h uses its selection
 * head's slots; d log g sums over that selection head's query heads (all G
 * of a KV head, or h alone).  sas_gate_score_bwd supports only flags = 0.
 */
#define SAS_FLAG_GATE_PER_QUERY_HEAD 1

/* Operation ids for sas_workspace_size(). */
enum {
  SAS_OP_GATE_SCORE = 0,
  SAS_OP_TOPK = 1,
  SAS_OP_FWD = 2,
  SAS_OP_BWD = 3,
  SAS_OP_GATE_BWD = 4,
  SAS_OP_WALK_ORDER = 5   /* bytes of the order buffer of sas_walk_order */
};

/*
 * Prefill / training-step dimensions.
 *   B batch, T tokens, Hq query heads, Hkv KV heads (G = Hq/Hkv query heads
 *   share one KV head and, with flags = 0, one gate), D head dim, dg gate
 *   hidden size, block KV block size (must be 64), topk historical blocks K
 *   per query (S = K + 1 slots per query: K historical + the current block),
 *   rope_theta gate-RoPE base, norm_eps RMSNorm epsilon, flags 0 or
 *   SAS_FLAG_GATE_PER_QUERY_HEAD.  The layouts below are written for
 *   flags = 0 (Hkv selection heads); with the flag, read Hq for Hkv in every
 *   gate-side shape (q_gate, wq [Hq,D,dg], idx, logg, dlogg, gate_lse, gate_probs).
 */
typedef struct {
  int32_t B, T, Hq, Hkv, D, dg, block, topk;
  double rope_theta;
  float norm_eps;
  int32_t flags;
} sas_dims;

/*
 * Decode dimensions.  B sequences with one new token each; KV cache holds up
 * to Lmax tokens per sequence, the gate-key cache NBmax = ceil(Lmax/64)
 * blocks.  apply_gate = 1 adds log g to the logits (same function as
 * training); 0 = selection only, no gate bias.  kg_dtype: element type of
 * the gate-key cache, 0 = fp32, 1 = bf16 (half the bytes of the scoring
 * step; the scores are the same fp32 dot products of the bf16 values).
 */
typedef struct {
  int32_t B, Hq, Hkv, D, dg, block, topk, Lmax, NBmax, apply_gate, kg_dtype;
  int32_t flags;   /* 0 or SAS_FLAG_GATE_PER_QUERY_HEAD (q_gate, idx_out, logg_out per query head) */
} sas_decode_dims;

/* Library version (SAS_VERSION). */
int sas_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char* sas_last_error(void);

/*
 * Optional timing hook (instrumentation for profiling; no effect on results).
 * events: n_events caller-created hipEvent_t handles (n_events <= 8), or
 * NULL / 0 to switch the hook off.  While set (per thread), each following
 * sas_sparse_attn_fwd / sas_sparse_attn_bwd call records events[i] on its
 * stream at stage boundary i (boundaries beyond n_events are skipped):
 *   fwd: 0 start, 1 after the staging order and the V transpose, 2 after
 *        the attention kernel;
 *   bwd: 0 start, 1 after Delta, the CSR build and the dQ staging order,
 *        2 after dK/dV, 3 after dQ.
 * The caller owns the events and keeps them alive while the hook is set.
 */
sas_status sas_set_timing_events(void* const* events, int n_events);

/*
 * Device fault flag of the attention kernels on the current device.  Their
 * waves share LDS staging slots without workgroup barriers and wait on LDS
 * counters; a wait that does not end within about 0.1 s (a protocol error,
 * never expected) is abandoned, the affected outputs are written as NaN and
 * the flag is set.  *fault receives the flag (0 = none) and the flag is
 * cleared.  Synchronises with the device.
 */
sas_status sas_take_device_fault(unsigned* fault);

/*
 * Staging order of the query-group walks (diagnostic; the forward and dQ
 * calls make it themselves, in their workspace).  Their kernels take a group
 * of tpw consecutive tokens of one selection head, tpw = min(64, 14 * TPT)
 * with TPT = floor(16 / Gs) tokens per 16-row tile (Gs query heads per
 * selection head), and copy every KV block some token of the group selected
 * (the union) through a small LDS ring shared by the group's tiles.  This
 * writes the order in which they take the union: per group
 * g = (b * Hs + sg) * ngrp + grp (ngrp = ceil(T / tpw)), at
 * order + g * stride with stride = (NB + 8) & ~7 entries, the count nU and
 * then nU distinct block indices.  The candidates are the first 64 union
 * blocks (ascending) not yet placed, ranked by how many of the last three
 * placed blocks their busiest tile needed (fewer first), then by how many
 * tiles need them (more first), then by block; each step ranks them once
 * and places up to two: the best, then the best whose tiles are disjoint
 * from the first's.  Any order gives the same attention up to
 * floating-point summation order; this one balances the tiles' work inside
 * each window of the ring.
 *   idx: [B,T,Hs,S] int32 as sas_topk_blocks writes it (entries outside
 *        0..c(t) are ignored, as in the forward);
 *   order: device, sas_workspace_size(SAS_OP_WALK_ORDER, d) bytes.
 * Errors: SAS_ERR_INVALID (null / unaligned pointer, order_bytes too small),
 * SAS_ERR_UNSUPPORTED (dims); nothing is launched on error.
 */
sas_status sas_walk_order(const sas_dims* d, const int32_t* idx, uint16_t* order,
                          size_t order_bytes, void* stream);

/* Workspace bytes needed by op (SAS_OP_*) for dims d; 0 if none; (size_t)-1
 * if d is invalid. */
size_t sas_workspace_size(int op, const sas_dims* d);

/* Workspace bytes needed by sas_decode; (size_t)-1 if d is invalid. */
size_t sas_decode_workspace_size(const sas_decode_dims* d);

/*
 * Gate router (model card table: Qproj, max+min+average key pooling, Q/K
 * normalisation, gate RoPE; abstract: "lightweight selector").
 *
 * For batch b, KV head kappa, token t with block c = t/64:
 *   q_gate[b,t,kappa,:] = RoPE_t( RMSNorm( x_t . wq[kappa] ) * w_qn )
 *       x_t = concatenation of q[b,t,kappa*G+i,:] for i = 0..G-1  (G*D wide)
 *   k_gate[b,t,kappa,:] = RoPE_{64c}( RMSNorm( p_t . wk[kappa] ) * w_kn )
 *       p_t = [max; min; mean] channel-wise over k[b,64c..t,kappa,:]  (3D)
 * RMSNorm(y) = y / sqrt(mean(y^2) + norm_eps); RoPE rotates pairs
 * (i, i+dg/2) by pos * rope_theta^(-2i/dg) (angles reduced in double).
 * k_gate of token 64j+63 is the key of complete block j; the current block
 * of token t uses its own causal prefix key k_gate[t].
 *
 *   q      [B,T,Hq,D]  bf16      k     [B,T,Hkv,D] bf16
 *   wq     [Hkv,G*D,dg] bf16     wk    [Hkv,3*D,dg] bf16
 *   w_qn, w_kn [dg] fp32
 *   q_gate, k_gate [B,T,Hkv,dg] fp32 (outputs, fully overwritten)
 *   ws: workspace of sas_workspace_size(SAS_OP_GATE_SCORE, d) bytes
 */
sas_status sas_gate_score(const sas_dims* d, const uint16_t* q, const uint16_t* k,
                          const uint16_t* wq, const uint16_t* wk, const float* w_qn,
                          const float* w_kn, float* q_gate, float* k_gate, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Router backward (GitHub README intro (b): the continuous gate on each
 * selected block gives the LM loss a gradient path to the selector; model
 * card "Checkpoint configuration": the router's layers).
 *
 * Gradients of the router, with the selection idx held fixed, from
 * dlogg = dL/d log g per slot as sas_sparse_attn_bwd produces it.  log g =
 * s - lse(s) over the row's candidate blocks, and the row's lse is one
 * constant inside all of the row's attention logits, so that dlogg sums to
 * zero over each row's valid slots; the gradient reaching the gate logits is
 * then dlogg on the selected blocks and zero on the others, which is what
 * this call uses (for a dlogg without that property the result is the
 * gradient of sum dlogg * (s_selected - lse) without the lse term).
 * Chain rule through s_j = q_gate . key_j / sqrt(dg), the gate RoPE (its
 * transpose rotates back), RMSNorm, the projections and the pooling: a
 * channel's max / min passes its gradient to the first row of the prefix
 * that attains it, the mean to every row of the prefix.
 *
 *   q, k, wq, wk, w_qn, w_kn as for sas_gate_score;
 *   q_gate, k_gate: that call's outputs for the same inputs;
 *   idx, dlogg [B,T,Hkv,K+1] (slots outside [0, t/64] are ignored);
 *   dq [B,T,Hq,D], dk [B,T,Hkv,D] fp32: the router's part of dL/dq, dL/dk
 *   (add it to the attention's); dwq [Hkv,G*D,dg], dwk [Hkv,3*D,dg],
 *   dw_qn, dw_kn [dg] fp32.  All outputs are fully overwritten.
 *   ws: sas_workspace_size(SAS_OP_GATE_BWD, d) bytes.
 *   Deterministic (bitwise repeatable); fp32 accumulation.
 */
sas_status sas_gate_score_bwd(const sas_dims* d, const uint16_t* q, const uint16_t* k,
                              const uint16_t* wq, const uint16_t* wk, const float* w_qn,
                              const float* w_kn, const float* q_gate, const float* k_gate,
                              const int32_t* idx, const float* dlogg, float* dq, float* dk,
                              float* dwq, float* dwk, float* dw_qn, float* dw_kn, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * Candidate softmax and Top-K selection (abstract: normalised softmax gates
 * calibrate history against the always-retained current block; README (a):
 * discrete Top-K).
 *
 * For each (b, t, kappa) with c = t/64:
 *   s_j = q_gate[t] . k_gate[64j+63] / sqrt(dg)   for historical j < c
 *   s_c = q_gate[t] . k_gate[t]      / sqrt(dg)   (current block)
 *   gate_lse = logsumexp_{j<=c} s_j;  log g_j = s_j - gate_lse
 *   selection = the min(K, c) largest s_j over j < c (equal scores: lower j
 *   first) in ascending order, then c.  Slots beyond are padding.
 *
 *   idx   [B,T,Hkv,K+1] int32  selected block ids, ascending, current last, pad -1
 *   logg  [B,T,Hkv,K+1] fp32   log g of each slot, pad -inf
 *   gate_lse [B,T,Hkv] fp32
 *   gate_probs [B,T,Hkv,NB] fp32 or NULL: dense g_j (0 for j > c), NB = ceil(T/64)
 *   ws: sas_workspace_size(SAS_OP_TOPK, d) bytes (may be 0 / NULL)
 */
sas_status sas_topk_blocks(const sas_dims* d, const float* q_gate, const float* k_gate,
                           int32_t* idx, float* logg, float* gate_lse, float* gate_probs,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Gated sparse attention forward (abstract: log gate inside the attention
 * softmax; README (b): a continuous gate on each selected block; the
 * FlashAttention-style kernel mentioned in the abstract).
 *
 * For query head h (KV head kappa = h/G) and token t:
 *   l_tau = scale * q[t,h] . k[tau,kappa] + logg[t,kappa,slot(tau)]
 *   over the keys tau of the blocks in idx[t,kappa,:] with tau <= t;
 *   o[t,h] = softmax(l) . v;  lse[t,h] = logsumexp(l)  (natural log).
 *
 *   q [B,T,Hq,D], k, v [B,T,Hkv,D] bf16;  idx, logg as produced by
 *   sas_topk_blocks (entries outside [0, t/64] are ignored; the valid
 *   entries must be distinct); o [B,T,Hq,D] bf16, lse [B,T,Hq] fp32 outputs;
 *   o_f32 [B,T,Hq,D] fp32 optional output (NULL = not written): the same
 *   result before bf16 rounding, for the backward's Delta.
 *   ws: sas_workspace_size(SAS_OP_FWD, d) bytes (holds a transposed copy of
 *   v, [B,Hkv,D,64*ceil(T/64)], rebuilt on every call, plus per-block maxima
 *   and per-head scales).  With o_f32 requested, the copy is bf16 and the
 *   softmax weights P enter the PV product as bf16 hi + lo parts (o_f32 exact
 *   to ~2^-16); otherwise the copy is fp16, scaled per (b, KV head) by a power
 *   of two that keeps it finite, and P enters once in fp16 (2^-11 relative).
 *   Deterministic (bitwise repeatable).
 */
sas_status sas_sparse_attn_fwd(const sas_dims* d, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* idx, const float* logg,
                               float scale, uint16_t* o, float* lse, float* o_f32, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * Gated sparse attention backward (README (b) / abstract: the LM loss
 * reaches the selector through log g).
 *
 * With P the forward probabilities (from lse), Delta = rowsum(dout * o),
 * dS = P (dout . v - Delta):
 *   dq = scale sum dS k;  dk = scale sum dS q;  dv = sum P dout;
 *   dlogg[t,kappa,slot] = sum over the G heads of kappa and the keys of the
 *   slot's block of dS  (gradient w.r.t. log g; pads 0).
 *
 *   q, k, v, o, dout bf16 as in the forward; lse from the forward;
 *   o_f32: the forward's optional fp32 output or NULL.  When given, Delta
 *   uses it, which removes the bf16 rounding of o from dS (that rounding,
 *   times |dout| sqrt(D), otherwise dominates the error of dlogg);
 *   dq [B,T,Hq,D], dk, dv [B,T,Hkv,D] bf16 (fully overwritten, fp32
 *   accumulation); dlogg [B,T,Hkv,K+1] fp32.
 *   ws: sas_workspace_size(SAS_OP_BWD, d) bytes; it includes dS of every
 *   selected (token, head, slot) as bf16 hi + lo parts, 256 bytes each
 *   (B * T * Hq * (K+1) * 256 bytes: 8.6 GB at T = 32768, Hq = 32, K = 31),
 *   written by the dK/dV kernel and read by the dQ kernel.
 *   Deterministic (bitwise repeatable).
 */
sas_status sas_sparse_attn_bwd(const sas_dims* d, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const uint16_t* o, const float* o_f32,
                               const uint16_t* dout,
                               const float* lse, const int32_t* idx, const float* logg,
                               float scale, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                               float* dlogg, void* ws, size_t ws_bytes, void* stream);

/*
 * Budgeted single-token decode (model card: sparse decode budget of 1,024 /
 * 2,048 / 4,096 tokens = 64 (topk + 1); usage guide pitfall 3: the budget
 * bounds the tokens each query attends, not the KV cache).
 *
 * Per sequence b with L = ctx_len[b] (the new token sits at position L-1,
 * c = (L-1)/64) and KV head kappa:
 *   s_j = q_gate[b,kappa] . kg_cache[b,kappa,j] / sqrt(dg), j = 0..c
 *   (entry c is the current block's causal prefix key), selection and log g
 *   as in sas_topk_blocks, then attention of the G query heads over the
 *   selected blocks' keys tau < L, with log g added when apply_gate = 1.
 *
 *   q [B,Hq,D] bf16;  q_gate [B,Hkv,dg] fp32;
 *   k_cache, v_cache [B,Hkv,Lmax,D] bf16 (head-major contiguous cache);
 *   kg_cache [B,Hkv,NBmax,dg] fp32 (bf16 with kg_dtype = 1);  ctx_len [B]
 *   int32 (device);
 *   o [B,Hq,D] bf16 output;  idx_out [B,Hkv,K+1] int32 and logg_out
 *   [B,Hkv,K+1] fp32 outputs (either may be NULL).
 *   A sequence with ctx_len outside [1, Lmax] gets o = NaN, idx = -1.
 *   ws: sas_decode_workspace_size(d) bytes.
 */
sas_status sas_decode(const sas_decode_dims* d, const uint16_t* q, const float* q_gate,
                      const uint16_t* k_cache, const uint16_t* v_cache,
                      const float* kg_cache, const int32_t* ctx_len, float scale,
                      uint16_t* o, int32_t* idx_out, float* logg_out, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * sas_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, kernels and outputs as sas_decode, with the workspace
 * taken from a fixed 16 MiB scratch array that the library holds on each GPU
 * it runs on until the process ends.  No workspace argument; nothing is
 * allocated.  The scratch is enough for the dimensions of a serving batch
 * (for example B = 256 sequences x 8 KV heads at Lmax = 131072); dimensions
 * whose sas_decode_workspace_size exceeds 16 MiB are rejected with
 * SAS_ERR_WORKSPACE before anything is launched.  Every call on one GPU uses
 * the same scratch, which keeps the previous call's contents (nothing in it
 * needs to start at zero): calls that can overlap on one GPU (different
 * streams, or threads) race and must be ordered by the caller.  Call with the
 * device that owns the buffers current.
 */
sas_status sas_decode_noalloc(const sas_decode_dims* d, const uint16_t* q, const float* q_gate,
                              const uint16_t* k_cache, const uint16_t* v_cache,
                              const float* kg_cache, const int32_t* ctx_len, float scale,
                              uint16_t* o, int32_t* idx_out, float* logg_out, void* stream);

/*
 * Gate key of each sequence's current block for decode (model card,
 * checkpoint configuration: block pooling max + min + average, K norm, gate
 * RoPE).  With L = ctx_len[b] (the new token already written at position
 * L-1 of the KV cache) and c = (L-1)/64, per KV head kappa:
 *   p = [max; min; mean] over the cache rows 64c .. L-1 (channel-wise),
 *   kg = RoPE_{64c}(RMSNorm(p Wk[kappa]) * w_kn)
 * — the prefill gate key of token L-1 (sas_gate_score's k_gate) — written to
 * the gate-key cache entry of block c, which sas_decode / sas_decode_paged
 * then score as the current block.  Called after each appended token.
 *
 *   k_cache: [B,Hkv,Lmax,D] bf16 (block_table NULL), or the paged pool
 *   [num_pages,Hkv,64,D] with block_table [B,NBmax] as in sas_decode_paged;
 *   wk [Hkv,3D,dg] bf16, w_kn [dg] fp32, rope_theta, norm_eps as in
 *   sas_gate_score;  kg_cache: [B,Hkv,NBmax,dg] (or [num_pages,Hkv,dg]),
 *   fp32 or bf16 per d->kg_dtype; only the entries of the current blocks
 *   are written.  Sequences with ctx_len outside [1, Lmax], or whose current
 *   block's page is outside the pool, are left untouched.  fp32 arithmetic,
 *   deterministic.  No workspace.
 */
sas_status sas_decode_gate_key(const sas_decode_dims* d, const uint16_t* k_cache,
                               const int32_t* block_table, int32_t num_pages, const uint16_t* wk,
                               const float* w_kn, double rope_theta, float norm_eps,
                               const int32_t* ctx_len, void* kg_cache, void* stream);

/*
 * sas_decode over a paged KV cache: a serving backend keeps each sequence's
 * 64-token blocks in pages of a shared pool (the model card's decode runs a
 * batch of sequences of different lengths; a page is one KV block, so a
 * selected block is one page read).  Same computation and outputs as
 * sas_decode; only where block j of sequence b lives differs.
 *
 *   k_pages, v_pages [num_pages, Hkv, 64, D] bf16: page p holds one block's
 *   64 keys / values of every KV head (16 KiB contiguous per head at D = 128);
 *   kg_pages [num_pages, Hkv, dg] fp32 (bf16 with kg_dtype = 1): the
 *   block's gate key (for a sequence's current block, its causal prefix key);
 *   block_table [B, NBmax] int32 (device): page of block j of sequence b for
 *   j <= (ctx_len[b] - 1) / 64; later entries are not read.  A page outside
 *   [0, num_pages) reads as zeros (gate score 0, zero keys and values): the
 *   result is then meaningless but nothing outside the pool is touched.
 *   d->Lmax bounds ctx_len (NBmax = ceil(Lmax / 64) table columns); other
 *   arguments as in sas_decode.  ws: sas_decode_workspace_size(d) bytes.
 */
sas_status sas_decode_paged(const sas_decode_dims* d, const uint16_t* q, const float* q_gate,
                            const uint16_t* k_pages, const uint16_t* v_pages,
                            const float* kg_pages, int32_t num_pages,
                            const int32_t* block_table, const int32_t* ctx_len, float scale,
                            uint16_t* o, int32_t* idx_out, float* logg_out, void* ws,
                            size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SAS_H_ */
