// C ABI of libsas: argument validation, workspace layout and dispatch.
// Every check runs before any launch; on failure nothing is written.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/sas.h"
#include "sas_kernels.h"

namespace {

thread_local std::string g_err;
constexpr int kMaxTimingEvents = 8;
thread_local hipEvent_t g_ev[kMaxTimingEvents];
thread_local int g_nev = 0;

sas_status fail(sas_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

sas_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SAS_OK;
  return fail(SAS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Selection heads (the heads that carry one gate each): the KV heads, whose
// gate the G query heads of each share, or with SAS_FLAG_GATE_PER_QUERY_HEAD
// every query head.  Gs query heads per selection head; selection head sg
// attends KV head sg / kdiv.
struct SelHeads { int Hs, Gs, kdiv; };
SelHeads sel_heads(int Hq, int Hkv, int flags) {
  const int G = Hq / Hkv;
  if (flags & SAS_FLAG_GATE_PER_QUERY_HEAD) return SelHeads{Hq, 1, G};
  return SelHeads{Hkv, G, 1};
}

sas_status check_dims(const sas_dims* d) {
  if (!d) return fail(SAS_ERR_INVALID, "dims pointer is null");
  if (d->flags & ~SAS_FLAG_GATE_PER_QUERY_HEAD)
    return fail(SAS_ERR_INVALID, "dims.flags: unknown bits 0x%x", d->flags & ~SAS_FLAG_GATE_PER_QUERY_HEAD);
  if (d->B < 1 || d->T < 1 || d->Hq < 1 || d->Hkv < 1)
    return fail(SAS_ERR_INVALID, "B, T, Hq, Hkv must be >= 1 (got %d, %d, %d, %d)", d->B, d->T,
                d->Hq, d->Hkv);
  if (d->Hq % d->Hkv) return fail(SAS_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)",
                                  d->Hq, d->Hkv);
  const int G = d->Hq / d->Hkv;
  if (G > 8) return fail(SAS_ERR_UNSUPPORTED, "G = Hq/Hkv = %d > 8 is not supported", G);
  if (d->block != 64) return fail(SAS_ERR_UNSUPPORTED, "block must be 64 (got %d)", d->block);
  if (d->D != 64 && d->D != 128)
    return fail(SAS_ERR_UNSUPPORTED, "head dim D must be 64 or 128 (got %d)", d->D);
  if (d->dg != 32 && d->dg != 64 && d->dg != 128)
    return fail(SAS_ERR_UNSUPPORTED, "gate hidden dg must be 32, 64 or 128 (got %d)", d->dg);
  if (d->topk < 0) return fail(SAS_ERR_INVALID, "topk must be >= 0 (got %d)", d->topk);
  if (d->topk + 1 > sas::kMaxS)
    return fail(SAS_ERR_UNSUPPORTED, "topk must be <= %d (got %d)", sas::kMaxS - 1, d->topk);
  if (d->T > sas::kMaxNB * 64)
    return fail(SAS_ERR_UNSUPPORTED, "T must be <= %d (got %d)", sas::kMaxNB * 64, d->T);
  if (static_cast<long long>(d->T) * d->Hkv * d->D > 0x7fffffffLL)
    return fail(SAS_ERR_UNSUPPORTED, "T * Hkv * D must be < 2^31 (one batch's K fits 32-bit offsets)");
  if (!(d->norm_eps >= 0.f) || !std::isfinite(d->norm_eps))
    return fail(SAS_ERR_INVALID, "norm_eps must be finite and >= 0");
  if (!(d->rope_theta > 0.0) || !std::isfinite(d->rope_theta))
    return fail(SAS_ERR_INVALID, "rope_theta must be finite and > 0");
  if (static_cast<long long>(d->B) * d->Hkv * ((d->T + 63) / 64) > 0x7fffffffLL)
    return fail(SAS_ERR_UNSUPPORTED, "grid too large");
  if (static_cast<long long>(d->B) * d->T * d->Hq > 0x7fffffffLL)
    return fail(SAS_ERR_UNSUPPORTED, "B*T*Hq must be < 2^31");
  return SAS_OK;
}

#define REQ_PTR(p)                                                                   \
  do {                                                                               \
    if (!(p)) return fail(SAS_ERR_INVALID, "pointer '%s' is null", #p);             \
    if (!aligned16(p)) return fail(SAS_ERR_INVALID, "pointer '%s' is not 16-byte aligned", #p); \
  } while (0)

// workspace layouts ------------------------------------------------------
struct GateWs { size_t wqT, wkT, rope, total; };
GateWs gate_ws(const sas_dims* d) {
  const SelHeads sh = sel_heads(d->Hq, d->Hkv, d->flags);
  GateWs w;
  w.wqT = 0;
  w.wkT = align_up(w.wqT + sizeof(uint16_t) * sh.Hs * d->dg * sh.Gs * d->D);
  w.rope = align_up(w.wkT + sizeof(uint16_t) * d->Hkv * d->dg * 3 * d->D);
  w.total = align_up(w.rope + sizeof(float2) * static_cast<size_t>(d->T) * (d->dg / 2));
  return w;
}

struct GateBwdWs {
  size_t wqT, wkT, rope, dqg, dkg, dy, dz, dzs, pmm, wq_part, wk_part, wn_part, bk_part, total;
  int nchunk, nq_part, nk_part;
};
GateBwdWs gate_bwd_ws(const sas_dims* d) {
  const int G = d->Hq / d->Hkv;
  const size_t NB = (d->T + 63) / 64;
  const size_t rows = static_cast<size_t>(d->B) * d->T;
  const size_t rk = rows * d->Hkv;
  GateBwdWs w;
  w.nchunk = static_cast<int>((rows + sas::kGateBwdChunk - 1) / sas::kGateBwdChunk);
  w.nq_part = static_cast<int>(d->Hkv * ((rows + 127) / 128));
  w.nk_part = static_cast<int>(d->B * d->Hkv * NB);
  w.wqT = 0;
  w.wkT = align_up(w.wqT + sizeof(uint16_t) * d->Hkv * d->dg * G * d->D);
  w.rope = align_up(w.wkT + sizeof(uint16_t) * d->Hkv * d->dg * 3 * d->D);
  w.dqg = align_up(w.rope + sizeof(float2) * static_cast<size_t>(d->T) * (d->dg / 2));
  w.dkg = align_up(w.dqg + sizeof(float) * rk * d->dg);
  w.dy = align_up(w.dkg + sizeof(float) * rk * d->dg);
  w.dz = align_up(w.dy + sizeof(float) * rk * d->dg);
  w.dzs = align_up(w.dz + sizeof(float) * rk * d->dg);
  w.pmm = align_up(w.dzs + sizeof(float) * rk * d->dg);
  w.wq_part = align_up(w.pmm + sizeof(uint16_t) * rk * 2 * d->D);
  w.wk_part = align_up(w.wq_part + sizeof(float) * w.nchunk * d->Hkv * G * d->D * d->dg);
  w.wn_part = align_up(w.wk_part + sizeof(float) * w.nchunk * d->Hkv * 3 * d->D * d->dg);
  w.bk_part = align_up(w.wn_part + sizeof(float) * (static_cast<size_t>(w.nq_part) + w.nk_part) * d->dg);
  const size_t ntc = (NB + sas::kGateBwdKeyChunk - 1) / sas::kGateBwdKeyChunk;
  w.total = align_up(w.bk_part + sizeof(float) * d->B * d->Hkv * ntc * NB * d->dg);
  return w;
}

// staging orders of the query-group walks (forward, dQ): one per token group
size_t walk_order_bytes(const sas_dims* d) {
  const SelHeads sh = sel_heads(d->Hq, d->Hkv, d->flags);
  const int NB = (d->T + 63) / 64;
  return sizeof(uint16_t) * sas::walk_order_stride(NB) *
         sas::walk_order_groups(d->B, d->T, sh.Hs, 16 / sh.Gs);
}

struct FwdWs { size_t vt, amax, vscale, order, total; };
FwdWs fwd_ws_layout(const sas_dims* d) {
  const size_t NB = (d->T + 63) / 64;
  FwdWs w;
  w.vt = 0;
  w.amax = align_up(sizeof(uint16_t) * d->B * d->Hkv * d->D * NB * 64);
  w.vscale = align_up(w.amax + sizeof(float) * d->B * d->Hkv * NB);
  w.order = align_up(w.vscale + sizeof(float) * d->B * d->Hkv);
  w.total = align_up(w.order + walk_order_bytes(d));
  return w;
}
size_t fwd_ws(const sas_dims* d) { return fwd_ws_layout(d).total; }

struct BwdWs { size_t delta, cnt2d, rowptr, entries, order, ds, total; };
BwdWs bwd_ws(const sas_dims* d) {
  const size_t NB = (d->T + 63) / 64;
  const size_t S = d->topk + 1;
  const size_t Hs = sel_heads(d->Hq, d->Hkv, d->flags).Hs;
  BwdWs w;
  w.delta = 0;
  w.cnt2d = align_up(w.delta + sizeof(float) * static_cast<size_t>(d->B) * d->T * d->Hq);
  w.rowptr = align_up(w.cnt2d + sizeof(int32_t) * d->B * Hs * NB * NB);
  w.entries = align_up(w.rowptr + sizeof(int32_t) * d->B * Hs * (NB + 1));
  w.order = align_up(w.entries + sizeof(int32_t) * static_cast<size_t>(d->B) * Hs * d->T * S);
  w.ds = align_up(w.order + walk_order_bytes(d));
  // dS of every selected (token, head, slot): 64 keys x (hi, lo) bf16
  w.total = align_up(w.ds + 256 * static_cast<size_t>(d->B) * d->T * d->Hq * S);
  return w;
}

struct DecWs { size_t idx, logg, part, score, total; int nsplit, spw; };
DecWs dec_ws(const sas_decode_dims* d) {
  const size_t S = d->topk + 1;
  const SelHeads sh = sel_heads(d->Hq, d->Hkv, d->flags);
  const size_t units = static_cast<size_t>(d->B) * sh.Hs;    // (sequence, selection head)
  DecWs w;
  sas::decode_split(static_cast<int>(S), static_cast<int>(units), &w.nsplit, &w.spw);
  w.idx = 0;
  w.logg = align_up(w.idx + sizeof(int32_t) * units * S);
  w.part = align_up(w.logg + sizeof(float) * units * S);
  // split partials (none with one split per unit)
  const size_t nparts = w.nsplit > 1 ? units * w.nsplit : 0;
  w.score = align_up(w.part + sizeof(float) * nparts * sas::decode_part_floats(sh.Gs, d->D));
  w.total = align_up(w.score + sizeof(float) * units * d->NBmax);
  return w;
}

sas_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return SAS_OK;
  if (!ws) return fail(SAS_ERR_WORKSPACE, "workspace is null but %zu bytes are required", need);
  if (!aligned16(ws)) return fail(SAS_ERR_INVALID, "workspace is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(SAS_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  return SAS_OK;
}

sas_status check_decode_dims(const sas_decode_dims* d) {
  if (!d) return fail(SAS_ERR_INVALID, "decode dims pointer is null");
  if (d->B < 1 || d->Hq < 1 || d->Hkv < 1)
    return fail(SAS_ERR_INVALID, "B, Hq, Hkv must be >= 1");
  if (d->Hq % d->Hkv) return fail(SAS_ERR_INVALID, "Hq must be a multiple of Hkv");
  const int G = d->Hq / d->Hkv;
  if (G > 8) return fail(SAS_ERR_UNSUPPORTED, "G = Hq/Hkv = %d > 8 is not supported", G);
  if (d->block != 64) return fail(SAS_ERR_UNSUPPORTED, "block must be 64");
  if (d->D != 128 && d->D != 64) return fail(SAS_ERR_UNSUPPORTED, "D must be 64 or 128");
  if (d->dg != 32 && d->dg != 64 && d->dg != 128)
    return fail(SAS_ERR_UNSUPPORTED, "dg must be 32, 64 or 128");
  if (d->topk < 0) return fail(SAS_ERR_INVALID, "topk must be >= 0");
  if (d->topk + 1 > sas::kMaxS) return fail(SAS_ERR_UNSUPPORTED, "topk must be <= %d", sas::kMaxS - 1);
  if (d->Lmax < 1) return fail(SAS_ERR_INVALID, "Lmax must be >= 1");
  if (d->NBmax != (d->Lmax + 63) / 64)
    return fail(SAS_ERR_INVALID, "NBmax must equal ceil(Lmax/64) (got %d, Lmax %d)", d->NBmax,
                d->Lmax);
  if (d->NBmax > sas::kMaxDecodeNB)
    return fail(SAS_ERR_UNSUPPORTED, "Lmax must be <= %d", sas::kMaxDecodeNB * 64);
  if (d->apply_gate != 0 && d->apply_gate != 1)
    return fail(SAS_ERR_INVALID, "apply_gate must be 0 or 1");
  if (d->kg_dtype != 0 && d->kg_dtype != 1)
    return fail(SAS_ERR_INVALID, "kg_dtype must be 0 (fp32) or 1 (bf16)");
  if (d->flags & ~SAS_FLAG_GATE_PER_QUERY_HEAD)
    return fail(SAS_ERR_INVALID, "decode dims.flags: unknown bits 0x%x",
                d->flags & ~SAS_FLAG_GATE_PER_QUERY_HEAD);
  return SAS_OK;
}

}  // namespace

// Device scratch of sas_decode_noalloc (for callers that cannot allocate):
// one fixed-size array per device, held until the process ends.  Host code
// never uses the array's name as an address: its device address on each GPU
// comes from hipGetSymbolAddress, looked up once per device.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the current device (first call per device
// looks it up with that device current).
sas_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(SAS_ERR_UNSUPPORTED, "device %d: at most %d devices are supported", dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(SAS_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SAS_OK;
}

}  // namespace

namespace sas {
// Records the caller's timing event of stage boundary i (see
// sas_set_timing_events) on stream st, if the hook is set.
void timing_mark(int i, hipStream_t st) {
  if (i < g_nev) (void)hipEventRecord(g_ev[i], st);
}
}  // namespace sas

extern "C" {

int sas_version(void) { return SAS_VERSION; }

sas_status sas_set_timing_events(void* const* events, int n_events) {
  if (n_events < 0 || n_events > kMaxTimingEvents || (n_events > 0 && !events))
    return fail(SAS_ERR_INVALID, "n_events must be in [0, %d] with a non-null array",
                kMaxTimingEvents);
  g_nev = n_events;
  for (int i = 0; i < n_events; ++i) g_ev[i] = static_cast<hipEvent_t>(events[i]);
  g_err.clear();
  return SAS_OK;
}

const char* sas_last_error(void) { return g_err.c_str(); }

sas_status sas_take_device_fault(unsigned* fault) {
  if (!fault) return fail(SAS_ERR_INVALID, "fault must be non-null");
  *fault = 0;
  hipError_t e = sas::take_ring_fault_fwd(fault);
  if (e == hipSuccess) e = sas::take_ring_fault_bwd(fault);
  if (e != hipSuccess) return fail(SAS_ERR_HIP, "reading the fault flag: %s", hipGetErrorString(e));
  g_err.clear();
  return SAS_OK;
}

size_t sas_workspace_size(int op, const sas_dims* d) {
  if (check_dims(d) != SAS_OK) return static_cast<size_t>(-1);
  switch (op) {
    case SAS_OP_GATE_SCORE: return gate_ws(d).total;
    case SAS_OP_TOPK: return 0;
    case SAS_OP_FWD: return fwd_ws(d);
    case SAS_OP_WALK_ORDER: return walk_order_bytes(d);
    case SAS_OP_BWD: return bwd_ws(d).total;
    case SAS_OP_GATE_BWD: return gate_bwd_ws(d).total;
    default: fail(SAS_ERR_INVALID, "unknown op %d", op); return static_cast<size_t>(-1);
  }
}

size_t sas_decode_workspace_size(const sas_decode_dims* d) {
  if (check_decode_dims(d) != SAS_OK) return static_cast<size_t>(-1);
  return dec_ws(d).total;
}

sas_status sas_gate_score(const sas_dims* d, const uint16_t* q, const uint16_t* k,
                          const uint16_t* wq, const uint16_t* wk, const float* w_qn,
                          const float* w_kn, float* q_gate, float* k_gate, void* ws,
                          size_t ws_bytes, void* stream) {
  sas_status st = check_dims(d);
  if (st) return st;
  REQ_PTR(q); REQ_PTR(k); REQ_PTR(wq); REQ_PTR(wk); REQ_PTR(w_qn); REQ_PTR(w_kn);
  REQ_PTR(q_gate); REQ_PTR(k_gate);
  const GateWs w = gate_ws(d);
  if ((st = check_ws(ws, ws_bytes, w.total))) return st;
  char* base = static_cast<char*>(ws);
  sas::RouterParams p{};
  p.q = q; p.k = k; p.w_qn = w_qn; p.w_kn = w_kn; p.q_gate = q_gate; p.k_gate = k_gate;
  p.B = d->B; p.T = d->T; p.Hq = d->Hq; p.Hkv = d->Hkv; p.D = d->D; p.dg = d->dg;
  p.G = d->Hq / d->Hkv; p.eps = d->norm_eps;
  const SelHeads sh = sel_heads(d->Hq, d->Hkv, d->flags);
  p.Hs = sh.Hs; p.Gs = sh.Gs;
  g_err.clear();
  return hip_status(sas::launch_router(p, wq, wk, reinterpret_cast<uint16_t*>(base + w.wqT),
                                       reinterpret_cast<uint16_t*>(base + w.wkT),
                                       reinterpret_cast<float2*>(base + w.rope), d->rope_theta,
                                       static_cast<hipStream_t>(stream)),
                    "sas_gate_score launch");
}

sas_status sas_topk_blocks(const sas_dims* d, const float* q_gate, const float* k_gate,
                           int32_t* idx, float* logg, float* gate_lse, float* gate_probs,
                           void* ws, size_t ws_bytes, void* stream) {
  (void)ws; (void)ws_bytes;
  sas_status st = check_dims(d);
  if (st) return st;
  REQ_PTR(q_gate); REQ_PTR(k_gate); REQ_PTR(idx); REQ_PTR(logg); REQ_PTR(gate_lse);
  if (gate_probs && !aligned16(gate_probs))
    return fail(SAS_ERR_INVALID, "pointer 'gate_probs' is not 16-byte aligned");
  sas::TopkParams p{};
  p.q_gate = q_gate; p.k_gate = k_gate; p.idx = idx; p.logg = logg; p.gate_lse = gate_lse;
  p.gate_probs = gate_probs;
  p.B = d->B; p.T = d->T; p.Hkv = d->Hkv; p.dg = d->dg; p.K = d->topk; p.S = d->topk + 1;
  {
    const SelHeads sh = sel_heads(d->Hq, d->Hkv, d->flags);
    p.Hs = sh.Hs; p.kdiv = sh.kdiv;
  }
  p.NB = (d->T + 63) / 64;
  const size_t smem = sas::topk_smem_bytes(p.NB, p.dg);
  if (smem > 160 * 1024) return fail(SAS_ERR_UNSUPPORTED, "T too large for the Top-K kernel");
  g_err.clear();
  return hip_status(sas::launch_topk(p, static_cast<hipStream_t>(stream)),
                    "sas_topk_blocks launch");
}

sas_status sas_sparse_attn_fwd(const sas_dims* d, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* idx, const float* logg,
                               float scale, uint16_t* o, float* lse, float* o_f32, void* ws,
                               size_t ws_bytes, void* stream) {
  sas_status st = check_dims(d);
  if (st) return st;
  REQ_PTR(q); REQ_PTR(k); REQ_PTR(v); REQ_PTR(idx); REQ_PTR(logg); REQ_PTR(o); REQ_PTR(lse);
  if (o_f32 && !aligned16(o_f32)) return fail(SAS_ERR_INVALID, "pointer 'o_f32' is not 16-byte aligned");
  if (!std::isfinite(scale)) return fail(SAS_ERR_INVALID, "scale must be finite");
  if ((st = check_ws(ws, ws_bytes, fwd_ws(d)))) return st;
  sas::FwdParams p{};
  const FwdWs fw = fwd_ws_layout(d);
  p.vt = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + fw.vt);
  p.vamax = reinterpret_cast<float*>(static_cast<char*>(ws) + fw.amax);
  p.vscale = reinterpret_cast<float*>(static_cast<char*>(ws) + fw.vscale);
  p.order = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + fw.order);
  p.ost = sas::walk_order_stride((d->T + 63) / 64);
  p.q = q; p.k = k; p.v = v; p.idx = idx; p.logg = logg; p.o = o; p.lse = lse; p.o32 = o_f32;
  p.B = d->B; p.T = d->T; p.Hq = d->Hq; p.Hkv = d->Hkv; p.D = d->D; p.G = d->Hq / d->Hkv;
  p.S = d->topk + 1; p.NB = (d->T + 63) / 64;
  {
    const SelHeads sh = sel_heads(d->Hq, d->Hkv, d->flags);
    p.Hs = sh.Hs; p.Gs = sh.Gs; p.kdiv = sh.kdiv;
  }
  p.TPT = 16 / p.Gs;
  p.ntiles = (64 + p.TPT - 1) / p.TPT;
  p.scale_log2 = scale * sas::kLog2e;
  g_err.clear();
  return hip_status(sas::launch_sparse_fwd(p, static_cast<hipStream_t>(stream)),
                    "sas_sparse_attn_fwd launch");
}

sas_status sas_walk_order(const sas_dims* d, const int32_t* idx, uint16_t* order,
                          size_t order_bytes, void* stream) {
  sas_status st = check_dims(d);
  if (st) return st;
  REQ_PTR(idx); REQ_PTR(order);
  const size_t need = walk_order_bytes(d);
  if (order_bytes < need)
    return fail(SAS_ERR_INVALID, "order buffer too small: %zu < %zu bytes", order_bytes, need);
  const SelHeads sh = sel_heads(d->Hq, d->Hkv, d->flags);
  const int NB = (d->T + 63) / 64;
  const sas::WalkOrderParams p{idx, order, d->B, d->T, sh.Hs, d->topk + 1, NB, 16 / sh.Gs,
                               sas::walk_order_stride(NB)};
  g_err.clear();
  return hip_status(sas::launch_walk_order(p, static_cast<hipStream_t>(stream)),
                    "sas_walk_order launch");
}

sas_status sas_gate_score_bwd(const sas_dims* d, const uint16_t* q, const uint16_t* k,
                              const uint16_t* wq, const uint16_t* wk, const float* w_qn,
                              const float* w_kn, const float* q_gate, const float* k_gate,
                              const int32_t* idx, const float* dlogg, float* dq, float* dk,
                              float* dwq, float* dwk, float* dw_qn, float* dw_kn, void* ws,
                              size_t ws_bytes, void* stream) {
  sas_status st = check_dims(d);
  if (st) return st;
  if (d->flags & SAS_FLAG_GATE_PER_QUERY_HEAD)
    return fail(SAS_ERR_UNSUPPORTED,
                "sas_gate_score_bwd covers one gate per KV head (flags must be 0)");
  REQ_PTR(q); REQ_PTR(k); REQ_PTR(wq); REQ_PTR(wk); REQ_PTR(w_qn); REQ_PTR(w_kn);
  REQ_PTR(q_gate); REQ_PTR(k_gate); REQ_PTR(idx); REQ_PTR(dlogg); REQ_PTR(dq); REQ_PTR(dk);
  REQ_PTR(dwq); REQ_PTR(dwk); REQ_PTR(dw_qn); REQ_PTR(dw_kn);
  const GateBwdWs w = gate_bwd_ws(d);
  if ((st = check_ws(ws, ws_bytes, w.total))) return st;
  char* base = static_cast<char*>(ws);
  const int G = d->Hq / d->Hkv;
  sas::GateBwdParams p{};
  p.q = q; p.k = k; p.w_qn = w_qn; p.w_kn = w_kn; p.q_gate = q_gate; p.k_gate = k_gate;
  p.idx = idx; p.dlogg = dlogg;
  p.dq = dq; p.dk = dk; p.dwq = dwq; p.dwk = dwk; p.dw_qn = dw_qn; p.dw_kn = dw_kn;
  uint16_t* wqT = reinterpret_cast<uint16_t*>(base + w.wqT);
  uint16_t* wkT = reinterpret_cast<uint16_t*>(base + w.wkT);
  float2* rope = reinterpret_cast<float2*>(base + w.rope);
  p.wq = wq; p.wk = wk; p.wqT = wqT; p.wkT = wkT; p.rope = rope;
  p.dqg = reinterpret_cast<float*>(base + w.dqg);
  p.dkg = reinterpret_cast<float*>(base + w.dkg);
  p.dy = reinterpret_cast<float*>(base + w.dy);
  p.dz = reinterpret_cast<float*>(base + w.dz);
  p.dzs = reinterpret_cast<float*>(base + w.dzs);
  p.pmm = reinterpret_cast<uint16_t*>(base + w.pmm);
  p.wq_part = reinterpret_cast<float*>(base + w.wq_part);
  p.wk_part = reinterpret_cast<float*>(base + w.wk_part);
  p.wn_part = reinterpret_cast<float*>(base + w.wn_part);
  p.bk_part = reinterpret_cast<float*>(base + w.bk_part);
  p.B = d->B; p.T = d->T; p.Hq = d->Hq; p.Hkv = d->Hkv; p.D = d->D; p.dg = d->dg; p.G = G;
  p.S = d->topk + 1; p.NB = (d->T + 63) / 64;
  p.nchunk = w.nchunk; p.nq_part = w.nq_part; p.nk_part = w.nk_part;
  p.eps = d->norm_eps;
  p.inv_sqrt_dg = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d->dg)));
  g_err.clear();
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = sas::launch_rope_table(rope, d->T, d->dg, d->rope_theta, hs);
  if (e == hipSuccess) e = sas::launch_transpose_w(wq, wqT, d->Hkv, G * d->D, d->dg, hs);
  if (e == hipSuccess) e = sas::launch_transpose_w(wk, wkT, d->Hkv, 3 * d->D, d->dg, hs);
  if (e == hipSuccess) e = sas::launch_gate_bwd(p, hs);
  return hip_status(e, "sas_gate_score_bwd launch");
}

sas_status sas_sparse_attn_bwd(const sas_dims* d, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const uint16_t* o, const float* o_f32,
                               const uint16_t* dout, const float* lse, const int32_t* idx,
                               const float* logg, float scale, uint16_t* dq, uint16_t* dk,
                               uint16_t* dv, float* dlogg, void* ws, size_t ws_bytes,
                               void* stream) {
  sas_status st = check_dims(d);
  if (st) return st;
  REQ_PTR(q); REQ_PTR(k); REQ_PTR(v); REQ_PTR(o); REQ_PTR(dout); REQ_PTR(lse); REQ_PTR(idx);
  REQ_PTR(logg); REQ_PTR(dq); REQ_PTR(dk); REQ_PTR(dv); REQ_PTR(dlogg);
  if (o_f32 && !aligned16(o_f32)) return fail(SAS_ERR_INVALID, "pointer 'o_f32' is not 16-byte aligned");
  if (!std::isfinite(scale)) return fail(SAS_ERR_INVALID, "scale must be finite");
  if (64LL * d->Hq * (d->topk + 1) * 256 >= (1LL << 31))
    return fail(SAS_ERR_UNSUPPORTED, "Hq * (topk + 1) too large (64 tokens' dS rows must fit 2 GiB)");
  const BwdWs w = bwd_ws(d);
  if ((st = check_ws(ws, ws_bytes, w.total))) return st;
  char* base = static_cast<char*>(ws);
  sas::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.o32 = o_f32; p.dout = dout; p.lse = lse; p.idx = idx;
  p.logg = logg;
  p.dq = dq; p.dk = dk; p.dv = dv; p.dlogg = dlogg;
  p.delta = reinterpret_cast<float*>(base + w.delta);
  p.cnt2d = reinterpret_cast<int32_t*>(base + w.cnt2d);
  p.rowptr = reinterpret_cast<int32_t*>(base + w.rowptr);
  p.entries = reinterpret_cast<int32_t*>(base + w.entries);
  p.dsbuf = reinterpret_cast<uint16_t*>(base + w.ds);
  p.order = reinterpret_cast<uint16_t*>(base + w.order);
  p.ost = sas::walk_order_stride((d->T + 63) / 64);
  p.B = d->B; p.T = d->T; p.Hq = d->Hq; p.Hkv = d->Hkv; p.D = d->D; p.G = d->Hq / d->Hkv;
  p.S = d->topk + 1; p.NB = (d->T + 63) / 64;
  {
    const SelHeads sh = sel_heads(d->Hq, d->Hkv, d->flags);
    p.Hs = sh.Hs; p.Gs = sh.Gs; p.kdiv = sh.kdiv;
  }
  p.TPT = 16 / p.Gs;
  p.ntiles = (64 + p.TPT - 1) / p.TPT;
  p.scale = scale;
  p.scale_log2 = scale * sas::kLog2e;
  g_err.clear();
  return hip_status(sas::launch_sparse_bwd(p, static_cast<hipStream_t>(stream)),
                    "sas_sparse_attn_bwd launch");
}

}  // extern "C"

namespace {

// Shared by sas_decode and sas_decode_noalloc: validation of the tensor
// arguments, then the launch over a workspace at `base` of at least
// dec_ws(d).total bytes.
sas_status decode_checked(const sas_decode_dims* d, const uint16_t* q, const float* q_gate,
                          const uint16_t* k_cache, const uint16_t* v_cache,
                          const float* kg_cache, const int32_t* ctx_len, float scale,
                          uint16_t* o, int32_t* idx_out, float* logg_out) {
  REQ_PTR(q); REQ_PTR(q_gate); REQ_PTR(k_cache); REQ_PTR(v_cache); REQ_PTR(kg_cache);
  REQ_PTR(ctx_len); REQ_PTR(o);
  if (idx_out && !aligned16(idx_out)) return fail(SAS_ERR_INVALID, "idx_out is not 16-byte aligned");
  if (logg_out && !aligned16(logg_out))
    return fail(SAS_ERR_INVALID, "logg_out is not 16-byte aligned");
  if (!std::isfinite(scale)) return fail(SAS_ERR_INVALID, "scale must be finite");
  return SAS_OK;
}

sas_status decode_launch(const sas_decode_dims* d, const uint16_t* q, const float* q_gate,
                         const uint16_t* k_cache, const uint16_t* v_cache,
                         const float* kg_cache, const int32_t* ctx_len, float scale,
                         uint16_t* o, int32_t* idx_out, float* logg_out, char* base,
                         const char* what, hipStream_t stream) {
  const DecWs w = dec_ws(d);
  sas::DecodeParams p{};
  p.q = q; p.q_gate = q_gate; p.k_cache = k_cache; p.v_cache = v_cache; p.kg_cache = kg_cache;
  p.ctx_len = ctx_len; p.o = o; p.idx_out = idx_out; p.logg_out = logg_out;
  p.ws_idx = reinterpret_cast<int32_t*>(base + w.idx);
  p.ws_logg = reinterpret_cast<float*>(base + w.logg);
  p.ws_part = reinterpret_cast<float*>(base + w.part);
  p.ws_score = reinterpret_cast<float*>(base + w.score);
  p.B = d->B; p.Hq = d->Hq; p.Hkv = d->Hkv; p.D = d->D; p.dg = d->dg;
  {
    const SelHeads sh = sel_heads(d->Hq, d->Hkv, d->flags);
    p.Hs = sh.Hs; p.Gs = sh.Gs; p.kdiv = sh.kdiv;
    p.G = sh.Gs;                 // query heads per unit
  }
  p.K = d->topk; p.S = d->topk + 1; p.Lmax = d->Lmax; p.NBmax = d->NBmax;
  p.apply_gate = d->apply_gate; p.nsplit = w.nsplit; p.spw = w.spw; p.kg_bf16 = d->kg_dtype;
  p.scale_log2 = scale * sas::kLog2e;
  g_err.clear();
  return hip_status(sas::launch_decode(p, stream), what);
}

}  // namespace

extern "C" {

sas_status sas_decode(const sas_decode_dims* d, const uint16_t* q, const float* q_gate,
                      const uint16_t* k_cache, const uint16_t* v_cache,
                      const float* kg_cache, const int32_t* ctx_len, float scale,
                      uint16_t* o, int32_t* idx_out, float* logg_out, void* ws,
                      size_t ws_bytes, void* stream) {
  sas_status st = check_decode_dims(d);
  if (st) return st;
  if ((st = decode_checked(d, q, q_gate, k_cache, v_cache, kg_cache, ctx_len, scale, o, idx_out,
                           logg_out)))
    return st;
  if ((st = check_ws(ws, ws_bytes, dec_ws(d).total))) return st;
  return decode_launch(d, q, q_gate, k_cache, v_cache, kg_cache, ctx_len, scale, o, idx_out,
                       logg_out, static_cast<char*>(ws), "sas_decode launch",
                       static_cast<hipStream_t>(stream));
}

sas_status sas_decode_noalloc(const sas_decode_dims* d, const uint16_t* q, const float* q_gate,
                              const uint16_t* k_cache, const uint16_t* v_cache,
                              const float* kg_cache, const int32_t* ctx_len, float scale,
                              uint16_t* o, int32_t* idx_out, float* logg_out, void* stream) {
  sas_status st = check_decode_dims(d);
  if (st) return st;
  if ((st = decode_checked(d, q, q_gate, k_cache, v_cache, kg_cache, ctx_len, scale, o, idx_out,
                           logg_out)))
    return st;
  const size_t need = dec_ws(d).total;
  if (need > kNoAllocScratchBytes)
    return fail(SAS_ERR_WORKSPACE,
                "sas_decode_noalloc: these dimensions need %zu bytes of scratch, more than the "
                "fixed %zu; call sas_decode with a workspace instead", need, kNoAllocScratchBytes);
  void* base = nullptr;
  if ((st = scratch_address(&base))) return st;
  return decode_launch(d, q, q_gate, k_cache, v_cache, kg_cache, ctx_len, scale, o, idx_out,
                       logg_out, static_cast<char*>(base), "sas_decode_noalloc launch",
                       static_cast<hipStream_t>(stream));
}

sas_status sas_decode_gate_key(const sas_decode_dims* d, const uint16_t* k_cache,
                               const int32_t* block_table, int32_t num_pages, const uint16_t* wk,
                               const float* w_kn, double rope_theta, float norm_eps,
                               const int32_t* ctx_len, void* kg_cache, void* stream) {
  sas_status st = check_decode_dims(d);
  if (st) return st;
  REQ_PTR(k_cache); REQ_PTR(wk); REQ_PTR(w_kn); REQ_PTR(ctx_len); REQ_PTR(kg_cache);
  if (block_table && !aligned16(block_table))
    return fail(SAS_ERR_INVALID, "block_table is not 16-byte aligned");
  if (block_table && num_pages < 1)
    return fail(SAS_ERR_INVALID, "num_pages must be positive (got %d)", num_pages);
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta))
    return fail(SAS_ERR_INVALID, "rope_theta must be positive and finite");
  if (!(norm_eps >= 0.f) || !std::isfinite(norm_eps))
    return fail(SAS_ERR_INVALID, "norm_eps must be non-negative and finite");
  sas::DecodeKeyParams p{};
  p.k = k_cache; p.btab = block_table; p.num_pages = num_pages; p.wk = wk; p.w_kn = w_kn;
  p.ctx_len = ctx_len; p.kg = kg_cache;
  p.B = d->B; p.Hkv = d->Hkv; p.D = d->D; p.dg = d->dg; p.Lmax = d->Lmax; p.NBmax = d->NBmax;
  p.kg_bf16 = d->kg_dtype; p.theta = rope_theta; p.eps = norm_eps;
  g_err.clear();
  return hip_status(sas::launch_decode_gate_key(p, static_cast<hipStream_t>(stream)),
                    "sas_decode_gate_key launch");
}

sas_status sas_decode_paged(const sas_decode_dims* d, const uint16_t* q, const float* q_gate,
                            const uint16_t* k_pages, const uint16_t* v_pages,
                            const float* kg_pages, int32_t num_pages,
                            const int32_t* block_table, const int32_t* ctx_len, float scale,
                            uint16_t* o, int32_t* idx_out, float* logg_out, void* ws,
                            size_t ws_bytes, void* stream) {
  sas_status st = check_decode_dims(d);
  if (st) return st;
  REQ_PTR(q); REQ_PTR(q_gate); REQ_PTR(k_pages); REQ_PTR(v_pages); REQ_PTR(kg_pages);
  REQ_PTR(block_table); REQ_PTR(ctx_len); REQ_PTR(o);
  if (num_pages < 1) return fail(SAS_ERR_INVALID, "num_pages must be positive (got %d)", num_pages);
  if (idx_out && !aligned16(idx_out)) return fail(SAS_ERR_INVALID, "idx_out is not 16-byte aligned");
  if (logg_out && !aligned16(logg_out))
    return fail(SAS_ERR_INVALID, "logg_out is not 16-byte aligned");
  if (!std::isfinite(scale)) return fail(SAS_ERR_INVALID, "scale must be finite");
  const DecWs w = dec_ws(d);
  if ((st = check_ws(ws, ws_bytes, w.total))) return st;
  char* base = static_cast<char*>(ws);
  sas::DecodeParams p{};
  p.q = q; p.q_gate = q_gate; p.k_cache = k_pages; p.v_cache = v_pages; p.kg_cache = kg_pages;
  p.btab = block_table; p.num_pages = num_pages;
  p.ctx_len = ctx_len; p.o = o; p.idx_out = idx_out; p.logg_out = logg_out;
  p.ws_idx = reinterpret_cast<int32_t*>(base + w.idx);
  p.ws_logg = reinterpret_cast<float*>(base + w.logg);
  p.ws_part = reinterpret_cast<float*>(base + w.part);
  p.ws_score = reinterpret_cast<float*>(base + w.score);
  p.B = d->B; p.Hq = d->Hq; p.Hkv = d->Hkv; p.D = d->D; p.dg = d->dg;
  {
    const SelHeads sh = sel_heads(d->Hq, d->Hkv, d->flags);
    p.Hs = sh.Hs; p.Gs = sh.Gs; p.kdiv = sh.kdiv;
    p.G = sh.Gs;                 // query heads per unit
  }
  p.K = d->topk; p.S = d->topk + 1; p.Lmax = d->Lmax; p.NBmax = d->NBmax;
  p.apply_gate = d->apply_gate; p.nsplit = w.nsplit; p.spw = w.spw; p.kg_bf16 = d->kg_dtype;
  p.scale_log2 = scale * sas::kLog2e;
  g_err.clear();
  return hip_status(sas::launch_decode(p, static_cast<hipStream_t>(stream)),
                    "sas_decode_paged launch");
}

}  // extern "C"
