// Device-side helpers shared by the libsas kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sas {

constexpr int kBlock = 64;     // KV block size (model card: 64 tokens)
constexpr int kWave = 64;      // CDNA wavefront width

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two fp32 -> packed bf16 pair (low = a), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Split two fp32 values into bf16 hi = rne(x) and lo = rne(x - hi) pairs, so
// that an MFMA fed hi and then lo reproduces x to ~2^-16 relative.
__device__ __forceinline__ void split_bf2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf2(a, b);
  lo = pack_bf2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// XOR swizzle of the 16-byte chunks of an LDS tile row of ROWB bytes, chosen
// so that 16 lanes reading the same logical chunk of 16 consecutive rows hit
// distinct banks (256-byte rows: chunk ^ (r & 15); 128-byte rows, where two
// rows share the bank space: chunk ^ ((r >> 1) & 7)).
template <int ROWB>
__device__ __forceinline__ int lds_swz(int r) {
  static_assert(ROWB == 256 || ROWB == 128, "row size");
  return ROWB == 256 ? (r & 15) : ((r >> 1) & 7);
}

// XOR swizzle of the 16-byte chunks of a 128-byte row d of a transposed
// (K^T / V^T) LDS tile, read as one 16-byte chunk of 16 consecutive rows per
// 16 lanes.  f(d) = (d & 7) ^ ((d >> 3) & 1) keeps any 8 consecutive rows on
// distinct chunks and, among rows of equal parity (which share one half of a
// 256-byte bank window), all 16 rows on distinct chunks: conflict-free both
// for 128-byte and for 256-byte bank windows.
__device__ __forceinline__ int tr_swz(int d) { return (d & 7) ^ ((d >> 3) & 1); }

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// l receives element l % 4 of the 8-byte words addressed by lanes l / 4 + 4 e
// (e = 0..3), i.e. one column of the 4 x 16 block of 16-bit values that the
// group's 16 addresses span when lane s addresses row s / 4, columns
// 4 (s % 4) .. 4 (s % 4) + 3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p));
  return __builtin_bit_cast(uint2, v);
}

// 16-byte load / store through a native vector type.  A plain uint4 struct
// copy becomes a memcpy, which keeps arrays of staged values that live across
// loop iterations from being promoted to registers (they end up in scratch).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(void* p, uint4 v) {
  *reinterpret_cast<u32x4*>(p) = u32x4{v.x, v.y, v.z, v.w};
}

// Raw buffer resources (stride 0, no swizzle) with the fourth descriptor word
// of the gfx9 family (32-bit data format).  A lane whose byte offset is at or
// beyond the resource's size reads zeros and makes no memory request.
constexpr int kBufferWord3 = 0x00020000;
__device__ __forceinline__ uint4 buffer_ld16(__amdgpu_buffer_rsrc_t rs, unsigned off) {
  typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v v = __builtin_bit_cast(
      u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(off), 0, 0));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16x16x4 fp32 MFMA: lane l holds A[l%16][l/16] and B[l/16][l%16]; C column
// l%16 holds rows 4*(l/16) .. +4.
__device__ __forceinline__ floatx4 mfma16x16x4f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// a.lo * b.lo + a.hi * b.hi + c for packed bf16 pairs (v_dot2_f32_bf16:
// exact bf16 products, fp32 accumulation).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                          __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

// Two fp32 -> packed fp16 pair (low = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  const h2_t v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// C[16x16] += A[16x32] * B[32x16], fp16 inputs, fp32 accumulate (same lane
// layout as the bf16 form below).
__device__ __forceinline__ floatx4 mfma16x16x32h(uint4 a, uint4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a),
                                                __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}

// C[16x16] += A[16x32] * B[32x16], bf16 inputs, fp32 accumulate.
// Lane l: A row l%16 / B column l%16 holds k = 8*(l/16) .. +8;
// C column l%16 holds rows 4*(l/16) .. +4.
__device__ __forceinline__ floatx4 mfma16x16x32(uint4 a, uint4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// Reductions over the four 16-lane rows of a wave, per position l = lane % 16
// (the xor-16 and xor-32 butterflies), with the gfx950 row-swap permutes:
// permlane16_swap(x, x) yields rows (r0, r0, r2, r2) and (r1, r1, r3, r3),
// permlane32_swap(x, x) yields (r0, r1, r0, r1) and (r2, r3, r2, r3).  Pure
// VALU (no LDS round trip); every lane ends with the same, order-fixed result.
__device__ __forceinline__ float row4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float row4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// DPP lane moves inside 16-lane rows (quad_perm / half-row mirror controls).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Maximum / sum over the whole wave without an LDS round trip: the four
// butterflies inside each 16-lane row on DPP, then the row swaps; every lane
// ends with the same, order-fixed result.
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));     // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_mov<0x4E>(x));     // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_mov<0x141>(x));    // row_half_mirror
  x = fmaxf(x, dpp_mov<0x140>(x));    // row_mirror
  return row4_max(x);
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  return row4_sum(x);
}
// Sum over aligned groups of n consecutive lanes, n in {1, 2, 4, 8}
// (wave-uniform n): xor-1, xor-2, then the 8-lane mirror.
__device__ __forceinline__ float group_sum_pow2(float x, int n) {
  if (n >= 2) x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  if (n >= 4) x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  if (n >= 8) x += dpp_mov<0x141>(x);   // row_half_mirror
  return x;
}

// Sum over each row of 16 lanes (the 8-lane sums, then the row mirror).
__device__ __forceinline__ float row16_sum(float x) {
  x = group_sum_pow2(x, 8);
  return x + dpp_mov<0x140>(x);        // row_mirror
}

// Order-preserving map fp32 -> uint32 (larger float -> larger key).  -0.0
// and +0.0 compare equal as numbers, so both map to the key of +0.0 and an
// exact tie between them goes to the lower block index like any other tie.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// Number of lanes of the wave for which p holds (ballot + scalar popcount:
// no cross-lane data movement, so no LDS round trip).
__device__ __forceinline__ int wave_count(bool p) { return __popcll(__ballot(p)); }

// 2^x with the bare hardware instruction (results below 2^-126 flush to 0,
// which is harmless for softmax weights).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait until every global load issued so far by this wave has returned.
// Used once before a software-pipelined loop so that registers loaded before
// the loop are not treated as possibly pending inside it (which would make
// the compiler wait for the loop's own prefetches every iteration).
__device__ __forceinline__ void wait_vmem_all() {
  // s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maxima
  __builtin_amdgcn_s_waitcnt(0x0f70);
}

// ---- LDS ring shared by the waves of a workgroup, without workgroup barriers.
// Slot n % R holds block n of the walk.  Each wave writes its share of block n
// once every wave is done reading block n - R (done[n % R] >= NW * (n / R))
// and then bumps fill[n % R]; a wave reads block u once
// fill[u % R] >= NW * (u / R + 1) and bumps done[u % R] after its last read of
// it.  The counters only grow, so a count names the use of the slot, and a
// wave can run up to R - 1 blocks ahead of the slowest one.  The LDS accesses
// of one wave are performed in order, so a bump issued after a wave's stores
// (or reads) of a slot is observed only after them; the asm statements keep the
// compiler from moving memory accesses across a bump or a poll.
constexpr int kSpinLimit = 1 << 21;   // polls (0.1 - 0.5 s) before a wait gives up
// s_sleep between polls (about 64 cycles per unit): a compute wave's poll
// takes SIMD issue slots from the waves that have work, so compute waves nap
// longer (512 cycles, a seventh of a block visit) than the stagers
constexpr int kComputeNap = 8;
constexpr int kStagerNap = 4;

// The counters are read with plain LDS loads and bumped with an LDS atomic
// add written as an instruction without results: the compiler treats atomic
// (or volatile) LDS accesses as possibly touching the destinations of pending
// asynchronous global -> LDS copies and would wait for all of them first.  A
// 32-bit LDS load is single-copy atomic.
__device__ __forceinline__ unsigned ring_count(const unsigned* c) {
  asm volatile("" ::: "memory");
  const unsigned v = *c;
  asm volatile("" ::: "memory");
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ void ring_bump(unsigned* c, int lane) {
  typedef __attribute__((address_space(3))) unsigned* lds_u32_ptr;
  const unsigned addr = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_u32_ptr)c));
  asm volatile("" ::: "memory");
  if (lane == 0) asm volatile("ds_add_u32 %0, %1" ::"v"(addr), "v"(1u) : "memory");
  asm volatile("" ::: "memory");
}

// Asynchronous 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4):
// lane i's 16 bytes land at lds + 16 * i.  `lds` must be wave-uniform.  The
// copy is complete once the wave's vector-memory counter says so (s_waitcnt
// vmcnt); the compiler orders later LDS reads that may touch the destination
// (the same LDS variable, or any atomic / volatile LDS access) after it.
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)(lds), 16, 0, 0);
}

// Set (never expected) when a ring wait gave up: the kernel then finishes
// with NaN outputs for the waves concerned instead of hanging.  One copy per
// source file; read and cleared from the host through take_ring_fault_*().
static __device__ unsigned g_ring_fault;

__device__ __forceinline__ void ring_fault(int lane) {
  if (lane == 0) atomicOr(&g_ring_fault, 1u);
}

}  // namespace sas
