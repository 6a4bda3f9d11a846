// Device-side helpers for the gfx950 kernels: vector types, MFMA wrappers,
// the in-register 2-bit unpack and exact dequantization, reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {

typedef _Float16 half_t;
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// C[16x16] += A[16x32] * B[32x16].  Operand layout (wave64): lane l holds
// A[row l%16][k 8*(l/16) .. +7], B[k 8*(l/16) .. +7][col l%16]; the result
// lane l holds C[row 4*(l/16)+v][col l%16], v = 0..3.
__device__ __forceinline__ f32x4 mfma16(const half8v& a, const half8v& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8v& a, const bf16x8v& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <typename T> struct Vec8;
template <> struct Vec8<half_t> { typedef half8v type; };
template <> struct Vec8<__bf16> { typedef bf16x8v type; };

__device__ __forceinline__ half8v as_half8(u32x4 v) { return __builtin_bit_cast(half8v, v); }
__device__ __forceinline__ u32x4 as_u32x4(half8v v) { return __builtin_bit_cast(u32x4, v); }

// ---- 2-bit unpack ---------------------------------------------------------
// A dword holds the 16 codes of two consecutive MFMA k-steps of one lane
// (8 inputs per step).  For step b (0 or 1) and input j = 2v + h of the step,
// the code sits at bit 16*h + pos(b, v) with pos(0, .) = {4, 6, 8, 0} and
// pos(1, .) = {10, 12, 14, 2}.  Each output register is a packed fp16 pair
// whose halves are 1 + q*c (exponent bits of 1.0 OR-ed over the code placed in
// the mantissa), with class c = 1/64, 1/16 or 1/4 given by the mantissa
// position.  One and-or per pair; two shifts per dword.
//   out[0..3] : step b=0, classes {1/64, 1/16, 1/4, 1/64}
//   out[4..7] : step b=1, classes {1/64, 1/16, 1/4, 1/16}
__device__ __forceinline__ uint32_t and_or_s(uint32_t a, uint32_t m, uint32_t c);
__device__ __forceinline__ void unpack16(uint32_t D, uint32_t out[8]) {
  const uint32_t M4 = 0x00300030u, M6 = 0x00C000C0u, M8 = 0x03000300u;
  const uint32_t ONE = 0x3C003C00u;
  const uint32_t E = D >> 6, F = D << 4;
  out[0] = and_or_s(D, M4, ONE);
  out[1] = and_or_s(D, M6, ONE);
  out[2] = and_or_s(D, M8, ONE);
  out[3] = and_or_s(F, M4, ONE);
  out[4] = and_or_s(E, M4, ONE);
  out[5] = and_or_s(E, M6, ONE);
  out[6] = and_or_s(E, M8, ONE);
  out[7] = and_or_s(F, M6, ONE);
}

// ---- buffer loads ----------------------------------------------------------
// Raw buffer resource over [base, base + bytes): the load address is an SGPR
// base + 32-bit lane offset + uniform SGPR offset, and a read past the end
// returns zeros (no fault).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2 bload64(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// ---- loads with an LDS destination (buffer_load ... lds) --------------------
// Each lane's bytes land at lds + lane * size; the LDS pointer must be
// wave-uniform.  Loads complete in issue order; a wave waits for its own with
// wait_vm<N>() and makes them visible to the workgroup with a barrier.
typedef __attribute__((address_space(3))) void lds_t;

// out-of-range voffset: the load returns zeros and reads no memory (only the
// vector offset is range checked, so every scalar offset must stay in range)
constexpr uint32_t OOB = 0x7FFFFFF0u;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_t*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff,
                                     uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_t*)lds, 4, voff, soff, 0, 0);
}

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// wait until every LDS / scalar-memory operation of this wave has completed
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// First round of a load ring whose prologue issued batches 0 .. D-1 either
// whole (NI loads each) or as all their early loads first and then the other
// NX loads of each: after batch u's last load at least (D - 1 - u) NX + u NI
// loads were issued either way (u NI by the ring's own stages), so
// wait_vm<(D - 1 - u) NX + u NI>() leaves batch u landed.  u in [0, D - 1)
// must fold to a constant (an unrolled loop index).
template <int NI, int NX, int D, int U = 0>
__device__ __forceinline__ void wait_vm_first(int u) {
  if constexpr (U < D - 1) {
    if (u == U) wait_vm<(D - 1 - U) * NX + U * NI>();
    else wait_vm_first<NI, NX, D, U + 1>(u);
  }
}

// Reads of data that no workgroup of the running kernel writes, at
// wave-uniform addresses: through the constant address space they become
// scalar loads, counted apart from the vector-memory loads in flight.
typedef __attribute__((address_space(4))) const int cint_t;
__device__ __forceinline__ int sload(const int* p, int i) {
  return ((cint_t*)p)[i];
}

// Lane l of a wave gets p[i0 + l % 16]: 16 wave-uniform scalar loads and a
// select chain (no array, so nothing goes through private memory).
template <int I = 0>
__device__ __forceinline__ int sload16(const int* p, int i0, int l16, int r = 0) {
  if constexpr (I == 16) {
    return r;
  } else {
    const int v = sload(p, i0 + I);
    return sload16<I + 1>(p, i0, l16, (l16 == I) ? v : r);
  }
}

// x, unknown to the optimizer from here on: values derived from it are
// computed where they are used instead of being hoisted out of loops (and
// held in registers across them)
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// workgroup barrier without a memory fence (a fenced barrier waits for every
// load in flight); the empty asm statements keep the compiler from moving
// LDS accesses across it
__device__ __forceinline__ void bar_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// (a & m) | c in one VALU op (the compiler otherwise emits an and plus an or).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm volatile("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
  return r;
}

// The same, free to be scheduled and merged like ordinary arithmetic.
__device__ __forceinline__ uint32_t and_or_s(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
  return r;
}

// The MFMA A operand of step b (0 or 1) of dword D alone (half of
// unpack16_frags).
__device__ __forceinline__ u32x4 unpack16_step(uint32_t D, int b) {
  const uint32_t M4 = 0x00300030u, M6 = 0x00C000C0u, M8 = 0x03000300u;
  const uint32_t ONE = 0x3C003C00u;
  u32x4 f;
  if (b == 0) {
    const uint32_t F = D << 4;
    f[0] = and_or(D, M4, ONE);
    f[1] = and_or(D, M6, ONE);
    f[2] = and_or(D, M8, ONE);
    f[3] = and_or(F, M4, ONE);
  } else {
    const uint32_t E = D >> 6, F = D << 4;
    f[0] = and_or(E, M4, ONE);
    f[1] = and_or(E, M6, ONE);
    f[2] = and_or(E, M8, ONE);
    f[3] = and_or(F, M6, ONE);
  }
  return f;
}

// unpack16 into the two MFMA A operands (step b = 0 and b = 1) of dword D.
__device__ __forceinline__ void unpack16_frags(uint32_t D, u32x4& f0, u32x4& f1) {
  const uint32_t M4 = 0x00300030u, M6 = 0x00C000C0u, M8 = 0x03000300u;
  const uint32_t ONE = 0x3C003C00u;
  const uint32_t E = D >> 6, F = D << 4;
  f0[0] = and_or(D, M4, ONE);
  f0[1] = and_or(D, M6, ONE);
  f0[2] = and_or(D, M8, ONE);
  f0[3] = and_or(F, M4, ONE);
  f1[0] = and_or(E, M4, ONE);
  f1[1] = and_or(E, M6, ONE);
  f1[2] = and_or(E, M8, ONE);
  f1[3] = and_or(F, M6, ONE);
}

// Per (row, group) constants turning 1 + q*c into the dequantized weight
// RND_f16(s * (q - z)):  ((1 + q c) - (1 + z c)) is exact (Sterbenz), equals
// (q - z) c, and the product with s/c (exact: power-of-two scaling, |s| < 1024)
// rounds the exact value (q - z) s once.
struct DeqConst {
  half2v k64, k16, k4;      // (c^-1 s, -(1 + z c)) for c = 1/64, 1/16, 1/4
};

// From the (s, z) word: (64 s, -(1 + z/64)) in one packed fma, then each
// next class by (x/4, 4 y + 3); every value is exact (powers of two, z an
// integer in 0..3, |64 s| <= 65504).  The scale lanes add -0, which keeps
// the sign of a zero scale.
__device__ __forceinline__ DeqConst deq_const(uint32_t szw) {
  const half2v sz = __builtin_bit_cast(half2v, szw);
  DeqConst c;
  c.k64 = __builtin_elementwise_fma(sz, half2v{(half_t)64.0f, (half_t)-0.015625f},
                                    half2v{(half_t)-0.0f, (half_t)-1.0f});
  c.k16 = __builtin_elementwise_fma(c.k64, half2v{(half_t)0.25f, (half_t)4.0f},
                                    half2v{(half_t)-0.0f, (half_t)3.0f});
  c.k4 = __builtin_elementwise_fma(c.k16, half2v{(half_t)0.25f, (half_t)4.0f},
                                   half2v{(half_t)-0.0f, (half_t)3.0f});
  return c;
}

__device__ __forceinline__ uint32_t deq_pair(uint32_t m, half2v k) {
  half2v v = __builtin_bit_cast(half2v, m);
  v = v + half2v{k.y, k.y};   // exact
  v = v * half2v{k.x, k.x};   // one rounding of (q - z) s
  return __builtin_bit_cast(uint32_t, v);
}

// Dequantized A operands of the two k-steps held by dword D.
__device__ __forceinline__ void deq_dword(uint32_t D, const DeqConst& c0, const DeqConst& c1,
                                          half8v& a0, half8v& a1) {
  uint32_t m[8];
  unpack16(D, m);
  u32x4 r0, r1;
  r0[0] = deq_pair(m[0], c0.k64);
  r0[1] = deq_pair(m[1], c0.k16);
  r0[2] = deq_pair(m[2], c0.k4);
  r0[3] = deq_pair(m[3], c0.k64);
  r1[0] = deq_pair(m[4], c1.k64);
  r1[1] = deq_pair(m[5], c1.k16);
  r1[2] = deq_pair(m[6], c1.k4);
  r1[3] = deq_pair(m[7], c1.k16);
  a0 = as_half8(r0);
  a1 = as_half8(r1);
}

// ---- dequantization for any finite fp16 scale and zero point --------------
// The four weights a (row, group) can take, RND_f16(fl32(fl32(q - z) * s))
// for q = 0..3, are formed once per group in fp32 and kept as a byte table:
// byte q of `lo` is the low byte of the value for code q, byte q of `hi` its
// high byte.  A code pair then becomes its two fp16 values with one
// v_perm_b32 (bytes 0-3 of the selector pick from `lo`, 4-7 from `hi`), so
// the values are the canonical ones whatever z and s are (a fractional zero
// point, a scale of any magnitude, a signed zero).
struct DeqLut {
  uint32_t lo, hi;
};

// fp32 value the compiler may not fold into a neighbouring operation: each
// rounding step below then happens exactly where written (no fused
// multiply-add, no mixed-precision multiply-convert, no sign-of-zero folding)
__device__ __forceinline__ float fence_f(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// RND_f16(fl32(fl32(q - z) * s)) as fp16 bits
__device__ __forceinline__ uint32_t deq_bits(float q, float z, float s) {
  const float d = fence_f(q - z);
  const float t = fence_f(d * s);
  return (uint32_t)__builtin_bit_cast(uint16_t, (half_t)t);   // round to nearest even
}

__device__ __forceinline__ DeqLut deq_lut(uint32_t szw) {
  const float s = (float)__builtin_bit_cast(half_t, (uint16_t)(szw & 0xFFFFu));
  const float z = (float)__builtin_bit_cast(half_t, (uint16_t)(szw >> 16));
  const uint32_t h0 = deq_bits(0.0f, z, s), h1 = deq_bits(1.0f, z, s);
  const uint32_t h2 = deq_bits(2.0f, z, s), h3 = deq_bits(3.0f, z, s);
  const uint32_t h01 = h0 | (h1 << 16), h23 = h2 | (h3 << 16);
  DeqLut t;
  t.lo = __builtin_amdgcn_perm(h23, h01, 0x06040200u);   // low bytes of h0, h1, h2, h3
  t.hi = __builtin_amdgcn_perm(h23, h01, 0x07050301u);   // high bytes
  return t;
}

// The fp16 pair of the codes at bit P (low half) and 16 + P (high half) of D.
template <int P>
__device__ __forceinline__ uint32_t lut_pair(uint32_t D, const DeqLut& t) {
  const uint32_t x = (D >> P) & 0x00030003u;                  // q0 | q1 << 16
  const uint32_t sel = __umul24(x, 0x101u) + 0x04000400u;     // bytes q0, q0 + 4, q1, q1 + 4
  return __builtin_amdgcn_perm(t.hi, t.lo, sel);
}

// deq_dword for any scale and zero point: the same operands, from the tables
// of the groups of k-steps 2d (t0) and 2d + 1 (t1).  Code positions as in
// unpack16: step 0 pairs at bits 4, 6, 8, 0; step 1 pairs at 10, 12, 14, 2.
__device__ __forceinline__ void deq_dword_lut(uint32_t D, const DeqLut& t0, const DeqLut& t1,
                                              half8v& a0, half8v& a1) {
  u32x4 r0, r1;
  r0[0] = lut_pair<4>(D, t0);
  r0[1] = lut_pair<6>(D, t0);
  r0[2] = lut_pair<8>(D, t0);
  r0[3] = lut_pair<0>(D, t0);
  r1[0] = lut_pair<10>(D, t1);
  r1[1] = lut_pair<12>(D, t1);
  r1[2] = lut_pair<14>(D, t1);
  r1[3] = lut_pair<2>(D, t1);
  a0 = as_half8(r0);
  a1 = as_half8(r1);
}

// ---- 3-bit codes ------------------------------------------------------------
// Per lane, a unit of 4 MFMA k-steps (32 codes: the lane's 8 inputs of each
// step) is three dwords D0, D1, D2.  Pair n = 0..15 is (step n / 4, register
// n % 4), i.e. inputs 2v and 2v + 1 (v = n % 4) of the step.  Pair n = 5j + f
// (f < 5) sits in dword j: the low input's code at bits 3f .. 3f + 2, the
// high input's at 16 + 3f ...; pair 15 is spread over the spare bits: bit b
// of its low code is bit 15 of dword b, bit b of its high code bit 31.
// Unpacked into packed fp16 pairs 1 + q c (exponent bits of 1.0 OR-ed over a
// code placed in the mantissa at bit p, c = 2^(p - 10)):
//   f = 0: (D << 4) at p = 4     f = 1: (D << 4) at p = 7    f = 2: D at p = 6
//   f = 3: (D >> 5) at p = 4     f = 4: (D >> 5) at p = 7    pair 15 at p = 4
// so the class of pair n is p = CLS3[n] below (c = 1/64, 1/8 or 1/16).
constexpr uint32_t U3_ONE = 0x3C003C00u, U3_M4 = 0x00700070u, U3_M7 = 0x03800380u,
                   U3_M6 = 0x01C001C0u;
// mantissa position of pair n's code (4, 6 or 7)
__host__ __device__ constexpr int cls3(int n) {
  return n == 15 ? 4 : ((n % 5) == 2 ? 6 : ((n % 5) == 1 || (n % 5) == 4 ? 7 : 4));
}

// (m & a) | (~m & b) in one v_bfi_b32
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
  return (m & a) | (~m & b);
}

// The source word and mask of pair n (f < 5) or the assembled spare pair.
template <int N>
__device__ __forceinline__ uint32_t raw3_pair(uint32_t D0, uint32_t D1, uint32_t D2) {
  if constexpr (N == 15) {
    uint32_t t = bfi(0x00200020u, D1 >> 10, D0 >> 11);
    t = bfi(0x00400040u, D2 >> 9, t);
    return and_or_s(t, U3_M4, U3_ONE);
  } else {
    constexpr int j = N / 5, f = N % 5;
    const uint32_t D = (j == 0) ? D0 : (j == 1 ? D1 : D2);
    if constexpr (f == 0) return and_or_s(D << 4, U3_M4, U3_ONE);
    else if constexpr (f == 1) return and_or_s(D << 4, U3_M7, U3_ONE);
    else if constexpr (f == 2) return and_or_s(D, U3_M6, U3_ONE);
    else if constexpr (f == 3) return and_or_s(D >> 5, U3_M4, U3_ONE);
    else return and_or_s(D >> 5, U3_M7, U3_ONE);
  }
}

// The raw A operand (1 + q c per half) of step S of a unit.
template <int S>
__device__ __forceinline__ u32x4 raw3_step(uint32_t D0, uint32_t D1, uint32_t D2) {
  u32x4 r;
  r[0] = raw3_pair<4 * S + 0>(D0, D1, D2);
  r[1] = raw3_pair<4 * S + 1>(D0, D1, D2);
  r[2] = raw3_pair<4 * S + 2>(D0, D1, D2);
  r[3] = raw3_pair<4 * S + 3>(D0, D1, D2);
  return r;
}

// The codes q0 | q1 << 16 of pair n (for table dequantization).
template <int N>
__device__ __forceinline__ uint32_t codes3_pair(uint32_t D0, uint32_t D1, uint32_t D2) {
  if constexpr (N == 15) {
    uint32_t t = bfi(0x00200020u, D1 >> 10, D0 >> 11);
    t = bfi(0x00400040u, D2 >> 9, t);
    return (t >> 4) & 0x00070007u;
  } else {
    constexpr int j = N / 5, f = N % 5;
    const uint32_t D = (j == 0) ? D0 : (j == 1 ? D1 : D2);
    return (D >> (3 * f)) & 0x00070007u;
  }
}

// Per (row, group) constants of the packed dequantization for the 3-bit
// classes c = 1/64, 1/16, 1/8: (c^-1 s, -(1 + z c)); exact for integer z in
// 0..7 and |s| < 1024 (as in deq_const).
struct DeqConst3 {
  half2v k64, k16, k8;
};
__device__ __forceinline__ DeqConst3 deq_const3(uint32_t szw) {
  const half2v sz = __builtin_bit_cast(half2v, szw);
  DeqConst3 c;
  c.k64 = __builtin_elementwise_fma(sz, half2v{(half_t)64.0f, (half_t)-0.015625f},
                                    half2v{(half_t)-0.0f, (half_t)-1.0f});
  c.k16 = __builtin_elementwise_fma(c.k64, half2v{(half_t)0.25f, (half_t)4.0f},
                                    half2v{(half_t)-0.0f, (half_t)3.0f});
  c.k8 = __builtin_elementwise_fma(c.k16, half2v{(half_t)0.5f, (half_t)2.0f},
                                   half2v{(half_t)-0.0f, (half_t)1.0f});
  return c;
}

template <int N>
__device__ __forceinline__ half2v k3_of(const DeqConst3& c) {
  if constexpr (cls3(N) == 4) return c.k64;
  else if constexpr (cls3(N) == 6) return c.k16;
  else return c.k8;
}

// Dequantized A operand RND_f16((q - z) s) of step S of a 3-bit unit.
template <int S>
__device__ __forceinline__ half8v deq3_step(uint32_t D0, uint32_t D1, uint32_t D2,
                                            const DeqConst3& c) {
  u32x4 r;
  r[0] = deq_pair(raw3_pair<4 * S + 0>(D0, D1, D2), k3_of<4 * S + 0>(c));
  r[1] = deq_pair(raw3_pair<4 * S + 1>(D0, D1, D2), k3_of<4 * S + 1>(c));
  r[2] = deq_pair(raw3_pair<4 * S + 2>(D0, D1, D2), k3_of<4 * S + 2>(c));
  r[3] = deq_pair(raw3_pair<4 * S + 3>(D0, D1, D2), k3_of<4 * S + 3>(c));
  return as_half8(r);
}

// Table dequantization for 3-bit codes (any finite scale and zero point):
// the eight values RND_f16(fl32(fl32(q - z) * s)) as byte tables, low bytes
// of q = 0..3 / 4..7 in lo0 / lo1, high bytes in hi0 / hi1.  A pair takes its
// low bytes from lo (selector bytes q0, 12, q1, 12; 12 selects a zero byte)
// and its high bytes from hi (12, q0, 12, q1).
struct DeqLut3 {
  uint32_t lo0, lo1, hi0, hi1;
};
__device__ __forceinline__ DeqLut3 deq_lut3(uint32_t szw) {
  const float s = (float)__builtin_bit_cast(half_t, (uint16_t)(szw & 0xFFFFu));
  const float z = (float)__builtin_bit_cast(half_t, (uint16_t)(szw >> 16));
  uint32_t h[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) h[q] = deq_bits((float)q, z, s);
  DeqLut3 t;
  const uint32_t h01 = h[0] | (h[1] << 16), h23 = h[2] | (h[3] << 16);
  const uint32_t h45 = h[4] | (h[5] << 16), h67 = h[6] | (h[7] << 16);
  t.lo0 = __builtin_amdgcn_perm(h23, h01, 0x06040200u);
  t.hi0 = __builtin_amdgcn_perm(h23, h01, 0x07050301u);
  t.lo1 = __builtin_amdgcn_perm(h67, h45, 0x06040200u);
  t.hi1 = __builtin_amdgcn_perm(h67, h45, 0x07050301u);
  return t;
}
__device__ __forceinline__ uint32_t lut3_pair(uint32_t x, const DeqLut3& t) {
  const uint32_t r1 = __builtin_amdgcn_perm(t.lo1, t.lo0, x | 0x0C000C00u);
  const uint32_t r2 = __builtin_amdgcn_perm(t.hi1, t.hi0, (x << 8) | 0x000C000Cu);
  return r1 | r2;
}
template <int S>
__device__ __forceinline__ half8v lut3_step(uint32_t D0, uint32_t D1, uint32_t D2,
                                            const DeqLut3& t) {
  u32x4 r;
  r[0] = lut3_pair(codes3_pair<4 * S + 0>(D0, D1, D2), t);
  r[1] = lut3_pair(codes3_pair<4 * S + 1>(D0, D1, D2), t);
  r[2] = lut3_pair(codes3_pair<4 * S + 2>(D0, D1, D2), t);
  r[3] = lut3_pair(codes3_pair<4 * S + 3>(D0, D1, D2), t);
  return as_half8(r);
}

// ---- reductions -----------------------------------------------------------
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int wave_incl_scan_i(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Sum over aligned groups of G lanes (G = 1, 2, 4, 8, 16 or 32): DPP moves
// inside 16-lane rows (xor 1, xor 2, half-row mirror, row mirror), one
// shuffle across rows for 32.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32, "group size");
  if constexpr (G >= 2) v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v += dpp_f<0x141>(v);   // row_half_mirror
  if constexpr (G >= 16) v += dpp_f<0x140>(v);  // row_mirror
  if constexpr (G >= 32) v += __shfl_xor(v, 16, 64);
  return v;
}

// Exclusive scan over the block (blockDim.x multiple of 64, <= 1024).
// s_w: shared int[17].  Returns the exclusive prefix; *total gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* s_w, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
  const int inc = wave_incl_scan_i(v, lane);
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  if (w == 0) {
    const int t = (lane < nw) ? s_w[lane] : 0;
    const int i2 = wave_incl_scan_i(t, lane);
    if (lane < nw) s_w[lane] = i2 - t;
    if (lane == nw - 1) s_w[16] = i2;
  }
  __syncthreads();
  const int res = s_w[w] + inc - v;
  *total = s_w[16];
  __syncthreads();
  return res;
}

// Segment of `tile` in a tile prefix toff[0..nseg] (toff[0] = 0,
// non-decreasing): the number of entries toff[1..nseg] <= tile, or -1 when
// tile >= toff[nseg].  Called by every thread; uses *s_res.
__device__ __forceinline__ int find_segment(const int* toff, int nseg, int tile, int* s_res) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int c = 0;
    for (int i = lane + 1; i <= nseg; i += 64) c += (toff[i] <= tile) ? 1 : 0;
    c = wave_sum_i(c);
    if (lane == 0) *s_res = (tile < toff[nseg]) ? c : -1;
  }
  __syncthreads();
  return *s_res;
}

// fp32 -> storage type (round to nearest even)
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ half_t from_f32<half_t>(float v) { return (half_t)v; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float v) { return (__bf16)v; }

template <typename T> __device__ __forceinline__ float to_f32(T v) { return (float)v; }

// silu(v) = v / (1 + e^-v) from the hardware base-2 exponential and
// reciprocal (each within about one ulp in fp32; the result is rounded to the
// activation dtype afterwards).  v -> -inf: e^-v overflows to inf and the
// reciprocal to 0.
__device__ __forceinline__ float silu_f(float v) {
  const float e = __builtin_amdgcn_exp2f(v * -1.4426950408889634f);
  return v * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace tq
