// Device helpers for gfx950 (CDNA4, wave64): fp16 conversion, int4 dot
// products with in-register dequantisation, lane-group reductions, top-K.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smd {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(f16, b); }
// fp32 -> fp16, round-to-nearest-even (the hardware default rounding mode).
__device__ __forceinline__ uint16_t f2h(float v) { return __builtin_bit_cast(uint16_t, (f16)v); }

__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// Load through the global address space. Pointers read out of device tables
// are generic; a generic (flat) load is also counted by the LDS wait counter,
// so every LDS wait would stall on it. Weights are always in global memory.
template <typename T>
__device__ __forceinline__ T ldg(const T* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ldg(const uint4* p) {
  const u32x4 v = *(const __attribute__((address_space(1))) u32x4*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float dot2(f16x2 a, f16x2 b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

// The eight int4 weights of one packed word as exact fp16 pairs.
//
// The word holds two's-complement nibbles n_0..n_7 (n_j at bits 4j). With
// 0x8 XOR-ed into a nibble it becomes the offset-binary u_j = q_j + 8 in
// [0, 15]; placed in the mantissa of fp16 1024.0 (0x6400) it reads
// 1024 + u exactly, and a nibble sitting 4 bits higher reads 1024 + 16u.
// Both steps are one bitwise select per register: C ^ (w & M), with M the
// nibble mask and C the 0x8 XOR bits inside M plus the 0x6400 exponent bits
// outside it. One packed fp16 subtract (or multiply-add by 1/16) then gives
// q exactly, two values per register:
//   p0 = (q0, q4)   p1 = (q1, q5)   p2 = (q2, q6)   p3 = (q3, q7)
// so activations must be supplied pair-permuted as
//   xp[0] = (x0, x4)  xp[1] = (x1, x5)  xp[2] = (x2, x6)  xp[3] = (x3, x7).
// AFF (the affine codec): the nibbles are unsigned values q in [0, 15];
// without the 0x8 XOR the mantissa reads 1024 + q (1024 + 16 q a nibble
// higher), so the same two instructions per register subtract 1024 (or
// scale by 1/16 and subtract 64).
template <bool AFF = false>
__device__ __forceinline__ void q4_pairs(uint32_t w, f16x2& p0, f16x2& p1, f16x2& p2,
                                         f16x2& p3) {
  const uint32_t v = w >> 8;
  const uint32_t c0 = AFF ? 0x64006400u : 0x64086408u, c1 = AFF ? 0x64006400u : 0x64806480u;
  const f16x2 k0 = {(f16)(AFF ? 1024.0f : 1032.0f), (f16)(AFF ? 1024.0f : 1032.0f)};
  const f16x2 k16 = {(f16)0.0625f, (f16)0.0625f};
  const f16x2 k1 = {(f16)(AFF ? 64.0f : 72.0f), (f16)(AFF ? 64.0f : 72.0f)};
  p0 = as_h2(c0 ^ (w & 0x000F000Fu)) - k0;
  p1 = as_h2(c1 ^ (w & 0x00F000F0u)) * k16 - k1;
  p2 = as_h2(c0 ^ (v & 0x000F000Fu)) - k0;
  p3 = as_h2(c1 ^ (v & 0x00F000F0u)) * k16 - k1;
}

// bf16 bit pattern to fp32 (exact).
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Eight int4 weights of one packed word against eight pair-permuted
// activations; q and x are exact in fp16, v_dot2_f32_f16 accumulates the
// products in fp32.
template <bool AFF = false>
__device__ __forceinline__ float q4_dot8(uint32_t w, const f16x2* xp, float acc) {
  f16x2 p0, p1, p2, p3;
  q4_pairs<AFF>(w, p0, p1, p2, p3);
  acc = dot2(p0, xp[0], acc);
  acc = dot2(p1, xp[1], acc);
  acc = dot2(p2, xp[2], acc);
  acc = dot2(p3, xp[3], acc);
  return acc;
}

// Position of element i inside its 8-element block after the pair
// permutation q4_dot8 expects: [x0 x4 x1 x5 x2 x6 x3 x7].
__device__ __forceinline__ int perm8(int i) {
  int j = i & 7;
  return (i & ~7) | (j < 4 ? 2 * j : 2 * (j - 4) + 1);
}

// DPP lane moves within a 16-lane row (bound_ctrl off, all lanes active).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LG lanes (LG in {1, 2, 4, 8, 16}); every lane of
// the group receives the group sum. quad_perm swaps, then half-row and row
// mirrors, so partner lanes never leave the group.
template <int LG>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LG >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (LG >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (LG >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if constexpr (LG >= 16) v += dpp_f<0x140>(v); // row_mirror
  return v;
}

template <int LG>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (LG >= 2) v = fmaxf(v, dpp_f<0xB1>(v));
  if constexpr (LG >= 4) v = fmaxf(v, dpp_f<0x4E>(v));
  if constexpr (LG >= 8) v = fmaxf(v, dpp_f<0x141>(v));
  if constexpr (LG >= 16) v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Wave-wide sum / max without LDS traffic: DPP inside each 16-lane row, then
// the four row results are read into scalars. The whole wave must be active.
__device__ __forceinline__ float wave_sum_rows(float v) {
  v = group_sum<16>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

__device__ __forceinline__ float wave_max_rows(float v) {
  v = group_max<16>(v);
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)),
               fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Wave-wide maximum of a uint32 (DPP in each 16-lane row, then the four row
// results); the whole wave must be active.
__device__ __forceinline__ uint32_t wave_max_u32_rows(uint32_t v) {
  v = umax32(v, dpp_u<0xB1>(v));
  v = umax32(v, dpp_u<0x4E>(v));
  v = umax32(v, dpp_u<0x141>(v));
  v = umax32(v, dpp_u<0x140>(v));
  return umax32(umax32((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                       (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
                umax32((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                       (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// Wave-wide maximum of 64-bit keys (score bits high, a distinct tag low):
// the maximal high word, then, only when several lanes hold it, the largest
// low word among them (the 64-bit maximum, found with 32-bit steps). The
// whole wave must be active.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  const uint32_t hi = (uint32_t)(k >> 32), lo = (uint32_t)k;
  const uint32_t mh = wave_max_u32_rows(hi);
  const uint64_t tied = __ballot(hi == mh);
  uint32_t ml;
  if (__popcll(tied) == 1)
    ml = (uint32_t)__builtin_amdgcn_readlane((int)lo, __ffsll((unsigned long long)tied) - 1);
  else
    ml = wave_max_u32_rows(hi == mh ? lo : 0u);
  return ((uint64_t)mh << 32) | ml;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t f2key(float v) {
  uint32_t b = __builtin_bit_cast(uint32_t, v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Split an fp32 vector value into fp16 hi + lo after scaling by 2^-e, so that
// dot products against fp16 weights keep ~22 bits of the activation:
// x * 2^-e = hi + lo + O(2^-22 |x|).
__device__ __forceinline__ void split_hilo(float v, float inv_scale, f16& hi, f16& lo) {
  float t = v * inv_scale;
  hi = (f16)t;
  lo = (f16)(t - (float)hi);
}

// Packed exchange words: two fp32 values rounded to 28 bits (19 stored
// mantissa bits, round to nearest even; relative error <= 2^-20) under an
// 8-bit launch tag in the top byte. The tag is 1 + epoch % 255; the host
// clears the buffer before a tag can recur.
__device__ __forceinline__ uint32_t round28(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  return (b + 0x7u + ((b >> 4) & 1u)) >> 4;
}
__device__ __forceinline__ void put2(uint64_t* p, float v0, float v1, uint32_t tag) {
  const uint64_t w = ((uint64_t)tag << 56) | ((uint64_t)(round28(v0) & 0xFFFFFFFu) << 28) |
                     (uint64_t)(round28(v1) & 0xFFFFFFFu);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The two values of a packed word given as its low and high 32-bit halves.
__device__ __forceinline__ float2 unpack2(uint32_t lo, uint32_t hi) {
  const uint32_t r0 = ((hi & 0x00FFFFFFu) << 4) | (lo >> 28);
  const uint32_t r1 = lo & 0x0FFFFFFFu;
  return make_float2(__builtin_bit_cast(float, r0 << 4), __builtin_bit_cast(float, r1 << 4));
}

}  // namespace smd
