// Device helpers shared by the codec and attention kernels (gfx950).
//
// Bit-exact arithmetic of the residual codec (see include/kvc.h): every helper
// here performs exactly one IEEE binary32 operation per step, rounding to
// nearest even; the translation units are compiled with -ffp-contract=off so
// no multiply-add is fused behind our back.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;   // MFMA operand
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));                // MFMA operand
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;  // 32x32 acc
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;    // 16x16 acc

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// float -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even: one
// v_cvt_pk_bf16_f32, the same bits as f32_to_bf16_bits for every finite input, denormals
// included (NaN payloads may differ). Inline asm, so that the compiler keeps one
// instruction per pair also where the pair is unpacked again; f32_to_bf16_bits costs
// three instructions per value.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  uint32_t r;
  asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
  return r;
}

// fp16 conversions through clang's _Float16 (fptrunc is round-to-nearest-even).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(b & 0xFFFFu));
}

// Load one element of an input tensor as fp32 (XT = float or uint16_t bf16 bits).
template <typename XT>
__device__ __forceinline__ float load_x(const XT* p);
template <>
__device__ __forceinline__ float load_x<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_x<uint16_t>(const uint16_t* p) {
  return bf16_bits_to_f32(*p);
}

template <typename XT>
__device__ __forceinline__ void store_x(XT* p, float v);
template <>
__device__ __forceinline__ void store_x<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_x<uint16_t>(uint16_t* p, float v) {
  *p = (uint16_t)f32_to_bf16_bits(v);
}

// Round a value to what the storage dtype holds (identity for fp32).
template <typename XT>
__device__ __forceinline__ float round_to(float v);
template <>
__device__ __forceinline__ float round_to<float>(float v) { return v; }
template <>
__device__ __forceinline__ float round_to<uint16_t>(float v) {
  return bf16_bits_to_f32(f32_to_bf16_bits(v));
}

// ---------------------------------------------------------------------------
// Group quantizer.  r[0..n) in registers -> scale/zero word and codes.
// z = fp16(min), s = fp16((max - min) / L) with IEEE division,
// code = clamp(rint((r - z) / s), 0, L), all codes 0 when s == 0.
// ---------------------------------------------------------------------------
struct GroupQ {
  float s, z;       // fp16 values widened to fp32
  uint32_t word;    // fp16(s) | fp16(z) << 16
};

__device__ __forceinline__ GroupQ group_scale_zero(float mn, float mx, int levels) {
  GroupQ g;
  uint32_t zb = f32_to_f16_bits(mn);
  float s32 = (mx - mn) / (float)levels;   // correctly rounded division (HIP default)
  uint32_t sb = f32_to_f16_bits(s32);
  g.s = f16_bits_to_f32(sb);
  g.z = f16_bits_to_f32(zb);
  g.word = sb | (zb << 16);
  return g;
}

__device__ __forceinline__ uint32_t quantize_one(float r, const GroupQ& g, int levels) {
  if (g.s == 0.0f) return 0u;
  float t = rintf((r - g.z) / g.s);
  t = fminf(fmaxf(t, 0.0f), (float)levels);
  return (uint32_t)t;
}

// (code * s) + z: code * s is exact (code <= 15, s has 11 significant bits), so a
// fused multiply-add gives the same single rounding as the two-step form.
__device__ __forceinline__ float dequant_one(uint32_t code, float s, float z) {
  return __builtin_fmaf((float)code, s, z);
}

// Lanes l and l ^ 32 exchange a 32-bit value (v_permlane32_swap); hf = lane >> 5.
__device__ __forceinline__ uint32_t swap_halves(uint32_t v, int hf) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return hf ? r[0] : r[1];
}

// The two bf16 values of a packed word, widened exactly to fp32.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Group quantizer of the codec contract on G residuals whose group min and max are
// mn and mx (a group may span lanes): scale/zero as group_scale_zero, codes
// clamp(rint(fl(fl(r - z) / s)), 0, L) packed BITS-wide into cw.  The quotient is taken as r * rcp(s) - z * rcp(s), which rounds to the same
// integer unless it lies within (|z / s| + L + 2) 2^-19 of a half-integer (the two
// forms differ by at most a quarter of that for the values that the clamp keeps); a
// group with such a value is redone with the IEEE division.
template <int BITS, int G>
__device__ __forceinline__ GroupQ quantize_with(const float (&r)[G], float mn, float mx,
                                                uint32_t (&cw)[G * BITS / 32]) {
  constexpr int L = (1 << BITS) - 1, PER = 32 / BITS, GW = G / PER;
  const GroupQ q = group_scale_zero(mn, mx, L);
#pragma unroll
  for (int w = 0; w < GW; ++w) cw[w] = 0u;
  if (q.s != 0.0f) {
    const float rinv = __builtin_amdgcn_rcpf(q.s);
    const float nzr = -(q.z * rinv);
    const float thr = 0.5f - (fabsf(nzr) + (float)(L + 2)) * 0x1p-19f;
    float dev = 0.0f;   // largest |y - rint(y)| of the group
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float y = __builtin_fmaf(r[i], rinv, nzr);
      const float k = __builtin_rintf(y);
      dev = fmaxf(dev, fabsf(y - k));
      const uint32_t code = (uint32_t)__builtin_amdgcn_fmed3f(k, 0.0f, (float)L);
      cw[i / PER] |= code << (BITS * (i % PER));
    }
    if (dev > thr) {
#pragma unroll
      for (int w = 0; w < GW; ++w) cw[w] = 0u;
#pragma unroll
      for (int i = 0; i < G; ++i) cw[i / PER] |= quantize_one(r[i], q, L) << (BITS * (i % PER));
    }
  }
  return q;
}

// The same with the group's min and max taken over r itself.
template <int BITS, int G>
__device__ __forceinline__ GroupQ quantize_group(const float (&r)[G], uint32_t (&cw)[G * BITS / 32]) {
  float mn = r[0], mx = r[0];
#pragma unroll
  for (int i = 1; i < G; ++i) { mn = fminf(mn, r[i]); mx = fmaxf(mx, r[i]); }
  return quantize_with<BITS, G>(r, mn, mx, cw);
}

// Code i of a group packed by quantize_group.
template <int BITS, int G>
__device__ __forceinline__ uint32_t group_code(const uint32_t (&cw)[G * BITS / 32], int i) {
  constexpr int PER = 32 / BITS;
  return (cw[i / PER] >> (BITS * (i % PER))) & ((1u << BITS) - 1u);
}

// XCD-aware remap of a linear workgroup id: hardware dispatches consecutive ids
// round-robin over the 8 XCDs; this gives each XCD a contiguous range of tiles so
// tiles that share data (same head) share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int nx = 8;
  int per = (nblocks + nx - 1) / nx;
  int xcd = bid % nx;
  int slot = bid / nx;
  // XCDs with index < nblocks % nx own `per` tiles, others `per - 1` (when uneven).
  int rem = nblocks % nx;
  int start;
  if (rem == 0) {
    start = xcd * per;
  } else {
    start = (xcd < rem) ? xcd * per : rem * per + (xcd - rem) * (per - 1);
  }
  return start + slot;
}

}  // namespace kvc
