// Decode-fused attention over a compressed K/V history.
//
// Method: queries attend to the compressed history of keys and values (NanoKV
// abstract: repeated attention over history is the cost to cut); O =
// softmax(Q K^T * scale) V per head, no mask.  The decoded cache is what a
// bf16 (or fp32) cache would hold: every decoded value is rounded to the cache
// dtype before it meets a query.
//
// bf16 path (d = 128), one workgroup = 8 wave64 = 256 queries of one head:
//   per 64-key tile: all 512 threads decode K (row-major bf16) and V (transposed
//   fp16) into one of two LDS buffers from compressed rows prefetched a tile earlier
//   with buffer loads (indices two tiles earlier), while the other buffer is consumed:
//   each wave computes S^T = K Q^T for its 32 queries with
//   v_mfma_f32_32x32x16_bf16 (a lane owns one query column, so the softmax row
//   reductions are in-lane plus one cross-half exchange), runs the online
//   softmax in fp32 with exp2, rounds P to fp16 (nearest even) and accumulates
//   O^T += V^T P^T with v_mfma_f32_32x32x16_f16.  The decoded values are rounded to
//   bf16 (the cache dtype) and then held in fp16, which represents every bf16 value
//   of magnitude 2^-14..65504 exactly; fp16 P carries 3 more mantissa bits than bf16,
//   which keeps the output within 2e-2 of the fp64 result on caches with x10 outlier
//   channels (bf16 P does not), at the same MFMA rate.  The P^T register layout that
//   the S^T tile produces is used directly as the B operand: the key order inside
//   each 16-key MFMA step is permuted, and V^T is read from LDS in the same order.
// fp32 path (d = 64 or 128): one lane per query, fp32 dot products and softmax.
#include <type_traits>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

enum { SRC_NONE = 0, SRC_CENTROID = 1 };

struct Src {
  const uint32_t* codes;
  const uint32_t* sz;
  const void* index;
  const void* cen;     // [H][C][D] cache dtype
  const uint16_t* cen16;   // fp16 image of cen (c * 2^cexp[h]), or null
  const int32_t* cexp;     // [H] per-head exponents of cen16
  int64_t cap;
  int bits, group, groups, words, idxb, C, mode;
  int rot;             // Hn residual transform width: 0, 16 or 64
};

struct AttnParams {
  const void* q;
  int64_t nq, nk;
  int H;
  float scale;        // softmax scale (fp32 path)
  float scale_log2;   // softmax scale * log2(e) (bf16 path)
  float* out;
  float* lse;
  Src k, v;
  const uint16_t* basis;   // mixed-dimensional keys: [d][m] bf16
  // key splitting: workgroup (head, query block, split) covers key tiles
  // [split * tps, min(ntiles, (split + 1) * tps)) and writes its normalized partial
  // output and log-sum-exp to part_o [splits][nq][H][D] / part_lse [splits][H][nq]
  int splits, tps;
  float* part_o;
  float* part_lse;
  int jensen;   // subtract the Jensen-bias correction from compressed keys' logits
};

// Decode channels ch0..ch0+7 of key `key` (head h) as fp32 (cache dtype XT rounding
// is applied by the caller).  Groups are >= 16 wide, so the 8 channels share one
// scale/zero word and their codes one 32-bit word.
template <typename XT, int D>
__device__ __forceinline__ void decode8(const Src& s, int h, int64_t key, int ch0, float v[8]) {
  const int64_t row = (int64_t)h * s.cap + key;
  const uint32_t szw = s.sz[row * s.groups + ch0 / s.group];
  const float sc = f16_bits_to_f32(szw & 0xFFFFu);
  const float ze = f16_bits_to_f32(szw >> 16);
  const int bitpos = ch0 * s.bits;
  const uint32_t bits8 = s.codes[row * s.words + (bitpos >> 5)] >> (bitpos & 31);
  const uint32_t mask = (1u << s.bits) - 1u;
  float base[8];
  if (s.mode == SRC_CENTROID) {
    int a = s.idxb == 1 ? reinterpret_cast<const uint8_t*>(s.index)[row]
                        : reinterpret_cast<const uint16_t*>(s.index)[row];
    a = min(a, s.C - 1);   // out-of-contract indices must not read past the table
    const XT* c = reinterpret_cast<const XT*>(s.cen) + ((int64_t)h * s.C + a) * D + ch0;
    if constexpr (sizeof(XT) == 2) {
      const uint4 w = *reinterpret_cast<const uint4*>(c);
      base[0] = bf16_bits_to_f32(w.x & 0xFFFFu); base[1] = bf16_bits_to_f32(w.x >> 16);
      base[2] = bf16_bits_to_f32(w.y & 0xFFFFu); base[3] = bf16_bits_to_f32(w.y >> 16);
      base[4] = bf16_bits_to_f32(w.z & 0xFFFFu); base[5] = bf16_bits_to_f32(w.z >> 16);
      base[6] = bf16_bits_to_f32(w.w & 0xFFFFu); base[7] = bf16_bits_to_f32(w.w >> 16);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) base[k] = load_x<XT>(c + k);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) base[k] = 0.0f;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t code = (bits8 >> (s.bits * k)) & mask;
    v[k] = base[k] + dequant_one(code, sc, ze);
  }
}

// ----------------------------------------------------------------------------
// bf16 MFMA path
// ----------------------------------------------------------------------------
constexpr int BK = 64;           // keys per tile
constexpr int NW = 8;            // waves per workgroup (two per SIMD)
constexpr int QW = 32;           // queries per wave
constexpr int BQ = NW * QW;      // queries per workgroup
constexpr int NT = NW * 64;      // threads per workgroup
constexpr int DM = 128;          // head dim of the MFMA path
constexpr int KROW = DM + 8;     // K tile row (bf16 elements), padded
constexpr int VROW = BK + 16;    // V^T tile row (fp16 elements), padded to 40 dwords: the
                                 // 32 lanes of a 16-byte fragment read then hit distinct
                                 // banks (rocprofv3 SQ_LDS_BANK_CONFLICT 3x lower than 36)

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// c + d for c the fp16 value in the low / high half of w scaled by sc (a power of two):
// one v_fma_mix_f32, c * sc + d with a single rounding, i.e. exactly fl(c * sc + d)
__device__ __forceinline__ float add_f16lo(uint32_t w, float sc, float d) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(sc), "v"(d));
  return r;
}
__device__ __forceinline__ float add_f16hi(uint32_t w, float sc, float d) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(sc), "v"(d));
  return r;
}
__device__ __forceinline__ float byte_f(uint32_t x, int k) { return (float)((x >> (8 * k)) & 0xFFu); }
// A code held in a 16-bit half of w, read as the f16 denormal q * 2^-24.  v_fma_mix_f32
// widens it exactly, so fma(code_lo(w), s * 2^24, z) == fma(q, s, z) bit for bit (s an
// fp16 value, s * 2^24 exact in fp32): one instruction per code, no integer conversion.
__device__ __forceinline__ float code_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float code_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 v = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}
// pk_bf16 kept opaque to the compiler: where the packed pair is unpacked again (the V
// tile's bf16-to-fp16 step) it would otherwise round each value with its own
// conversion and shift (three instructions per value instead of two per pair)
__device__ __forceinline__ uint32_t pk_bf16_asm(float a, float b) {
  uint32_t r;
  asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// packed bf16 pair -> packed fp16 pair holding the same values (exact for |v| in
// 2^-14..65504; nearest even otherwise)
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 v = {(_Float16)lo_bf16(w), (_Float16)hi_bf16(w)};
  return __builtin_bit_cast(uint32_t, v);
}

// Value held by lane l ^ 32 (v_permlane32_swap: the upper half of the first operand
// and the lower half of the second trade places).
__device__ __forceinline__ float other_half(float x, int half) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(half ? r[0] : r[1]);
}

// Registers a thread prefetches for one tile.
template <int BITS>
struct KPre {                     // key kk, channels 16w..16w+15
  uint32_t code[BITS / 2];
  uint32_t sz;
  uint4 c0, c1;
};
struct VPre {                     // keys 2kp, 2kp+1, channels 8c8..8c8+7
  uint32_t code[2];
  uint32_t sz[2];
  uint4 c[2];
};

// V^T tile layout: row r (a channel) holds the tile's 64 keys as fp16.  Inside each
// group of 16 keys, bits 2 and 3 of the key index are swapped, so the 8 keys one lane
// feeds to a PV MFMA ({4 h .. 4 h + 3, 8 + 4 h .. 8 + 4 h + 3} of the group, h = lane's
// half) are 8 consecutive elements: one 16-byte read.  The 8-element blocks of row r
// are XOR-permuted by (r / 16) mod 8; with the 40-dword row stride the 32 lanes served
// together by a 16-byte read then touch 32 distinct 4-bank slots, and the transposed
// decode writes are at most two-way.
__device__ __forceinline__ int vpos(int row, int key) {
  const int k16 = key & 15;
  const int p = (key & ~15) | (k16 & 3) | ((k16 & 4) << 1) | ((k16 & 8) >> 1);
  return (((p >> 3) ^ ((row >> 4) & 7)) << 3) | (p & 7);
}

// DENSE: K and V are uncompressed bf16 caches [capacity][H][d] (e.g. what kvc_decode
// writes for a predictor chain); the tile loaders copy rows instead of decoding.
// MIXED: keys are NanoKV-Fast coefficient records.  The K tile then holds, per key,
// the centroid row C[a] (128 bf16) followed by the dequantized coefficients c split
// into bf16 high and low parts (16 + 16); the queries carry B^T q split the same way,
// and three extra MFMA steps add (B^T q) . c to q . C[a] with about 2^-16 relative
// error - the score is formed without reconstructing the key.
// The value of the lane M = 1, 2 or 4 apart within aligned groups of 8 lanes, by DPP
// (quad_perm [1,0,3,2] / [2,3,0,1]; for 4, lanes 0-3 of each group read 4-7 by
// row_shl:4 and lanes 4-7 read 0-3 by row_shr:4, selected by bank masks).
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  const int x = __builtin_bit_cast(int, v);
  int r;
  if constexpr (M == 1) {
    r = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);
  } else if constexpr (M == 2) {
    r = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);
  } else {
    static_assert(M == 4, "lane distance");
    r = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xF, 0x5, false);
    r = __builtin_amdgcn_update_dpp(r, x, 0x114, 0xF, 0xA, false);
  }
  return __builtin_bit_cast(float, r);
}

// One butterfly stage between lanes M apart: the lower piece takes a + b, the upper
// a - b, both as fma(own, +-1, partner) - one rounding of the exact sum or difference.
template <int M, int W>
__device__ __forceinline__ void hn_lane_stage(float (&v)[W], int piece) {
  const float sg = (piece & M) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < W; ++i) v[i] = __builtin_fmaf(v[i], sg, lane_xor<M>(v[i]));
}

// Hn transform back (Coral-KV Fig. 5: residuals were rotated per group of n channels
// before quantization) on a lane's W consecutive channels of one vector, pieces of the
// vector on consecutive lanes (piece = lane's index within the vector, groups of 8
// lanes aligned): butterflies at channel distance 1 .. W/2 in the lane, then W, 2W, ..
// n/2 with the lanes 1, 2, 4 apart - the order of the Sylvester recursion, so the
// result is the codec decoder's to the bit.  The values come in already scaled by
// 1/sqrt(n) (exact).
template <int W>
__device__ __forceinline__ void hn_back(float (&v)[W], int piece, int n) {
#pragma unroll
  for (int h = 1; h < W; h <<= 1) {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
  if (n > W) hn_lane_stage<1>(v, piece);
  if (n > 2 * W) hn_lane_stage<2>(v, piece);
  if constexpr (W < 16) {
    if (n > 4 * W) hn_lane_stage<4>(v, piece);
  }
}

// JB (Jensen-bias correction, the INT2 Jensen-bias abstract on the Coral-KV listing
// page): a compressed key with step s_g on scale group g has rounding noise of variance
// s_g^2 / 12 per channel, which raises E[exp(logit)] by (scale^2 / 24) sum_g s_g^2
// ||q_g||^2 to second order; the kernel subtracts that from the logit.  The K decode
// writes s_g^2 (bf16) next to each key row (columns DM + g, zero for g >= d/group) and
// every lane holds -(scale / 24) ||q_g||^2 of its query as a B operand (k = g), so one
// more v_mfma_f32_32x32x16_bf16 per 32-key block adds the correction to the raw scores.
template <int BITS, int VBITS, bool KCEN, bool VCEN, bool MIXED, bool DENSE = false, bool ROT = false,
          bool JB = false, bool CF16 = false>
__global__ __launch_bounds__(NT, 1) void attend_bf16_kernel(AttnParams p) {
  constexpr int KR = MIXED ? DM + 32 + 8 : (JB ? DM + 16 + 8 : KROW);   // K tile row (bf16 elements)
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BK * KR];     // bf16
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][DM * VROW];   // fp16 bits

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int nqb = (int)((p.nq + BQ - 1) / BQ);
  const int nk = (int)p.nk;
  const int ntiles = (nk + BK - 1) / BK;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int split = tile % p.splits, hq = tile / p.splits;
  const int tb = split * p.tps, te = min(ntiles, tb + p.tps);   // this split's key tiles
  const int h = hq / nqb;
  const int64_t myq = (int64_t)(hq % nqb) * BQ + wave * QW + col;

  // Per-head buffer resources (SGPRs): every prefetch is a buffer load with a 32-bit
  // byte offset, and the descriptor's record count bounds it.  The count covers the
  // n_keys attended rows only (not the store's capacity), so the tail of the last tile
  // reads zeros - codes 0, scale and zero 0, centroid 0: finite values whose weight is
  // masked to 0 - never whatever unwritten rows past n_keys hold.
  auto rsrc = [](const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
  };
  const int kwb = p.k.words * 4, kgb = p.k.groups * 4;   // bytes per key row
  const int vwb = p.v.words * 4, vgb = p.v.groups * 4;
  const int64_t khrow = (int64_t)h * p.k.cap, vhrow = (int64_t)h * p.v.cap;
  const int64_t nkr = p.nk;   // rows visible to the loads (n_keys <= capacity)
  const auto rk_code = rsrc(p.k.codes + khrow * p.k.words, nkr * kwb);
  const auto rk_sz = rsrc(p.k.sz + khrow * p.k.groups, nkr * kgb);
  const auto rv_code = rsrc(p.v.codes + vhrow * p.v.words, nkr * vwb);
  const auto rv_sz = rsrc(p.v.sz + vhrow * p.v.groups, nkr * vgb);
  const auto rk_idx = rsrc(reinterpret_cast<const uint8_t*>(p.k.index) + khrow * p.k.idxb,
                           KCEN ? nkr * p.k.idxb : 0);
  const auto rv_idx = rsrc(reinterpret_cast<const uint8_t*>(p.v.index) + vhrow * p.v.idxb,
                           VCEN ? nkr * p.v.idxb : 0);
  // CF16: the tables' fp16 images (c * 2^e_h, same layout and size) and the per-head
  // powers of two 2^-e_h that restore c inside the centroid add
  const uint16_t* kcen = CF16 ? p.k.cen16 : reinterpret_cast<const uint16_t*>(p.k.cen);
  const uint16_t* vcen = CF16 ? p.v.cen16 : reinterpret_cast<const uint16_t*>(p.v.cen);
  const auto rk_cen = rsrc(kcen + (int64_t)h * p.k.C * DM, KCEN ? (int64_t)p.k.C * DM * 2 : 0);
  const auto rv_cen = rsrc(vcen + (int64_t)h * p.v.C * DM, VCEN ? (int64_t)p.v.C * DM * 2 : 0);
  const float ksc = CF16 ? __int_as_float((127 - p.k.cexp[h]) << 23) : 1.0f;
  const float vsc = CF16 ? __int_as_float((127 - p.v.cexp[h]) << 23) : 1.0f;
  // centroid + dequantized residual (fp32, one rounding), channel pair in word w
  auto cadd_lo = [&](uint32_t w, float sc, float d) {
    if constexpr (CF16) return add_f16lo(w, sc, d);
    else return lo_bf16(w) + d;
  };
  auto cadd_hi = [&](uint32_t w, float sc, float d) {
    if constexpr (CF16) return add_f16hi(w, sc, d);
    else return hi_bf16(w) + d;
  };

  // DENSE: one resource over the whole token-major cache, rows H*d apart
  const int hdb = p.H * DM * 2;
  const auto rk_dense = rsrc(p.k.codes, DENSE ? nkr * hdb : 0);
  const auto rv_dense = rsrc(p.v.codes, DENSE ? nkr * hdb : 0);

  // decode roles: 8 lanes share a K row (16 channels each), 16 lanes share a V row (8
  // channels each), so every load instruction reads whole contiguous rows
  const int kk = tid >> 3, kw = tid & 7;          // K: key kk, channels 16kw..16kw+15
  const int c8 = tid & 15, kp = tid >> 4;         // V: keys 2kp, 2kp+1, channels 8c8..8c8+7
  // first code word of the thread's 16 channels (MIXED: of coefficients 8kw..8kw+7)
  const int kword = MIXED ? (2 * kw * BITS) >> 5 : (16 * kw * BITS) >> 5;
  const int kcsh = MIXED ? (2 * kw * BITS) & 31 : 0;
  const int kgrp = MIXED ? 0 : (16 * kw) / p.k.group;   // coefficients: one group per key
  const int vword = (8 * c8 * VBITS) >> 5;
  const int vgrp = (8 * c8) / p.v.group;
  const int vsh = (8 * c8 * VBITS) & 31;          // bit offset of the 8 codes in their word
  // INT2 V: byte selector that puts the two keys' 16 code bits side by side
  const uint32_t vsel = vsh ? 0x07060302u : 0x05040100u;
  // index entries are read one at a time (byte or short buffer loads), so the range
  // check of the buffer resource covers exactly the stored entries
  auto load_index = [](__amdgpu_buffer_rsrc_t r, uint32_t key, int idxb) -> int {
    return idxb == 1 ? (int)__builtin_amdgcn_raw_buffer_load_b8(r, key, 0, 0)
                     : (int)__builtin_amdgcn_raw_buffer_load_b16(r, 2u * key, 0, 0);
  };
  auto idx_of = [](int v, int C) -> uint32_t { return min((uint32_t)v, (uint32_t)(C - 1)); };
  // the index entries are kept in registers; the clamp happens at use
  auto load_idx = [&](int t, int& ki, int (&vi)[2]) {
    const uint32_t k0 = (uint32_t)(t * BK);
    if constexpr (KCEN)
      ki = load_index(rk_idx, k0 + kk, p.k.idxb);
    else
      ki = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (VCEN)
        vi[j] = load_index(rv_idx, k0 + 2 * kp + j, p.v.idxb);
      else
        vi[j] = 0;
    }
  };
  auto load_data = [&](int t, int ki, const int (&vi)[2], KPre<BITS>& kpr, VPre& vp) {
    const uint32_t k0 = (uint32_t)(t * BK);
    const uint32_t n = k0 + kk;
    if constexpr (DENSE) {
      typedef uint32_t u4 __attribute__((ext_vector_type(4)));
      const uint32_t ko = n * hdb + h * DM * 2 + 32 * kw;
      const u4 a0 = __builtin_amdgcn_raw_buffer_load_b128(rk_dense, ko, 0, 0);
      const u4 a1 = __builtin_amdgcn_raw_buffer_load_b128(rk_dense, ko + 16, 0, 0);
      kpr.c0 = uint4{a0.x, a0.y, a0.z, a0.w};
      kpr.c1 = uint4{a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u4 a = __builtin_amdgcn_raw_buffer_load_b128(
            rv_dense, (k0 + 2 * kp + j) * hdb + h * DM * 2 + 16 * c8, 0, 0);
        vp.c[j] = uint4{a.x, a.y, a.z, a.w};
      }
      return;
    }
    if constexpr (BITS == 2 || MIXED) {
      kpr.code[0] = __builtin_amdgcn_raw_buffer_load_b32(rk_code, n * kwb + kword * 4, 0, 0);
    } else {
      typedef uint32_t u2 __attribute__((ext_vector_type(2)));
      const u2 c = __builtin_amdgcn_raw_buffer_load_b64(rk_code, n * kwb + kword * 4, 0, 0);
      kpr.code[0] = c.x;
      kpr.code[1] = c.y;
    }
    kpr.sz = __builtin_amdgcn_raw_buffer_load_b32(rk_sz, n * kgb + kgrp * 4, 0, 0);
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    if constexpr (KCEN) {
      const uint32_t off = idx_of(ki, p.k.C) * (DM * 2) + 32 * kw;
      const u4 a0 = __builtin_amdgcn_raw_buffer_load_b128(rk_cen, off, 0, 0);
      const u4 a1 = __builtin_amdgcn_raw_buffer_load_b128(rk_cen, off + 16, 0, 0);
      kpr.c0 = uint4{a0.x, a0.y, a0.z, a0.w};
      kpr.c1 = uint4{a1.x, a1.y, a1.z, a1.w};
    } else {
      kpr.c0 = uint4{0u, 0u, 0u, 0u};
      kpr.c1 = kpr.c0;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t m = k0 + 2 * kp + j;
      vp.code[j] = __builtin_amdgcn_raw_buffer_load_b32(rv_code, m * vwb + vword * 4, 0, 0);
      vp.sz[j] = __builtin_amdgcn_raw_buffer_load_b32(rv_sz, m * vgb + vgrp * 4, 0, 0);
      if constexpr (VCEN) {
        const uint32_t off =
            idx_of(vi[j], p.v.C) * (DM * 2) + 16 * c8;
        const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rv_cen, off, 0, 0);
        vp.c[j] = uint4{a.x, a.y, a.z, a.w};
      } else {
        vp.c[j] = uint4{0u, 0u, 0u, 0u};
      }
    }
  };
  // Pieces of load_idx / load_data for the centroid/plain kernels, whose K decode runs
  // among the score MFMAs: the K and V prefetches (and their index words) are issued at
  // different points of a tile, each one tile ahead of its use.
  auto load_kidx = [&](int t, int& ki) {
    if constexpr (KCEN)
      ki = load_index(rk_idx, (uint32_t)(t * BK) + kk, p.k.idxb);
    else
      ki = 0;
  };
  auto load_vidx = [&](int t, int (&vi)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (VCEN)
        vi[j] = load_index(rv_idx, (uint32_t)(t * BK) + 2 * kp + j, p.v.idxb);
      else
        vi[j] = 0;
    }
  };
  auto load_k = [&](int t, int ki, KPre<BITS>& kpr) {
    const uint32_t n = (uint32_t)(t * BK) + kk;
    if constexpr (BITS == 2) {
      kpr.code[0] = __builtin_amdgcn_raw_buffer_load_b32(rk_code, n * kwb + kword * 4, 0, 0);
    } else {
      typedef uint32_t u2 __attribute__((ext_vector_type(2)));
      const u2 c = __builtin_amdgcn_raw_buffer_load_b64(rk_code, n * kwb + kword * 4, 0, 0);
      kpr.code[0] = c.x;
      kpr.code[1] = c.y;
    }
    kpr.sz = __builtin_amdgcn_raw_buffer_load_b32(rk_sz, n * kgb + kgrp * 4, 0, 0);
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    if constexpr (KCEN) {
      const uint32_t off = idx_of(ki, p.k.C) * (DM * 2) + 32 * kw;
      const u4 a0 = __builtin_amdgcn_raw_buffer_load_b128(rk_cen, off, 0, 0);
      const u4 a1 = __builtin_amdgcn_raw_buffer_load_b128(rk_cen, off + 16, 0, 0);
      kpr.c0 = uint4{a0.x, a0.y, a0.z, a0.w};
      kpr.c1 = uint4{a1.x, a1.y, a1.z, a1.w};
    } else {
      kpr.c0 = uint4{0u, 0u, 0u, 0u};
      kpr.c1 = kpr.c0;
    }
  };
  auto load_v = [&](int t, const int (&vi)[2], VPre& vp) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t m = (uint32_t)(t * BK) + 2 * kp + j;
      vp.code[j] = __builtin_amdgcn_raw_buffer_load_b32(rv_code, m * vwb + vword * 4, 0, 0);
      vp.sz[j] = __builtin_amdgcn_raw_buffer_load_b32(rv_sz, m * vgb + vgrp * 4, 0, 0);
      if constexpr (VCEN) {
        const uint32_t off =
            idx_of(vi[j], p.v.C) * (DM * 2) + 16 * c8;
        const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rv_cen, off, 0, 0);
        vp.c[j] = uint4{a.x, a.y, a.z, a.w};
      } else {
        vp.c[j] = uint4{0u, 0u, 0u, 0u};
      }
    }
  };
  // JB: s_g^2 of a key row's scale group at column DM + g, written by the group's first lane
  auto store_step_sq = [&](int dbuf, uint32_t szw) {
    if constexpr (JB) {
      if (((16 * kw) & (p.k.group - 1)) == 0) {
        const float stp = f16_bits_to_f32(szw & 0xFFFFu);
        k_lds[dbuf][kk * KR + DM + kgrp] = (uint16_t)f32_to_bf16_bits(stp * stp);
      }
    }
  };
  auto dequant = [&](const KPre<BITS>& kpr, const VPre& vp, int buf, bool do_k = true) {
    if constexpr (DENSE) {
      uint4* dst = reinterpret_cast<uint4*>(&k_lds[buf][kk * KR + 16 * kw]);
      dst[0] = kpr.c0;
      dst[1] = kpr.c1;
      const uint32_t v0[4] = {vp.c[0].x, vp.c[0].y, vp.c[0].z, vp.c[0].w};
      const uint32_t v1[4] = {vp.c[1].x, vp.c[1].y, vp.c[1].z, vp.c[1].w};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int row = 8 * c8 + c;
        const uint32_t a = (c & 1) ? (v0[c >> 1] >> 16) : (v0[c >> 1] & 0xFFFFu);
        const uint32_t b = (c & 1) ? (v1[c >> 1] >> 16) : (v1[c >> 1] & 0xFFFFu);
        *reinterpret_cast<uint32_t*>(&v_lds[buf][row * VROW + vpos(row, 2 * kp)]) =
            bf16x2_to_f16x2(a | (b << 16));
      }
      return;
    }
    if constexpr (MIXED) {
      // ---- K: centroid row chunk as is; lane kw adds coefficients 2 kw, 2 kw + 1 (hi, lo)
      uint4* dst = reinterpret_cast<uint4*>(&k_lds[buf][kk * KR + 16 * kw]);
      dst[0] = kpr.c0;
      dst[1] = kpr.c1;
      {
        const float sc = f16_bits_to_f32(kpr.sz & 0xFFFFu), ze = f16_bits_to_f32(kpr.sz >> 16);
        const uint32_t w = kpr.code[0] >> kcsh;
        const float c0 = __builtin_fmaf((float)(w & ((1u << BITS) - 1u)), sc, ze);
        const float c1 = __builtin_fmaf((float)((w >> BITS) & ((1u << BITS) - 1u)), sc, ze);
        const uint32_t hi = pk_bf16(c0, c1);
        const uint32_t lo = pk_bf16(c0 - lo_bf16(hi), c1 - hi_bf16(hi));
        *reinterpret_cast<uint32_t*>(&k_lds[buf][kk * KR + DM + 2 * kw]) = hi;
        *reinterpret_cast<uint32_t*>(&k_lds[buf][kk * KR + DM + 16 + 2 * kw]) = lo;
      }
    } else {
    // ---- K: 16 consecutive channels of key kk -> row-major bf16
     if (do_k) {
      float s24 = f16_bits_to_f32(kpr.sz & 0xFFFFu) * 0x1p24f, ze = f16_bits_to_f32(kpr.sz >> 16);
      if constexpr (ROT) {   // the 1/sqrt(n) of the transform, folded in exactly
        const float sc = p.k.rot == 64 ? 0.125f : (p.k.rot == 16 ? 0.25f : 1.0f);
        s24 *= sc;
        ze *= sc;
      }
      float dq[16];   // code * s + z per channel
      if constexpr (BITS == 2) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const uint32_t b = (kpr.code[0] >> (2 * r)) & 0x00030003u;   // codes r, r+8
          dq[r] = __builtin_fmaf(code_lo(b), s24, ze);
          dq[r + 8] = __builtin_fmaf(code_hi(b), s24, ze);
        }
      } else {
#pragma unroll
        for (int wd = 0; wd < 2; ++wd)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t b = (kpr.code[wd] >> (4 * r)) & 0x000F000Fu;   // codes r, r+4 of word wd
            dq[8 * wd + r] = __builtin_fmaf(code_lo(b), s24, ze);
            dq[8 * wd + r + 4] = __builtin_fmaf(code_hi(b), s24, ze);
          }
      }
      if constexpr (ROT) {
        if (p.k.rot) hn_back<16>(dq, kw, p.k.rot);   // 8 lanes per key row, 16 channels each
      }
      const uint32_t cw[8] = {kpr.c0.x, kpr.c0.y, kpr.c0.z, kpr.c0.w, kpr.c1.x, kpr.c1.y, kpr.c1.z, kpr.c1.w};
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x0 = cadd_lo(cw[i], ksc, dq[2 * i]);
        const float x1 = cadd_hi(cw[i], ksc, dq[2 * i + 1]);
        o[i] = pk_bf16(x0, x1);
      }
      uint4* dst = reinterpret_cast<uint4*>(&k_lds[buf][kk * KR + 16 * kw]);
      dst[0] = uint4{o[0], o[1], o[2], o[3]};
      dst[1] = uint4{o[4], o[5], o[6], o[7]};
      store_step_sq(buf, kpr.sz);
     }
    }
    // ---- V: channels 8c8..8c8+7 of keys 2kp, 2kp+1 -> transposed fp16 (swizzled)
    {
      float x[2][8];   // [key j][channel c]
      float dq[2][8];  // code * s + z
      float s24[2], ze[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        s24[j] = f16_bits_to_f32(vp.sz[j] & 0xFFFFu) * 0x1p24f;
        ze[j] = f16_bits_to_f32(vp.sz[j] >> 16);
        if constexpr (ROT) {   // the 1/sqrt(n) of the transform, folded in exactly
          const float sc = p.v.rot == 64 ? 0.125f : (p.v.rot == 16 ? 0.25f : 1.0f);
          s24[j] *= sc;
          ze[j] *= sc;
        }
      }
      if constexpr (VBITS == 2) {
        // the two keys' 8 codes side by side (key 0 low half, key 1 high half)
        const uint32_t w = __builtin_amdgcn_perm(vp.code[1], vp.code[0], vsel);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const uint32_t b = (w >> (2 * r)) & 0x00030003u;     // channel r of both keys
          dq[0][r] = __builtin_fmaf(code_lo(b), s24[0], ze[0]);
          dq[1][r] = __builtin_fmaf(code_hi(b), s24[1], ze[1]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t b = (vp.code[j] >> (4 * r)) & 0x000F000Fu;   // channels r, r+4
            dq[j][r] = __builtin_fmaf(code_lo(b), s24[j], ze[j]);
            dq[j][r + 4] = __builtin_fmaf(code_hi(b), s24[j], ze[j]);
          }
      }
      if constexpr (ROT) {
        if (p.v.rot) {   // 16 lanes per value row, 8 channels each
          hn_back<8>(dq[0], c8, p.v.rot);
          hn_back<8>(dq[1], c8, p.v.rot);
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t cw[4] = {vp.c[j].x, vp.c[j].y, vp.c[j].z, vp.c[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[j][2 * i] = cadd_lo(cw[i], vsc, dq[j][2 * i]);
          x[j][2 * i + 1] = cadd_hi(cw[i], vsc, dq[j][2 * i + 1]);
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int row = 8 * c8 + c;
        // the decoded value is the codec's bf16 reconstruction; fp16 holds it exactly
        // inside fp16's range (|v| <= 65504, a limit the API states for this path)
        const uint32_t w = bf16x2_to_f16x2(pk_bf16_asm(x[0][c], x[1][c]));   // keys 2kp, 2kp+1
        *reinterpret_cast<uint32_t*>(&v_lds[buf][row * VROW + vpos(row, 2 * kp)]) = w;
      }
    }
  };

  // Q^T operand: lane holds Q[myq][16*ks + 8*half .. +7] for ks = 0..7
  bf16x8_t qreg[8];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + (myq * p.H + h) * DM + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (myq < p.nq) qreg[ks] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * ks);
      else qreg[ks] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  // JB: -(scale / 24) ||q_g||^2 for groups g = 0..7 (lanes of half 0; k = 8..15 and
  // groups beyond d/group stay zero), and zeros in the unused step columns of both
  // K buffers
  bf16x8_t jbq = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (JB) {
    float full[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qv = bf16_bits_to_f32((uint16_t)qreg[ks][e]);
        a = __builtin_fmaf(qv, qv, a);
      }
      full[ks] = a + other_half(a, half);   // channels 16 ks .. 16 ks + 15
    }
    const int ksh = __builtin_ctz((unsigned)p.k.group) - 4;   // 16-channel blocks per group: 2^ksh
    const float cf = -p.scale * (1.0f / 24.0f);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      float n = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) n += ((ks >> ksh) == g) ? full[ks] : 0.0f;
      jbq[g] = half ? (short)0 : (short)f32_to_bf16_bits(cf * n);
    }
    const int g0 = DM / p.k.group;
    for (int e = tid; e < 2 * BK * 16; e += NT) {
      const int b = e / (BK * 16), r = (e >> 4) % BK, g = e & 15;
      if (g >= g0) k_lds[b][r * KR + DM + g] = 0;
    }
  }

  // MIXED: (B^T q) for the lane's query as bf16 high / low parts, k-slice 8*half..+7
  bf16x8_t phi = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0}, plo = phi;
  if constexpr (MIXED) {
    uint16_t* bst = &v_lds[1][0];   // the basis is staged in the not yet used V buffer
    for (int e = tid; e < DM * 16 / 8; e += NT)
      *reinterpret_cast<uint4*>(&bst[8 * e]) = *reinterpret_cast<const uint4*>(p.basis + 8 * e);
    __syncthreads();
    float part[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) part[j] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 16 * ks + 8 * half + e;
        const float qv = bf16_bits_to_f32((uint16_t)qreg[ks][e]);
        const uint4 b0 = *reinterpret_cast<const uint4*>(&bst[16 * i]);
        const uint4 b1 = *reinterpret_cast<const uint4*>(&bst[16 * i + 8]);
        const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          part[2 * jj] = __builtin_fmaf(qv, lo_bf16(bw[jj]), part[2 * jj]);
          part[2 * jj + 1] = __builtin_fmaf(qv, hi_bf16(bw[jj]), part[2 * jj + 1]);
        }
      }
    float pj[8];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float full = part[j] + other_half(part[j], half);
      if ((j >> 3) == half) pj[j & 7] = full;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t h2 = pk_bf16(pj[2 * i], pj[2 * i + 1]);
      const uint32_t l2 = pk_bf16(pj[2 * i] - lo_bf16(h2), pj[2 * i + 1] - hi_bf16(h2));
      phi[2 * i] = (short)(h2 & 0xFFFFu); phi[2 * i + 1] = (short)(h2 >> 16);
      plo[2 * i] = (short)(l2 & 0xFFFFu); plo[2 * i + 1] = (short)(l2 >> 16);
    }
    __syncthreads();
  }

  f32x16_t oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.0f;
  float m_run = -__builtin_inff();
  float l_run = 0.0f;
  const float c2 = p.scale_log2;

  // prefetch state: the next tile's compressed rows, the index words of the one after
  KPre<BITS> kpre;
  VPre vpre;
  int kidx, vidx[2];

  // The K decode of the next tile cut into 16 steps, one per score MFMA: steps 0..7
  // dequantize two channels each (codes as f16 denormals through v_fma_mix), steps
  // 8..15 add the centroid and round one channel pair, step 15 stores the row (with
  // rotated residuals step 8 first rotates the 16 dequantized channels back).
  struct KDec {
    float s24, ze, dq[16];
    uint32_t o[8];
  };
  auto kstep = [&](int j, KDec& st, const KPre<BITS>& kpr, int dbuf) {
    if (j == 0) {
      st.s24 = f16_bits_to_f32(kpr.sz & 0xFFFFu) * 0x1p24f;
      st.ze = f16_bits_to_f32(kpr.sz >> 16);
      if constexpr (ROT) {   // the 1/sqrt(n) of the transform, folded in exactly
        const float sc = p.k.rot == 64 ? 0.125f : (p.k.rot == 16 ? 0.25f : 1.0f);
        st.s24 *= sc;
        st.ze *= sc;
      }
    }
    if (j < 8) {
      if constexpr (BITS == 2) {
        const uint32_t b = (kpr.code[0] >> (2 * j)) & 0x00030003u;   // codes j, j+8
        st.dq[j] = __builtin_fmaf(code_lo(b), st.s24, st.ze);
        st.dq[j + 8] = __builtin_fmaf(code_hi(b), st.s24, st.ze);
      } else {
        const int wd = j >> 2, r = j & 3;
        const uint32_t b = (kpr.code[wd] >> (4 * r)) & 0x000F000Fu;   // codes r, r+4 of word wd
        st.dq[8 * wd + r] = __builtin_fmaf(code_lo(b), st.s24, st.ze);
        st.dq[8 * wd + r + 4] = __builtin_fmaf(code_hi(b), st.s24, st.ze);
      }
    } else {
      if constexpr (ROT) {   // all 16 channels dequantized: rotate back before the centroid
        if (j == 8 && p.k.rot) hn_back<16>(st.dq, kw, p.k.rot);
      }
      const int i = j - 8;
      const uint32_t cwi = (i < 4) ? (i == 0 ? kpr.c0.x : i == 1 ? kpr.c0.y : i == 2 ? kpr.c0.z : kpr.c0.w)
                                   : (i == 4 ? kpr.c1.x : i == 5 ? kpr.c1.y : i == 6 ? kpr.c1.z : kpr.c1.w);
      st.o[i] = pk_bf16(cadd_lo(cwi, ksc, st.dq[2 * i]), cadd_hi(cwi, ksc, st.dq[2 * i + 1]));
      if (j == 15) {
        uint4* dst = reinterpret_cast<uint4*>(&k_lds[dbuf][kk * KR + 16 * kw]);
        dst[0] = uint4{st.o[0], st.o[1], st.o[2], st.o[3]};
        dst[1] = uint4{st.o[4], st.o[5], st.o[6], st.o[7]};
        store_step_sq(dbuf, kpr.sz);
      }
    }
  };

  // MASK: the tile runs past the last key (only the final tile of a ragged history)
  // KDEC: the next tile's K rows are decoded among the score MFMAs (hard scheduling
  // fences keep one decode step after each MFMA, so the wave's VALU work issues while
  // its MFMAs run), then tile t+2's K rows and tile t+3's K index words are requested.
  auto compute = [&](int t, int buf, auto mask_tag, auto kdec_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool KDEC = decltype(kdec_tag)::value;
    const int k0 = t * BK;
    // S^T = K Q^T (raw scores)
    // K fragments stream through two groups of 4 registers: the reads of group g+1
    // are in flight while the 4 MFMAs of group g run
    f32x16_t sacc[2];
    const uint16_t* krow = &k_lds[buf][col * KR + 8 * half];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
    bf16x8_t kf[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kf[0][i] = *reinterpret_cast<const bf16x8_t*>(krow + 16 * i);
    if constexpr (KDEC) {
      KDec st;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < 4; ++g) {   // g: (kb, ks half) = (g >> 1, g & 1)
        if (g + 1 < 4) {
          const int kb1 = (g + 1) >> 1, k1 = 4 * ((g + 1) & 1);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            kf[(g + 1) & 1][i] =
                *reinterpret_cast<const bf16x8_t*>(krow + kb1 * 32 * KR + 16 * (k1 + i));
        }
        const int kb = g >> 1, k0s = 4 * (g & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[g & 1][i], qreg[k0s + i], sacc[kb], 0, 0, 0);
          kstep(4 * g + i, st, kpre, buf ^ 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // past the last tile the prefetches repeat it (valid rows, no branches)
      load_k(min(t + 2, te - 1), kidx, kpre);
      load_kidx(min(t + 3, te - 1), kidx);
    } else {
#pragma unroll
    for (int g = 0; g < 4; ++g) {   // g: (kb, ks half) = (g >> 1, g & 1)
      if (g + 1 < 4) {
        const int kb1 = (g + 1) >> 1, k1 = 4 * ((g + 1) & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          kf[(g + 1) & 1][i] =
              *reinterpret_cast<const bf16x8_t*>(krow + kb1 * 32 * KR + 16 * (k1 + i));
      }
      const int kb = g >> 1, k0s = 4 * (g & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[g & 1][i], qreg[k0s + i], sacc[kb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int g = 0; g < 3; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      if (g < 2) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    // all V^T fragments of the tile are read now, so they arrive during the softmax
    // (one 16-byte read each: row 32 d + col, block (2 kh + half) ^ (2 d + col / 16) =
    // 2 (kh ^ d) + (half ^ col / 16)); (kb, hf) = kh covers keys 32*kb + 16*hf +
    // {4*half+0..3, 8+4*half+0..3}
    // (the mixed-dimensional kernel, which holds B^T q as well, and the rotated kernel
    // with the Jensen correction read the last two channel blocks during the PV MFMAs
    // instead, to stay within 256 registers)
    constexpr int VE = (MIXED || (ROT && JB)) ? 2 : 4;   // channel blocks read before the softmax
    f16x8_t vf[4][4];
    const uint16_t* vbase = &v_lds[buf][col * VROW + 8 * (half ^ (col >> 4))];
    auto read_vf = [&](int d) {
#pragma unroll
      for (int kh = 0; kh < 4; ++kh)
        vf[d][kh] = *reinterpret_cast<const f16x8_t*>(vbase + 32 * d * VROW + 16 * (kh ^ d));
    };
#pragma unroll
    for (int d = 0; d < VE; ++d) read_vf(d);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MIXED) {   // + (B^T q) . c: hi*hi + hi*lo + lo*hi
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint16_t* r0 = &k_lds[buf][(kb * 32 + col) * KR + DM + 8 * half];
        const bf16x8_t ch = *reinterpret_cast<const bf16x8_t*>(r0);
        const bf16x8_t cl = *reinterpret_cast<const bf16x8_t*>(r0 + 16);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ch, phi, sacc[kb], 0, 0, 0);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ch, plo, sacc[kb], 0, 0, 0);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cl, phi, sacc[kb], 0, 0, 0);
      }
    }
    if constexpr (JB) {   // - (scale / 24) sum_g s_g^2 ||q_g||^2 into the raw scores
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t sq = *reinterpret_cast<const bf16x8_t*>(&k_lds[buf][(kb * 32 + col) * KR + DM + 8 * half]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sq, jbq, sacc[kb], 0, 0, 0);
      }
    }
    if constexpr (MASK) {   // last, partial tile: mask keys >= nk
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (k0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= nk) sacc[kb][r] = -__builtin_inff();
    }
    float mloc = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[kb][r]);
    mloc = fmaxf(mloc, other_half(mloc, half));
    // Lazy rescaling: the reference max moves only when a lane's scores exceed it by
    // more than 2^8 (log2 domain, scale > 0), so P stays <= 256 - exact range for
    // fp16 - and the output accumulators are rescaled on a few tiles only.
    if (__builtin_expect(__any(mloc * c2 > m_run + 8.0f), 0)) {
      const float m_new = fmaxf(m_run, mloc * c2);
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= corr;
      m_run = m_new;
    }
    const float negm = -m_run;
    f16x8_t pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f16x8_t t8;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          t8[j] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * hf + j], c2, negm));
        pb[kb][hf] = t8;
      }
    // row sums of the fp16 P that the MFMAs use (two products per v_dot2_f32_f16,
    // fp32 accumulation), so numerator and denominator see the same weights
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kh = 0; kh < 4; ++kh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const h2 pr = {pb[kh >> 1][kh & 1][2 * i], pb[kh >> 1][kh & 1][2 * i + 1]};
        ls[kh] = __builtin_amdgcn_fdot2(pr, one2, ls[kh], false);
      }
    float lsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    lsum += other_half(lsum, half);
    l_run = l_run + lsum;
    // O^T += V^T P^T
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if (d + VE < 4) read_vf(d + VE);
#pragma unroll
      for (int kh = 0; kh < 4; ++kh)
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[d][kh], pb[kh >> 1][kh & 1], oacc[d], 0, 0, 0);
    }
  };

  // ---- prologue: first tile decoded into buffer 0, the next prefetched, indices of
  //      the one after
  load_idx(tb, kidx, vidx);
  load_data(tb, kidx, vidx, kpre, vpre);
  if (tb + 1 < te) load_idx(tb + 1, kidx, vidx);
  dequant(kpre, vpre, 0);
  if (tb + 1 < te) load_data(tb + 1, kidx, vidx, kpre, vpre);
  if (tb + 2 < te) load_idx(tb + 2, kidx, vidx);
  __syncthreads();

  // ---- main loop: decode tile t+1 into the other buffer, prefetch tile t+2's
  //      compressed rows (and t+3's indices), then attend tile t
  // the final tile of a ragged history (the only one that masks keys) runs after the
  // loop, so the loop body has one variant
  const int tfull = (te * BK > nk) ? te - 1 : te;
  if constexpr (!DENSE && !MIXED) {
    // V decode first, K decode among the score MFMAs (see compute)
    int t = tb;
    for (; t < min(tfull, te - 1); ++t) {
      const int buf = (t - tb) & 1;
      dequant(kpre, vpre, buf ^ 1, false);
      load_v(min(t + 2, te - 1), vidx, vpre);
      load_vidx(min(t + 3, te - 1), vidx);
      compute(t, buf, std::false_type{}, std::true_type{});
      __syncthreads();
    }
    if (t < tfull) {   // the last tile, complete: nothing left to decode
      compute(t, (t - tb) & 1, std::false_type{}, std::false_type{});
      __syncthreads();
    }
  } else {
    for (int t = tb; t < tfull; ++t) {
      const int buf = (t - tb) & 1;
      // past the last tile the decode and the prefetches repeat it into the buffer
      // nobody reads (valid rows, no branches)
      dequant(kpre, vpre, buf ^ 1);
      load_data(min(t + 2, te - 1), kidx, vidx, kpre, vpre);
      load_idx(min(t + 3, te - 1), kidx, vidx);
      compute(t, buf, std::false_type{}, std::false_type{});
      __syncthreads();
    }
  }
  if (tfull < te) compute(tfull, (tfull - tb) & 1, std::true_type{}, std::false_type{});

  // ---- epilogue: O[q][h][c] = O^T[c][q] / l (a split's partial output when splitting)
  float* const outp = p.splits > 1 ? p.part_o + (int64_t)split * p.nq * p.H * DM : p.out;
  float* const lsep = p.splits > 1 ? p.part_lse + (int64_t)split * p.H * p.nq : p.lse;
  if (myq < p.nq) {
    const float inv = 1.0f / l_run;
    float* op = outp + (myq * p.H + h) * DM;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 o;
        o.x = oacc[d][4 * g + 0] * inv;
        o.y = oacc[d][4 * g + 1] * inv;
        o.z = oacc[d][4 * g + 2] * inv;
        o.w = oacc[d][4 * g + 3] * inv;
        *reinterpret_cast<float4*>(op + d * 32 + 8 * g + 4 * half) = o;
      }
    if (lsep && half == 0)
      lsep[(int64_t)h * p.nq + myq] = (m_run + __log2f(l_run)) * 0.69314718055994531f;
  }
}

constexpr int MAX_PARTS = 9;   // partial results one merge takes (8 key splits + a chunk)

// Merge of the key splits: O = sum_s w_s O_s, w_s = exp(lse_s - lse) with
// lse = log sum_s exp(lse_s); one thread per (query, head, 4 channels).
__global__ __launch_bounds__(256) void attend_combine_kernel(AttnParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nqh = p.nq * p.H;
  if (i >= nqh * (DM / 4)) return;
  const int64_t qh = i / (DM / 4);
  const int c4 = (int)(i % (DM / 4));
  const int64_t q = qh / p.H;
  const int h = (int)(qh % p.H);
  float ls[MAX_PARTS];
  float m = -__builtin_inff();
  for (int s = 0; s < p.splits; ++s) {
    ls[s] = p.part_lse[((int64_t)s * p.H + h) * p.nq + q];
    m = fmaxf(m, ls[s]);
  }
  float wsum = 0.0f;
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s = 0; s < p.splits; ++s) {
    const float w = __expf(ls[s] - m);
    wsum += w;
    const float4 v = *reinterpret_cast<const float4*>(p.part_o + ((int64_t)s * nqh + qh) * DM + 4 * c4);
    o.x = __builtin_fmaf(w, v.x, o.x);
    o.y = __builtin_fmaf(w, v.y, o.y);
    o.z = __builtin_fmaf(w, v.z, o.z);
    o.w = __builtin_fmaf(w, v.w, o.w);
  }
  const float inv = 1.0f / wsum;
  *reinterpret_cast<float4*>(p.out + qh * DM + 4 * c4) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  if (p.lse && c4 == 0) p.lse[(int64_t)h * p.nq + q] = m + __logf(wsum);
}

// ----------------------------------------------------------------------------
// Mixed-dimensional attention over cluster-ordered keys
// ----------------------------------------------------------------------------
// The NanoKV-Fast score of key n is q . C_k[a_n] + (B^T q) . c_n (NanoKV abstract and
// project page: scores on the low-dimensional coefficients, without reconstructing
// K).  Keys whose centroids fall in one block of CL_BLK consecutive centroids share
// the 32 x CL_BLK table Q C_blk^T of a wave's queries, so the history is first put in
// centroid-block order (attention does not depend on the order of its keys; the
// values move with their keys), the table is formed once per block with 8 MFMAs, and
// a key's first term enters the score MFMA as a one-hot product: the K tile row holds,
// next to the key's coefficients, a one-hot row over the block's 32 centroids, and the
// table (split into bf16 high and low parts, exact to about 2^-16) is the other
// operand.  Per 64-key tile a wave runs 8 one-hot MFMAs, the 6 coefficient MFMAs
// (16-dimensional contraction, bf16 high/low parts) and the 16 PV MFMAs, against
// 16 + 6 + 16 when the centroid rows are gathered into a 128-wide K tile.
//
// Ordering: a stable counting sort by block (block = min(a, C - 1) / CL_BLK) per head,
// in three launches: per-chunk block counts, per-head prefix sums (block offsets,
// each chunk's first destination per block, and the tile table: a block's keys are
// cut into 64-key tiles, the last one ragged), and a scatter that copies each key's K
// coefficient row and V row to its sorted place (rank within a chunk from wave
// ballots, so equal blocks keep token order and the result is deterministic).
constexpr int CL_BLK = 32;        // centroids per block (one 32 x 32 MFMA tile)
constexpr int CL_CHUNK = 2048;    // keys per counting / scatter workgroup
constexpr int CL_THREADS = 256;
constexpr int CL_MAXNB = 128;     // blocks at most (C <= 4096)

struct ClusterParams {
  int64_t n;                      // keys per head
  int H, nb, nchunk, tmax;
  Src k, v;                       // source stores (rows h * cap + i)
  uint32_t* kcodes;               // cluster-ordered copies, rows h * n + j
  uint32_t* ksz;
  uint8_t* kidx;
  uint32_t* vcodes;
  uint32_t* vsz;
  uint8_t* vidx;
  int* cnt;                       // [H][nchunk][nb]: counts, then first destinations
  int2* tiles;                    // [H][tmax]: (first sorted position, block | keys << 8
                                  //   | first tile of its block << 16)
  int* ntiles;                    // [H]
};

__device__ __forceinline__ int cl_index(const Src& s, int64_t row) {
  return s.idxb == 1 ? (int)reinterpret_cast<const uint8_t*>(s.index)[row]
                     : (int)reinterpret_cast<const uint16_t*>(s.index)[row];
}
__device__ __forceinline__ int cl_bin(const ClusterParams& c, int h, int64_t i) {
  return min(cl_index(c.k, (int64_t)h * c.k.cap + i), c.k.C - 1) / CL_BLK;
}

__global__ __launch_bounds__(CL_THREADS) void cluster_count_kernel(ClusterParams c) {
  __shared__ int hist[CL_MAXNB];
  const int chunk = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  for (int b = tid; b < c.nb; b += CL_THREADS) hist[b] = 0;
  __syncthreads();
  const int64_t i0 = (int64_t)chunk * CL_CHUNK;
  for (int j = tid; j < CL_CHUNK; j += CL_THREADS)
    if (i0 + j < c.n) atomicAdd(&hist[cl_bin(c, h, i0 + j)], 1);
  __syncthreads();
  for (int b = tid; b < c.nb; b += CL_THREADS)
    c.cnt[((int64_t)h * c.nchunk + chunk) * c.nb + b] = hist[b];
}

__global__ __launch_bounds__(CL_THREADS) void cluster_scan_kernel(ClusterParams c) {
  __shared__ int boff[CL_MAXNB + 1];
  __shared__ int tbase[CL_MAXNB + 1];
  const int h = blockIdx.x, tid = threadIdx.x;
  int* cnt = c.cnt + (int64_t)h * c.nchunk * c.nb;
  for (int b = tid; b < c.nb; b += CL_THREADS) {   // per block: prefix over chunks
    int run = 0;
    for (int k0 = 0; k0 < c.nchunk; k0 += 8) {      // 8 loads in flight
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = k0 + j < c.nchunk ? cnt[(k0 + j) * c.nb + b] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (k0 + j < c.nchunk) cnt[(k0 + j) * c.nb + b] = run;
        run += v[j];
      }
    }
    boff[b] = run;   // the block's size for now
  }
  __syncthreads();
  if (tid == 0) {   // block offsets and first tiles (at most CL_MAXNB steps)
    int off = 0, tb = 0;
    for (int b = 0; b < c.nb; ++b) {
      const int sz = boff[b];
      boff[b] = off;
      tbase[b] = tb;
      off += sz;
      tb += (sz + BK - 1) / BK;
    }
    boff[c.nb] = off;
    tbase[c.nb] = tb;
    c.ntiles[h] = tb;
  }
  __syncthreads();
  for (int e = tid; e < c.nchunk * c.nb; e += CL_THREADS) cnt[e] += boff[e % c.nb];
  const int T = tbase[c.nb];
  for (int t = tid; t < T; t += CL_THREADS) {
    int lo = 0, hi = c.nb - 1;   // the last block with tbase <= t (it holds tile t)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tbase[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    const int st = boff[lo] + (t - tbase[lo]) * BK;
    const int cnt = min(BK, boff[lo + 1] - st);
    c.tiles[(int64_t)h * c.tmax + t] = make_int2(st, lo | (cnt << 8) | ((t == tbase[lo]) << 16));
  }
}

__device__ __forceinline__ void cl_copy_words(uint32_t* dst, const uint32_t* src, int n) {
  if ((n & 3) == 0) {
    for (int w = 0; w < n; w += 4)
      *reinterpret_cast<uint4*>(dst + w) = *reinterpret_cast<const uint4*>(src + w);
  } else if ((n & 1) == 0) {
    for (int w = 0; w < n; w += 2)
      *reinterpret_cast<uint2*>(dst + w) = *reinterpret_cast<const uint2*>(src + w);
  } else {
    for (int w = 0; w < n; ++w) dst[w] = src[w];
  }
}

__global__ __launch_bounds__(CL_THREADS) void cluster_scatter_kernel(ClusterParams c) {
  constexpr int NWV = CL_THREADS / 64;
  __shared__ int run[CL_MAXNB];
  __shared__ int wh[NWV][CL_MAXNB];
  const int chunk = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  for (int b = tid; b < c.nb; b += CL_THREADS) {
    run[b] = c.cnt[((int64_t)h * c.nchunk + chunk) * c.nb + b];
#pragma unroll
    for (int w = 0; w < NWV; ++w) wh[w][b] = 0;
  }
  __syncthreads();
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  for (int r = 0; r < CL_CHUNK / CL_THREADS; ++r) {
    const int64_t i = (int64_t)chunk * CL_CHUNK + r * CL_THREADS + tid;
    const bool live = i < c.n;
    const int bin = live ? cl_bin(c, h, i) : CL_MAXNB;   // 8 bits
    uint64_t same = ~0ull;   // lanes of the wave with this lane's block
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint64_t bk = __ballot((bin >> k) & 1);
      same &= ((bin >> k) & 1) ? bk : ~bk;
    }
    const int rank = __popcll(same & below);
    if (live && rank == 0) wh[wave][bin] = __popcll(same);
    __syncthreads();
    if (live) {
      int j = run[bin] + rank;
      for (int w = 0; w < wave; ++w) j += wh[w][bin];
      const int64_t src = (int64_t)h * c.k.cap + i, dk = (int64_t)h * c.n + j;
      const int64_t vsrc = (int64_t)h * c.v.cap + i;
      cl_copy_words(c.kcodes + dk * c.k.words, c.k.codes + src * c.k.words, c.k.words);
      cl_copy_words(c.ksz + dk * c.k.groups, c.k.sz + src * c.k.groups, c.k.groups);
      cl_copy_words(c.vcodes + dk * c.v.words, c.v.codes + vsrc * c.v.words, c.v.words);
      cl_copy_words(c.vsz + dk * c.v.groups, c.v.sz + vsrc * c.v.groups, c.v.groups);
      if (c.k.idxb == 1) c.kidx[dk] = reinterpret_cast<const uint8_t*>(c.k.index)[src];
      else reinterpret_cast<uint16_t*>(c.kidx)[dk] = reinterpret_cast<const uint16_t*>(c.k.index)[src];
      if (c.v.idxb == 1) c.vidx[dk] = reinterpret_cast<const uint8_t*>(c.v.index)[vsrc];
      else if (c.v.idxb == 2)
        reinterpret_cast<uint16_t*>(c.vidx)[dk] = reinterpret_cast<const uint16_t*>(c.v.index)[vsrc];
    }
    __syncthreads();
    for (int b = tid; b < c.nb; b += CL_THREADS) {
      int add = 0;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        add += wh[w][b];
        wh[w][b] = 0;
      }
      run[b] += add;
    }
    __syncthreads();
  }
}

// The tile table of the ordered history.
struct ClusterTabs {
  const int2* tiles;   // [H][tmax], as ClusterParams::tiles
  const int* ntiles;   // [H]
  int tmax;
};
constexpr int MWIN = 1024;   // tile records a workgroup stages in LDS at a time

// One workgroup = 8 waves x 32 queries of one head, as attend_bf16_kernel; p.k and p.v
// are the cluster-ordered stores (capacity n), p.k.cen the key centroid table.
template <int KBITS, int VBITS, bool VCEN, bool CF16 = false>
__global__ __launch_bounds__(NT, 1) void attend_mixed_cl_kernel(AttnParams p, ClusterTabs ct) {
  // K tile row: 16 high + 16 low coefficient parts, the one-hot row over the block's 32
  // centroids, pad
  constexpr int KR = 32 + CL_BLK + 8;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BK * KR];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][DM * VROW];
  __shared__ __attribute__((aligned(16))) uint16_t c_lds[2][CL_BLK * KROW];
  __shared__ int2 m_lds[MWIN];   // the tile records of the current window

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int nqb = (int)((p.nq + BQ - 1) / BQ);
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int split = tile % p.splits, hq = tile / p.splits;
  const int h = hq / nqb;
  const int64_t myq = (int64_t)(hq % nqb) * BQ + wave * QW + col;
  const int nth = ct.ntiles[h];
  // this workgroup's tiles of the head's table (none for a late split of a head with
  // fewer tiles than the longest)
  const int tb = min(nth, split * p.tps), te = min(nth, tb + p.tps);
  const int2* tab = ct.tiles + (int64_t)h * ct.tmax;
  int w0 = tb, w1 = tb;   // the window of tile records in m_lds

  auto rsrc = [](const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
  };
  const int64_t n = p.nk;
  const int kwb = p.k.words * 4;
  const int vwb = p.v.words * 4, vgb = p.v.groups * 4;
  const int64_t hr = (int64_t)h * n;   // the ordered stores have capacity n
  const auto rk_code = rsrc(p.k.codes + hr * p.k.words, n * kwb);
  const auto rk_sz = rsrc(p.k.sz + hr, n * 4);
  const auto rk_idx = rsrc(reinterpret_cast<const uint8_t*>(p.k.index) + hr * p.k.idxb, n * p.k.idxb);
  const auto rv_code = rsrc(p.v.codes + hr * p.v.words, n * vwb);
  const auto rv_sz = rsrc(p.v.sz + hr * p.v.groups, n * vgb);
  const auto rv_idx = rsrc(reinterpret_cast<const uint8_t*>(p.v.index) + hr * p.v.idxb,
                           VCEN ? n * p.v.idxb : 0);
  const auto rk_cen = rsrc(reinterpret_cast<const uint16_t*>(p.k.cen) + (int64_t)h * p.k.C * DM,
                           (int64_t)p.k.C * DM * 2);
  // CF16: V's centroid rows from the table's fp16 image (c * 2^e_h), restored by 2^-e_h
  const uint16_t* vcen = CF16 ? p.v.cen16 : reinterpret_cast<const uint16_t*>(p.v.cen);
  const auto rv_cen = rsrc(vcen + (int64_t)h * p.v.C * DM, VCEN ? (int64_t)p.v.C * DM * 2 : 0);
  const float vsc = CF16 ? __int_as_float((127 - p.v.cexp[h]) << 23) : 1.0f;

  // roles: 8 lanes per K row (2 coefficients and 4 one-hot columns each), 16 lanes per V
  // row pair (8 channels each), 16 lanes per centroid row
  const int kk = tid >> 3, kw = tid & 7;
  const int c8 = tid & 15, kp = tid >> 4;
  const int kword = (2 * kw * KBITS) >> 5;
  const int kcsh = (2 * kw * KBITS) & 31;
  const int vword = (8 * c8 * VBITS) >> 5;
  const int vgrp = (8 * c8) / p.v.group;
  const int vsh = (8 * c8 * VBITS) & 31;
  const uint32_t vsel = vsh ? 0x07060302u : 0x05040100u;
  auto load_index = [](__amdgpu_buffer_rsrc_t r, uint32_t key, int idxb) -> int {
    return idxb == 1 ? (int)__builtin_amdgcn_raw_buffer_load_b8(r, key, 0, 0)
                     : (int)__builtin_amdgcn_raw_buffer_load_b16(r, 2u * key, 0, 0);
  };

  struct Pre {
    uint32_t kcode, ksz;
    int kidx;
    uint32_t vcode[2], vsz[2];
    uint4 vc[2];
    uint4 crow;
  };
  // a tile record of the window: first sorted position, block, keys of the block in it,
  // and whether the block's Q C^T table has to be formed (its first tile, or the
  // window's); the records of tiles t+1 .. t+4 ride in registers, one LDS read per tile
  struct Meta {
    int st, blk, cnt;
    bool fresh;
  };
  auto meta_of = [&](int2 e, int t) {
    Meta m;
    m.st = __builtin_amdgcn_readfirstlane(e.x);
    const int y = __builtin_amdgcn_readfirstlane(e.y);
    m.blk = y & 0xFF;
    m.cnt = (y >> 8) & 0xFF;
    m.fresh = t == w0 || ((y >> 16) & 1);
    return m;
  };
  auto meta = [&](int t) { return meta_of(m_lds[t - w0], t); };
  auto load_vidx = [&](const Meta& mt, int (&vi)[2]) {
    const uint32_t st = (uint32_t)mt.st;
#pragma unroll
    for (int j = 0; j < 2; ++j) vi[j] = VCEN ? load_index(rv_idx, st + 2 * kp + j, p.v.idxb) : 0;
  };
  auto load_data = [&](const Meta& mt, const int (&vi)[2], Pre& pr) {
    const int st = mt.st, blk = mt.blk;
    const uint32_t key = (uint32_t)st + kk;
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    pr.kcode = __builtin_amdgcn_raw_buffer_load_b32(rk_code, key * kwb + kword * 4, 0, 0);
    pr.ksz = __builtin_amdgcn_raw_buffer_load_b32(rk_sz, key * 4, 0, 0);
    pr.kidx = load_index(rk_idx, key, p.k.idxb);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t m = (uint32_t)st + 2 * kp + j;
      pr.vcode[j] = __builtin_amdgcn_raw_buffer_load_b32(rv_code, m * vwb + vword * 4, 0, 0);
      pr.vsz[j] = __builtin_amdgcn_raw_buffer_load_b32(rv_sz, m * vgb + vgrp * 4, 0, 0);
      if constexpr (VCEN) {
        const uint32_t off = min((uint32_t)vi[j], (uint32_t)(p.v.C - 1)) * (DM * 2) + 16 * c8;
        const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rv_cen, off, 0, 0);
        pr.vc[j] = uint4{a.x, a.y, a.z, a.w};
      } else {
        pr.vc[j] = uint4{0u, 0u, 0u, 0u};
      }
    }
    {   // the block's centroid rows, zero past C (the range check); staged every tile,
        // used on a block's first (branch-free prefetch)
      const uint32_t row = (uint32_t)(CL_BLK * blk) + (tid >> 4);
      const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rk_cen, row * (DM * 2) + 16 * (tid & 15), 0, 0);
      pr.crow = uint4{a.x, a.y, a.z, a.w};
    }
  };
  auto dequant = [&](const Meta& mt, const Pre& pr, int buf) {
    const int blk = mt.blk;
    // ---- K: coefficients 2 kw, 2 kw + 1 (hi, lo) and the key's row in the wave's Q C^T
    //      table
    {
      const float sc = f16_bits_to_f32(pr.ksz & 0xFFFFu), ze = f16_bits_to_f32(pr.ksz >> 16);
      const uint32_t w = pr.kcode >> kcsh;
      const float c0 = __builtin_fmaf((float)(w & ((1u << KBITS) - 1u)), sc, ze);
      const float c1 = __builtin_fmaf((float)((w >> KBITS) & ((1u << KBITS) - 1u)), sc, ze);
      const uint32_t hi = pk_bf16(c0, c1);
      const uint32_t lo = pk_bf16(c0 - lo_bf16(hi), c1 - hi_bf16(hi));
      *reinterpret_cast<uint32_t*>(&k_lds[buf][kk * KR + 2 * kw]) = hi;
      *reinterpret_cast<uint32_t*>(&k_lds[buf][kk * KR + 16 + 2 * kw]) = lo;
    }
    {   // one-hot row: centroids 4kw..4kw+3 of the block (keys of the next block, which
        // are masked, get a row inside the block)
      const int a = min(max(min(pr.kidx, p.k.C - 1) - CL_BLK * blk, 0), CL_BLK - 1) - 4 * kw;
      const uint32_t o0 = (a == 0 ? 0x3F80u : 0u) | (a == 1 ? 0x3F800000u : 0u);
      const uint32_t o1 = (a == 2 ? 0x3F80u : 0u) | (a == 3 ? 0x3F800000u : 0u);
      *reinterpret_cast<uint2*>(&k_lds[buf][kk * KR + 32 + 4 * kw]) = make_uint2(o0, o1);
    }
    *reinterpret_cast<uint4*>(&c_lds[buf][(tid >> 4) * KROW + 8 * (tid & 15)]) = pr.crow;
    // ---- V: channels 8c8..8c8+7 of keys 2kp, 2kp+1 -> transposed fp16 (swizzled)
    float x[2][8];
    float dq[2][8];
    float s24[2], ze2[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      s24[j] = f16_bits_to_f32(pr.vsz[j] & 0xFFFFu) * 0x1p24f;
      ze2[j] = f16_bits_to_f32(pr.vsz[j] >> 16);
    }
    if constexpr (VBITS == 2) {
      const uint32_t w = __builtin_amdgcn_perm(pr.vcode[1], pr.vcode[0], vsel);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint32_t b = (w >> (2 * r)) & 0x00030003u;
        dq[0][r] = __builtin_fmaf(code_lo(b), s24[0], ze2[0]);
        dq[1][r] = __builtin_fmaf(code_hi(b), s24[1], ze2[1]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t b = (pr.vcode[j] >> (4 * r)) & 0x000F000Fu;
          dq[j][r] = __builtin_fmaf(code_lo(b), s24[j], ze2[j]);
          dq[j][r + 4] = __builtin_fmaf(code_hi(b), s24[j], ze2[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t cw[4] = {pr.vc[j].x, pr.vc[j].y, pr.vc[j].z, pr.vc[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (CF16) {
          x[j][2 * i] = add_f16lo(cw[i], vsc, dq[j][2 * i]);
          x[j][2 * i + 1] = add_f16hi(cw[i], vsc, dq[j][2 * i + 1]);
        } else {
          x[j][2 * i] = lo_bf16(cw[i]) + dq[j][2 * i];
          x[j][2 * i + 1] = hi_bf16(cw[i]) + dq[j][2 * i + 1];
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int row = 8 * c8 + c;
      const uint32_t w = bf16x2_to_f16x2(pk_bf16_asm(x[0][c], x[1][c]));
      *reinterpret_cast<uint32_t*>(&v_lds[buf][row * VROW + vpos(row, 2 * kp)]) = w;
    }
  };

  // Q^T operand: lane holds Q[myq][16*ks + 8*half .. +7] for ks = 0..7
  bf16x8_t qreg[8];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + (myq * p.H + h) * DM + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (myq < p.nq) qreg[ks] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * ks);
      else qreg[ks] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  // (B^T q) for the lane's query as bf16 high / low parts, k-slice 8*half..+7
  bf16x8_t phi, plo;
  {
    uint16_t* bst = &v_lds[1][0];   // the basis is staged in the not yet used V buffer
    for (int e = tid; e < DM * 16 / 8; e += NT)
      *reinterpret_cast<uint4*>(&bst[8 * e]) = *reinterpret_cast<const uint4*>(p.basis + 8 * e);
    __syncthreads();
    float part[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) part[j] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 16 * ks + 8 * half + e;
        const float qv = bf16_bits_to_f32((uint16_t)qreg[ks][e]);
        const uint4 b0 = *reinterpret_cast<const uint4*>(&bst[16 * i]);
        const uint4 b1 = *reinterpret_cast<const uint4*>(&bst[16 * i + 8]);
        const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          part[2 * jj] = __builtin_fmaf(qv, lo_bf16(bw[jj]), part[2 * jj]);
          part[2 * jj + 1] = __builtin_fmaf(qv, hi_bf16(bw[jj]), part[2 * jj + 1]);
        }
      }
    float pj[8];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float full = part[j] + other_half(part[j], half);
      if ((j >> 3) == half) pj[j & 7] = full;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t h2 = pk_bf16(pj[2 * i], pj[2 * i + 1]);
      const uint32_t l2 = pk_bf16(pj[2 * i] - lo_bf16(h2), pj[2 * i + 1] - hi_bf16(h2));
      phi[2 * i] = (short)(h2 & 0xFFFFu); phi[2 * i + 1] = (short)(h2 >> 16);
      plo[2 * i] = (short)(l2 & 0xFFFFu); plo[2 * i + 1] = (short)(l2 >> 16);
    }
    __syncthreads();
  }

  f32x16_t oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.0f;
  float m_run = -__builtin_inff();
  float l_run = 0.0f;
  const float c2 = p.scale_log2;
  // Q C_blk^T of this wave's queries as the B operand of the one-hot MFMAs: k-step s
  // covers the block's centroids 16 s .. 16 s + 15, high and low bf16 parts
  bf16x8_t qch[2], qcl[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    qch[s2] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    qcl[s2] = qch[s2];
  }

  auto compute = [&](const Meta& mt, int buf) {
    const int cnt = mt.cnt;
    const bool fresh = mt.fresh;
    if (fresh) {   // Q C_blk^T of this wave's queries (uniform over the workgroup)
      f32x16_t qc;
#pragma unroll
      for (int r = 0; r < 16; ++r) qc[r] = 0.0f;
      const uint16_t* crow = &c_lds[buf][col * KROW + 8 * half];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        qc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(crow + 16 * ks),
                                                      qreg[ks], qc, 0, 0, 0);
      // accumulator row m = 8 (r / 4) + 4 half + r % 4 (a centroid), column = the lane's
      // query; the B operand of k-step s wants rows 16 s + 8 half .. + 7 in the lane:
      // trading rows 4..7 of half 1 for rows 8..11 of half 0 (and so on) between the
      // register pairs (r, r + 4) puts them there
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(qc[8 * s2 + j]),
                                                           __float_as_uint(qc[8 * s2 + 4 + j]), false, false);
          v[j] = __uint_as_float(sw[0]);
          v[4 + j] = __uint_as_float(sw[1]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t h2 = pk_bf16(v[2 * i], v[2 * i + 1]);
          const uint32_t l2 = pk_bf16(v[2 * i] - lo_bf16(h2), v[2 * i + 1] - hi_bf16(h2));
          qch[s2][2 * i] = (short)(h2 & 0xFFFFu); qch[s2][2 * i + 1] = (short)(h2 >> 16);
          qcl[s2][2 * i] = (short)(l2 & 0xFFFFu); qcl[s2][2 * i + 1] = (short)(l2 >> 16);
        }
      }
    }
    // S^T = one-hot(a) (Q C_blk^T) + the coefficient part (hi*hi + hi*lo + lo*hi)
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
      const uint16_t* r0 = &k_lds[buf][(kb * 32 + col) * KR + 8 * half];
      const bf16x8_t ch = *reinterpret_cast<const bf16x8_t*>(r0);
      const bf16x8_t cl = *reinterpret_cast<const bf16x8_t*>(r0 + 16);
      const bf16x8_t oh0 = *reinterpret_cast<const bf16x8_t*>(r0 + 32);
      const bf16x8_t oh1 = *reinterpret_cast<const bf16x8_t*>(r0 + 48);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oh0, qch[0], sacc[kb], 0, 0, 0);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oh1, qch[1], sacc[kb], 0, 0, 0);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oh0, qcl[0], sacc[kb], 0, 0, 0);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oh1, qcl[1], sacc[kb], 0, 0, 0);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ch, phi, sacc[kb], 0, 0, 0);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ch, plo, sacc[kb], 0, 0, 0);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cl, phi, sacc[kb], 0, 0, 0);
    }
    f16x8_t vf[4][4];
    const uint16_t* vbase = &v_lds[buf][col * VROW + 8 * (half ^ (col >> 4))];
    auto read_vf = [&](int d) {
#pragma unroll
      for (int kh = 0; kh < 4; ++kh)
        vf[d][kh] = *reinterpret_cast<const f16x8_t*>(vbase + 32 * d * VROW + 16 * (kh ^ d));
    };
    read_vf(0);   // the other channel blocks are read during the PV MFMAs (registers)
    if (cnt < BK) {   // the block's last, partial tile: keys of the next block are masked
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= cnt) sacc[kb][r] = -__builtin_inff();
    }
    float mloc = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[kb][r]);
    mloc = fmaxf(mloc, other_half(mloc, half));
    if (__builtin_expect(__any(mloc * c2 > m_run + 8.0f), 0)) {   // lazy rescaling (2^8)
      const float m_new = fmaxf(m_run, mloc * c2);
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= corr;
      m_run = m_new;
    }
    const float negm = -m_run;
    f16x8_t pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f16x8_t t8;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          t8[j] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * hf + j], c2, negm));
        pb[kb][hf] = t8;
      }
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kh = 0; kh < 4; ++kh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const h2 pr = {pb[kh >> 1][kh & 1][2 * i], pb[kh >> 1][kh & 1][2 * i + 1]};
        ls[kh] = __builtin_amdgcn_fdot2(pr, one2, ls[kh], false);
      }
    float lsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    lsum += other_half(lsum, half);
    l_run = l_run + lsum;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if (d + 1 < 4) read_vf(d + 1);
#pragma unroll
      for (int kh = 0; kh < 4; ++kh)
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[d][kh], pb[kh >> 1][kh & 1], oacc[d], 0, 0, 0);
    }
  };

  // ---- prologue / main loop: decode tile t+1 into the other buffer and prefetch tile
  //      t+2's rows (t+3's value indices) while tile t is attended
  Pre pre;
  int vidx[2] = {0, 0};
  for (w0 = tb; w0 < te; w0 = w1) {   // windows of MWIN tiles, each its own pipeline
    w1 = min(te, w0 + MWIN);
    for (int i = tid; i < w1 - w0; i += NT) m_lds[i] = tab[w0 + i];
    __syncthreads();
    // past the window's last tile the pipeline repeats that tile's loads and decode into
    // the buffer nobody reads (valid rows, no branches in the loop)
    const int wl = w1 - 1;
    Meta m0 = meta(w0), m1 = meta(min(w0 + 1, wl)), m2 = meta(min(w0 + 2, wl)),
         m3 = meta(min(w0 + 3, wl));
    load_vidx(m0, vidx);
    load_data(m0, vidx, pre);
    load_vidx(m1, vidx);
    dequant(m0, pre, 0);
    load_data(m1, vidx, pre);
    load_vidx(m2, vidx);
    __syncthreads();
    for (int t = w0; t < w1; ++t) {
      const int buf = (t - w0) & 1;
      const int t4 = min(t + 4, wl);
      const int2 r4 = m_lds[t4 - w0];   // decoded at the end of the tile
      dequant(m1, pre, buf ^ 1);
      load_data(m2, vidx, pre);
      load_vidx(m3, vidx);
      compute(m0, buf);
      __syncthreads();
      m0 = m1;
      m1 = m2;
      m2 = m3;
      m3 = meta_of(r4, t4);
    }
  }

  // ---- epilogue (a split without tiles writes O = 0 with log-sum-exp -inf)
  float* const outp = p.splits > 1 ? p.part_o + (int64_t)split * p.nq * p.H * DM : p.out;
  float* const lsep = p.splits > 1 ? p.part_lse + (int64_t)split * p.H * p.nq : p.lse;
  if (myq < p.nq) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float* op = outp + (myq * p.H + h) * DM;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 o;
        o.x = oacc[d][4 * g + 0] * inv;
        o.y = oacc[d][4 * g + 1] * inv;
        o.z = oacc[d][4 * g + 2] * inv;
        o.w = oacc[d][4 * g + 3] * inv;
        *reinterpret_cast<float4*>(op + d * 32 + 8 * g + 4 * half) = o;
      }
    if (lsep && half == 0)
      lsep[(int64_t)h * p.nq + myq] =
          l_run > 0.0f ? (m_run + __log2f(l_run)) * 0.69314718055994531f : -__builtin_inff();
  }
}

// ----------------------------------------------------------------------------
// fp32 path: one lane per query, 32-key tiles decoded into LDS as fp32
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attend_f32_kernel(AttnParams p) {
  constexpr int TK = 32;
  __shared__ float kt[TK][D + 1];
  __shared__ float vt[TK][D + 1];
  const int tid = threadIdx.x;
  const int nqb = (int)((p.nq + 63) / 64);
  const int h = blockIdx.x / nqb;
  const int64_t qi = (int64_t)(blockIdx.x % nqb) * 64 + tid;
  float q[D], o[D];
  const float* qp = reinterpret_cast<const float*>(p.q) + (qi * p.H + h) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    q[i] = qi < p.nq ? qp[i] : 0.0f;
    o[i] = 0.0f;
  }
  float m_run = -__builtin_inff(), l_run = 0.0f;
  for (int64_t k0 = 0; k0 < p.nk; k0 += TK) {
    __syncthreads();
    for (int item = tid; item < TK * (D / 8); item += 64) {
      const int kk = item / (D / 8), c8 = item % (D / 8);
      const int64_t key = k0 + kk;
      float a[8], b[8];
      if (key < p.nk) {
        decode8<float, D>(p.k, h, key, c8 * 8, a);
        decode8<float, D>(p.v, h, key, c8 * 8, b);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = b[k] = 0.0f;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        kt[kk][c8 * 8 + k] = a[k];
        vt[kk][c8 * 8 + k] = b[k];
      }
    }
    __syncthreads();
    float s[TK];
    float mt = -__builtin_inff();
    for (int j = 0; j < TK; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < D; ++i) acc = __builtin_fmaf(q[i], kt[j][i], acc);
      acc *= p.scale;
      s[j] = (k0 + j < p.nk) ? acc : -__builtin_inff();
      mt = fmaxf(mt, s[j]);
    }
    const float m_new = fmaxf(m_run, mt);
    const float corr = expf(m_run - m_new);
    l_run *= corr;
#pragma unroll
    for (int i = 0; i < D; ++i) o[i] *= corr;
    for (int j = 0; j < TK; ++j) {
      const float e = expf(s[j] - m_new);
      l_run += e;
#pragma unroll
      for (int i = 0; i < D; ++i) o[i] = __builtin_fmaf(e, vt[j][i], o[i]);
    }
    m_run = m_new;
  }
  if (qi < p.nq) {
    float* op = p.out + (qi * p.H + h) * D;
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int i = 0; i < D; ++i) op[i] = o[i] * inv;
    if (p.lse) p.lse[(int64_t)h * p.nq + qi] = m_run + logf(l_run);
  }
}

Src make_src(const CodecArgs& c, const StoreArgs& st, const BaseArgs& b) {
  Src s{};
  s.codes = st.codes;
  s.sz = st.sz;
  s.index = st.index;
  s.cen = b.centroids;
  s.cap = st.capacity;
  s.bits = c.bits;
  s.group = c.group;
  s.groups = c.groups;
  s.words = c.code_words;
  s.idxb = c.index_bytes;
  s.C = c.C;
  s.mode = (c.base == KVC_BASE_CENTROID || c.base == KVC_BASE_COEFF) ? SRC_CENTROID : SRC_NONE;
  s.rot = c.rot;
  if (b.centroid_tables && s.mode == SRC_CENTROID && c.x_dtype == KVC_BF16) {
    s.cexp = reinterpret_cast<const int32_t*>(b.centroid_tables);
    s.cen16 = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(b.centroid_tables) +
                                                centroid_tables_header_bytes(c.H));
  }
  return s;
}

// Key splits of the bf16 path.  One workgroup fills a CU (its registers), so a launch of
// W workgroups takes ceil(W / CUs) rounds of equal length; splitting the keys s ways
// shortens a workgroup's run s-fold but multiplies the workgroups by s and adds a partial
// output per split.  The count kept minimizes rounds x key tiles per split: at most 8
// splits, at least 8 key tiles each, none empty.
int even_cost(int64_t base, int ntiles, int64_t cus, int s) {
  const int64_t tps = (ntiles + s - 1) / s;
  return (int)(((base * s + cus - 1) / cus) * tps);
}

int choose_splits(int H, int64_t nq, int64_t nk) {
  const int64_t base = (int64_t)H * ((nq + BQ - 1) / BQ);
  const int ntiles = (int)((nk + BK - 1) / BK);
  const int64_t cus = cu_count();
  const int smax = std::max(1, std::min(8, ntiles / 8));
  int sp = 1;
  for (int s = 2; s <= smax; ++s)
    if (even_cost(base, ntiles, cus, s) < even_cost(base, ntiles, cus, sp)) sp = s;
  // a split pays a partial output and a merge: keep one pass unless 5% shorter
  if (sp > 1 && (int64_t)even_cost(base, ntiles, cus, sp) * 20 > (int64_t)ntiles * 19) sp = 1;
  const int tps = (ntiles + sp - 1) / sp;
  return (ntiles + tps - 1) / tps;
}

// Sets p.splits / p.tps / partial buffers (one split when the workspace is too small).
void plan_splits(const AttendLaunch& a, AttnParams& p) {
  const int ntiles = (int)((a.n_keys + BK - 1) / BK);
  p.splits = 1;
  p.tps = ntiles;
  const int sp = choose_splits(a.kc.H, a.n_queries, a.n_keys);
  if (sp > 1 && a.workspace && a.workspace_bytes >= attend_workspace_bytes(a.kc, a.n_keys, a.n_queries)) {
    p.splits = sp;
    p.tps = (ntiles + sp - 1) / sp;
    p.part_o = reinterpret_cast<float*>(a.workspace);
    p.part_lse = p.part_o + (int64_t)sp * a.n_queries * a.kc.H * DM;
  }
}

hipError_t launch_combine(const AttnParams& p, hipStream_t s) {
  if (p.splits <= 1) return hipGetLastError();
  const int64_t n = p.nq * p.H * (DM / 4);
  hipLaunchKernelGGL(attend_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

// The bf16 kernel over compressed K and V of the given bit widths and bases: every
// (K bits, V bits, K base, V base) combination is its own kernel so the prefetch loads
// stay branch-free.
hipError_t launch_compressed_bf16(const AttnParams& p, int kbits, int vbits, dim3 grid, hipStream_t s) {
  const bool kc = p.k.mode == SRC_CENTROID, vc = p.v.mode == SRC_CENTROID;
  const dim3 block(NT);
  const bool rot = p.k.rot || p.v.rot, jb = p.jensen != 0;
  const bool cf = kc && vc && p.k.cen16 && p.v.cen16;   // both tables' fp16 images given
  if (rot || jb) {   // rotated residuals / Jensen correction: centroid K and V (validated by the caller)
    if (!kc || !vc) return hipErrorInvalidValue;
#define KVC_ATT_RJ(KB_, VB_, R_, J_)                                                             \
    if (kbits == KB_ && vbits == VB_ && rot == R_ && jb == J_) {                                 \
      if (cf)                                                                                    \
        hipLaunchKernelGGL((attend_bf16_kernel<KB_, VB_, true, true, false, false, R_, J_, true>), \
                           grid, block, 0, s, p);                                                \
      else                                                                                       \
        hipLaunchKernelGGL((attend_bf16_kernel<KB_, VB_, true, true, false, false, R_, J_>), grid, block, 0, s, p); \
      return hipGetLastError();                                                                  \
    }
#define KVC_ATT_RJ_BITS(R_, J_) \
    KVC_ATT_RJ(2, 2, R_, J_) KVC_ATT_RJ(2, 4, R_, J_) KVC_ATT_RJ(4, 2, R_, J_) KVC_ATT_RJ(4, 4, R_, J_)
    KVC_ATT_RJ_BITS(true, false)
    KVC_ATT_RJ_BITS(false, true)
    KVC_ATT_RJ_BITS(true, true)
#undef KVC_ATT_RJ_BITS
#undef KVC_ATT_RJ
    return hipErrorInvalidValue;
  }
  if (cf) {
#define KVC_ATT16(KB_, VB_)                                                                       \
    if (kbits == KB_ && vbits == VB_) {                                                           \
      hipLaunchKernelGGL((attend_bf16_kernel<KB_, VB_, true, true, false, false, false, false, true>), \
                         grid, block, 0, s, p);                                                   \
      return hipGetLastError();                                                                   \
    }
    KVC_ATT16(2, 2) KVC_ATT16(2, 4) KVC_ATT16(4, 2) KVC_ATT16(4, 4)
#undef KVC_ATT16
    return hipErrorInvalidValue;
  }
#define KVC_ATT(KB_, VB_, KC_, VC_)                                                       \
  if (kbits == KB_ && vbits == VB_ && kc == KC_ && vc == VC_) {                         \
    hipLaunchKernelGGL((attend_bf16_kernel<KB_, VB_, KC_, VC_, false>), grid, block, 0, s, p); \
    return hipGetLastError();                                                            \
  }
#define KVC_ATT_BITS(KC_, VC_) \
  KVC_ATT(2, 2, KC_, VC_) KVC_ATT(2, 4, KC_, VC_) KVC_ATT(4, 2, KC_, VC_) KVC_ATT(4, 4, KC_, VC_)
  KVC_ATT_BITS(true, true)
  KVC_ATT_BITS(true, false)
  KVC_ATT_BITS(false, true)
  KVC_ATT_BITS(false, false)
#undef KVC_ATT_BITS
#undef KVC_ATT
  return hipErrorInvalidValue;
}

// Key splits of the history when a current chunk is attended as well: one part more
// than the splits must fit the merge.
int chunk_history_splits(int H, int64_t nq, int64_t nk) {
  const int ntiles = (int)((nk + BK - 1) / BK);
  const int sp = std::min(choose_splits(H, nq, nk), MAX_PARTS - 1);
  const int tps = (ntiles + sp - 1) / sp;
  return (ntiles + tps - 1) / tps;
}

}  // namespace

size_t attend_workspace_bytes(const CodecArgs& kc, int64_t n_keys, int64_t n_queries) {
  if (kc.x_dtype != KVC_BF16 || kc.D != DM || n_queries <= 0 || n_keys <= 0) return 0;
  const int sp = choose_splits(kc.H, n_queries, n_keys);
  if (sp <= 1) return 0;
  return (size_t)sp * n_queries * kc.H * (DM + 1) * sizeof(float);
}

hipError_t launch_attend(const AttendLaunch& a, hipStream_t s) {
  if (a.n_queries == 0) return hipSuccess;
  AttnParams p{};
  p.q = a.q;
  p.nq = a.n_queries;
  p.nk = a.n_keys;
  p.H = a.kc.H;
  p.scale = a.scale;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.out = a.out;
  p.lse = a.lse;
  p.k = make_src(a.kc, a.ks, a.kb);
  p.v = make_src(a.vc, a.vs, a.vb);
  p.jensen = a.jensen;
  if (a.kc.x_dtype == KVC_BF16) {
    plan_splits(a, p);
    const int nqb = (int)((a.n_queries + BQ - 1) / BQ);
    const dim3 grid(nqb * a.kc.H * p.splits), block(NT);
    if (a.kc.bits == 16) {   // uncompressed bf16 caches (validated: both K and V)
      hipLaunchKernelGGL((attend_bf16_kernel<2, 2, false, false, false, true>), grid, block, 0, s, p);
      return launch_combine(p, s);
    }
    const hipError_t e = launch_compressed_bf16(p, a.kc.bits, a.vc.bits, grid, s);
    if (e != hipSuccess) return e;
    return launch_combine(p, s);
  } else {
    p.splits = 1;
    const int nqb = (int)((a.n_queries + 63) / 64);
    if (a.kc.D == 128)
      hipLaunchKernelGGL(attend_f32_kernel<128>, dim3(nqb * a.kc.H), dim3(64), 0, s, p);
    else
      hipLaunchKernelGGL(attend_f32_kernel<64>, dim3(nqb * a.kc.H), dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

size_t attend_chunk_workspace_bytes(const CodecArgs& kc, int64_t n_keys, int64_t n_queries) {
  if (kc.x_dtype != KVC_BF16 || kc.D != DM || n_queries <= 0 || n_keys <= 0) return 0;
  const int sp = chunk_history_splits(kc.H, n_queries, n_keys);
  return (size_t)(sp + 1) * n_queries * kc.H * (DM + 1) * sizeof(float);
}

// Compressed history (key splits 0 .. S-1) and the uncompressed current chunk (part S)
// attended as separate parts of one softmax; attend_combine_kernel merges the S + 1
// normalized partial outputs by their log-sum-exp.
hipError_t launch_attend_chunk(const AttendLaunch& a, const void* chunk_k, const void* chunk_v,
                               int64_t n_chunk, hipStream_t s) {
  if (a.n_queries == 0) return hipSuccess;
  const int H = a.kc.H;
  const int64_t nq = a.n_queries;
  AttnParams p{};
  p.q = a.q;
  p.nq = nq;
  p.nk = a.n_keys;
  p.H = H;
  p.scale = a.scale;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.k = make_src(a.kc, a.ks, a.kb);
  p.v = make_src(a.vc, a.vs, a.vb);
  p.jensen = a.jensen;
  const int ntiles = (int)((a.n_keys + BK - 1) / BK);
  const int sp = chunk_history_splits(H, nq, a.n_keys);
  p.splits = sp;
  p.tps = (ntiles + sp - 1) / sp;
  p.part_o = reinterpret_cast<float*>(a.workspace);
  p.part_lse = p.part_o + (int64_t)(sp + 1) * nq * H * DM;
  if (sp == 1) {   // a single history part writes its normalized result as part 0
    p.out = p.part_o;
    p.lse = p.part_lse;
  }
  const int nqb = (int)((nq + BQ - 1) / BQ);
  hipError_t e = launch_compressed_bf16(p, a.kc.bits, a.vc.bits, dim3(nqb * H * sp), s);
  if (e != hipSuccess) return e;
  // the chunk: a dense bf16 cache [n_chunk][H][d], part sp
  AttnParams pc = p;
  pc.nk = n_chunk;
  pc.splits = 1;
  pc.tps = (int)((n_chunk + BK - 1) / BK);
  pc.k = Src{};
  pc.v = Src{};
  pc.k.codes = reinterpret_cast<const uint32_t*>(chunk_k);
  pc.v.codes = reinterpret_cast<const uint32_t*>(chunk_v);
  pc.k.cap = pc.v.cap = n_chunk;
  pc.k.bits = pc.v.bits = 16;
  pc.out = p.part_o + (int64_t)sp * nq * H * DM;
  pc.lse = p.part_lse + (int64_t)sp * H * nq;
  hipLaunchKernelGGL((attend_bf16_kernel<2, 2, false, false, false, true>), dim3(nqb * H), dim3(NT), 0, s, pc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  AttnParams pm = p;
  pm.splits = sp + 1;
  pm.out = a.out;
  pm.lse = a.lse;
  return launch_combine(pm, s);
}

namespace {

// Workspace of the cluster-ordered mixed path: the tables, the ordered K and V copies
// (V sized for the widest value codec: 16 code words, 8 scale/zero words and 2-byte
// indices per row), then the key splits' partial results.
struct MixedLayout {
  size_t cnt, tiles, ntiles, kcodes, ksz, kidx, vcodes, vsz, vidx, part, total;
  int nb, nchunk, tmax, splits;
};

bool mixed_clusterable(const CodecArgs& kc) {
  return kc.base == KVC_BASE_COEFF && kc.x_dtype == KVC_BF16 && kc.D == DM && kc.m == 16 &&
         kc.groups == 1 && kc.C >= 1 && kc.C <= CL_BLK * CL_MAXNB;
}

MixedLayout mixed_layout(const CodecArgs& kc, int64_t n, int64_t nq) {
  MixedLayout L{};
  L.nb = (kc.C + CL_BLK - 1) / CL_BLK;
  L.nchunk = (int)((n + CL_CHUNK - 1) / CL_CHUNK);
  L.tmax = (int)((n + BK - 1) / BK) + L.nb;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t H = (size_t)kc.H, rows = H * (size_t)n;
  size_t o = 0;
  L.cnt = o;    o = al(o + H * L.nchunk * L.nb * 4);
  L.tiles = o;  o = al(o + H * L.tmax * 8);
  L.ntiles = o; o = al(o + H * 4);
  L.kcodes = o; o = al(o + rows * kc.code_words * 4);
  L.ksz = o;    o = al(o + rows * 4);
  L.kidx = o;   o = al(o + rows * kc.index_bytes);
  L.vcodes = o; o = al(o + rows * 16 * 4);
  L.vsz = o;    o = al(o + rows * 8 * 4);
  L.vidx = o;   o = al(o + rows * 2);
  L.splits = choose_splits(kc.H, nq, (int64_t)L.tmax * BK);
  L.part = o;
  if (L.splits > 1) o = al(o + (size_t)L.splits * nq * H * (DM + 1) * 4);
  L.total = o;
  return L;
}

}  // namespace

size_t attend_mixed_workspace_bytes(const CodecArgs& kc, int64_t n_keys, int64_t n_queries) {
  if (n_queries <= 0 || n_keys <= 0) return 0;
  if (!mixed_clusterable(kc)) return attend_workspace_bytes(kc, n_keys, n_queries);
  return mixed_layout(kc, n_keys, n_queries).total;
}

// With a workspace of attend_mixed_workspace_bytes: order the keys by centroid block
// (three small launches), attend the ordered copies with attend_mixed_cl_kernel, merge
// the key splits.  Otherwise the centroid rows are gathered into the K tiles
// (attend_bf16_kernel<..., MIXED>).
hipError_t launch_attend_mixed(const AttendLaunch& a, hipStream_t s) {
  if (a.n_queries == 0) return hipSuccess;
  if (a.kc.m != 16 || a.kc.groups != 1) return hipErrorInvalidValue;
  AttnParams p{};
  p.q = a.q;
  p.nq = a.n_queries;
  p.nk = a.n_keys;
  p.H = a.kc.H;
  p.scale = a.scale;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.out = a.out;
  p.lse = a.lse;
  p.k = make_src(a.kc, a.ks, a.kb);
  p.v = make_src(a.vc, a.vs, a.vb);
  p.jensen = a.jensen;
  p.basis = reinterpret_cast<const uint16_t*>(a.kb.basis);
  const bool vc = p.v.mode == SRC_CENTROID;
  const int nqb = (int)((a.n_queries + BQ - 1) / BQ);
  if (mixed_clusterable(a.kc) && vc && a.vc.code_words <= 16 && a.vc.groups <= 8 && a.vc.index_bytes <= 2 &&
      a.workspace && a.workspace_bytes >= attend_mixed_workspace_bytes(a.kc, a.n_keys, a.n_queries)) {
    const MixedLayout L = mixed_layout(a.kc, a.n_keys, a.n_queries);
    char* ws = reinterpret_cast<char*>(a.workspace);
    ClusterParams c{};
    c.n = a.n_keys;
    c.H = a.kc.H;
    c.nb = L.nb;
    c.nchunk = L.nchunk;
    c.tmax = L.tmax;
    c.k = p.k;
    c.v = p.v;
    c.cnt = reinterpret_cast<int*>(ws + L.cnt);
    c.tiles = reinterpret_cast<int2*>(ws + L.tiles);
    c.ntiles = reinterpret_cast<int*>(ws + L.ntiles);
    c.kcodes = reinterpret_cast<uint32_t*>(ws + L.kcodes);
    c.ksz = reinterpret_cast<uint32_t*>(ws + L.ksz);
    c.kidx = reinterpret_cast<uint8_t*>(ws + L.kidx);
    c.vcodes = reinterpret_cast<uint32_t*>(ws + L.vcodes);
    c.vsz = reinterpret_cast<uint32_t*>(ws + L.vsz);
    c.vidx = reinterpret_cast<uint8_t*>(ws + L.vidx);
    const dim3 cg((unsigned)L.nchunk, (unsigned)a.kc.H);
    hipLaunchKernelGGL(cluster_count_kernel, cg, dim3(CL_THREADS), 0, s, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(cluster_scan_kernel, dim3((unsigned)a.kc.H), dim3(CL_THREADS), 0, s, c);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(cluster_scatter_kernel, cg, dim3(CL_THREADS), 0, s, c);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    AttnParams pc = p;
    pc.k.codes = c.kcodes;
    pc.k.sz = c.ksz;
    pc.k.index = c.kidx;
    pc.k.cap = a.n_keys;
    pc.v.codes = c.vcodes;
    pc.v.sz = c.vsz;
    pc.v.index = c.vidx;
    pc.v.cap = a.n_keys;
    pc.splits = L.splits;
    pc.tps = (L.tmax + L.splits - 1) / L.splits;
    if (pc.splits > 1) {
      pc.part_o = reinterpret_cast<float*>(ws + L.part);
      pc.part_lse = pc.part_o + (int64_t)pc.splits * a.n_queries * a.kc.H * DM;
    }
    ClusterTabs ct{c.tiles, c.ntiles, L.tmax};
    const dim3 grid((unsigned)(nqb * a.kc.H * pc.splits)), block(NT);
#define KVC_MIXCL(KB_, VB_)                                                               \
    if (a.kc.bits == KB_ && a.vc.bits == VB_) {                                           \
      if (pc.v.cen16)                                                                     \
        hipLaunchKernelGGL((attend_mixed_cl_kernel<KB_, VB_, true, true>), grid, block, 0, s, pc, ct); \
      else                                                                                \
        hipLaunchKernelGGL((attend_mixed_cl_kernel<KB_, VB_, true>), grid, block, 0, s, pc, ct); \
      e = hipGetLastError();                                                              \
      if (e != hipSuccess) return e;                                                      \
      return launch_combine(pc, s);                                                       \
    }
    KVC_MIXCL(4, 2) KVC_MIXCL(4, 4) KVC_MIXCL(2, 2) KVC_MIXCL(2, 4)
#undef KVC_MIXCL
    return hipErrorInvalidValue;
  }
  plan_splits(a, p);
  const dim3 grid(nqb * a.kc.H * p.splits), block(NT);
#define KVC_MIX(KB_, VB_, VC_)                                                           \
  if (a.kc.bits == KB_ && a.vc.bits == VB_ && vc == VC_) {                              \
    hipLaunchKernelGGL((attend_bf16_kernel<KB_, VB_, true, VC_, true>), grid, block, 0, s, p); \
    return launch_combine(p, s);                                                         \
  }
  KVC_MIX(4, 2, true) KVC_MIX(4, 4, true) KVC_MIX(2, 2, true) KVC_MIX(2, 4, true)
#undef KVC_MIX
  return hipErrorInvalidValue;
}

}  // namespace kvc
