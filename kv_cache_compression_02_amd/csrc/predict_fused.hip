// Fused predictor + quantizer for bf16 d = 128 data.
//
// * Cross-layer block-DPLR (Coral-KV arXiv 2610.12514, Fig. 3):
//       pred[h] = W_h [in0_h ; in1_h] + U_h t,   t = v_lr [in0 ; in1]   (rank r)
// * Temporal values (TempoKV arXiv 2610.15324, Fig. 2b): pred[h] = M_h aux_h + beta_h * in0_h.
// * Temporal keys: pred = (a * in0) + (b * in1) per channel; anchors: pred = 0.
//
// rank_kernel forms t (fp32), 16 tokens per wave, each element one MFMA accumulation
// chain over the whole contraction in ascending order, so every call with the same
// inputs gives the same t.  pred_kernel keeps one head's W_h (and U_h) in LDS and walks
// that head's 16-token tiles; in a wave, lane (t, q) = (lane & 15, lane >> 4) owns
// channels 32 q .. 32 q + 31 of token t.  The MFMA rows of the weight operand are
// permuted (row 4 q + s of output block ob holds channel 32 q + 4 ob + s), so accumulator
// s of block ob is a channel of the lane's own quarter row: the prediction reaches the
// group quantizer from registers.  The contraction runs in natural channel order, lane q
// feeding channels 32 ks + 8 q .. + 7 of k-step ks.  t enters as bf16 high and
// low parts (about 2^-16 relative).  With no input to encode the same kernel only
// writes the prediction, for the decoder: encoder and decoder see identical bases.
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int D = 128;

struct RankParams {
  const uint16_t* in0;
  const uint16_t* in1;
  int64_t ps;            // token stride of the inputs (elements)
  const uint16_t* vlr;   // [r][nin * hd]
  float* t;              // [n][r]
  int n, r, hd, nin;
};



typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// t = v_lr [in0 ; in1] on v_mfma_f32_16x16x32_bf16.  A workgroup of eight waves takes
// 128 tokens, each wave 16 of them over the whole contraction, so every t element is one
// MFMA accumulation chain in ascending k and the same on every call.  v_lr is staged
// through LDS in chunks of 128 columns shared by the eight waves; every global load
// reads 64 contiguous bytes of 16 rows.  The pass only streams its inputs, so it is
// bound by how many bytes are in flight: each wave keeps the next three chunks of its
// input fragments in registers (a ring of three), and the v_lr chunk for the LDS buffer
// two chunks ahead is requested an iteration before it is stored.  Past the last chunk
// the requests repeat it (valid addresses, no branches around the loads).
constexpr int RK_KC = 128;              // contraction chunk
constexpr int RK_ROW = RK_KC + 8;       // padded LDS row (bf16)
constexpr int RK_TOK = 128;             // tokens per workgroup
template <int RB>        // r <= 16 RB
__global__ __launch_bounds__(512) void rank_kernel(RankParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t vl[2][16 * RB * RK_ROW];
  constexpr int PIECES = 16 * RB * (RK_KC / 8);        // 16-byte pieces of a chunk
  constexpr int PPT = (PIECES + 511) / 512;            // per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, q = lane >> 4;
  const int n = blockIdx.x * RK_TOK + wave * 16 + col;   // token of B-operand column col
  const bool tok = n < p.n;
  // Rows past the last token and v_lr rows past r are read from the last valid row: they
  // only feed t columns and rows that are never stored, and every load stays unconditional
  // (no divergent branch makes the compiler drain the loads in flight).
  const int64_t trow = (int64_t)min(n, p.n - 1) * p.ps;
  const int K = p.nin * p.hd, nch = K / RK_KC;           // hd is a multiple of 128
  static_assert(PIECES % 512 == 0 && PPT <= 2, "whole chunk pieces per thread");
  // a chunk's v_lr pieces of this thread on their way to LDS (one or two 16-byte pieces)
  struct Stage { uint4 a, b; };
  auto load_stage = [&](int c, Stage& v) {
    auto piece = [&](int e) {
      const int row = min(e >> 4, p.r - 1), pc = e & 15;
      return *reinterpret_cast<const uint4*>(p.vlr + (int64_t)row * K + c * RK_KC + 8 * pc);
    };
    v.a = piece(tid);
    if constexpr (PPT == 2) v.b = piece(tid + 512);
  };
  auto store_stage = [&](int b, const Stage& v) {
    *reinterpret_cast<uint4*>(&vl[b][(tid >> 4) * RK_ROW + 8 * (tid & 15)]) = v.a;
    if constexpr (PPT == 2)
      *reinterpret_cast<uint4*>(&vl[b][((tid + 512) >> 4) * RK_ROW + 8 * (tid & 15)]) = v.b;
  };
  auto load_b = [&](int c, bf16x8_t (&bx)[4]) {
    const int k0 = c * RK_KC;
    const int j = k0 >= p.hd ? 1 : 0;   // a chunk never straddles the two inputs
    const uint16_t* src = (j ? p.in1 : p.in0) + (k0 - j * p.hd) + trow + 8 * q;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      bx[ks] = *reinterpret_cast<const bf16x8_t*>(src + 32 * ks);
  };
  f32x4_t acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // sa / sb: the v_lr chunk of even / odd index on its way to LDS; b0, b1, b2: the input
  // fragments of chunk c with c % 3 == 0, 1, 2
  Stage sa, sb;
  bf16x8_t b0[4], b1[4], b2[4];
  load_stage(0, sa);
  load_stage(min(1, nch - 1), sb);
  load_b(0, b0);
  load_b(min(1, nch - 1), b1);
  load_b(min(2, nch - 1), b2);
  store_stage(0, sa);
  __syncthreads();
  // chunk c: LDS buffer lb = c & 1 holds it, sfree (same parity) is free, snext holds
  // chunk c + 1, bcur holds its input fragments
  auto step = [&](int c, int lb, Stage& sfree, Stage& snext,
                  bf16x8_t (&bcur)[4]) __attribute__((always_inline)) {
    load_stage(min(c + 2, nch - 1), sfree);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t*>(&vl[lb][(16 * rb + col) * RK_ROW + 32 * ks + 8 * q]);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bcur[ks], acc[rb], 0, 0, 0);
      }
    load_b(min(c + 3, nch - 1), bcur);
    store_stage(lb ^ 1, snext);
    __syncthreads();
  };
  // six chunks per pass, so that both rings are indexed statically; the passes have no
  // branches inside, the chunks of a last partial pass (nch % 6) follow
  int c0 = 0;
#pragma unroll 1
  for (; c0 + 6 <= nch; c0 += 6) {
    step(c0, 0, sa, sb, b0);
    step(c0 + 1, 1, sb, sa, b1);
    step(c0 + 2, 0, sa, sb, b2);
    step(c0 + 3, 1, sb, sa, b0);
    step(c0 + 4, 0, sa, sb, b1);
    step(c0 + 5, 1, sb, sa, b2);
  }
  if (c0 < nch) step(c0, 0, sa, sb, b0);
  if (c0 + 1 < nch) step(c0 + 1, 1, sb, sa, b1);
  if (c0 + 2 < nch) step(c0 + 2, 0, sa, sb, b2);
  if (c0 + 3 < nch) step(c0 + 3, 1, sb, sa, b0);
  if (c0 + 4 < nch) step(c0 + 4, 0, sa, sb, b1);
  // lane (col, q) holds t[n][16 rb + 4 q + i]: 64 contiguous bytes per token and block
  if (tok) {
    float* trow_out = p.t + (int64_t)n * p.r;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int c0 = 16 * rb + 4 * q;
      if (c0 < p.r)
        *reinterpret_cast<float4*>(trow_out + c0) = make_float4(acc[rb][0], acc[rb][1], acc[rb][2], acc[rb][3]);
    }
  }
}

enum { PM_NONE = 0, PM_TEMPORAL_K = 1, PM_DPLR = 2, PM_TEMPORAL_V = 3 };

struct PredParams {
  const uint16_t* x;       // encode input [n][H][D] (token stride x_stride)
  int64_t x_stride;
  const uint16_t* g0;      // matrix-product inputs (DPLR: in0, in1; temporal V: aux)
  const uint16_t* g1;
  const uint16_t* e0;      // element-wise inputs (temporal K: K_{t-1}, K_{t-2}; temporal V: V_{t-1})
  const uint16_t* e1;
  int64_t ps;              // token stride of g0 / g1 / e0 / e1
  const uint16_t* w;       // [H][D][nin D]
  const uint16_t* u;       // [H D][r]
  const float* t;          // [n][r]
  const float* ca;         // [H][D]
  const float* cb;
  int n, H, r, segs;
  int64_t token_offset, capacity;
  uint32_t* codes;
  uint32_t* sz;
  uint16_t* recon;         // [n][H][D] bf16 or null
  float* pred;             // [n][H][D] fp32 or null
  int rot;                 // Hn residual transform width: 0, 16 or 64
};

// Output channel held by MFMA row i of output block ob (16 x 16 blocks): row 4 q + s
// of block ob is channel 32 q + 4 ob + s, so lane (t, q) receives channels 32 q + 4 ob + s.
__device__ __forceinline__ int out_channel(int ob, int i) { return 32 * (i >> 2) + 4 * ob + (i & 3); }

// LDS geometry: permuted weight rows, U with permuted columns (64 wide, zero past r),
// then one 16-token staging tile per wave.  Rows are padded by 16 elements (U rows 40
// dwords, weight rows 72 or 136) so that the 32 lanes served together by a 16-byte LDS
// read (rows t = 0..15, column blocks q and q + 1) fall on distinct 4-bank slots.
constexpr int URW = 64 + 16;
constexpr int STG = 16 * D;                  // staging tile (bf16 elements)
__host__ __device__ constexpr int w_row(int nin) { return nin * D + 16; }
__host__ __device__ constexpr int w_elems(int nin) { return 128 * w_row(nin); }

// 16-byte loads that give zeros when `ok` is false (a branch, not a select of addresses)
__device__ __forceinline__ uint4 ld_u4(const void* p, bool ok) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (ok) v = *reinterpret_cast<const uint4*>(p);
  return v;
}
__device__ __forceinline__ float4 ld_f4(const float* p, bool ok) {
  float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (ok) v = *reinterpret_cast<const float4*>(p);
  return v;
}

// Staging tile slot (16-byte units) of chunk c (8 channels) of token tok: chunk index
// XOR token spreads both access patterns below over all 16 bank groups.
__device__ __forceinline__ int stg_slot(int tok, int c) { return tok * 16 + (c ^ tok); }

// Hn transform (Coral-KV Fig. 5 and Fig. 9b-c: each group of n residual channels is
// rotated by the n-point Walsh-Hadamard matrix) of a lane's GL contiguous channels in the
// layout below (lane q of a token holds channels 32 q .. 32 q + 31), with the rounding of
// the Sylvester recursion H_2m [a; b] = [H_m a + H_m b; H_m a - H_m b]: butterflies at
// channel distance 1, 2, 4, 8 (and 16 for n = 64) inside the lane, for n = 64 then 32
// with the lane 16 apart (quarter q ^ 1); the lower channel of a pair takes a + b, the
// upper a - b; then the exact 1/sqrt(n) scale.  H_n / sqrt(n) is its own inverse, so
// the same call rotates the residual before the quantizer and the dequantized vector
// back.  n divides the group (validated), so every block lies in one lane or one pair.
template <int GL>
__device__ __forceinline__ void hn_rotate_lane(float (&r)[GL], int n, int q) {
#pragma unroll
  for (int h = 1; h < 32 && h < GL; h <<= 1) {
    if (h >= 16 && n != 64) break;
#pragma unroll
    for (int i = 0; i < GL; ++i) {
      if (i & h) continue;
      const float a = r[i], b = r[i + h];
      r[i] = a + b;
      r[i + h] = a - b;
    }
  }
  if constexpr (GL == 32) {
    if (n == 64) {
      const bool up = (q & 1) != 0;
#pragma unroll
      for (int i = 0; i < GL; ++i) {
        const float o = __shfl_xor(r[i], 16);
        r[i] = up ? o - r[i] : r[i] + o;
      }
    }
  }
  const float sc = n == 64 ? 0.125f : 0.25f;
#pragma unroll
  for (int i = 0; i < GL; ++i) r[i] *= sc;
}

template <int BITS, int G, int PM, int NIN>
__global__ __launch_bounds__(512) void pred_kernel(PredParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  constexpr bool MAT = PM == PM_DPLR || PM == PM_TEMPORAL_V;
  constexpr bool LR = PM == PM_DPLR;
  constexpr int WROW = w_row(NIN);           // padded weight row (bf16)
  constexpr int PER = 32 / BITS;             // codes per word
  constexpr int LW = 32 / PER;               // code words of a lane (32 values)
  constexpr int GL = G < 32 ? G : 32;        // values of one group in a lane
  constexpr int NGL = 32 / GL;               // groups (or group halves) in a lane
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = lane & 15, q = lane >> 4;
  // coalesced role of the lane: token 4 i + ct of a 16-token tile in instruction i,
  // channel chunk cc (16 lanes cover one token's 256-byte row)
  const int ct = lane >> 4, cc = lane & 15;
  // matrix modes: workgroup = (head, segment) with the head's weights in LDS, its waves
  // walking that head's tiles; other modes walk the flattened (head, tile) list
  const int hw = MAT ? blockIdx.x / p.segs : 0, seg = MAT ? blockIdx.x % p.segs : (int)blockIdx.x;
  uint16_t* wl = lds;                                   // [128][WROW], permuted rows
  uint16_t* ul = lds + (MAT ? w_elems(NIN) : 0);        // [128][URW]
  uint16_t* stg = lds + (MAT ? w_elems(NIN) : 0) + (LR ? 128 * URW : 0) + wave * STG;
  if constexpr (MAT) {
    const uint16_t* wh = p.w + (int64_t)hw * D * (NIN * D);
    for (int e = tid; e < 128 * NIN * 16; e += 512) {
      const int i2 = e / (NIN * 16), c = e % (NIN * 16);
      const int ch = out_channel(i2 >> 4, i2 & 15);
      *reinterpret_cast<uint4*>(&wl[i2 * WROW + 8 * c]) =
          *reinterpret_cast<const uint4*>(wh + (int64_t)ch * (NIN * D) + 8 * c);
    }
    if constexpr (LR) {
      // U row ch in permuted row order; its 4-column piece m of 32-block kb goes to
      // position 32 kb + 8 (m & 3) + 4 (m >> 2), matching how a lane reads t below
      for (int e = tid; e < 128 * 16; e += 512) {
        const int i2 = e >> 4, piece = e & 15, kb = piece >> 3, m = piece & 7;
        const int ch = out_channel(i2 >> 4, i2 & 15);
        const int col = 32 * kb + 4 * m;
        uint2 v = make_uint2(0u, 0u);
        if (col < p.r) v = *reinterpret_cast<const uint2*>(p.u + ((int64_t)hw * D + ch) * p.r + col);
        *reinterpret_cast<uint2*>(&ul[i2 * URW + 32 * kb + 8 * (m & 3) + 4 * (m >> 2)]) = v;
      }
    }
    __syncthreads();
  }
  const int tiles = (p.n + 15) / 16;
  constexpr int NG = MAT ? NIN : 0;                                 // matrix inputs
  constexpr int NE = PM == PM_TEMPORAL_K ? 2 : (PM == PM_TEMPORAL_V ? 1 : 0);   // element-wise
  constexpr int NT = LR ? 2 : 0;                                    // t k-steps (r <= 64)
  // everything a tile reads, so the next tile's reads are in flight while this one computes
  struct TileIn {
    uint4 xv[4];                       // row to encode, coalesced layout
    bf16x8_t gin[NG > 0 ? NG : 1][4];  // matrix-product inputs, k-step ks = chunk 4 ks + q
    uint4 ev[NE > 0 ? NE : 1][4];      // element-wise inputs, coalesced layout
    float4 tv[NT > 0 ? NT : 1][2];     // t[32 ks + 4 q ..], t[32 ks + 16 + 4 q ..]
  };
  const int items = MAT ? tiles : tiles * p.H;
  const int istride = MAT ? p.segs * 8 : gridDim.x * 8;
  auto load_tile = [&](int item, TileIn& in) __attribute__((always_inline)) {
    const bool ok = item < items;
    const int h = MAT ? hw : (ok ? item / tiles : 0), tile = MAT ? item : (ok ? item % tiles : 0);
    const int n = tile * 16 + t;
    const bool live = ok && n < p.n;
    // coalesced: instruction i reads tokens 4 i .. 4 i + 3 whole
    if (p.x) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nc = tile * 16 + 4 * i + ct;
        in.xv[i] = ld_u4(p.x + (int64_t)nc * p.x_stride + (int64_t)h * D + 8 * cc, ok && nc < p.n);
      }
    }
    const uint16_t* esrc[2] = {p.e0, p.e1};
#pragma unroll
    for (int j = 0; j < NE; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nc = tile * 16 + 4 * i + ct;
        in.ev[j][i] = ld_u4(esrc[j] + (int64_t)nc * p.ps + (int64_t)h * D + 8 * cc, ok && nc < p.n);
      }
    const int64_t grow = (int64_t)(live ? n : 0) * p.ps + (int64_t)h * D;
    const uint16_t* gsrc[2] = {p.g0, p.g1};
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        in.gin[j][ks] = __builtin_bit_cast(bf16x8_t, ld_u4(gsrc[j] + grow + 32 * ks + 8 * q, live));
#pragma unroll
    for (int ks = 0; ks < NT; ++ks) {
      const float* tp = p.t + (int64_t)(live ? n : 0) * p.r + 32 * ks + 4 * q;
      in.tv[ks][0] = ld_f4(tp, live && 32 * ks + 4 * q < p.r);
      in.tv[ks][1] = ld_f4(tp + 16, live && 32 * ks + 16 + 4 * q < p.r);
    }
  };
  // coalesced rows -> this lane's quarter row (channels 32 q .. 32 q + 31), through the
  // wave's staging tile (a wave's LDS operations complete in order)
  auto to_quarter = [&](const uint4 (&v)[4], uint4 (&o)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&stg[8 * stg_slot(4 * i + ct, cc)]) = v[i];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = *reinterpret_cast<const uint4*>(&stg[8 * stg_slot(t, 4 * q + i)]);
    __builtin_amdgcn_wave_barrier();
  };

  TileIn cur;
  const int first = seg * 8 + wave;
  load_tile(first, cur);
#pragma unroll 1
  for (int item = first; item < items; item += istride) {
    TileIn nxt;
    load_tile(item + istride, nxt);   // past the last item: no reads (zeros)
    const int h = MAT ? hw : item / tiles, tile = MAT ? item : item % tiles;
    const int n = tile * 16 + t;
    const bool live = n < p.n;
    uint4 xv[4];
    if (p.x) to_quarter(cur.xv, xv);
    float pred[32];
    if constexpr (PM == PM_NONE) {
#pragma unroll
      for (int i = 0; i < 32; ++i) pred[i] = 0.0f;
    } else if constexpr (PM == PM_TEMPORAL_K) {
      uint4 e0[4], e1[4];
      to_quarter(cur.ev[0], e0);
      to_quarter(cur.ev[NE - 1], e1);
      const float* ca = p.ca + h * D + 32 * q;
      const float* cb = p.cb + h * D + 32 * q;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v0 = e0[i];
        const uint4 v1 = e1[i];
        const float4 ca0 = *reinterpret_cast<const float4*>(ca + 8 * i);
        const float4 ca1 = *reinterpret_cast<const float4*>(ca + 8 * i + 4);
        const float4 cb0 = *reinterpret_cast<const float4*>(cb + 8 * i);
        const float4 cb1 = *reinterpret_cast<const float4*>(cb + 8 * i + 4);
        const float av[8] = {ca0.x, ca0.y, ca0.z, ca0.w, ca1.x, ca1.y, ca1.z, ca1.w};
        const float bv[8] = {cb0.x, cb0.y, cb0.z, cb0.w, cb1.x, cb1.y, cb1.z, cb1.w};
        const uint32_t a0[4] = {v0.x, v0.y, v0.z, v0.w}, a1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float p0 = av[2 * k] * lo_bf16(a0[k]), q0 = bv[2 * k] * lo_bf16(a1[k]);
          const float p1 = av[2 * k + 1] * hi_bf16(a0[k]), q1 = bv[2 * k + 1] * hi_bf16(a1[k]);
          pred[8 * i + 2 * k] = p0 + q0;
          pred[8 * i + 2 * k + 1] = p1 + q1;
        }
      }
    } else {
      // matrix products, one input at a time; k-step ks: lane q feeds channels
      // 32 ks + 8 q .. + 7 (its part of a contiguous 64-byte read per token)
      f32x4_t acc[8];
#pragma unroll
      for (int ob = 0; ob < 8; ++ob) acc[ob] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < NG; ++j) {
#pragma unroll
        for (int ob = 0; ob < 8; ++ob) {
          const uint16_t* arow = wl + (16 * ob + t) * WROW + j * D + 8 * q;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(arow + 32 * ks);
            acc[ob] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, cur.gin[j][ks], acc[ob], 0, 0, 0);
          }
          // keep one block's weight fragments live at a time
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (LR) {
        // rank part: t as bf16 high + low parts, its own accumulator, added at the end
        bf16x8_t thi[NT], tlo[NT];
#pragma unroll
        for (int ks = 0; ks < NT; ++ks) {
          const float4 a = cur.tv[ks][0], b = cur.tv[ks][1];
          const float tv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            const uint32_t hw = pack_bf16x2(tv[i], tv[i + 1]);
            const uint32_t lw = pack_bf16x2(tv[i] - lo_bf16(hw), tv[i + 1] - hi_bf16(hw));
            thi[ks][i] = (short)(hw & 0xFFFFu);
            thi[ks][i + 1] = (short)(hw >> 16);
            tlo[ks][i] = (short)(lw & 0xFFFFu);
            tlo[ks][i + 1] = (short)(lw >> 16);
          }
        }
        const int rsteps = (p.r + 31) / 32;
#pragma unroll
        for (int ob = 0; ob < 8; ++ob) {
          f32x4_t au = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int ks = 0; ks < NT; ++ks) {
            if (ks < rsteps) {
              const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(ul + (16 * ob + t) * URW + 32 * ks + 8 * q);
              au = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, thi[ks], au, 0, 0, 0);
              au = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, tlo[ks], au, 0, 0, 0);
            }
          }
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) pred[4 * ob + s2] = acc[ob][s2] + au[s2];
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int ob = 0; ob < 8; ++ob)
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) pred[4 * ob + s2] = acc[ob][s2];
      }
      if constexpr (PM == PM_TEMPORAL_V) {
        uint4 e0[4];
        to_quarter(cur.ev[0], e0);
        const float* ca = p.ca + h * D + 32 * q;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v0 = e0[i];
          const float4 ca0 = *reinterpret_cast<const float4*>(ca + 8 * i);
          const float4 ca1 = *reinterpret_cast<const float4*>(ca + 8 * i + 4);
          const float av[8] = {ca0.x, ca0.y, ca0.z, ca0.w, ca1.x, ca1.y, ca1.z, ca1.w};
          const uint32_t a0[4] = {v0.x, v0.y, v0.z, v0.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float b0 = av[2 * k] * lo_bf16(a0[k]), b1 = av[2 * k + 1] * hi_bf16(a0[k]);
            pred[8 * i + 2 * k] = pred[8 * i + 2 * k] + b0;
            pred[8 * i + 2 * k + 1] = pred[8 * i + 2 * k + 1] + b1;
          }
        }
      }
    }
    const int64_t orow = ((int64_t)(live ? n : 0) * p.H + h) * D + 32 * q;   // [n][H][D]
    if (live && p.pred) {
#pragma unroll
      for (int i = 0; i < 32; i += 4)
        *reinterpret_cast<float4*>(p.pred + orow + i) = make_float4(pred[i], pred[i + 1], pred[i + 2], pred[i + 3]);
    }
    if (p.x) {
      uint32_t words[LW], szw[NGL];
      uint4 rq[4];   // reconstructed quarter row (bf16)
#pragma unroll
      for (int gi = 0; gi < NGL; ++gi) {
        float r[GL];
#pragma unroll
        for (int i = 0; i < GL / 8; ++i) {
          const uint4 xw = xv[(GL * gi) / 8 + i];
          const uint32_t xa[4] = {xw.x, xw.y, xw.z, xw.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int c = GL * gi + 8 * i + 2 * k;
            r[8 * i + 2 * k] = lo_bf16(xa[k]) - pred[c];
            r[8 * i + 2 * k + 1] = hi_bf16(xa[k]) - pred[c + 1];
          }
        }
        if (p.rot) hn_rotate_lane<GL>(r, p.rot, q);   // the rotated residual is quantized
        uint32_t cw[GL * BITS / 32];
        GroupQ gq;
        if constexpr (G == 64) {
          // the group spans this lane and lane ^ 16: combine min and max first
          float mn = r[0], mx = r[0];
#pragma unroll
          for (int i = 1; i < GL; ++i) { mn = fminf(mn, r[i]); mx = fmaxf(mx, r[i]); }
          mn = fminf(mn, __shfl_xor(mn, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          gq = quantize_with<BITS, GL>(r, mn, mx, cw);
        } else {
          gq = quantize_group<BITS, GL>(r, cw);
        }
        szw[gi] = gq.word;
#pragma unroll
        for (int w = 0; w < GL * BITS / 32; ++w) words[gi * (GL * BITS / 32) + w] = cw[w];
        if (p.recon) {
          float dq[GL];   // dequantized residual, rotated back when the codec rotates
#pragma unroll
          for (int i = 0; i < GL; ++i) dq[i] = dequant_one(group_code<BITS, GL>(cw, i), gq.s, gq.z);
          if (p.rot) hn_rotate_lane<GL>(dq, p.rot, q);
#pragma unroll
          for (int i = 0; i < GL; i += 8) {
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int i0 = i + 2 * k;
              const float v0 = pred[GL * gi + i0] + dq[i0];
              const float v1 = pred[GL * gi + i0 + 1] + dq[i0 + 1];
              o[k] = pack_bf16x2(v0, v1);
            }
            rq[(GL * gi + i) / 8] = make_uint4(o[0], o[1], o[2], o[3]);
          }
        }
      }
      if (p.recon) {
        // quarter rows -> whole rows through the staging tile, stored 1 KB at a time
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<uint4*>(&stg[8 * stg_slot(t, 4 * q + i)]) = rq[i];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = *reinterpret_cast<const uint4*>(&stg[8 * stg_slot(4 * i + ct, cc)]);
          const int nc = tile * 16 + 4 * i + ct;
          if (nc < p.n) *reinterpret_cast<uint4*>(p.recon + ((int64_t)nc * p.H + h) * D + 8 * cc) = v;
        }
        __builtin_amdgcn_wave_barrier();
      }
      if (live) {
        const int64_t row = (int64_t)h * p.capacity + p.token_offset + n;
        uint32_t* cd = p.codes + row * (4 * LW) + LW * q;
        if constexpr (LW == 4) *reinterpret_cast<uint4*>(cd) = make_uint4(words[0], words[1], words[2], words[3]);
        else *reinterpret_cast<uint2*>(cd) = make_uint2(words[0], words[1]);
        uint32_t* sd = p.sz + row * (D / G);
        if constexpr (G == 16) *reinterpret_cast<uint2*>(sd + 2 * q) = make_uint2(szw[0], szw[1]);
        else if constexpr (G == 32) sd[q] = szw[0];
        else if ((q & 1) == 0) sd[q >> 1] = szw[0];
      }
    }
    cur = nxt;
  }
}

// Persistent grid: as many workgroups as are resident at once (the kernel's register and
// LDS use decide how many per CU), matrix modes split evenly over the heads.
template <int BITS, int G, int PM, int NIN>
hipError_t launch_pred_t(PredParams p, size_t lds, hipStream_t s) {
  auto k = pred_kernel<BITS, G, PM, NIN>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  int occ = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(k), 512, lds);
  if (e != hipSuccess) return e;
  const int64_t resident = (int64_t)std::max(1, occ) * cu_count();
  const int64_t tiles = (p.n + 15) / 16;
  int grid;
  if (PM == PM_DPLR || PM == PM_TEMPORAL_V) {
    const int64_t per_head = (tiles + 7) / 8;
    p.segs = (int)std::max<int64_t>(1, std::min<int64_t>(per_head, resident / p.H));
    grid = p.segs * p.H;
  } else {
    grid = (int)std::max<int64_t>(1, std::min<int64_t>((tiles * p.H + 7) / 8, resident));
    p.segs = grid;
  }
  hipLaunchKernelGGL(k, dim3(grid), dim3(512), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_rank(const EncodeLaunch& a, float* t, hipStream_t s) {
  RankParams r{};
  r.in0 = reinterpret_cast<const uint16_t*>(a.b.prev0);
  r.in1 = reinterpret_cast<const uint16_t*>(a.b.prev1);
  r.ps = a.b.prev_stride;
  r.vlr = reinterpret_cast<const uint16_t*>(a.b.v_lr);
  r.t = t;
  r.n = (int)a.n_tokens;
  r.r = a.c.rank;
  r.hd = a.c.H * D;
  r.nin = a.c.n_inputs;
  const dim3 grid((unsigned)((a.n_tokens + RK_TOK - 1) / RK_TOK));
  if (r.r <= 32) hipLaunchKernelGGL(rank_kernel<2>, grid, dim3(512), 0, s, r);
  else hipLaunchKernelGGL(rank_kernel<4>, grid, dim3(512), 0, s, r);
  return hipGetLastError();
}

// Which fused mode a call maps to (-1: none).
int fused_mode(const EncodeLaunch& a) {
  const CodecArgs& c = a.c;
  if (c.x_dtype != KVC_BF16 || c.D != D || a.n_tokens >= (1ll << 31)) return -1;
  if ((a.b.prev_stride % 8) != 0) return -1;
  switch (c.base) {
    case KVC_BASE_NONE: return PM_NONE;
    case KVC_BASE_TEMPORAL: return a.b.w_block ? PM_TEMPORAL_V : PM_TEMPORAL_K;
    case KVC_BASE_DPLR:
      if (c.rank % 16 != 0 || c.rank > 64 || c.n_inputs < 1 || c.n_inputs > 2) return -1;
      return PM_DPLR;
    default: return -1;
  }
}

size_t lds_bytes(int mode, int nin, int r) {
  (void)r;
  size_t b = (size_t)8 * STG * 2;   // staging tiles
  if (mode == PM_DPLR || mode == PM_TEMPORAL_V) b += (size_t)w_elems(nin) * 2;
  if (mode == PM_DPLR) b += (size_t)128 * URW * 2;
  return b;
}

PredParams make_params(const EncodeLaunch& a, int mode, float* pred) {
  PredParams p{};
  p.x = reinterpret_cast<const uint16_t*>(a.x);
  p.x_stride = a.x_stride;
  p.ps = a.b.prev_stride;
  if (mode == PM_DPLR) {
    p.g0 = reinterpret_cast<const uint16_t*>(a.b.prev0);
    p.g1 = reinterpret_cast<const uint16_t*>(a.b.prev1);
    p.u = reinterpret_cast<const uint16_t*>(a.b.u);
    p.t = rank_intermediate(a);
  } else if (mode == PM_TEMPORAL_V) {
    p.g0 = reinterpret_cast<const uint16_t*>(a.b.aux);
    p.e0 = reinterpret_cast<const uint16_t*>(a.b.prev0);
  } else if (mode == PM_TEMPORAL_K) {
    p.e0 = reinterpret_cast<const uint16_t*>(a.b.prev0);
    p.e1 = reinterpret_cast<const uint16_t*>(a.b.prev1);
  }
  p.w = reinterpret_cast<const uint16_t*>(a.b.w_block);
  p.ca = a.b.coef_a;
  p.cb = a.b.coef_b;
  p.n = (int)a.n_tokens;
  p.H = a.c.H;
  p.r = a.c.rank;
  p.token_offset = a.token_offset;
  p.capacity = a.st.capacity;
  p.codes = a.st.codes;
  p.sz = a.st.sz;
  p.recon = reinterpret_cast<uint16_t*>(a.recon);
  p.pred = pred;
  p.rot = a.c.rot;
  p.segs = 1;   // set at launch
  return p;
}


// One dispatch for the encoder and the decoder's prediction, so the two always run the
// same instantiation on the same calls.
hipError_t dispatch(const EncodeLaunch& a, int mode, const PredParams& p, hipStream_t s) {
  const int bits = a.c.bits, g = a.c.group;
  // the temporal value map has one matrix input whatever n_inputs says
  const size_t lds = lds_bytes(mode, mode == PM_DPLR ? a.c.n_inputs : 1, a.c.rank);
#define KVC_PRED(B, G_, M, N)                                                       \
  if (bits == B && g == G_ && mode == M && (M != PM_DPLR || a.c.n_inputs == N))   \
    return launch_pred_t<B, G_, M, N>(p, lds, s);
#define KVC_PRED_ALL(B, G_)                                                        \
  KVC_PRED(B, G_, PM_NONE, 1) KVC_PRED(B, G_, PM_TEMPORAL_K, 1)                    \
  KVC_PRED(B, G_, PM_TEMPORAL_V, 1) KVC_PRED(B, G_, PM_DPLR, 1) KVC_PRED(B, G_, PM_DPLR, 2)
  KVC_PRED_ALL(2, 16) KVC_PRED_ALL(2, 32) KVC_PRED_ALL(2, 64)
  KVC_PRED_ALL(4, 16) KVC_PRED_ALL(4, 32) KVC_PRED_ALL(4, 64)
#undef KVC_PRED_ALL
#undef KVC_PRED
  return hipErrorInvalidValue;
}

bool fused_codec(const EncodeLaunch& a) {
  const int bits = a.c.bits, g = a.c.group;
  return (bits == 2 || bits == 4) && (g == 16 || g == 32 || g == 64);
}

}  // namespace

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

bool encode_fused_shape(const EncodeLaunch& a) {
  return fused_mode(a) >= 0 && fused_codec(a) && a.x_stride % 8 == 0;
}

bool launch_encode_fused(const EncodeLaunch& a, hipStream_t s, hipError_t* err) {
  const int mode = fused_mode(a);
  if (!encode_fused_shape(a)) return false;
  if (a.n_tokens == 0) { *err = hipSuccess; return true; }
  if (mode == PM_DPLR) {
    float* t = rank_intermediate(a);
    const hipError_t e = launch_rank(a, t, s);
    if (e != hipSuccess) { *err = e; return true; }
  }
  *err = dispatch(a, mode, make_params(a, mode, a.pred), s);
  return true;
}

bool launch_predict_fused(const EncodeLaunch& a, float* out, hipStream_t s, hipError_t* err) {
  const int mode = fused_mode(a);
  if ((mode != PM_DPLR && mode != PM_TEMPORAL_V) || !fused_codec(a)) return false;
  if (a.n_tokens == 0) { *err = hipSuccess; return true; }
  if (mode == PM_DPLR) {
    float* t = rank_intermediate(a);
    const hipError_t e = launch_rank(a, t, s);
    if (e != hipSuccess) { *err = e; return true; }
  }
  PredParams p = make_params(a, mode, out);
  p.x = nullptr;   // prediction only
  *err = dispatch(a, mode, p, s);
  return true;
}

}  // namespace kvc
