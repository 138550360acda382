// Encode: base formation, residual, group scale/zero, quantize, pack.
//
// Method (Coral-KV arXiv 2610.12514 abstract and Fig. 2c: cluster-based bases and
// quantized residual errors; Fig. 5c: one shared scale per group of values;
// TempoKV arXiv 2610.15324 Fig. 2b: temporal prediction of keys; NanoKV abstract:
// low-bit coefficients of the centroid residual).
//
// One workgroup (256 threads, 4 wave64) owns a tile of 64 tokens of one head.
//  1. the x tile is staged in LDS as fp32;
//  2. centroid bases: every (token, centroid) squared distance is summed in fp32 in
//     ascending channel order (one lane per token, one wave per centroid residue
//     class, centroid rows broadcast from LDS), ties to the lowest index;
//  3. coefficient bases: c_j = sum_i B_ij r_i in fp32, ascending i;
//  4. one thread per (token, group): min/max, fp16 scale/zero, codes, packing and a
//     coalesced store of the head-major code rows.
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int TOK = 64;       // tokens per workgroup
constexpr int CCHUNK = 128;   // centroid rows staged in LDS at a time
constexpr int NTHREADS = 256;

enum BaseMode { MODE_NONE = 0, MODE_CENTROID = 1, MODE_COEFF = 2, MODE_TEMPORAL_K = 3,
                MODE_BUFFER = 4 };

struct EncodeParams {
  const void* x;
  int64_t n_tokens, x_stride, token_offset, capacity;
  int H, C, bits, group, groups, code_words, vec_len, m, index_bytes, mode;
  const void* centroids;
  const uint16_t* basis;   // [D][m] bf16
  const void* prev0;
  const void* prev1;
  int64_t prev_stride;
  const float* coef_a;
  const float* coef_b;
  const float* base_buf;   // MODE_BUFFER: fp32 [N][H][D]
  uint32_t* codes;
  uint32_t* sz;
  void* index;
  void* recon;
  float* pred;
  // a second tensor encoded by the same launch (the keys and the values of a chunk):
  // its input, centroid table and store; same codec, token count, stride and offset
  int pair;
  const void* x2;
  const void* centroids2;
  uint32_t* codes2;
  uint32_t* sz2;
  void* index2;
  int64_t capacity2;
  int index_only;   // encode_c16_kernel: store the centroid index only
};

template <typename XT, int D>
__global__ __launch_bounds__(NTHREADS) void encode_kernel(EncodeParams p) {
  __shared__ float xs[TOK][D + 1];
  __shared__ XT cs[CCHUNK][D];
  __shared__ float bd[NTHREADS / 64][TOK];
  __shared__ int bi[NTHREADS / 64][TOK];
  __shared__ int aidx[TOK];
  __shared__ float cbuf[TOK][17];   // coefficients (m <= 16)

  const int tid = threadIdx.x;
  const int ntiles = (int)((p.n_tokens + TOK - 1) / TOK);
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int h = tile / ntiles;
  const int64_t n0 = (int64_t)(tile % ntiles) * TOK;
  const XT* x = reinterpret_cast<const XT*>(p.x);

  // 1. stage x tile
  for (int e = tid; e < TOK * D; e += NTHREADS) {
    int t = e / D, i = e % D;
    int64_t n = n0 + t;
    xs[t][i] = (n < p.n_tokens) ? load_x<XT>(x + n * p.x_stride + (int64_t)h * D + i) : 0.0f;
  }
  __syncthreads();

  const XT* cen = reinterpret_cast<const XT*>(p.centroids) + (int64_t)h * p.C * D;

  // 2. nearest centroid
  if (p.mode == MODE_CENTROID || p.mode == MODE_COEFF) {
    const int lane = tid & 63, w = tid >> 6;
    float xr[D];
#pragma unroll
    for (int i = 0; i < D; ++i) xr[i] = xs[lane][i];
    float best = __builtin_inff();
    int besti = 0;
    for (int c0 = 0; c0 < p.C; c0 += CCHUNK) {
      const int nc = min(CCHUNK, p.C - c0);
      __syncthreads();
      {
        // 16-byte vector copy of rows c0..c0+nc
        const int4* src = reinterpret_cast<const int4*>(cen + (int64_t)c0 * D);
        int4* dst = reinterpret_cast<int4*>(&cs[0][0]);
        const int nvec = nc * D * (int)sizeof(XT) / 16;
        for (int e = tid; e < nvec; e += NTHREADS) dst[e] = src[e];
      }
      __syncthreads();
      for (int j = w; j < nc; j += NTHREADS / 64) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < D; ++i) {
          float t = xr[i] - load_x<XT>(&cs[j][i]);
          float t2 = t * t;
          acc = acc + t2;
        }
        if (acc < best) { best = acc; besti = c0 + j; }
      }
    }
    bd[w][lane] = best;
    bi[w][lane] = besti;
    __syncthreads();
    if (tid < TOK) {
      float d = bd[0][tid];
      int ii = bi[0][tid];
#pragma unroll
      for (int ww = 1; ww < NTHREADS / 64; ++ww) {
        float d2 = bd[ww][tid];
        int i2 = bi[ww][tid];
        if (d2 < d || (d2 == d && i2 < ii)) { d = d2; ii = i2; }
      }
      aidx[tid] = ii;
      int64_t n = n0 + tid;
      if (n < p.n_tokens) {
        int64_t row = (int64_t)h * p.capacity + p.token_offset + n;
        if (p.index_bytes == 1) reinterpret_cast<uint8_t*>(p.index)[row] = (uint8_t)ii;
        else reinterpret_cast<uint16_t*>(p.index)[row] = (uint16_t)ii;
      }
    }
    __syncthreads();
  }

  // 3. coefficients of the centroid residual
  if (p.mode == MODE_COEFF) {
    for (int e = tid; e < TOK * p.m; e += NTHREADS) {
      int t = e / p.m, j = e % p.m;
      const XT* crow = cen + (int64_t)aidx[t] * D;
      float acc = 0.0f;
      for (int i = 0; i < D; ++i) {
        float r = xs[t][i] - load_x<XT>(crow + i);
        float b = bf16_bits_to_f32(p.basis[i * p.m + j]);
        float prod = r * b;
        acc = acc + prod;
      }
      cbuf[t][j] = acc;
    }
    __syncthreads();
  }

  // 4. quantize + pack, one thread per (token, group)
  const int levels = (1 << p.bits) - 1;
  const int per_word = 32 / p.bits;
  const int g = p.group;
  for (int item = tid; item < TOK * p.groups; item += NTHREADS) {
    const int t = item / p.groups, gi = item % p.groups;
    const int64_t n = n0 + t;
    if (n >= p.n_tokens) continue;
    const int i0 = gi * g;
    const XT* crow = (p.mode == MODE_CENTROID) ? cen + (int64_t)aidx[t] * D : nullptr;
    const XT* p0 = reinterpret_cast<const XT*>(p.prev0);
    const XT* p1 = reinterpret_cast<const XT*>(p.prev1);
    const int64_t prow = n * p.prev_stride + (int64_t)h * D;
    const int64_t xrow = (n * p.H + h) * (int64_t)D;   // [N][H][D] dense outputs

    auto base_at = [&](int i) -> float {
      switch (p.mode) {
        case MODE_CENTROID: return load_x<XT>(crow + i);
        case MODE_TEMPORAL_K: {
          float a = p.coef_a[h * D + i] * load_x<XT>(p0 + prow + i);
          float b = p.coef_b[h * D + i] * load_x<XT>(p1 + prow + i);
          return a + b;
        }
        case MODE_BUFFER: return p.base_buf[xrow + i];
        default: return 0.0f;
      }
    };
    auto value_at = [&](int i) -> float {
      if (p.mode == MODE_COEFF) return cbuf[t][i];
      float b = base_at(i);
      return xs[t][i] - b;
    };

    float mn = __builtin_inff(), mx = -__builtin_inff();
    for (int i = 0; i < g; ++i) {
      float r = value_at(i0 + i);
      mn = fminf(mn, r);
      mx = fmaxf(mx, r);
    }
    GroupQ q = group_scale_zero(mn, mx, levels);
    const int64_t row = (int64_t)h * p.capacity + p.token_offset + n;
    p.sz[row * p.groups + gi] = q.word;
    const int words = g / per_word;
    for (int wd = 0; wd < words; ++wd) {
      uint32_t word = 0;
      for (int k = 0; k < per_word; ++k) {
        int i = i0 + wd * per_word + k;
        float r = value_at(i);
        uint32_t code = quantize_one(r, q, levels);
        word |= code << (p.bits * k);
        if (p.mode != MODE_COEFF && (p.recon || p.pred)) {
          float b = base_at(i);
          if (p.pred) p.pred[xrow + i] = b;
          if (p.recon) {
            float xh = b + dequant_one(code, q.s, q.z);
            store_x<XT>(reinterpret_cast<XT*>(p.recon) + xrow + i, xh);
          }
        }
      }
      p.codes[row * p.code_words + (i0 / per_word) + wd] = word;
    }
  }
}

// ---------------------------------------------------------------------------
// Nearest centroid with an MFMA shortlist (bf16, d = 128).
//
// x . c_j for every centroid runs on v_mfma_f32_32x32x16_bf16 (bf16 products are
// exact; fp32 accumulation).  With n_j = ||c_j||^2 and the token norm, the expanded
// distance A_j = n_j - 2 x.c_j differs from the exact D_j - ||x||^2 by at most
// E_j = 2 (d + 4) u (n_j + 2 ||x|| ||c_j||), u = 2^-24 (both sums carry at most d
// rounding errors of relative size u; the factor 2 is slack).  U = min_j (A_j + E_j)
// bounds the best exact distance from above; every centroid whose lower bound
// A_j - E_j lies within U + 8 (d + 4) u (|U| + ||x||^2) - a margin covering the
// oracle's own fp32 rounding of the direct-form sums - is rescored with exactly
// the oracle's arithmetic (fp32, ascending channels, ties to the lowest index).
// Every centroid outside that set is provably farther in the oracle's arithmetic,
// so the index equals the oracle's bit for bit.
// ---------------------------------------------------------------------------
template <int TOK>
__global__ __launch_bounds__(NTHREADS, 1) void encode_shortlist_kernel(EncodeParams p) {
  constexpr int D = 128;
  constexpr int XROW = D + 8;                 // bf16 elements per staged token row
  constexpr int CCH = 256;                    // centroid rows per staged chunk
  constexpr int CROW = D + 8;
  constexpr int CMAX = TOK == 64 ? 256 : 512;
  constexpr int SROW = CMAX + 1;              // fp32 expanded distances per token
  constexpr int PARTS = NTHREADS / TOK;       // threads cooperating on one token
  __shared__ __attribute__((aligned(16))) uint16_t xs[TOK * XROW];
  __shared__ __attribute__((aligned(16))) uint16_t ct[CCH * CROW];
  __shared__ float sm[TOK * SROW];
  __shared__ float cn2[CMAX], cn1[CMAX];
  __shared__ float xn2[TOK], xn1[TOK];
  __shared__ int aidx[TOK];
  // after the argmin the distance buffer holds the coefficients and the chosen rows
  float (*cbuf)[17] = reinterpret_cast<float (*)[17]>(sm);
  uint16_t* brow = reinterpret_cast<uint16_t*>(sm + TOK * 17);   // [TOK][XROW] bf16

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntiles = (int)((p.n_tokens + TOK - 1) / TOK);
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int h = tile / ntiles;
  const int64_t n0 = (int64_t)(tile % ntiles) * TOK;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(p.x);
  const uint16_t* cen = reinterpret_cast<const uint16_t*>(p.centroids) + (int64_t)h * p.C * D;

  // 1. token tile (16-byte rows pieces), zero rows past the end
  for (int e = tid; e < TOK * (D / 8); e += NTHREADS) {
    const int t = e / (D / 8), c = e % (D / 8);
    const int64_t n = n0 + t;
    uint4 v = {0u, 0u, 0u, 0u};
    if (n < p.n_tokens) v = *reinterpret_cast<const uint4*>(x + n * p.x_stride + (int64_t)h * D + 8 * c);
    *reinterpret_cast<uint4*>(&xs[t * XROW + 8 * c]) = v;
  }
  __syncthreads();
  // squared norm of a staged bf16 row (any order: it only feeds the error bound)
  auto row_norm2 = [](const uint16_t* row) {
    float s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < D; i += 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + i);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lo = bf16_bits_to_f32(w[k] & 0xFFFFu), hi = bf16_bits_to_f32(w[k] >> 16);
        s2 = __builtin_fmaf(lo, lo, s2);
        s2 = __builtin_fmaf(hi, hi, s2);
      }
    }
    return s2;
  };
  if (tid < TOK) {
    const float s2 = row_norm2(&xs[tid * XROW]);
    xn2[tid] = s2;
    xn1[tid] = sqrtf(s2);
  }

  // 2. expanded distances, one staged chunk of centroids at a time
  const int col = lane & 31, half = lane >> 5;
  int last_c0 = 0, last_nc = 0;
  for (int c0 = 0; c0 < p.C; c0 += CCH) {
    const int nc = min(CCH, p.C - c0);
    __syncthreads();
    for (int e = tid; e < CCH * (D / 8); e += NTHREADS) {
      const int j = e / (D / 8), c = e % (D / 8);
      uint4 v = {0u, 0u, 0u, 0u};
      if (j < nc) v = *reinterpret_cast<const uint4*>(cen + (int64_t)(c0 + j) * D + 8 * c);
      *reinterpret_cast<uint4*>(&ct[j * CROW + 8 * c]) = v;
    }
    __syncthreads();
    for (int j = tid; j < nc; j += NTHREADS) {
      const float s2 = row_norm2(&ct[j * CROW]);
      cn2[c0 + j] = s2;
      cn1[c0 + j] = sqrtf(s2);
    }
    __syncthreads();
    constexpr int NB = (TOK / 32) * (CCH / 32);      // 32x32 output blocks
    for (int b = wave; b < NB; b += NTHREADS / 64) {
      const int tb = b / (CCH / 32), cb = b % (CCH / 32);
      if (cb * 32 >= nc) continue;
      f32x16_t acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&xs[(32 * tb + col) * XROW + 16 * ks + 8 * half]);
        const bf16x8_t bb = *reinterpret_cast<const bf16x8_t*>(&ct[(32 * cb + col) * CROW + 16 * ks + 8 * half]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc, 0, 0, 0);
      }
      const int j = 32 * cb + col;
      if (j < nc) {
        const float nj = cn2[c0 + j];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = 32 * tb + 8 * (r >> 2) + 4 * half + (r & 3);
          sm[t * SROW + c0 + j] = nj - 2.0f * acc[r];
        }
      }
    }
    last_c0 = c0;
    last_nc = nc;
  }
  __syncthreads();

  // 3. shortlist bound per token: PARTS consecutive lanes share a token, each owning a
  //    contiguous run of SPAN centroids read as 16-byte LDS vectors
  constexpr int SPAN = CMAX / PARTS;     // 64 in both configurations
  const int t = tid / PARTS, q = tid % PARTS;
  const int j0 = q * SPAN;
  const float g = 2.0f * (float)(D + 4) * 5.9604645e-8f;   // 2 (d + 4) 2^-24
  const float xn2x = 2.0f * xn1[t], xx = xn2[t];
  float lbv[SPAN];
  float ub = __builtin_inff();
#pragma unroll
  for (int i = 0; i < SPAN; i += 4) {
    const float4 a4 = *reinterpret_cast<const float4*>(&sm[t * SROW + j0 + i]);
    const float4 n2 = *reinterpret_cast<const float4*>(&cn2[j0 + i]);
    const float4 n1 = *reinterpret_cast<const float4*>(&cn1[j0 + i]);
    const float av[4] = {a4.x, a4.y, a4.z, a4.w}, nv2[4] = {n2.x, n2.y, n2.z, n2.w},
                nv1[4] = {n1.x, n1.y, n1.z, n1.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool valid = j0 + i + k < p.C;
      const float e = g * __builtin_fmaf(xn2x, nv1[k], nv2[k]);
      ub = valid ? fminf(ub, av[k] + e) : ub;
      lbv[i + k] = valid ? av[k] - e : __builtin_inff();
    }
  }
#pragma unroll
  for (int o = 1; o < PARTS; o <<= 1) ub = fminf(ub, __shfl_xor(ub, o));
  const float T = ub + 4.0f * g * (fabsf(ub) + xx);
  uint64_t cand = 0;
#pragma unroll
  for (int i = 0; i < SPAN; ++i) cand |= (uint64_t)(lbv[i] <= T) << i;

  // 4. exact rescoring of the shortlist (the oracle's fp32 direct form), ascending j
  float best = __builtin_inff();
  int bestj = 0x7FFFFFFF;
  while (cand) {
    const int i = __builtin_ctzll(cand);
    cand &= cand - 1;
    const int j = j0 + i;
    const bool resident = j >= last_c0 && j < last_c0 + last_nc;
    const uint16_t* crow = resident ? &ct[(j - last_c0) * CROW] : cen + (int64_t)j * D;
    float acc = 0.0f;
    for (int ii = 0; ii < D; ii += 8) {
      const uint4 xv = *reinterpret_cast<const uint4*>(&xs[t * XROW + ii]);
      const uint4 cv = *reinterpret_cast<const uint4*>(crow + ii);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, cw[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float d0 = bf16_bits_to_f32(xw[k] & 0xFFFFu) - bf16_bits_to_f32(cw[k] & 0xFFFFu);
        float sq0 = d0 * d0;
        acc = acc + sq0;
        float d1 = bf16_bits_to_f32(xw[k] >> 16) - bf16_bits_to_f32(cw[k] >> 16);
        float sq1 = d1 * d1;
        acc = acc + sq1;
      }
    }
    if (acc < best) { best = acc; bestj = j; }   // ascending j: first minimum wins ties
  }
#pragma unroll
  for (int o = 1; o < PARTS; o <<= 1) {
    const float ob = __shfl_xor(best, o);
    const int oj = __shfl_xor(bestj, o);
    if (ob < best || (ob == best && oj < bestj)) { best = ob; bestj = oj; }
  }
  if (q == 0) {
    aidx[t] = bestj;
    const int64_t n = n0 + t;
    if (n < p.n_tokens) {
      const int64_t row = (int64_t)h * p.capacity + p.token_offset + n;
      if (p.index_bytes == 1) reinterpret_cast<uint8_t*>(p.index)[row] = (uint8_t)bestj;
      else reinterpret_cast<uint16_t*>(p.index)[row] = (uint16_t)bestj;
    }
  }
  __syncthreads();
  // stage each token's centroid row (16-byte pieces)
  for (int e = tid; e < TOK * (D / 8); e += NTHREADS) {
    const int tt = e / (D / 8), c = e % (D / 8);
    *reinterpret_cast<uint4*>(&brow[tt * XROW + 8 * c]) =
        *reinterpret_cast<const uint4*>(cen + (int64_t)aidx[tt] * D + 8 * c);
  }
  __syncthreads();

  // 5. coefficients of the centroid residual (fp32, ascending channels)
  if (p.mode == MODE_COEFF) {
    for (int e = tid; e < TOK * p.m; e += NTHREADS) {
      const int tt = e / p.m, j = e % p.m;
      const uint16_t* crow = &brow[tt * XROW];
      float acc = 0.0f;
      for (int i = 0; i < D; ++i) {
        const float r = bf16_bits_to_f32(xs[tt * XROW + i]) - bf16_bits_to_f32(crow[i]);
        const float b = bf16_bits_to_f32(p.basis[i * p.m + j]);
        const float prod = r * b;
        acc = acc + prod;
      }
      cbuf[tt][j] = acc;
    }
    __syncthreads();
  }

  // 6. quantize + pack, one thread per (token, group)
  const int levels = (1 << p.bits) - 1;
  const int per_word = 32 / p.bits;
  const int gsz = p.group;
  for (int item = tid; item < TOK * p.groups; item += NTHREADS) {
    const int tt = item / p.groups, gi = item % p.groups;
    const int64_t n = n0 + tt;
    if (n >= p.n_tokens) continue;
    const int i0 = gi * gsz;
    const uint16_t* crow = &brow[tt * XROW];
    const int64_t xrow = (n * p.H + h) * (int64_t)D;
    auto value_at = [&](int i) -> float {
      if (p.mode == MODE_COEFF) return cbuf[tt][i];
      return bf16_bits_to_f32(xs[tt * XROW + i]) - bf16_bits_to_f32(crow[i]);
    };
    float mn = __builtin_inff(), mx = -__builtin_inff();
    for (int i = 0; i < gsz; ++i) {
      const float r = value_at(i0 + i);
      mn = fminf(mn, r);
      mx = fmaxf(mx, r);
    }
    const GroupQ gq = group_scale_zero(mn, mx, levels);
    const int64_t row = (int64_t)h * p.capacity + p.token_offset + n;
    p.sz[row * p.groups + gi] = gq.word;
    const int words = gsz / per_word;
    for (int wd = 0; wd < words; ++wd) {
      uint32_t word = 0;
      for (int k = 0; k < per_word; ++k) {
        const int i = i0 + wd * per_word + k;
        const uint32_t code = quantize_one(value_at(i), gq, levels);
        word |= code << (p.bits * k);
        if (p.mode != MODE_COEFF && (p.recon || p.pred)) {
          const float bsv = bf16_bits_to_f32(crow[i]);
          if (p.pred) p.pred[xrow + i] = bsv;
          if (p.recon) {
            const float xh = bsv + dequant_one(code, gq.s, gq.z);
            reinterpret_cast<uint16_t*>(p.recon)[xrow + i] = (uint16_t)f32_to_bf16_bits(xh);
          }
        }
      }
      p.codes[row * p.code_words + (i0 / per_word) + wd] = word;
    }
  }
}

// ---------------------------------------------------------------------------
// Centroid and coefficient codecs for bf16 d = 128 data with at most CM (256 or 512)
// centroids per head.
//
// One wave encodes 32 tokens of one head at a time; lane (t, hf) owns channels 64 hf ..
// 64 hf + 63 of token t in registers.  The head's centroid table sits in LDS, loaded
// once per workgroup of NW waves (four, or eight when one workgroup fills the CU's LDS),
// which then walks the head's tiles of 32 NW tokens.
//
// Assignment.  v_j = x.c_j - |c_j|^2 / 2 comes out of v_mfma_f32_32x32x16_bf16
// (accumulator seeded with -|c_j|^2 / 2; the contraction index is permuted so that
// every lane feeds its own half row), one lane per (token, half) holding 128 of the
// CM values.  A lane keeps the top three of its values with the centroid's
// position packed into the low 8 (CM = 256) or 9 (CM = 512) mantissa bits (the
// position within the half replaces the low byte, the half bit goes above it), and
// merges them with its partner half.  With E >= |v_j - V_j| (the MFMA error, counted at two units in the last
// place per addition), g = (d + 3) 2^-24 the relative error of the exact fp32
// distance, and V the true values, d_j > d_w for the exact fp32 distances whenever
//     (v_w - v_j) - g (|x|^2 - v_w - v_j) > 2 E,
// since |x - c_j|^2 = |x|^2 - 2 V_j.  If that holds between the best and the second
// best value, the best centroid is the nearest one; if it holds between the best
// and the third, the nearest is one of the top two, and both are rescored in the
// exact fp32 order; otherwise every centroid the test cannot exclude is rescored.
// Ties in the exact distance go to the lower index.
//
// Coefficients (COEFF).  c_j = sum_i B_ij r_i over the full residual row in ascending
// i, multiply and add rounded separately; lane hf forms c_8hf .. c_8hf+7, and the m = 16
// coefficients are one quantization group spanning the two lanes.
//
// Quantization.  code = clamp(rint(fl(fl(r - z) / s))) is evaluated as
// rint(r * rcp(s) - z * rcp(s)); the two agree unless the product lies within
// (|z / s| + L + 2) 2^-19 of a half-integer, and a group with such an element is
// redone with the IEEE division.
// |lo|^2 + |hi|^2 + acc for a packed bf16 pair (v_dot2_f32_bf16; the products are
// exact in fp32).  Used only for norm bounds, which carry a relative slack of 2^-10.
__device__ __forceinline__ float sq2_bf16(uint32_t w, float acc) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 v = __builtin_bit_cast(bf2, w);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}

// waves per workgroup of the centroid codec: eight when the LDS allows one workgroup
// per CU (two waves per SIMD either way)
__host__ __device__ constexpr int cen_waves(int cm, bool coeff) { return (cm == 512 || coeff) ? 8 : 4; }

template <int BITS, int G, int CM, bool COEFF>
__global__ __launch_bounds__(64 * cen_waves(CM, COEFF), 2 * 4 / cen_waves(CM, COEFF)) void encode_centroid_kernel(EncodeParams p) {
  constexpr int D = 128, ROW = D + 8;
  constexpr int NW = cen_waves(CM, COEFF), NT = 64 * NW, TT = 32 * NW;   // waves, threads, tokens
  constexpr int NBM = CM / 32;                 // centroid blocks at most
  constexpr int LOCB = CM == 256 ? 7 : 8;      // bits of a value's position in a half
  constexpr uint32_t TAGM = (2u << LOCB) - 1u; // position + half bit
  constexpr float TSLACK = CM == 256 ? 0x1p-15f : 0x1p-14f;   // relative change by the tag
  constexpr int L = (1 << BITS) - 1;
  constexpr int NG = 64 / G;          // groups in a half row
  constexpr int PER = 32 / BITS;      // codes per word
  constexpr int WPL = 64 / PER;       // code words per half row
  constexpr int GW = G / PER;         // code words per group
  __shared__ __attribute__((aligned(16))) uint16_t tab[CM * ROW];
  __shared__ __attribute__((aligned(16))) float hn[CM];
  __shared__ float cnu[CM];   // |c_j| (upper bound), 0 beyond C
  __shared__ float wmax[NW];
  __shared__ uint32_t tq[NW][64];   // rescoring tasks of each wave: lane << 10 | centroid
  // per lane, the least (distance bits << 32 | centroid) of its tasks in a round
  __shared__ unsigned long long tres[NW][64];
  __shared__ __attribute__((aligned(16))) float bt[COEFF ? D * 16 : 4];   // basis [i][j], fp32

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = lane & 31, hf = lane >> 5;
  const int ntile = (int)((p.n_tokens + TT - 1) / TT);
  const int wph = (int)gridDim.x / p.H;   // workgroups per head
  const int b = xcd_remap(blockIdx.x, gridDim.x);
  const int h = b / wph, first = b % wph;
  const int C = p.C;
  const int nb = (C + 31) >> 5;
  const uint16_t* cen = reinterpret_cast<const uint16_t*>(p.centroids) + (int64_t)h * C * D;

  // this lane's half row of a tile's token (zeros past the last token); the first
  // tile's rows are requested before the table is staged, each next tile's while the
  // current one is encoded
  auto load_half_row = [&](int tl, uint4 (&dst)[8]) {
    const int64_t nn = (int64_t)tl * TT + wave * 32 + t;
    const bool lv = tl < ntile && nn < p.n_tokens;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(p.x) + (lv ? nn : 0) * p.x_stride +
                          (int64_t)h * D + 64 * hf;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dst[i] = lv ? *reinterpret_cast<const uint4*>(src + 8 * i) : make_uint4(0u, 0u, 0u, 0u);
  };
  uint4 xv[8];
  load_half_row(first, xv);

  // 1. the head's centroid table (rows C .. 32 nb - 1 zero), row norms, the basis
#pragma unroll
  for (int half16 = 0; half16 < (CM + NT - 1) / NT; ++half16) {   // rounds of 16 pieces a thread
    // sixteen 16-byte pieces of this thread in flight at once
    uint4 v[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int j = (NT / 16) * (16 * half16 + it) + (tid >> 4), c = tid & 15;
      v[it] = make_uint4(0u, 0u, 0u, 0u);
      if (j < C) v[it] = *reinterpret_cast<const uint4*>(cen + (int64_t)j * D + 8 * c);
    }
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int j = (NT / 16) * (16 * half16 + it) + (tid >> 4), c = tid & 15;
      if (j < 32 * nb) *reinterpret_cast<uint4*>(&tab[j * ROW + 8 * c]) = v[it];
    }
  }
  if constexpr (COEFF) {
    for (int e = tid; e < D * 16; e += NT) bt[e] = bf16_bits_to_f32(p.basis[e]);
  }
  __syncthreads();
  {
    float cnw = 0.0f;
#pragma unroll
    for (int jj = 0; jj < (CM + NT - 1) / NT; ++jj) {
      const int j = tid + NT * jj;
      if (j >= CM) break;
      float s2 = 0.0f;
      if (j < C) {
#pragma unroll
        for (int i = 0; i < D; i += 8) {
          const uint4 v = *reinterpret_cast<const uint4*>(&tab[j * ROW + i]);
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            s2 = sq2_bf16(w[k], s2);
          }
        }
      }
      hn[j] = j < C ? -0.5f * s2 : -1e30f;
      const float cn = sqrtf(s2) * (1.0f + 0x1p-10f);
      cnu[j] = cn;
      cnw = fmaxf(cnw, cn);
    }
#pragma unroll
    for (int o = 32; o; o >>= 1) cnw = fmaxf(cnw, __shfl_xor(cnw, o));
    if (lane == 0) wmax[wave] = cnw;
  }
  __syncthreads();
  float cmax = wmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) cmax = fmaxf(cmax, wmax[w]);

#pragma unroll 1
  for (int tile = first; tile < ntile; tile += wph) {
  const int64_t n = (int64_t)tile * TT + wave * 32 + t;
  const bool live = n < p.n_tokens;
  uint4 xnext[8];
  load_half_row(tile + wph, xnext);

  // 2. v_j for the 128 centroids of this half; top three with packed positions
  float m1 = -3.0e38f, m2 = -3.0e38f, m3 = -3.0e38f;
  auto block_values = [&](int cb, f32x16_t& acc) {
    const float4* hp = reinterpret_cast<const float4*>(&hn[32 * cb + 4 * hf]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = hp[2 * q];
      acc[4 * q] = v.x; acc[4 * q + 1] = v.y; acc[4 * q + 2] = v.z; acc[4 * q + 3] = v.w;
    }
    const uint16_t* arow = &tab[(32 * cb + t) * ROW + 64 * hf];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(arow + 8 * ks);
      bf16x8_t bx;
      __builtin_memcpy(&bx, &xv[ks], 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bx, acc, 0, 0, 0);
    }
  };
  auto top3 = [&](const f32x16_t& acc, int cb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // the position 16 cb + r (< 2^LOCB <= 256) replaces the low byte: one v_perm_b32
      const float pv = __uint_as_float(
          __builtin_amdgcn_perm(__float_as_uint(acc[r]), (uint32_t)(16 * cb + r), 0x07060500u));
      m3 = __builtin_amdgcn_fmed3f(m2, m3, pv);
      m2 = __builtin_amdgcn_fmed3f(m1, m2, pv);
      // max(m1, pv) for finite values, written as a median so that no canonicalizing
      // instruction is added for the tag-modified operand
      m1 = __builtin_amdgcn_fmed3f(m1, pv, 3.40282347e38f);
    }
  };
  // software-pipelined over the blocks: the MFMAs of block cb+1 are issued among the
  // top-three updates of block cb (two accumulators, the loop body one basic block)
  {
    f32x16_t acc0, acc1;
    block_values(0, acc0);
    int cb = 0;
    for (; cb + 2 < nb; cb += 2) {
      block_values(cb + 1, acc1);
      top3(acc0, cb);
      block_values(cb + 2, acc0);
      top3(acc1, cb + 1);
    }
    if (cb + 1 < nb) {
      block_values(cb + 1, acc1);
      top3(acc0, cb);
      top3(acc1, cb + 1);
    } else {
      top3(acc0, cb);
    }
  }
  // tag the half above the position bits, merge the two halves' top three
  auto half_tag = [&](float v) {   // bit LOCB := hf (for CM = 256 it is a tag bit, 0)
    return __uint_as_float((__float_as_uint(v) & ~(1u << LOCB)) | ((uint32_t)hf << LOCB));
  };
  m1 = half_tag(m1);
  m2 = half_tag(m2);
  m3 = half_tag(m3);
  auto swf = [&](float v) { return __uint_as_float(swap_halves(__float_as_uint(v), hf)); };
  const float b1 = swf(m1), b2 = swf(m2), b3 = swf(m3);
  const float t1 = fmaxf(m1, b1);
  const float t2 = fmaxf(fmaxf(m2, b2), fminf(m1, b1));
  const float t3 = fmaxf(fmaxf(m3, b3), fmaxf(fminf(m2, b1), fminf(m1, b2)));

  // |x|^2 (upper bound) and the separation test
  float xs = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      xs = sq2_bf16(w[k], xs);
    }
  }
  const float xxu = (xs + swf(xs)) * (1.0f + 0x1p-10f);
  const float xn = sqrtf(xxu) * (1.0f + 0x1p-10f);
  // error bound of one value v_j, from |c_j| (and E for any row: |c_j| <= cmax)
  auto erow = [&](float cj) {
    return (2.0f * (D + 2) * 0x1p-24f) * cj * (cj + xn) * (1.0f + 0x1p-10f) + 1e-30f;
  };
  const float E = erow(cmax);
  const float go = (D + 3) * 0x1p-24f * (1.0f + 0x1p-10f);
  // a (packed best) beats every centroid whose value is at most c, given the sum of
  // the two values' error bounds
  auto separated = [&](float a, float c, float esum) {
    const float va = a - TSLACK * fabsf(a), vc = c + TSLACK * fabsf(c);
    const float rhs = esum + go * (xxu - va - vc) + 0x1p-20f * (fabsf(va) + fabsf(vc) + xxu);
    return va - vc > rhs;
  };
  auto cidx = [](float v) {
    const uint32_t tg = __float_as_uint(v) & TAGM;
    const int hw = (int)(tg >> LOCB), loc = (int)(tg & (TAGM >> 1)), cb = loc >> 4, r = loc & 15;
    return 32 * cb + 8 * (r >> 2) + 4 * hw + (r & 3);
  };
  int best = cidx(t1);
  // with every error at its largest (E) most tokens are settled; the rest are
  // tested again with the row bounds of the best (and second) centroid
  bool uniq = !live || separated(t1, t2, 2.0f * E), pair = false;
  if (!uniq) {
    const float e1 = erow(cnu[best]), e2 = erow(cnu[cidx(t2)]);
    const bool beats_rest = separated(t1, t3, e1 + E);
    uniq = beats_rest && separated(t1, t2, e1 + e2);
    pair = beats_rest && !uniq;
  }

  // 3. exact rescoring: every (token, candidate) pair is a task in this wave's LDS
  //    queue; lane i computes task i in the exact fp32 order from the token's row
  if (__any(!uniq)) {
    uint32_t* q = &tq[wave][0];
    unsigned long long* rs = &tres[wave][0];
    int single = pair ? cidx(hf ? t2 : t1) : -1;   // one candidate per lane of a pair token
    uint32_t mask[NBM / 2];                         // bit 16 cb + r: candidate value of this lane
#pragma unroll
    for (int w = 0; w < NBM / 2; ++w) mask[w] = 0u;
    const bool full = !uniq && !pair;
    if (__any(full)) {
      // every value below tau is separated from the best one (the right-hand side of
      // the test grows far slower than the gap), so the values >= tau are a superset of
      // the centroids that can still be nearest; all of them are rescored
      const float va = t1 - TSLACK * fabsf(t1);
      const float tau = va - 2.0f * (2.0f * E + go * (xxu + 2.0f * fabsf(va)) +
                                     0x1p-20f * (2.0f * fabsf(va) + xxu) + 0x1p-14f * fabsf(va));
      for (int cb = 0; cb < nb; ++cb) {
        f32x16_t acc;
        block_values(cb, acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = 32 * cb + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (full && j < C && acc[r] >= tau) mask[cb >> 1] |= 1u << (16 * (cb & 1) + r);
        }
      }
    }
    const int64_t nw0 = n - t;   // first token of this wave
    float bd = __builtin_inff();
    int bj = 0x7FFFFFFF;
    // Task list without atomics: lane l's tasks (its `single` candidate, then its mask
    // bits in ascending order) take the consecutive slots from the exclusive prefix sum
    // of the lanes' task counts, 64 slots per round.  Each task lane folds its exact
    // distance into its owner lane's slot with a 64-bit LDS minimum on
    // (distance bits << 32 | centroid): distances are non-negative, so the bit order is
    // the numeric order, and equal distances go to the lower index.
    int cnt = single >= 0 ? 1 : 0;
#pragma unroll
    for (int w = 0; w < NBM / 2; ++w) cnt += __builtin_popcount(mask[w]);
    int off = cnt;   // inclusive prefix sum over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(off, d);
      if (lane >= d) off += o;
    }
    const int total = __shfl(off, 63);
    off -= cnt;
    for (int r0 = 0; r0 < total; r0 += 64) {
      rs[lane] = ~0ull;
      {
        int g = off;
        if (single >= 0) {
          if (g >= r0 && g < r0 + 64) q[g - r0] = ((uint32_t)lane << 10) | (uint32_t)single;
          ++g;
        }
        for (int w = 0; w < NBM / 2; ++w) {
          uint32_t m = mask[w];
          while (m) {
            const int bit = __builtin_ctz(m);
            m &= m - 1u;
            if (g >= r0 && g < r0 + 64) {
              const int cb = 2 * w + (bit >> 4), r = bit & 15;
              const int j = 32 * cb + 8 * (r >> 2) + 4 * hf + (r & 3);
              q[g - r0] = ((uint32_t)lane << 10) | (uint32_t)j;
            }
            ++g;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      const int ntask = min(total - r0, 64);
      if (lane < ntask) {
        const uint32_t tk = q[lane];
        const int j = (int)(tk & 0x3FFu);
        const int64_t nt = nw0 + (int)((tk >> 10) & 31u);
        const uint16_t* xr = reinterpret_cast<const uint16_t*>(p.x) + nt * p.x_stride + (int64_t)h * D;
        const uint16_t* crow = &tab[j * ROW];
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint4 xw = *reinterpret_cast<const uint4*>(xr + 8 * i);
          const uint4 cw = *reinterpret_cast<const uint4*>(crow + 8 * i);
          const uint32_t xa[4] = {xw.x, xw.y, xw.z, xw.w}, ca[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float d0 = lo_bf16(xa[k]) - lo_bf16(ca[k]);
            const float q0 = d0 * d0;
            acc = acc + q0;
            const float d1 = hi_bf16(xa[k]) - hi_bf16(ca[k]);
            const float q1 = d1 * d1;
            acc = acc + q1;
          }
        }
        atomicMin(&rs[tk >> 10], ((unsigned long long)__float_as_uint(acc) << 32) | (uint32_t)j);
      }
      __builtin_amdgcn_wave_barrier();
      const unsigned long long mine = rs[lane];
      if (mine != ~0ull) {
        const float d = __uint_as_float((uint32_t)(mine >> 32));
        const int j = (int)(uint32_t)mine;
        if (d < bd || (d == bd && j < bj)) { bd = d; bj = j; }
      }
      __builtin_amdgcn_wave_barrier();
    }
    const float od = swf(bd);
    const int oj = (int)swap_halves((uint32_t)bj, hf);
    if (!uniq) best = (od < bd || (od == bd && oj < bj)) ? oj : bj;
  }

  // 4. residual, group scale/zero, codes
  auto store_index = [&](int64_t row) {
    if (p.index_bytes == 2) reinterpret_cast<uint16_t*>(p.index)[row] = (uint16_t)best;
    else reinterpret_cast<uint8_t*>(p.index)[row] = (uint8_t)best;
  };
  if constexpr (COEFF) {
    // 4'. coefficients of the residual row; the partner's half of x by a lane swap
    uint4 xo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      xo[i] = make_uint4(swap_halves(xv[i].x, hf), swap_halves(xv[i].y, hf),
                         swap_halves(xv[i].z, hf), swap_halves(xv[i].w, hf));
    const uint16_t* crow = &tab[best * ROW];
    float cf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) cf[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {   // channels 8 k .. 8 k + 7, ascending
      const uint4 xw = ((k >> 3) == hf) ? xv[k & 7] : xo[k & 7];
      const uint4 cv = *reinterpret_cast<const uint4*>(crow + 8 * k);
      const uint32_t xa[4] = {xw.x, xw.y, xw.z, xw.w}, ca[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xe = (e & 1) ? hi_bf16(xa[e >> 1]) : lo_bf16(xa[e >> 1]);
        const float ce = (e & 1) ? hi_bf16(ca[e >> 1]) : lo_bf16(ca[e >> 1]);
        const float r = xe - ce;
        const float4 b0 = *reinterpret_cast<const float4*>(&bt[(8 * k + e) * 16 + 8 * hf]);
        const float4 b1 = *reinterpret_cast<const float4*>(&bt[(8 * k + e) * 16 + 8 * hf + 4]);
        const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float prod = r * bb[j];
          cf[j] = cf[j] + prod;
        }
      }
    }
    // one group of 16 across the two lanes
    float mn = cf[0], mx = cf[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) { mn = fminf(mn, cf[j]); mx = fmaxf(mx, cf[j]); }
    mn = fminf(mn, swf(mn));
    mx = fmaxf(mx, swf(mx));
    uint32_t cw[8 * BITS / 32];
    const GroupQ gq = quantize_with<BITS, 8>(cf, mn, mx, cw);
    if (live) {
      const int64_t row = (int64_t)h * p.capacity + p.token_offset + n;
      p.codes[row * 2 + hf] = cw[0];   // 16 INT4 codes: two words, one per lane
      if (hf == 0) {
        p.sz[row] = gq.word;
        store_index(row);
      }
    }
  } else {
  const uint16_t* crow = &tab[best * ROW + 64 * hf];
  uint32_t words[WPL], szw[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    float r[G];
#pragma unroll
    for (int i = 0; i < G / 8; ++i) {
      const uint4 cv = *reinterpret_cast<const uint4*>(crow + G * gi + 8 * i);
      const uint4 xw = xv[(G * gi) / 8 + i];
      const uint32_t xa[4] = {xw.x, xw.y, xw.z, xw.w}, ca[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        r[8 * i + 2 * k] = lo_bf16(xa[k]) - lo_bf16(ca[k]);
        r[8 * i + 2 * k + 1] = hi_bf16(xa[k]) - hi_bf16(ca[k]);
      }
    }
    uint32_t cw[GW];
    const GroupQ q = quantize_group<BITS, G>(r, cw);
    szw[gi] = q.word;
#pragma unroll
    for (int w = 0; w < GW; ++w) words[gi * GW + w] = cw[w];
    if (live && (p.recon || p.pred)) {
      const int64_t xrow = (n * p.H + h) * (int64_t)D + 64 * hf + G * gi;
      if (p.recon) {
        uint16_t* rec = reinterpret_cast<uint16_t*>(p.recon) + xrow;
#pragma unroll
        for (int i = 0; i < G; i += 8) {
          uint32_t o[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int i0 = i + 2 * k, i1 = i0 + 1;
            const uint32_t c0 = group_code<BITS, G>(cw, i0);
            const uint32_t c1 = group_code<BITS, G>(cw, i1);
            const uint32_t cw2 = crow[G * gi + i0] | ((uint32_t)crow[G * gi + i1] << 16);
            const float e0 = lo_bf16(cw2) + dequant_one(c0, q.s, q.z);
            const float e1 = hi_bf16(cw2) + dequant_one(c1, q.s, q.z);
            o[k] = pack_bf16x2(e0, e1);
          }
          *reinterpret_cast<uint4*>(rec + i) = make_uint4(o[0], o[1], o[2], o[3]);
        }
      }
      if (p.pred) {
        float* pd = p.pred + xrow;
#pragma unroll
        for (int i = 0; i < G; i += 4) {
          const uint2 cw2 = *reinterpret_cast<const uint2*>(crow + G * gi + i);
          *reinterpret_cast<float4*>(pd + i) =
              make_float4(lo_bf16(cw2.x), hi_bf16(cw2.x), lo_bf16(cw2.y), hi_bf16(cw2.y));
        }
      }
    }
  }

  // 5. stores: whole 16-byte pieces of the token's code and scale/zero rows
  if (live) {
    const int64_t row = (int64_t)h * p.capacity + p.token_offset + n;
    uint32_t* cd = p.codes + row * (2 * WPL) + WPL * hf;
#pragma unroll
    for (int w = 0; w < WPL; w += 4)
      *reinterpret_cast<uint4*>(cd + w) = make_uint4(words[w], words[w + 1], words[w + 2], words[w + 3]);
    uint32_t* sd = p.sz + row * (2 * NG) + NG * hf;
    if constexpr (NG == 4) *reinterpret_cast<uint4*>(sd) = make_uint4(szw[0], szw[1], szw[2], szw[3]);
    else if constexpr (NG == 2) *reinterpret_cast<uint2*>(sd) = make_uint2(szw[0], szw[1]);
    else sd[0] = szw[0];
    if (hf == 0) store_index(row);
  }
  }   // !COEFF
#pragma unroll
  for (int i = 0; i < 8; ++i) xv[i] = xnext[i];
  }   // tiles
}

// ---------------------------------------------------------------------------
// Centroid codec with 16-token waves (bf16 d = 128, at most CM = 256 or 512 centroids,
// no reconstruction output).  The same computation as encode_centroid_kernel, laid out
// for more waves per SIMD: on v_mfma_f32_16x16x32_bf16 a wave scores 16 tokens, and
// lane (t, q) = (lane & 15, lane >> 4) holds channels 32 ks + 8 q .. 32 ks + 8 q + 7
// (ks = 0..3) of token t, i.e. a quarter of its row.  Per 16-centroid block the lane
// gets the values of centroids 16 cb + 4 q + r (r = 0..3) for its token; it keeps their
// top three with the position 4 cb + r in the low byte and q above it (8 tag bits for
// CM = 256, 9 for 512), and the four lanes of a token merge their top threes.  The
// separation test, the exact rescoring (tasks from a wave-wide prefix sum, results by
// 64-bit LDS minimum, token rows re-read from memory in the oracle's fp32 order) and
// the quantizer are those of encode_centroid_kernel; a quantization group spans two
// (g = 16) or four (g = 32, 64) lanes, whose min and max are joined by lane exchanges.
// With at most 128 registers per lane, four waves share a SIMD (two workgroups of
// eight waves per CU with 256 centroids, one of sixteen with 512), which hides the
// latency of small launches that one tile per workgroup cannot.
__host__ __device__ constexpr int c16_waves(int cm) { return cm == 512 ? 16 : 8; }

// Hn residual transform (Coral-KV Fig. 5: each group of N residual channels is
// rotated independently) of one quantization step's residuals in the lane layout of
// encode_c16_kernel: value 8 u + e of lane quarter q is channel 32 (kg + u) + 8 q + e.
// The rounding is that of the Sylvester recursion H_2m [a; b] = [H_m a + H_m b;
// H_m a - H_m b]: butterflies at channel distance 1, 2, 4 inside the lane, 8 with the
// lane 16 apart (quarter q ^ 1), for N = 64 then 16 with the lane 32 apart (q ^ 2) and
// 32 between the lane's two k-steps; the lower channel of a pair takes a + b, the
// upper a - b.  The 1/sqrt(N) scale (1/4, 1/8) is exact.
template <int N, int KG>
__device__ __forceinline__ void hn_rotate_c16(float (&r)[8 * KG], int q) {
  static_assert(N == 16 || (N == 64 && KG == 2), "rotation width and quantization step");
#pragma unroll
  for (int u = 0; u < KG; ++u) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i & h) continue;
        const float a = r[8 * u + i], b = r[8 * u + i + h];
        r[8 * u + i] = a + b;
        r[8 * u + i + h] = a - b;
      }
    }
  }
  const bool up8 = (q & 1) != 0;
#pragma unroll
  for (int i = 0; i < 8 * KG; ++i) {
    const float o = __shfl_xor(r[i], 16);
    r[i] = up8 ? o - r[i] : r[i] + o;
  }
  if constexpr (N == 64) {
    const bool up16 = (q & 2) != 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float o = __shfl_xor(r[i], 32);
      r[i] = up16 ? o - r[i] : r[i] + o;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a = r[i], b = r[8 + i];
      r[i] = a + b;
      r[8 + i] = a - b;
    }
  }
  constexpr float sc = N == 64 ? 0.125f : 0.25f;
#pragma unroll
  for (int i = 0; i < 8 * KG; ++i) r[i] *= sc;
}

template <int BITS, int G, int CM, int ROT>
__global__ __launch_bounds__(64 * c16_waves(CM), 4) void encode_c16_kernel(EncodeParams p) {
  constexpr int D = 128, ROW = D + 8;
  constexpr int NW = c16_waves(CM), NT = 64 * NW, TT = 16 * NW;   // waves, threads, tokens
  constexpr int NBM = CM / 16;                 // centroid blocks at most
  constexpr int LOCB = CM == 256 ? 6 : 7;      // bits of a value's position in a lane
  constexpr uint32_t TAGM = (4u << LOCB) - 1u; // position + quarter
  constexpr float TSLACK = CM == 256 ? 0x1p-15f : 0x1p-14f;   // relative change by the tag
  constexpr int MW = (4 * NBM + 31) / 32;      // mask words of a lane
  constexpr int L = (1 << BITS) - 1;
  __shared__ __attribute__((aligned(16))) uint16_t tab[CM * ROW];
  __shared__ __attribute__((aligned(16))) float hn[CM];
  __shared__ float cnu[CM];   // |c_j| (upper bound), 0 beyond C
  __shared__ float wmax[NW];
  __shared__ uint32_t tq[NW][64];                 // rescoring tasks: lane << 10 | centroid
  __shared__ unsigned long long tres[NW][64];     // per lane: least (distance bits, centroid)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = lane & 15, q = lane >> 4;
  const int ntile = (int)((p.n_tokens + TT - 1) / TT);
  const int wph = (int)gridDim.x / (p.pair ? 2 * p.H : p.H);   // workgroups per head
  const int b = xcd_remap(blockIdx.x, gridDim.x);
  const int hs = b / wph, first = b % wph;
  // a paired launch: head slots H .. 2H - 1 are the second tensor's heads
  const bool second = hs >= p.H;
  const int h = second ? hs - p.H : hs;
  const void* const px = second ? p.x2 : p.x;
  uint32_t* const pcodes = second ? p.codes2 : p.codes;
  uint32_t* const psz = second ? p.sz2 : p.sz;
  void* const pidx = second ? p.index2 : p.index;
  const int64_t pcap = second ? p.capacity2 : p.capacity;
  const int C = p.C;
  const int nb = (C + 15) >> 4;
  const uint16_t* cen = reinterpret_cast<const uint16_t*>(second ? p.centroids2 : p.centroids) + (int64_t)h * C * D;

  // this lane's quarter row of a tile's token (zeros past the last token)
  auto load_quarter = [&](int tl, uint4 (&dst)[4]) {
    const int64_t nn = (int64_t)tl * TT + wave * 16 + t;
    const bool lv = tl < ntile && nn < p.n_tokens;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(px) + (lv ? nn : 0) * p.x_stride +
                          (int64_t)h * D + 8 * q;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      dst[ks] = lv ? *reinterpret_cast<const uint4*>(src + 32 * ks) : make_uint4(0u, 0u, 0u, 0u);
  };
  uint4 xv[4];
  load_quarter(first, xv);

  // 1. the head's centroid table (rows C .. 16 nb - 1 zero) and row norms
#pragma unroll
  for (int rnd = 0; rnd < (CM + NT / 16 * 8 - 1) / (NT / 16 * 8); ++rnd) {
    uint4 v[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int j = (NT / 16) * (8 * rnd + it) + (tid >> 4), c = tid & 15;
      v[it] = make_uint4(0u, 0u, 0u, 0u);
      if (j < C) v[it] = *reinterpret_cast<const uint4*>(cen + (int64_t)j * D + 8 * c);
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int j = (NT / 16) * (8 * rnd + it) + (tid >> 4), c = tid & 15;
      if (j < 16 * nb && j < CM) *reinterpret_cast<uint4*>(&tab[j * ROW + 8 * c]) = v[it];
    }
  }
  __syncthreads();
  {
    float cnw = 0.0f;
    for (int j = tid; j < CM; j += NT) {
      float s2 = 0.0f;
      if (j < C) {
#pragma unroll
        for (int i = 0; i < D; i += 8) {
          const uint4 v = *reinterpret_cast<const uint4*>(&tab[j * ROW + i]);
          s2 = sq2_bf16(v.x, s2);
          s2 = sq2_bf16(v.y, s2);
          s2 = sq2_bf16(v.z, s2);
          s2 = sq2_bf16(v.w, s2);
        }
      }
      hn[j] = j < C ? -0.5f * s2 : -1e30f;
      const float cn = sqrtf(s2) * (1.0f + 0x1p-10f);
      cnu[j] = cn;
      cnw = fmaxf(cnw, cn);
    }
#pragma unroll
    for (int o = 32; o; o >>= 1) cnw = fmaxf(cnw, __shfl_xor(cnw, o));
    if (lane == 0) wmax[wave] = cnw;
  }
  __syncthreads();
  float cmax = wmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) cmax = fmaxf(cmax, wmax[w]);

  auto xq = [&](float v, int m) { return __shfl_xor(v, m); };
  auto xqi = [&](uint32_t v, int m) { return (uint32_t)__shfl_xor((int)v, m); };

#pragma unroll 1
  for (int tile = first; tile < ntile; tile += wph) {
  const int64_t n = (int64_t)tile * TT + wave * 16 + t;
  const bool live = n < p.n_tokens;
  uint4 xnext[4];
  load_quarter(tile + wph, xnext);

  // 2. v_j = x.c_j - |c_j|^2 / 2 for the lane's 4 centroids of each block; top three
  float m1 = -3.0e38f, m2 = -3.0e38f, m3 = -3.0e38f;
  auto block_values = [&](int cb, f32x4_t& acc) {
    const float4 hv = *reinterpret_cast<const float4*>(&hn[16 * cb + 4 * q]);
    acc[0] = hv.x; acc[1] = hv.y; acc[2] = hv.z; acc[3] = hv.w;
    const uint16_t* arow = &tab[(16 * cb + t) * ROW + 8 * q];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(arow + 32 * ks);
      bf16x8_t bx;
      __builtin_memcpy(&bx, &xv[ks], 16);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bx, acc, 0, 0, 0);
    }
  };
  auto top3 = [&](const f32x4_t& acc, int cb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // the position 4 cb + r (< 2^LOCB) replaces the low byte: one v_perm_b32
      const float pv = __uint_as_float(
          __builtin_amdgcn_perm(__float_as_uint(acc[r]), (uint32_t)(4 * cb + r), 0x07060500u));
      m3 = __builtin_amdgcn_fmed3f(m2, m3, pv);
      m2 = __builtin_amdgcn_fmed3f(m1, m2, pv);
      m1 = __builtin_amdgcn_fmed3f(m1, pv, 3.40282347e38f);   // max, as a median
    }
  };
  {
    f32x4_t acc0, acc1;
    block_values(0, acc0);
    int cb = 0;
    for (; cb + 2 < nb; cb += 2) {
      block_values(cb + 1, acc1);
      top3(acc0, cb);
      block_values(cb + 2, acc0);
      top3(acc1, cb + 1);
    }
    if (cb + 1 < nb) {
      block_values(cb + 1, acc1);
      top3(acc0, cb);
      top3(acc1, cb + 1);
    } else {
      top3(acc0, cb);
    }
  }
  // the quarter above the position bits; merge the four lanes' top threes
  auto q_tag = [&](float v) {
    return __uint_as_float((__float_as_uint(v) & ~(3u << LOCB)) | ((uint32_t)q << LOCB));
  };
  m1 = q_tag(m1);
  m2 = q_tag(m2);
  m3 = q_tag(m3);
#pragma unroll
  for (int mk = 16; mk <= 32; mk <<= 1) {
    const float b1 = xq(m1, mk), b2 = xq(m2, mk), b3 = xq(m3, mk);
    const float n1 = fmaxf(m1, b1);
    const float n2 = fmaxf(fmaxf(m2, b2), fminf(m1, b1));
    const float n3 = fmaxf(fmaxf(m3, b3), fmaxf(fminf(m2, b1), fminf(m1, b2)));
    m1 = n1; m2 = n2; m3 = n3;
  }
  const float t1 = m1, t2 = m2, t3 = m3;

  // |x|^2 (upper bound) and the separation test
  float xs = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    xs = sq2_bf16(xv[ks].x, xs);
    xs = sq2_bf16(xv[ks].y, xs);
    xs = sq2_bf16(xv[ks].z, xs);
    xs = sq2_bf16(xv[ks].w, xs);
  }
  xs = xs + xq(xs, 16);
  xs = xs + xq(xs, 32);
  const float xxu = xs * (1.0f + 0x1p-10f);
  const float xn = sqrtf(xxu) * (1.0f + 0x1p-10f);
  auto erow = [&](float cj) {
    return (2.0f * (D + 2) * 0x1p-24f) * cj * (cj + xn) * (1.0f + 0x1p-10f) + 1e-30f;
  };
  const float E = erow(cmax);
  const float go = (D + 3) * 0x1p-24f * (1.0f + 0x1p-10f);
  auto separated = [&](float a, float c, float esum) {
    const float va = a - TSLACK * fabsf(a), vc = c + TSLACK * fabsf(c);
    const float rhs = esum + go * (xxu - va - vc) + 0x1p-20f * (fabsf(va) + fabsf(vc) + xxu);
    return va - vc > rhs;
  };
  auto cidx = [](float v) {
    const uint32_t tg = __float_as_uint(v) & TAGM;
    const int qq = (int)(tg >> LOCB), pos = (int)(tg & ((1u << LOCB) - 1u));
    return 16 * (pos >> 2) + 4 * qq + (pos & 3);
  };
  int best = cidx(t1);
  bool uniq = !live || separated(t1, t2, 2.0f * E), pair = false;
  if (!uniq) {
    const float e1 = erow(cnu[best]), e2 = erow(cnu[cidx(t2)]);
    const bool beats_rest = separated(t1, t3, e1 + E);
    uniq = beats_rest && separated(t1, t2, e1 + e2);
    pair = beats_rest && !uniq;
  }

  // 3. exact rescoring of the tokens the test leaves open
  if (__any(!uniq)) {
    uint32_t* qt = &tq[wave][0];
    unsigned long long* rs = &tres[wave][0];
    // a pair token's two candidates go to its lanes q = 0 and 1
    const int single = (pair && q < 2) ? cidx(q ? t2 : t1) : -1;
    uint32_t mask[MW];   // bit 4 cb + r: candidate value of this lane
#pragma unroll
    for (int w = 0; w < MW; ++w) mask[w] = 0u;
    const bool full = !uniq && !pair;
    if (__any(full)) {
      const float va = t1 - TSLACK * fabsf(t1);
      const float tau = va - 2.0f * (2.0f * E + go * (xxu + 2.0f * fabsf(va)) +
                                     0x1p-20f * (2.0f * fabsf(va) + xxu) + 0x1p-14f * fabsf(va));
      for (int cb = 0; cb < nb; ++cb) {
        f32x4_t acc;
        block_values(cb, acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * cb + 4 * q + r, pos = 4 * cb + r;
          if (full && j < C && acc[r] >= tau) mask[pos >> 5] |= 1u << (pos & 31);
        }
      }
    }
    const int64_t nw0 = n - t;   // first token of this wave
    float bd = __builtin_inff();
    int bj = 0x7FFFFFFF;
    int cnt = single >= 0 ? 1 : 0;
#pragma unroll
    for (int w = 0; w < MW; ++w) cnt += __builtin_popcount(mask[w]);
    int off = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(off, d);
      if (lane >= d) off += o;
    }
    const int total = __shfl(off, 63);
    off -= cnt;
    for (int r0 = 0; r0 < total; r0 += 64) {
      rs[lane] = ~0ull;
      {
        int g = off;
        if (single >= 0) {
          if (g >= r0 && g < r0 + 64) qt[g - r0] = ((uint32_t)lane << 10) | (uint32_t)single;
          ++g;
        }
        for (int w = 0; w < MW; ++w) {
          uint32_t m = mask[w];
          while (m) {
            const int pos = 32 * w + __builtin_ctz(m);
            m &= m - 1u;
            if (g >= r0 && g < r0 + 64)
              qt[g - r0] = ((uint32_t)lane << 10) | (uint32_t)(16 * (pos >> 2) + 4 * q + (pos & 3));
            ++g;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      const int ntask = min(total - r0, 64);
      if (lane < ntask) {
        const uint32_t tk = qt[lane];
        const int j = (int)(tk & 0x3FFu);
        const int64_t nt = nw0 + (int)((tk >> 10) & 15u);
        const uint16_t* xr = reinterpret_cast<const uint16_t*>(px) + nt * p.x_stride + (int64_t)h * D;
        const uint16_t* crow = &tab[j * ROW];
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {   // channels in ascending order
          const uint4 xw = *reinterpret_cast<const uint4*>(xr + 8 * i);
          const uint4 cw = *reinterpret_cast<const uint4*>(crow + 8 * i);
          const uint32_t xa[4] = {xw.x, xw.y, xw.z, xw.w}, ca[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float d0 = lo_bf16(xa[k]) - lo_bf16(ca[k]);
            const float q0 = d0 * d0;
            acc = acc + q0;
            const float d1 = hi_bf16(xa[k]) - hi_bf16(ca[k]);
            const float q1 = d1 * d1;
            acc = acc + q1;
          }
        }
        atomicMin(&rs[tk >> 10], ((unsigned long long)__float_as_uint(acc) << 32) | (uint32_t)j);
      }
      __builtin_amdgcn_wave_barrier();
      const unsigned long long mine = rs[lane];
      if (mine != ~0ull) {
        const float d = __uint_as_float((uint32_t)(mine >> 32));
        const int j = (int)(uint32_t)mine;
        if (d < bd || (d == bd && j < bj)) { bd = d; bj = j; }
      }
      __builtin_amdgcn_wave_barrier();
    }
    // the token's four lanes agree on the least (distance, index)
#pragma unroll
    for (int mk = 16; mk <= 32; mk <<= 1) {
      const float od = xq(bd, mk);
      const int oj = (int)xqi((uint32_t)bj, mk);
      if (od < bd || (od == bd && oj < bj)) { bd = od; bj = oj; }
    }
    if (!uniq) best = bj;
  }

  // 4. residual, group scale/zero, codes of the lane's quarter row (none when only the
  //    index is asked for)
  const uint16_t* crow = &tab[best * ROW + 8 * q];
  const int64_t row = (int64_t)h * pcap + p.token_offset + n;
  constexpr int KG = G == 64 ? 2 : 1;   // k-steps of one group
  if (!p.index_only) {
#pragma unroll
    for (int kg = 0; kg < 4; kg += KG) {
      float r[8 * KG];
#pragma unroll
      for (int u = 0; u < KG; ++u) {
        const uint4 cv = *reinterpret_cast<const uint4*>(crow + 32 * (kg + u));
        const uint4 xw = xv[kg + u];
        const uint32_t xa[4] = {xw.x, xw.y, xw.z, xw.w}, ca[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          r[8 * u + 2 * k] = lo_bf16(xa[k]) - lo_bf16(ca[k]);
          r[8 * u + 2 * k + 1] = hi_bf16(xa[k]) - hi_bf16(ca[k]);
        }
      }
      if constexpr (ROT != 0) hn_rotate_c16<ROT, KG>(r, q);
      float mn = r[0], mx = r[0];
#pragma unroll
      for (int i = 1; i < 8 * KG; ++i) { mn = fminf(mn, r[i]); mx = fmaxf(mx, r[i]); }
      // the group's other lanes: q ^ 1 (g = 16), all four (g = 32, 64)
      mn = fminf(mn, xq(mn, 16));
      mx = fmaxf(mx, xq(mx, 16));
      if constexpr (G >= 32) {
        mn = fminf(mn, xq(mn, 32));
        mx = fmaxf(mx, xq(mx, 32));
      }
      const GroupQ gq = group_scale_zero(mn, mx, L);
      // codes, 8 per k-step: the reciprocal quotient, redone with the IEEE division
      // when an element lies within the bound of a rounding boundary (see quantize_with)
      uint32_t cw[KG];
#pragma unroll
      for (int u = 0; u < KG; ++u) cw[u] = 0u;
      if (gq.s != 0.0f) {
        const float rinv = __builtin_amdgcn_rcpf(gq.s);
        const float nzr = -(gq.z * rinv);
        const float thr = 0.5f - (fabsf(nzr) + (float)(L + 2)) * 0x1p-19f;
        float dev = 0.0f;   // largest |y - rint(y)| of the group
#pragma unroll
        for (int i = 0; i < 8 * KG; ++i) {
          const float y = __builtin_fmaf(r[i], rinv, nzr);
          const float k = __builtin_rintf(y);
          dev = fmaxf(dev, fabsf(y - k));
          const uint32_t code = (uint32_t)__builtin_amdgcn_fmed3f(k, 0.0f, (float)L);
          cw[i >> 3] |= code << (BITS * (i & 7));
        }
        if (dev > thr) {
#pragma unroll
          for (int u = 0; u < KG; ++u) cw[u] = 0u;
#pragma unroll
          for (int i = 0; i < 8 * KG; ++i) cw[i >> 3] |= quantize_one(r[i], gq, L) << (BITS * (i & 7));
        }
      }
      // stores: channel piece (ks, q) holds bits 8 BITS (4 ks + q) .. of the token's row
#pragma unroll
      for (int u = 0; u < KG; ++u) {
        const int ks = kg + u;
        if constexpr (BITS == 4) {
          if (live) pcodes[row * 16 + 4 * ks + q] = cw[u];
        } else {
          const uint32_t pw = xqi(cw[u], 16);   // the partner quarter's 16 bits
          if (live && (q & 1) == 0) pcodes[row * 8 + 2 * ks + (q >> 1)] = cw[u] | (pw << 16);
        }
      }
      // scale/zero word of the group (one lane per group)
      const int gi = G == 16 ? 2 * kg + (q >> 1) : (G == 32 ? kg : kg >> 1);
      const bool owner = G == 16 ? (q & 1) == 0 : q == 0;
      if (live && owner) psz[row * (D / G) + gi] = gq.word;
    }
  }
  if (live && q == 0) {
    if (p.index_bytes == 2) reinterpret_cast<uint16_t*>(pidx)[row] = (uint16_t)best;
    else reinterpret_cast<uint8_t*>(pidx)[row] = (uint8_t)best;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) xv[i] = xnext[i];
  }   // tiles
}

template <int BITS, int G, int CM, int ROT>
hipError_t launch_c16_t(const EncodeParams& p, hipStream_t s) {
  auto k = encode_c16_kernel<BITS, G, CM, ROT>;
  constexpr int NT = 64 * c16_waves(CM), TT = NT / 4;
  int occ = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(k), NT, 0);
  if (e != hipSuccess) return e;
  const int64_t ntile = (p.n_tokens + TT - 1) / TT;
  const int64_t resident = (int64_t)std::max(1, occ) * cu_count();
  const int slots = p.pair ? 2 * p.H : p.H;
  const int wph = (int)std::max<int64_t>(1, std::min<int64_t>(ntile, resident / slots));
  hipLaunchKernelGGL(k, dim3((unsigned)(wph * slots)), dim3(NT), 0, s, p);
  return hipGetLastError();
}

// Persistent grid: workgroups per head = how many are resident at once (LDS and
// registers decide) divided over the heads, at most one per tile.
template <int BITS, int G, int CM, bool COEFF>
hipError_t launch_centroid_t(const EncodeParams& p, hipStream_t s) {
  auto k = encode_centroid_kernel<BITS, G, CM, COEFF>;
  constexpr int NT = 64 * cen_waves(CM, COEFF), TT = NT / 2;
  int occ = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(k), NT, 0);
  if (e != hipSuccess) return e;
  const int64_t ntile = (p.n_tokens + TT - 1) / TT;
  const int64_t resident = (int64_t)std::max(1, occ) * cu_count();
  const int wph = (int)std::max<int64_t>(1, std::min<int64_t>(ntile, resident / p.H));
  hipLaunchKernelGGL(k, dim3((unsigned)(wph * p.H)), dim3(NT), 0, s, p);
  return hipGetLastError();
}

template <typename XT, int D>
hipError_t launch_encode_t(const EncodeParams& p, int H, hipStream_t s) {
  const int ntiles = (int)((p.n_tokens + TOK - 1) / TOK);
  dim3 grid(ntiles * H);
  hipLaunchKernelGGL((encode_kernel<XT, D>), grid, dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}

// The fields of EncodeParams that come straight from the validated call.
EncodeParams encode_params(const EncodeLaunch& a) {
  EncodeParams p{};
  p.x = a.x;
  p.n_tokens = a.n_tokens;
  p.x_stride = a.x_stride;
  p.token_offset = a.token_offset;
  p.capacity = a.st.capacity;
  p.H = a.c.H;
  p.C = a.c.C;
  p.bits = a.c.bits;
  p.group = a.c.group;
  p.groups = a.c.groups;
  p.code_words = a.c.code_words;
  p.vec_len = a.c.vec_len;
  p.m = a.c.m;
  p.index_bytes = a.c.index_bytes;
  p.centroids = a.b.centroids;
  p.basis = reinterpret_cast<const uint16_t*>(a.b.basis);
  p.prev0 = a.b.prev0;
  p.prev1 = a.b.prev1;
  p.prev_stride = a.b.prev_stride;
  p.coef_a = a.b.coef_a;
  p.coef_b = a.b.coef_b;
  p.codes = a.st.codes;
  p.sz = a.st.sz;
  p.index = a.st.index;
  p.recon = a.recon;
  p.pred = a.pred;
  p.index_only = a.index_only ? 1 : 0;
  return p;
}

// The 16-token-wave centroid encoder, if it serves the codec (bf16 d = 128, <= 512
// centroids, group 16 / 32 / 64, no reconstruction or prediction output, input stride a
// multiple of 8): launches it and sets *done.
hipError_t dispatch_c16(const EncodeParams& p, const CodecArgs& c, hipStream_t s, bool* done) {
  *done = false;
  if (!(c.x_dtype == KVC_BF16 && c.D == 128 && p.mode == MODE_CENTROID && !p.recon && !p.pred &&
        c.C <= 512 && p.x_stride % 8 == 0 && (c.group == 16 || c.group == 32 || c.group == 64)))
    return hipSuccess;
#define KVC_ENC_C16(B, G, CM, R)                                                         \
  if (c.bits == B && c.group == G && (c.C <= 256) == (CM == 256) && c.rot == R) {       \
    *done = true;                                                                       \
    return launch_c16_t<B, G, CM, R>(p, s);                                             \
  }
#define KVC_ENC_C16_CM(CM)                                                                \
  KVC_ENC_C16(2, 16, CM, 0) KVC_ENC_C16(2, 32, CM, 0) KVC_ENC_C16(2, 64, CM, 0)          \
  KVC_ENC_C16(4, 16, CM, 0) KVC_ENC_C16(4, 32, CM, 0) KVC_ENC_C16(4, 64, CM, 0)          \
  KVC_ENC_C16(2, 16, CM, 16) KVC_ENC_C16(2, 32, CM, 16) KVC_ENC_C16(2, 64, CM, 16)       \
  KVC_ENC_C16(4, 16, CM, 16) KVC_ENC_C16(4, 32, CM, 16) KVC_ENC_C16(4, 64, CM, 16)       \
  KVC_ENC_C16(2, 64, CM, 64) KVC_ENC_C16(4, 64, CM, 64)
  KVC_ENC_C16_CM(256)
  KVC_ENC_C16_CM(512)
#undef KVC_ENC_C16_CM
#undef KVC_ENC_C16
  return hipSuccess;
}

}  // namespace

hipError_t launch_predict(const EncodeLaunch& a, float* base_out, hipStream_t s);

hipError_t launch_encode(const EncodeLaunch& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  {
    hipError_t e = hipSuccess;
    if (launch_encode_fused(a, s, &e)) return e;
  }
  // rotated predictor and plain codecs are encoded by the fused predictor + quantizer
  // only; refuse before any prediction kernel is launched
  if (a.c.rot != 0 && a.c.base != KVC_BASE_CENTROID) return hipErrorInvalidValue;
  EncodeParams p = encode_params(a);
  switch (a.c.base) {
    case KVC_BASE_NONE: p.mode = MODE_NONE; break;
    case KVC_BASE_CENTROID: p.mode = MODE_CENTROID; break;
    case KVC_BASE_COEFF: p.mode = MODE_COEFF; break;
    case KVC_BASE_TEMPORAL:
      if (a.b.w_block == nullptr) { p.mode = MODE_TEMPORAL_K; break; }
      [[fallthrough]];
    case KVC_BASE_DPLR: {
      // matrix-product bases: the prediction kernel writes the fp32 base first
      float* buf = a.pred ? a.pred : reinterpret_cast<float*>(a.workspace);
      hipError_t e = launch_predict(a, buf, s);
      if (e != hipSuccess) return e;
      p.mode = MODE_BUFFER;
      p.base_buf = buf;
      p.pred = nullptr;   // already written by the prediction kernel when requested
      break;
    }
    default: return hipErrorInvalidValue;
  }
  const bool bf16 = a.c.x_dtype == KVC_BF16;
  const bool c16_ok = bf16 && a.c.D == 128 && p.mode == MODE_CENTROID && !p.recon && !p.pred &&
                      a.c.C <= 512 && p.x_stride % 8 == 0;
  if (a.c.rot != 0 && !c16_ok) return hipErrorInvalidValue;   // rotation: 16-token-wave kernel only
  // centroid and coefficient (m = 16, INT4) bases, bf16 d = 128, <= 512 centroids:
  // register-resident MFMA assignment, persistent workgroups per head
  const bool cen_ok = p.mode == MODE_CENTROID && (a.c.group == 16 || a.c.group == 32 || a.c.group == 64);
  const bool coeff_ok = p.mode == MODE_COEFF && a.c.m == 16 && a.c.group == 16 && a.c.bits == 4;
  {
    bool done = false;
    const hipError_t e = dispatch_c16(p, a.c, s, &done);
    if (done || e != hipSuccess) return e;
  }
  if (a.c.rot != 0) return hipErrorInvalidValue;   // a width / group pair without a kernel
  if (bf16 && a.c.D == 128 && (cen_ok || coeff_ok) && a.c.C <= 512 && p.x_stride % 8 == 0) {
#define KVC_ENC_CEN(B, G, CM, CF)                                                        \
    if (a.c.bits == B && a.c.group == G && (a.c.C <= 256) == (CM == 256) && coeff_ok == CF) \
      return launch_centroid_t<B, G, CM, CF>(p, s);
    KVC_ENC_CEN(2, 16, 256, false) KVC_ENC_CEN(2, 32, 256, false) KVC_ENC_CEN(2, 64, 256, false)
    KVC_ENC_CEN(4, 16, 256, false) KVC_ENC_CEN(4, 32, 256, false) KVC_ENC_CEN(4, 64, 256, false)
    KVC_ENC_CEN(2, 16, 512, false) KVC_ENC_CEN(2, 32, 512, false) KVC_ENC_CEN(2, 64, 512, false)
    KVC_ENC_CEN(4, 16, 512, false) KVC_ENC_CEN(4, 32, 512, false) KVC_ENC_CEN(4, 64, 512, false)
    KVC_ENC_CEN(4, 16, 256, true) KVC_ENC_CEN(4, 16, 512, true)
#undef KVC_ENC_CEN
  }
  // centroid and coefficient bases on bf16 d = 128 data: MFMA shortlist + exact rescoring
  if (bf16 && a.c.D == 128 && (p.mode == MODE_CENTROID || p.mode == MODE_COEFF) &&
      p.x_stride % 8 == 0 && a.c.C <= 512) {
    if (a.c.C <= 256) {
      const int ntiles = (int)((p.n_tokens + 63) / 64);
      hipLaunchKernelGGL(encode_shortlist_kernel<64>, dim3(ntiles * a.c.H), dim3(NTHREADS), 0, s, p);
    } else {
      const int ntiles = (int)((p.n_tokens + 31) / 32);
      hipLaunchKernelGGL(encode_shortlist_kernel<32>, dim3(ntiles * a.c.H), dim3(NTHREADS), 0, s, p);
    }
    return hipGetLastError();
  }
  if (a.c.D == 128) {
    return bf16 ? launch_encode_t<uint16_t, 128>(p, a.c.H, s) : launch_encode_t<float, 128>(p, a.c.H, s);
  }
  return bf16 ? launch_encode_t<uint16_t, 64>(p, a.c.H, s) : launch_encode_t<float, 64>(p, a.c.H, s);
}

// The keys and the values of a chunk (same codec, token count, stride and offset): one
// launch of the 16-token-wave centroid encoder over both tensors' heads when it serves
// the codec, else the two tensors one after the other.
hipError_t launch_encode_pair(const EncodeLaunch& a, const EncodeLaunch& b, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  if (a.c.base == KVC_BASE_CENTROID) {
    EncodeParams p = encode_params(a);
    p.mode = MODE_CENTROID;
    p.pair = 1;
    p.x2 = b.x;
    p.centroids2 = b.b.centroids;
    p.codes2 = b.st.codes;
    p.sz2 = b.st.sz;
    p.index2 = b.st.index;
    p.capacity2 = b.st.capacity;
    bool done = false;
    const hipError_t e = dispatch_c16(p, a.c, s, &done);
    if (done || e != hipSuccess) return e;
  }
  const hipError_t e = launch_encode(a, s);
  if (e != hipSuccess) return e;
  return launch_encode(b, s);
}

}  // namespace kvc
