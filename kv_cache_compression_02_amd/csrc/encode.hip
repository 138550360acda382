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

template <typename XT, int D>
hipError_t launch_encode_t(const EncodeParams& p, int H, hipStream_t s) {
  const int ntiles = (int)((p.n_tokens + TOK - 1) / TOK);
  dim3 grid(ntiles * H);
  hipLaunchKernelGGL((encode_kernel<XT, D>), grid, dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_predict(const EncodeLaunch& a, float* base_out, hipStream_t s);

hipError_t launch_encode(const EncodeLaunch& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
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
  if (a.c.D == 128) {
    return bf16 ? launch_encode_t<uint16_t, 128>(p, a.c.H, s) : launch_encode_t<float, 128>(p, a.c.H, s);
  }
  return bf16 ? launch_encode_t<uint16_t, 64>(p, a.c.H, s) : launch_encode_t<float, 64>(p, a.c.H, s);
}

}  // namespace kvc
