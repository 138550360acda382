// Decode: reconstruction = base + ((code * s) + z), written token-major.
//
// Method: the stored residual codes, scales and assignments are what the
// compressed state holds (Coral-KV arXiv 2610.12514 Table 9 caption); adding the
// dequantized residual to the base gives the reconstruction (Coral-KV Fig. 3).
//
// One thread per (token, head, 16 consecutive channels), heads on the grid's y axis: loads
// its code words, the group's scale/zero word and 32 bytes of the base row, writes 16
// outputs with 16-byte vector stores.  HBM-bound streaming kernel.
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

struct DecodeParams {
  int64_t n_tokens, token_offset, capacity;
  int H, D, C, bits, group, groups, code_words, index_bytes, mode;
  int rot;             // Hn residual transform width (0, 16 or 64)
  uint32_t total;      // threads per head of this launch: n_tokens * (D / 16) < 2^31
  int cshift, gshift;  // log2(D / 16), log2(group)
  const uint32_t* codes;
  const uint32_t* sz;
  const void* index;
  const void* centroids;
  const void* prev0;
  const void* prev1;
  int64_t prev_stride;
  const float* coef_a;
  const float* coef_b;
  const float* base_buf;
  void* out;
  float* pred;
};

enum { DM_NONE = 0, DM_CENTROID = 1, DM_TEMPORAL_K = 3, DM_BUFFER = 4 };

// 16 consecutive values of a row in dtype XT (16-byte aligned) as fp32.
template <typename XT>
__device__ __forceinline__ void load16(const XT* src, float (&v)[16]) {
  if constexpr (sizeof(XT) == 2) {
    const uint4 a = *reinterpret_cast<const uint4*>(src);
    const uint4 b = *reinterpret_cast<const uint4*>(src + 8);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[2 * k] = bf16_bits_to_f32(w[k] & 0xFFFFu);
      v[2 * k + 1] = bf16_bits_to_f32(w[k] >> 16);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 u = *reinterpret_cast<const float4*>(src + 4 * k);
      v[4 * k] = u.x; v[4 * k + 1] = u.y; v[4 * k + 2] = u.z; v[4 * k + 3] = u.w;
    }
  }
}

// One thread per (token, head, 16 consecutive channels): the 16 codes are one (INT2)
// or two (INT4) aligned words, the channels share one scale/zero word (groups are >= 16
// wide), and the outputs go out as 16-byte stores, consecutive threads writing
// consecutive pieces of the token-major output rows.
template <typename XT, typename OT>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  // head-major walk (blockIdx.y = head): the store's rows are read in order and the
  // concurrently used centroid rows are one head's, which stay in L2 while the output
  // streams through it
  const uint32_t e = blockIdx.x * 256u + threadIdx.x;
  if (e >= p.total) return;
  const uint32_t c16 = e & ((1u << p.cshift) - 1u);
  const uint32_t n = e >> p.cshift;
  const uint32_t h = blockIdx.y;
  const int i0 = (int)c16 * 16;
  const int64_t row = (int64_t)h * p.capacity + p.token_offset + n;

  const uint32_t szw = p.sz[row * p.groups + (i0 >> p.gshift)];
  const float s = f16_bits_to_f32(szw & 0xFFFFu);
  const float z = f16_bits_to_f32(szw >> 16);
  const uint32_t* cw = p.codes + row * p.code_words + (int64_t)c16 * (p.bits >> 1);
  const uint32_t w0 = cw[0];
  const uint32_t w1 = p.bits == 4 ? cw[1] : 0u;

  float base[16];
  if (p.mode == DM_CENTROID) {
    int a = p.index_bytes == 1 ? reinterpret_cast<const uint8_t*>(p.index)[row]
                               : reinterpret_cast<const uint16_t*>(p.index)[row];
    a = min(a, p.C - 1);   // out-of-contract indices must not read past the table
    load16<XT>(reinterpret_cast<const XT*>(p.centroids) + ((int64_t)h * p.C + a) * p.D + i0, base);
  } else if (p.mode == DM_TEMPORAL_K) {
    float x0[16], x1[16];
    load16<XT>(reinterpret_cast<const XT*>(p.prev0) + (int64_t)n * p.prev_stride + (int64_t)h * p.D + i0, x0);
    load16<XT>(reinterpret_cast<const XT*>(p.prev1) + (int64_t)n * p.prev_stride + (int64_t)h * p.D + i0, x1);
    float ca[16], cb[16];
    load16<float>(p.coef_a + h * p.D + i0, ca);
    load16<float>(p.coef_b + h * p.D + i0, cb);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float a = ca[k] * x0[k];
      const float b = cb[k] * x1[k];
      base[k] = a + b;
    }
  } else if (p.mode == DM_BUFFER) {
    load16<float>(p.base_buf + ((int64_t)n * p.H + h) * p.D + i0, base);
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) base[k] = 0.0f;
  }

  const int64_t orow = ((int64_t)n * p.H + h) * p.D + i0;
  float v[16];
  const uint32_t mask = (1u << p.bits) - 1u;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int bit = p.bits * k;   // 0..60
    const uint32_t code = ((bit < 32 ? (w0 >> bit) : (w1 >> (bit - 32)))) & mask;
    v[k] = dequant_one(code, s, z);
  }
  if (p.rot != 0) {
    // Hn transform back (H_n / sqrt(n) is its own inverse) with the rounding of the
    // Sylvester recursion: butterflies at channel distance 1, 2, 4, 8 inside the
    // thread, then for n = 64 at 16 and 32 with the threads 1 and 2 lanes apart (the
    // neighbouring 16-channel pieces of the row; rows start at multiples of 8 lanes
    // and a launch covers whole rows, so the partner is live).  Lower channel of a
    // pair: a + b, upper: a - b; the 1/sqrt(n) scale is exact.
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k & h) continue;
        const float a = v[k], b = v[k + h];
        v[k] = a + b;
        v[k + h] = a - b;
      }
    }
    if (p.rot == 64) {
#pragma unroll
      for (int m = 1; m <= 2; m <<= 1) {
        const bool up = (c16 & (uint32_t)m) != 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float o = __shfl_xor(v[k], m);
          v[k] = up ? o - v[k] : v[k] + o;
        }
      }
    }
    const float sc = p.rot == 64 ? 0.125f : 0.25f;
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] *= sc;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = base[k] + v[k];
  OT* out = reinterpret_cast<OT*>(p.out) + orow;
  if constexpr (sizeof(OT) == 2) {     // 16 bf16 (round to nearest even): two 16-byte stores
    uint32_t o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
    *reinterpret_cast<uint4*>(out) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4*>(out + 8) = make_uint4(o[4], o[5], o[6], o[7]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<float4*>(out + 4 * k) = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
  if (p.pred && p.mode != DM_BUFFER) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<float4*>(p.pred + orow + 4 * k) =
          make_float4(base[4 * k], base[4 * k + 1], base[4 * k + 2], base[4 * k + 3]);
  }
}

// Launches in token ranges whose thread count stays below 2^31 (32-bit indexing in
// the kernel); every pointer that is indexed by the token moves with the range.
template <typename XT>
hipError_t launch_decode_x(const DecodeParams& p0, int out_dtype, hipStream_t s) {
  const int64_t per_token = p0.D / 16;   // threads per token of one head
  const int64_t step = std::max<int64_t>(1, ((int64_t)1 << 31) / per_token - 256);
  const int osz = out_dtype == KVC_BF16 ? 2 : 4;
  for (int64_t t0 = 0; t0 < p0.n_tokens; t0 += step) {
    DecodeParams p = p0;
    p.n_tokens = std::min(step, p0.n_tokens - t0);
    p.token_offset = p0.token_offset + t0;
    p.total = (uint32_t)(p.n_tokens * per_token);
    const int64_t elems = t0 * p0.H * p0.D;
    p.out = reinterpret_cast<char*>(p0.out) + elems * osz;
    if (p0.pred) p.pred = p0.pred + elems;
    if (p0.base_buf) p.base_buf = p0.base_buf + elems;
    if (p0.prev0) p.prev0 = reinterpret_cast<const XT*>(p0.prev0) + t0 * p0.prev_stride;
    if (p0.prev1) p.prev1 = reinterpret_cast<const XT*>(p0.prev1) + t0 * p0.prev_stride;
    const dim3 grid((p.total + 255u) / 256u, (unsigned)p0.H);
    if (out_dtype == KVC_BF16)
      hipLaunchKernelGGL((decode_kernel<XT, uint16_t>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((decode_kernel<XT, float>), grid, dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_predict(const EncodeLaunch& a, float* base_out, hipStream_t s);

hipError_t launch_decode(const DecodeLaunch& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  DecodeParams p{};
  p.n_tokens = a.n_tokens;
  p.token_offset = a.token_offset;
  p.capacity = a.st.capacity;
  p.H = a.c.H;
  p.D = a.c.D;
  p.C = a.c.C;
  p.bits = a.c.bits;
  p.group = a.c.group;
  p.groups = a.c.groups;
  p.code_words = a.c.code_words;
  p.index_bytes = a.c.index_bytes;
  p.codes = a.st.codes;
  p.sz = a.st.sz;
  p.index = a.st.index;
  p.centroids = a.b.centroids;
  p.prev0 = a.b.prev0;
  p.prev1 = a.b.prev1;
  p.prev_stride = a.b.prev_stride;
  p.coef_a = a.b.coef_a;
  p.coef_b = a.b.coef_b;
  p.out = a.out;
  p.pred = a.pred;
  p.rot = a.c.rot;
  p.cshift = __builtin_ctz((unsigned)(a.c.D / 16));
  p.gshift = __builtin_ctz((unsigned)a.c.group);
  if (a.c.D % 16 != 0 || (a.c.group & (a.c.group - 1)) != 0 || a.c.group < 16 || (a.c.bits != 2 && a.c.bits != 4))
    return hipErrorInvalidValue;
  switch (a.c.base) {
    case KVC_BASE_NONE: p.mode = DM_NONE; break;
    case KVC_BASE_CENTROID: p.mode = DM_CENTROID; break;
    case KVC_BASE_TEMPORAL:
      if (a.b.w_block == nullptr) { p.mode = DM_TEMPORAL_K; break; }
      [[fallthrough]];
    case KVC_BASE_DPLR: {
      EncodeLaunch e{};
      e.c = a.c;
      e.b = a.b;
      e.n_tokens = a.n_tokens;
      e.pred = a.pred;
      e.workspace = a.workspace;
      float* buf = a.pred ? a.pred : reinterpret_cast<float*>(a.workspace);
      hipError_t err = launch_predict(e, buf, s);
      if (err != hipSuccess) return err;
      p.mode = DM_BUFFER;
      p.base_buf = buf;
      break;
    }
    default: return hipErrorInvalidValue;
  }
  return a.c.x_dtype == KVC_BF16 ? launch_decode_x<uint16_t>(p, a.out_dtype, s)
                                 : launch_decode_x<float>(p, a.out_dtype, s);
}

}  // namespace kvc
