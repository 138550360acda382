// Decode: reconstruction = base + ((code * s) + z), written token-major.
//
// Method: the stored residual codes, scales and assignments are what the
// compressed state holds (Coral-KV arXiv 2610.12514 Table 9 caption); adding the
// dequantized residual to the base gives the reconstruction (Coral-KV Fig. 3).
//
// One thread per (token, head, 8 consecutive channels): loads its code bits, the
// group's scale/zero word and 16 bytes of the base row, writes 8 outputs with one
// vector store.  HBM-bound streaming kernel.
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

struct DecodeParams {
  int64_t n_tokens, token_offset, capacity;
  int H, D, C, bits, group, groups, code_words, index_bytes, mode;
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

template <typename XT, typename OT>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  const int64_t chunks_per_vec = p.D / 8;
  const int64_t total = p.n_tokens * p.H * chunks_per_vec;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int c8 = (int)(e % chunks_per_vec);
  const int64_t nh = e / chunks_per_vec;
  const int h = (int)(nh % p.H);
  const int64_t n = nh / p.H;
  const int i0 = c8 * 8;
  const int64_t row = (int64_t)h * p.capacity + p.token_offset + n;

  // scale / zero of the group holding channels i0..i0+7 (groups are >= 16 wide)
  const uint32_t szw = p.sz[row * p.groups + i0 / p.group];
  const float s = f16_bits_to_f32(szw & 0xFFFFu);
  const float z = f16_bits_to_f32(szw >> 16);
  // 8 codes = 8*bits consecutive bits starting at bit i0*bits
  const int bitpos = i0 * p.bits;
  const uint32_t word = p.codes[row * p.code_words + bitpos / 32];
  const uint32_t bits8 = word >> (bitpos % 32);
  const uint32_t mask = (1u << p.bits) - 1u;

  float base[8];
  if (p.mode == DM_CENTROID) {
    int a = p.index_bytes == 1 ? reinterpret_cast<const uint8_t*>(p.index)[row]
                               : reinterpret_cast<const uint16_t*>(p.index)[row];
    a = min(a, p.C - 1);   // out-of-contract indices must not read past the table
    const XT* crow = reinterpret_cast<const XT*>(p.centroids) + ((int64_t)h * p.C + a) * p.D + i0;
    if constexpr (sizeof(XT) == 2) {   // one 16-byte read of 8 bf16 values
      const uint4 w = *reinterpret_cast<const uint4*>(crow);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        base[2 * k] = bf16_bits_to_f32(ww[k] & 0xFFFFu);
        base[2 * k + 1] = bf16_bits_to_f32(ww[k] >> 16);
      }
    } else {                           // two 16-byte reads of 8 fp32 values
      const float4 u0 = *reinterpret_cast<const float4*>(crow);
      const float4 u1 = *reinterpret_cast<const float4*>(crow + 4);
      base[0] = u0.x; base[1] = u0.y; base[2] = u0.z; base[3] = u0.w;
      base[4] = u1.x; base[5] = u1.y; base[6] = u1.z; base[7] = u1.w;
    }
  } else if (p.mode == DM_TEMPORAL_K) {
    const XT* p0 = reinterpret_cast<const XT*>(p.prev0) + n * p.prev_stride + (int64_t)h * p.D + i0;
    const XT* p1 = reinterpret_cast<const XT*>(p.prev1) + n * p.prev_stride + (int64_t)h * p.D + i0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float a = p.coef_a[h * p.D + i0 + k] * load_x<XT>(p0 + k);
      float b = p.coef_b[h * p.D + i0 + k] * load_x<XT>(p1 + k);
      base[k] = a + b;
    }
  } else if (p.mode == DM_BUFFER) {
    const float* bb = p.base_buf + (n * p.H + h) * (int64_t)p.D + i0;
#pragma unroll
    for (int k = 0; k < 8; ++k) base[k] = bb[k];
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) base[k] = 0.0f;
  }

  const int64_t orow = (n * p.H + h) * (int64_t)p.D + i0;
  OT* out = reinterpret_cast<OT*>(p.out) + orow;
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t code = (bits8 >> (p.bits * k)) & mask;
    v[k] = base[k] + dequant_one(code, s, z);
  }
  if constexpr (sizeof(OT) == 2) {     // 8 bf16 (round to nearest even): one 16-byte store
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = f32_to_bf16_bits(v[2 * k]) | (f32_to_bf16_bits(v[2 * k + 1]) << 16);
    *reinterpret_cast<uint4*>(out) = make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    *reinterpret_cast<float4*>(out) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(out + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  if (p.pred && p.mode != DM_BUFFER) {
#pragma unroll
    for (int k = 0; k < 8; ++k) p.pred[orow + k] = base[k];
  }
}

template <typename XT>
hipError_t launch_decode_x(const DecodeParams& p, int out_dtype, hipStream_t s) {
  const int64_t total = p.n_tokens * p.H * (p.D / 8);
  dim3 grid((unsigned)((total + 255) / 256));
  if (out_dtype == KVC_BF16)
    hipLaunchKernelGGL((decode_kernel<XT, uint16_t>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((decode_kernel<XT, float>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
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
