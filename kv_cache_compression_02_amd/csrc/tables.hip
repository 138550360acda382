// fp16 images of bf16 centroid tables for the decode-fused attention.
//
// The tile decode adds a key's centroid row to its dequantized residual in fp32.  From
// an fp16 value c16 = c * 2^k that is one v_fma_mix_f32, c16 * 2^-k + r with a single
// rounding, i.e. exactly the fp32 sum c + r, where a bf16 value needs an unpack and an
// add.  Each head gets the power of two 2^k that brings its largest magnitude closest
// below 65504 (the largest fp16), and every entry is checked: c * 2^k must be an fp16
// value exactly (non-finite entries, or a head whose nonzero magnitudes span more than
// fp16's range, fail and keep the bf16 path).
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int CT_THREADS = 256;

// One workgroup per head.  Header: k per head, then 1 / 0 per head for exact / not.
__global__ __launch_bounds__(CT_THREADS) void centroid_tables_kernel(const uint4* cen, int H, int n8,
                                                                      int32_t* hdr, uint4* out) {
  __shared__ float red[CT_THREADS / 64];
  __shared__ int okw[CT_THREADS / 64];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint4* src = cen + (int64_t)h * n8;   // 8 bf16 per 16-byte piece
  uint4* dst = out + (int64_t)h * n8;
  float m = 0.0f;
  int ok = 1;
  for (int i = tid; i < n8; i += CT_THREADS) {
    const uint4 v = src[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = __uint_as_float(w[j] << 16), b = __uint_as_float(w[j] & 0xFFFF0000u);
      if (!(fabsf(a) <= 3.0e38f) || !(fabsf(b) <= 3.0e38f)) ok = 0;   // inf / nan
      m = fmaxf(m, fmaxf(fabsf(a), fabsf(b)));
    }
  }
#pragma unroll
  for (int o = 32; o; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < CT_THREADS / 64; ++w) m = fmaxf(m, red[w]);
  int k = 0;
  if (m > 0.0f && m <= 3.0e38f) {
    int e;
    const float f = frexpf(m, &e);   // m = f 2^e, f in [0.5, 1)
    k = (f * 65536.0f <= 65504.0f) ? 16 - e : 15 - e;
    k = max(-100, min(100, k));
  }
  const float sc = __int_as_float((127 + k) << 23);
  auto img = [&](float c) {   // fp16 bits of c * 2^k (exact scaling) and the check
    const float y = c * sc;
    const _Float16 hv = (_Float16)y;
    if (!((float)hv == y)) ok = 0;
    return (uint32_t)__builtin_bit_cast(uint16_t, hv);
  };
  for (int i = tid; i < n8; i += CT_THREADS) {
    const uint4 v = src[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = img(__uint_as_float(w[j] << 16)) | (img(__uint_as_float(w[j] & 0xFFFF0000u)) << 16);
    dst[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  ok = __all(ok) ? 1 : 0;
  if (lane == 0) okw[wave] = ok;
  __syncthreads();
  if (tid == 0) {
    int all = 1;
    for (int w = 0; w < CT_THREADS / 64; ++w) all &= okw[w];
    hdr[h] = k;
    hdr[H + h] = all;
  }
}

}  // namespace

size_t centroid_tables_header_bytes(int H) { return ((size_t)8 * H + 255) / 256 * 256; }

hipError_t launch_centroid_tables(const void* centroids, int H, int C, int D, void* tables,
                                  hipStream_t s) {
  // d = 128: every head's table is a whole number of 16-byte pieces, 16-byte aligned
  int32_t* hdr = reinterpret_cast<int32_t*>(tables);
  uint4* out = reinterpret_cast<uint4*>(reinterpret_cast<char*>(tables) + centroid_tables_header_bytes(H));
  hipLaunchKernelGGL(centroid_tables_kernel, dim3((unsigned)H), dim3(CT_THREADS), 0, s,
                     reinterpret_cast<const uint4*>(centroids), H, C * D / 8, hdr, out);
  return hipGetLastError();
}

}  // namespace kvc
