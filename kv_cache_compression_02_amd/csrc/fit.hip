// Online centroid fitting at block fill: Lloyd iterations on one block of tokens.
//
// Method: QVG fits video-specific centroids online when a cache block reaches its token
// limit (Coral-KV arXiv 2610.12514 Fig. 2c); the codec's nearest-centroid base then
// searches that table.  One iteration = assignment + update:
//   - assignment: the encoder itself (launch_encode into a scratch store in the
//     workspace), so the fitted table is searched exactly as the codec will search it
//     (fp32 distances, ascending channels, ties to the lowest index);
//   - update: every centroid that received tokens becomes the mean of its tokens,
//     rounded to bf16 (nearest even); a centroid that received none keeps its value.
//
// fit_update_kernel: a wave owns 64 channels of one centroid and walks the head's
// assignments 64 tokens at a time; a ballot marks the tokens of its centroid and only
// those rows are read, so the sums run in ascending token order (deterministic, fp32)
// and the reads are the assignments once per wave plus each token's row once per
// centroid half.  The mean is the fp32 sum divided by the count (IEEE division).
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int FD = 128;   // head dimension of the bf16 path

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct FitLayout {
  size_t codes, sz, index, total;
};

FitLayout fit_layout(const CodecArgs& c, int64_t n) {
  FitLayout l{};
  l.codes = 0;
  l.sz = align256((size_t)c.H * n * c.code_words * 4);
  l.index = l.sz + align256((size_t)c.H * n * c.groups * 4);
  l.total = l.index + align256((size_t)c.H * n * c.index_bytes);
  return l;
}

// grid: H * ceil(C / 4) workgroups of 8 waves; wave w of block b: centroid 4 b + (w >> 1),
// channels 64 (w & 1) .. + 63
__global__ __launch_bounds__(512) void fit_update_kernel(const uint16_t* x, int64_t x_stride,
                                                         const void* index, int idxb, int64_t n,
                                                         int H, int C, uint16_t* centroids) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int blocks = (C + 3) / 4;
  const int h = blockIdx.x / blocks;
  const int j = 4 * (blockIdx.x % blocks) + (wave >> 1);
  if (j >= C) return;   // no barriers below: a wave past the table just ends
  const int c = 64 * (wave & 1) + lane;
  const uint8_t* idx8 = reinterpret_cast<const uint8_t*>(index) + (int64_t)h * n * idxb;
  const uint16_t* xh = x + (int64_t)h * FD + c;
  float acc = 0.0f;
  int64_t count = 0;
  for (int64_t t0 = 0; t0 < n; t0 += 64) {
    const int64_t t = t0 + lane;
    int a = -1;
    if (t < n) a = idxb == 1 ? (int)idx8[t] : (int)reinterpret_cast<const uint16_t*>(idx8)[t];
    uint64_t m = __ballot(a == j);
    count += __popcll(m);
    while (m) {   // wave-uniform: the same tokens for every lane, ascending
      const int b = __builtin_ctzll(m);
      m &= m - 1;
      acc += bf16_bits_to_f32(xh[(t0 + b) * x_stride]);
    }
  }
  if (count) centroids[((int64_t)h * C + j) * FD + c] = (uint16_t)f32_to_bf16_bits(acc / (float)count);
}

}  // namespace

size_t fit_workspace_bytes(const CodecArgs& c, int64_t n_tokens) {
  if (n_tokens <= 0) return 0;
  return fit_layout(c, n_tokens).total;
}

hipError_t launch_fit(const EncodeLaunch& a0, int iterations, hipStream_t s) {
  if (a0.n_tokens == 0 || iterations <= 0) return hipSuccess;
  if (a0.c.D != FD || a0.c.x_dtype != KVC_BF16 || a0.c.base != KVC_BASE_CENTROID)
    return hipErrorInvalidValue;
  const FitLayout l = fit_layout(a0.c, a0.n_tokens);
  char* w = reinterpret_cast<char*>(a0.workspace);
  EncodeLaunch a = a0;   // assignment: the encoder into a scratch store of n rows
  a.st.codes = reinterpret_cast<uint32_t*>(w + l.codes);
  a.st.sz = reinterpret_cast<uint32_t*>(w + l.sz);
  a.st.index = w + l.index;
  a.st.capacity = a0.n_tokens;
  a.token_offset = 0;
  a.recon = nullptr;
  a.pred = nullptr;
  a.workspace = nullptr;
  uint16_t* table = const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(a0.b.centroids));
  const dim3 grid((unsigned)(a0.c.H * ((a0.c.C + 3) / 4))), block(512);
  for (int it = 0; it < iterations; ++it) {
    hipError_t e = launch_encode(a, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fit_update_kernel, grid, block, 0, s,
                       reinterpret_cast<const uint16_t*>(a0.x), a0.x_stride, a.st.index,
                       a0.c.index_bytes, a0.n_tokens, a0.c.H, a0.c.C, table);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvc
