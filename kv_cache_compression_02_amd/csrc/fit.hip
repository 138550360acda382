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
// fit_update_kernel: a workgroup owns 4 centroids (a wave: 64 channels of one); it
// stages a chunk of the head's assignments in LDS, its 8 waves split the chunk and list
// each centroid's tokens in ascending order (ballots), and only those rows are read (8
// loads in flight), so the sums run in ascending token order (deterministic, fp32) and
// each token's row is read once per centroid half.  The mean is the fp32 sum divided by
// the count (IEEE division).
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

// grid: H * ceil(C / 4) workgroups of 8 waves, each for 4 centroids 4 b .. 4 b + 3.
// Per chunk of FCH tokens: the workgroup stages the head's assignments in LDS; wave w
// scans tokens [w FCH/8, (w + 1) FCH/8) of the chunk for the 4 centroids (a count pass,
// then a pass that writes each hit at its wave's offset, so every centroid's list is in
// ascending token order); then waves 2 q and 2 q + 1 (channel halves) read the rows of
// centroid 4 b + q's list, 8 loads in flight, and add them in list order.
constexpr int FCH = 2048;
constexpr int FSEG = FCH / 8;   // tokens a wave scans per chunk

__global__ __launch_bounds__(512) void fit_update_kernel(const uint16_t* x, int64_t x_stride,
                                                         const void* index, int idxb, int64_t n,
                                                         int H, int C, uint16_t* centroids) {
  __shared__ uint16_t sidx[FCH];
  __shared__ uint16_t list[4][FCH];
  __shared__ int cnt[8][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int blocks = (C + 3) / 4;
  const int h = blockIdx.x / blocks;
  const int j0 = 4 * (blockIdx.x % blocks);
  const int q = wave >> 1, j = j0 + q;
  const bool live = j < C;   // waves past the table still take part in the barriers
  const int c = 64 * (wave & 1) + lane;
  const uint8_t* idx8 = reinterpret_cast<const uint8_t*>(index) + (int64_t)h * n * idxb;
  const uint16_t* xh = x + (int64_t)h * FD + c;
  const uint64_t below = (1ull << lane) - 1;
  float acc = 0.0f;
  int64_t count = 0;
  for (int64_t base = 0; base < n; base += FCH) {
    const int len = (int)min<int64_t>(FCH, n - base);
    uint16_t st[FCH / 512];   // all of the thread's loads in flight before the stores
#pragma unroll
    for (int u = 0; u < FCH / 512; ++u) {
      const int e = tid + 512 * u;
      st[u] = e >= len ? (uint16_t)0xFFFFu
                       : (idxb == 1 ? (uint16_t)idx8[base + e]
                                    : reinterpret_cast<const uint16_t*>(idx8)[base + e]);
    }
#pragma unroll
    for (int u = 0; u < FCH / 512; ++u) sidx[tid + 512 * u] = st[u];   // 0xFFFF past len
    __syncthreads();
    // count pass over the wave's segment (tokens past len hold 0xFFFF: no centroid)
    int a[FSEG / 64];
#pragma unroll
    for (int u = 0; u < FSEG / 64; ++u) a[u] = (int)sidx[FSEG * wave + 64 * u + lane] - j0;
    int n4[4] = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < FSEG / 64; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) n4[r] += __popcll(__ballot(a[u] == r));
    if (lane < 4) cnt[wave][lane] = lane == 0 ? n4[0] : lane == 1 ? n4[1] : lane == 2 ? n4[2] : n4[3];
    __syncthreads();
    // write pass: each hit at (earlier waves' count) + (earlier hits of this wave)
    int off[4], tot[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      off[r] = 0;
      tot[r] = 0;
      for (int w = 0; w < 8; ++w) {
        const int v = cnt[w][r];
        if (w < wave) off[r] += v;
        tot[r] += v;
      }
    }
#pragma unroll
    for (int u = 0; u < FSEG / 64; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool hit = a[u] == r;
        const uint64_t m = __ballot(hit);
        if (hit) list[r][off[r] + __popcll(m & below)] = (uint16_t)(FSEG * wave + 64 * u + lane);
        off[r] += __popcll(m);
      }
    __syncthreads();
    if (live) {
      const int nm = q == 0 ? tot[0] : q == 1 ? tot[1] : q == 2 ? tot[2] : tot[3];
      count += nm;
      for (int k0 = 0; k0 < nm; k0 += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {   // unconditional loads (the last entry repeated) stay in flight together
          const int e = min(k0 + k, nm - 1);
          v[k] = bf16_bits_to_f32(xh[(base + list[q][e]) * x_stride]);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k0 + k < nm) acc += v[k];   // ascending token order
      }
    }
    __syncthreads();   // sidx, cnt and the lists are rewritten by the next chunk
  }
  if (live && count)
    centroids[((int64_t)h * C + j) * FD + c] = (uint16_t)f32_to_bf16_bits(acc / (float)count);
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
  a.index_only = true;   // the update reads the assignment only
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
