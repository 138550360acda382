// Matrix-product predictor bases.
//
// * Cross-layer block-DPLR (Coral-KV arXiv 2610.12514, Fig. 3): at layer l the
//   reconstructed cache of layer l-1 predicts keys, and [K_l, V_{l-1}] predicts
//   values, each through a per-head block-diagonal map plus a global rank-r map:
//       pred[h] = W_h [prev0_h ; prev1_h] + U (v_lr [prev0 ; prev1])[h].
// * Temporal key->value cross predictor (TempoKV arXiv 2610.15324, Fig. 2b): the
//   value of frame t is predicted from the aligned reconstructed key and the
//   previous reconstructed value: pred[h] = M_h aux_h + beta_h * prev0_h.
//
// Every product runs on one tiled kernel, C (+)= A W^T with bf16 operands and fp32
// accumulation on v_mfma_f32_32x32x16_bf16; both operands are contiguous along the
// contraction, so each lane loads 16-byte fragments straight from global memory
// (the weights are small and stay in L2).  The rank-r intermediate is kept in fp32
// and enters the second product as bf16 high + low parts (about 2^-16 relative).
// The result is the fp32 base the quantizer subtracts.
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

struct GemmParams {
  const void* A;        // M x K rows, bf16 or fp32
  int64_t lda, a_bs;    // row stride, batch stride (elements)
  const uint16_t* W;    // N x K rows, bf16
  int64_t ldw, w_bs;
  float* C;             // M x N fp32
  int64_t ldc, c_bs;
  int M, N, K, accumulate;
};

template <bool AF32>
__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int z = blockIdx.z;
  const int m = blockIdx.x * 64 + 32 * (wave & 1) + col;     // A row this lane feeds
  const int n = blockIdx.y * 64 + 32 * (wave >> 1) + col;    // W row this lane feeds
  const bool mok = m < p.M, nok = n < p.N;
  const uint16_t* wrow = p.W + z * p.w_bs + (int64_t)(nok ? n : 0) * p.ldw + 8 * half;
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  for (int k0 = 0; k0 < p.K; k0 += 16) {
    bf16x8_t b = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    if (nok) b = *reinterpret_cast<const bf16x8_t*>(wrow + k0);
    if constexpr (AF32) {
      const float* arow = reinterpret_cast<const float*>(p.A) + z * p.a_bs +
                          (int64_t)(mok ? m : 0) * p.lda + 8 * half + k0;
      float av[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (mok) {
        const float4 x0 = *reinterpret_cast<const float4*>(arow);
        const float4 x1 = *reinterpret_cast<const float4*>(arow + 4);
        av[0] = x0.x; av[1] = x0.y; av[2] = x0.z; av[3] = x0.w;
        av[4] = x1.x; av[5] = x1.y; av[6] = x1.z; av[7] = x1.w;
      }
      bf16x8_t ahi, alo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t hb = f32_to_bf16_bits(av[i]);
        ahi[i] = (short)hb;
        alo[i] = (short)f32_to_bf16_bits(av[i] - bf16_bits_to_f32(hb));
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, b, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, b, acc, 0, 0, 0);
    } else {
      const uint16_t* arow = reinterpret_cast<const uint16_t*>(p.A) + z * p.a_bs +
                             (int64_t)(mok ? m : 0) * p.lda + 8 * half + k0;
      bf16x8_t a = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      if (mok) a = *reinterpret_cast<const bf16x8_t*>(arow);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
  }
  // acc[r] = C[row 8(r/4) + 4 half + r%4 of the wave's block][column col]
  const int cn = blockIdx.y * 64 + 32 * (wave >> 1) + col;
  if (cn >= p.N) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int cm = blockIdx.x * 64 + 32 * (wave & 1) + 8 * (r >> 2) + 4 * half + (r & 3);
    if (cm < p.M) {
      float* c = p.C + z * p.c_bs + (int64_t)cm * p.ldc + cn;
      *c = p.accumulate ? *c + acc[r] : acc[r];
    }
  }
}

hipError_t gemm(bool af32, const void* A, int64_t lda, int64_t a_bs, const uint16_t* W,
                int64_t ldw, int64_t w_bs, float* C, int64_t ldc, int64_t c_bs, int M, int N,
                int K, int batch, bool accumulate, hipStream_t s) {
  GemmParams p{A, lda, a_bs, W, ldw, w_bs, C, ldc, c_bs, M, N, K, accumulate ? 1 : 0};
  dim3 grid((M + 63) / 64, (N + 63) / 64, batch);
  if (af32)
    hipLaunchKernelGGL(gemm_nt_kernel<true>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(gemm_nt_kernel<false>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// base[n][h][c] = base[n][h][c] + coef[h][c] * prev[n][h][c]  (one rounded fp32 op each)
__global__ void add_scaled_kernel(float* base, const float* coef, const uint16_t* prev,
                                  int64_t prev_stride, int64_t n_tokens, int HD) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n_tokens * HD) return;
  const int64_t n = e / HD;
  const int j = (int)(e % HD);
  const float t = coef[j] * bf16_bits_to_f32(prev[n * prev_stride + j]);
  base[e] = base[e] + t;
}

}  // namespace

bool predict_available() { return true; }

float* rank_intermediate(const EncodeLaunch& a) {
  if (a.rank_buf) return a.rank_buf;
  return reinterpret_cast<float*>(reinterpret_cast<char*>(a.workspace) +
                                  (size_t)a.n_tokens * a.c.H * a.c.D * sizeof(float));
}

size_t encode_workspace_bytes(const CodecArgs& c, int64_t n_tokens) {
  const size_t pred = (size_t)n_tokens * c.H * c.D * sizeof(float);
  if (c.base == KVC_BASE_DPLR) return pred + (size_t)n_tokens * c.rank * sizeof(float);
  if (c.base == KVC_BASE_TEMPORAL) return pred;
  return 0;
}

// Writes the fp32 prediction [n][H][D] into base_out.  DPLR also uses the workspace
// after the prediction block for the rank-r intermediate.
hipError_t launch_predict(const EncodeLaunch& a, float* base_out, hipStream_t s) {
  const int H = a.c.H, D = a.c.D;
  const int64_t N = a.n_tokens, HD = (int64_t)H * D, ps = a.b.prev_stride;
  const int M = (int)N;
  if (N == 0) return hipSuccess;
  hipError_t e;
  if (launch_predict_fused(a, base_out, s, &e)) return e;
  if (a.c.base == KVC_BASE_TEMPORAL) {
    // M_h aux_h, then + beta_h * prev0_h
    e = gemm(false, a.b.aux, ps, D, reinterpret_cast<const uint16_t*>(a.b.w_block), D,
             (int64_t)D * D, base_out, HD, D, M, D, D, H, false, s);
    if (e != hipSuccess) return e;
    const int64_t total = N * HD;
    hipLaunchKernelGGL(add_scaled_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       base_out, a.b.coef_a, reinterpret_cast<const uint16_t*>(a.b.prev0), ps, N,
                       (int)HD);
    return hipGetLastError();
  }
  if (a.c.base != KVC_BASE_DPLR) return hipErrorInvalidValue;
  const int r = a.c.rank, nin = a.c.n_inputs;
  float* t = rank_intermediate(a);
  const uint16_t* vlr = reinterpret_cast<const uint16_t*>(a.b.v_lr);     // [r][nin*H*D]
  const uint16_t* wb = reinterpret_cast<const uint16_t*>(a.b.w_block);   // [H][D][nin*D]
  const uint16_t* u = reinterpret_cast<const uint16_t*>(a.b.u);          // [H*D][r]
  const void* in[2] = {a.b.prev0, a.b.prev1};
  // rank-r intermediate t = v_lr [prev0 ; prev1]  (fp32, [N][r])
  for (int j = 0; j < nin; ++j) {
    e = gemm(false, in[j], ps, 0, vlr + (int64_t)j * HD, (int64_t)nin * HD, 0, t, r, 0, M, r,
             (int)HD, 1, j > 0, s);
    if (e != hipSuccess) return e;
  }
  // per head: W_h [prev0_h ; prev1_h] + U_h t
  for (int j = 0; j < nin; ++j) {
    e = gemm(false, reinterpret_cast<const uint16_t*>(in[j]), ps, D, wb + (int64_t)j * D,
             (int64_t)nin * D, (int64_t)D * nin * D, base_out, HD, D, M, D, D, H, j > 0, s);
    if (e != hipSuccess) return e;
  }
  return gemm(true, t, r, 0, u, r, (int64_t)D * r, base_out, HD, D, M, D, r, H, true, s);
}

}  // namespace kvc
