// Decode-fused attention over a compressed K/V history.
//
// Method: queries attend to the compressed history of keys and values (NanoKV
// abstract: repeated attention over history is the cost to cut); O =
// softmax(Q K^T * scale) V per head, no mask.  The decoded cache is what a
// bf16 (or fp32) cache would hold: every decoded value is rounded to the cache
// dtype before it meets a query.
//
// bf16 path (d = 128), one workgroup = 4 wave64 = 128 queries of one head:
//   per 64-key tile: all 256 threads decode K (row-major) and V (transposed) into
//   LDS as bf16, then each wave computes S^T = K Q^T for its 32 queries with
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
  int64_t cap;
  int bits, group, groups, words, idxb, C, mode;
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
constexpr int NW = 4;            // waves per workgroup
constexpr int QW = 32;           // queries per wave
constexpr int BQ = NW * QW;      // queries per workgroup
constexpr int DM = 128;          // head dim of the MFMA path
constexpr int KROW = DM + 8;     // K tile row (bf16 elements), padded
constexpr int VROW = BK + 4;     // V^T tile row (bf16 elements), padded

__global__ __launch_bounds__(NW * 64, 2) void attend_bf16_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[BK * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[DM * VROW];   // fp16 bits

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;     // which 8-wide k-slice of an MFMA operand
  const int col = lane & 31;      // query (S^T column) / row index of an operand
  const int nqb = (int)((p.nq + BQ - 1) / BQ);
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int h = tile / nqb;
  const int64_t q0 = (int64_t)(tile % nqb) * BQ + wave * QW;
  const int64_t myq = q0 + col;

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

  f32x16_t oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.0f;
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  for (int64_t k0 = 0; k0 < p.nk; k0 += BK) {
    __syncthreads();
    // ---- decode K tile: item -> (key = item / 16, chunk = item % 16), row-major
#pragma unroll
    for (int it = 0; it < (BK * DM / 8) / (NW * 64); ++it) {
      const int item = tid + it * NW * 64;
      const int kk = item >> 4, c8 = item & 15;
      const int64_t key = k0 + kk;
      uint4 w = {0u, 0u, 0u, 0u};
      if (key < p.nk) {
        float v[8];
        decode8<uint16_t, DM>(p.k, h, key, c8 * 8, v);
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        w.z = pack_bf16x2(v[4], v[5]);
        w.w = pack_bf16x2(v[6], v[7]);
      }
      *reinterpret_cast<uint4*>(&k_lds[kk * KROW + c8 * 8]) = w;
    }
    // ---- decode V tile transposed: thread -> (chunk = tid / 16, keys 4*(tid%16)..+3)
    {
      const int c8 = tid >> 4;
      const int kq = tid & 15;
      float v[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t key = k0 + 4 * kq + j;
        if (key < p.nk) decode8<uint16_t, DM>(p.v, h, key, c8 * 8, v[j]);
        else {
#pragma unroll
          for (int k = 0; k < 8; ++k) v[j][k] = 0.0f;
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        // bf16 cache value, held exactly in fp16 (round-toward-zero is exact here)
        uint2 w;
        w.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(round_bf16_f32(v[0][c]),
                                                                      round_bf16_f32(v[1][c])));
        w.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(round_bf16_f32(v[2][c]),
                                                                      round_bf16_f32(v[3][c])));
        *reinterpret_cast<uint2*>(&v_lds[(c8 * 8 + c) * VROW + 4 * kq]) = w;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for 64 keys (two 32-key blocks)
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t*>(&k_lds[(kb * 32 + col) * KROW + 16 * ks + 8 * half]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], sacc[kb], 0, 0, 0);
      }
    }

    // ---- online softmax (log2 domain); lane = query `col`, 32 of the tile's keys
    float s[32];
    float mloc = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t key = k0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        float x = sacc[kb][r] * p.scale_log2;
        x = (key < p.nk) ? x : -__builtin_inff();
        s[kb * 16 + r] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
    float lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      s[i] = __builtin_amdgcn_exp2f(s[i] - m_new);
      lsum += s[i];
    }
    lsum += __shfl_xor(lsum, 32);
    l_run = l_run * corr + lsum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[d][r] *= corr;

    // ---- P^T operands (fp16, nearest even): (kb, hf) covers keys
    //      32*kb + 16*hf + {4*half+0..3, 8+4*half+0..3}
    f16x8_t pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const float* sp = &s[kb * 16 + hf * 8];
        f16x8_t t;
#pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = (_Float16)sp[j];
        pb[kb][hf] = t;
      }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint16_t* vrow = &v_lds[(d * 32 + col) * VROW];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int kbase = kb * 32 + hf * 16 + 4 * half;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + kbase);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + kbase + 8);
          const uint4 w = {lo.x, lo.y, hi.x, hi.y};
          const f16x8_t a = __builtin_bit_cast(f16x8_t, w);
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[kb][hf], oacc[d], 0, 0, 0);
        }
    }
  }

  // ---- epilogue: O[q][h][c] = O^T[c][q] / l
  if (myq < p.nq) {
    const float inv = 1.0f / l_run;
    float* op = p.out + (myq * p.H + h) * DM;
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
    if (p.lse && half == 0)
      p.lse[(int64_t)h * p.nq + myq] = (m_run + __log2f(l_run)) * 0.69314718055994531f;
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
  s.mode = c.base == KVC_BASE_CENTROID ? SRC_CENTROID : SRC_NONE;
  return s;
}

}  // namespace

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
  if (a.kc.x_dtype == KVC_BF16) {
    const int nqb = (int)((a.n_queries + BQ - 1) / BQ);
    hipLaunchKernelGGL(attend_bf16_kernel, dim3(nqb * a.kc.H), dim3(NW * 64), 0, s, p);
  } else {
    const int nqb = (int)((a.n_queries + 63) / 64);
    if (a.kc.D == 128)
      hipLaunchKernelGGL(attend_f32_kernel<128>, dim3(nqb * a.kc.H), dim3(64), 0, s, p);
    else
      hipLaunchKernelGGL(attend_f32_kernel<64>, dim3(nqb * a.kc.H), dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace kvc
