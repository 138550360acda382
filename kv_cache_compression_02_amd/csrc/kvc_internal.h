// Internal interface between the C-ABI entry points (api.hip) and the kernel
// translation units.  Host-side plain structs; no torch types anywhere.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

// Everything a codec kernel needs, resolved and validated on the host.
struct CodecArgs {
  int H = 0, D = 0, bits = 0, group = 0, base = 0, C = 0, rank = 0, n_inputs = 0, m = 0;
  int x_dtype = 0;
  int rot = 0;         // Hn residual transform width: 0, 16 or 64
  int vec_len = 0;     // values quantized per token-head (D, or m for COEFF)
  int code_words = 0;  // uint32 words per token-head
  int groups = 0;      // scale/zero words per token-head
  int index_bytes = 0; // 1 or 2 (0 when no index)
};

struct StoreArgs {
  uint32_t* codes = nullptr;
  uint32_t* sz = nullptr;
  void* index = nullptr;
  int64_t capacity = 0;
};

struct BaseArgs {
  const void* centroids = nullptr;
  const void* basis = nullptr;
  const void* prev0 = nullptr;
  const void* prev1 = nullptr;
  const void* aux = nullptr;
  const void* w_block = nullptr;
  const void* u = nullptr;
  const void* v_lr = nullptr;
  const float* coef_a = nullptr;
  const float* coef_b = nullptr;
  int64_t prev_stride = 0;
  const void* centroid_tables = nullptr;   // fp16 image of centroids (attention only)
};

struct EncodeLaunch {
  CodecArgs c;
  StoreArgs st;
  BaseArgs b;
  const void* x = nullptr;
  int64_t n_tokens = 0, x_stride = 0, token_offset = 0;
  void* recon = nullptr;
  float* pred = nullptr;
  void* workspace = nullptr;
  float* rank_buf = nullptr;   // DPLR rank-r intermediate [n][r] fp32; nullptr: in the workspace
  // only the centroid index is read back (the fit's assignment pass): the 16-token-wave
  // centroid encoder then writes the index alone; the other encoders write everything
  bool index_only = false;
};

struct DecodeLaunch {
  CodecArgs c;
  StoreArgs st;
  BaseArgs b;
  int64_t n_tokens = 0, token_offset = 0;
  void* out = nullptr;
  int out_dtype = 0;
  float* pred = nullptr;
  void* workspace = nullptr;
};

struct AttendLaunch {
  CodecArgs kc, vc;
  StoreArgs ks, vs;
  BaseArgs kb, vb;
  int64_t n_keys = 0, n_queries = 0;
  const void* q = nullptr;
  float scale = 0.f;
  float* out = nullptr;
  float* lse = nullptr;
  void* workspace = nullptr;      // optional: enables splitting the keys across workgroups
  size_t workspace_bytes = 0;
  int jensen = 0;                 // KVC_ATTEND_JENSEN: correct the compressed keys' logits
};

// Launchers (return hipSuccess or the launch error).
hipError_t launch_encode(const EncodeLaunch& a, hipStream_t s);
hipError_t launch_encode_pair(const EncodeLaunch& a, const EncodeLaunch& b, hipStream_t s);
hipError_t launch_decode(const DecodeLaunch& a, hipStream_t s);
hipError_t launch_attend(const AttendLaunch& a, hipStream_t s);
hipError_t launch_attend_mixed(const AttendLaunch& a, hipStream_t s);
hipError_t launch_attend_chunk(const AttendLaunch& a, const void* chunk_k, const void* chunk_v,
                               int64_t n_chunk, hipStream_t s);

// Fused predictor + quantizer for bf16 d = 128 (anchors, temporal keys and values,
// block-DPLR): returns false when a call is outside its shapes, else launches and
// stores the launch status in *err.  launch_predict_fused writes the prediction only
// (the decoder's base), with the same kernels and arithmetic as the encoder.
bool launch_encode_fused(const EncodeLaunch& a, hipStream_t s, hipError_t* err);
// compute units of the current device (256 if the query fails)
int cu_count();
bool launch_predict_fused(const EncodeLaunch& a, float* out, hipStream_t s, hipError_t* err);

// Whether the matrix-product predictor bases (DPLR, temporal values) are built.
bool predict_available();

// Workspace bytes that let attention split the keys across workgroups (0 when one
// pass is used anyway).
size_t attend_workspace_bytes(const CodecArgs& kc, int64_t n_keys, int64_t n_queries);
size_t attend_chunk_workspace_bytes(const CodecArgs& kc, int64_t n_keys, int64_t n_queries);
size_t attend_mixed_workspace_bytes(const CodecArgs& kc, int64_t n_keys, int64_t n_queries);
// fp16 centroid images for the decode-fused attention: header (per-head exponents and
// exactness flags, 256-byte padded) + [H][C][D] fp16
size_t centroid_tables_header_bytes(int H);
hipError_t launch_centroid_tables(const void* centroids, int H, int C, int D, void* tables,
                                  hipStream_t s);
// Online centroid fitting: `iterations` Lloyd steps on a.x (n_tokens rows) updating the
// table a.b.centroids in place; a.workspace holds a scratch store of n_tokens rows.
size_t fit_workspace_bytes(const CodecArgs& c, int64_t n_tokens);
hipError_t launch_fit(const EncodeLaunch& a, int iterations, hipStream_t s);

// Workspace bytes of the predictor paths (0 otherwise).
size_t encode_workspace_bytes(const CodecArgs& c, int64_t n_tokens);
// Where the DPLR rank-r intermediate t [n][r] fp32 lives: a.rank_buf when set, else the
// workspace after room for an fp32 prediction [n][H][d].
float* rank_intermediate(const EncodeLaunch& a);
// Whether an encode runs the fused predictor + quantizer kernel (the prediction then
// stays in registers; otherwise matrix-product bases first write an fp32 prediction).
bool encode_fused_shape(const EncodeLaunch& a);

}  // namespace kvc
