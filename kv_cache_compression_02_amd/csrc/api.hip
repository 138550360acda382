// C-ABI entry points: host-side validation, then an asynchronous launch on the
// caller's stream.  No device memory is allocated here; no exception crosses the
// ABI.  See include/kvc.h for the contract of every call.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "kvc.h"
#include "kvc_internal.h"

#include <vector>

using namespace kvc;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validate a codec and derive the per-vector layout.
kvc_status resolve_codec(const kvc_codec* c, CodecArgs* out) {
  if (!c) return KVC_E_NULL;
  CodecArgs a;
  a.H = c->heads;
  a.D = c->head_dim;
  a.bits = c->bits;
  a.group = c->group;
  a.base = c->base;
  a.C = c->n_centroids;
  a.rank = c->rank;
  a.n_inputs = c->n_inputs;
  a.m = c->coeff_dim;
  a.x_dtype = c->x_dtype;
  a.rot = c->rotation;
  if (a.H < 1 || a.H > 4096) return KVC_E_SHAPE;
  if (a.D != 64 && a.D != 128) return KVC_E_UNSUPPORTED;
  if (a.bits == 16) {   // uncompressed bf16 cache, token-major (attention inputs only)
    if (a.base != KVC_BASE_NONE || a.x_dtype != KVC_BF16 || a.rot != 0) return KVC_E_UNSUPPORTED;
    a.vec_len = a.D;
    a.group = a.D;
    a.code_words = a.D / 2;
    a.groups = 0;
    a.index_bytes = 0;
    *out = a;
    return KVC_OK;
  }
  if (a.bits != 2 && a.bits != 4) return KVC_E_UNSUPPORTED;
  if (a.group != 16 && a.group != 32 && a.group != 64 && a.group != 128) return KVC_E_UNSUPPORTED;
  if (a.x_dtype != KVC_F32 && a.x_dtype != KVC_BF16) return KVC_E_UNSUPPORTED;
  a.vec_len = a.D;
  switch (a.base) {
    case KVC_BASE_NONE: break;
    case KVC_BASE_CENTROID:
      if (a.C < 1 || a.C > 65535) return KVC_E_SHAPE;
      break;
    case KVC_BASE_COEFF:
      if (a.C < 1 || a.C > 65535) return KVC_E_SHAPE;
      if (a.m != 16) return KVC_E_UNSUPPORTED;
      a.vec_len = a.m;
      break;
    case KVC_BASE_TEMPORAL:
      if (a.x_dtype != KVC_BF16) return KVC_E_UNSUPPORTED;
      break;
    case KVC_BASE_DPLR:
      if (a.x_dtype != KVC_BF16 || a.D != 128) return KVC_E_UNSUPPORTED;
      if (a.rank < 16 || a.rank > 256 || a.rank % 16) return KVC_E_SHAPE;
      if (a.n_inputs != 1 && a.n_inputs != 2) return KVC_E_SHAPE;
      break;
    default: return KVC_E_UNSUPPORTED;
  }
  if ((a.base == KVC_BASE_DPLR || a.base == KVC_BASE_TEMPORAL) && !predict_available()) {
    // temporal keys are elementwise and always available; the matrix-product
    // predictors are checked again where the base parameters are known
    if (a.base == KVC_BASE_DPLR) return KVC_E_UNSUPPORTED;
  }
  if (a.vec_len % a.group) return KVC_E_SHAPE;
  if (a.rot != 0) {   // Hn residual transform: the 16-token-wave centroid encoder and the
                      // fused predictor + quantizer (anchors, temporal and block-DPLR bases)
    if (a.rot != 16 && a.rot != 64) return KVC_E_UNSUPPORTED;
    if (a.x_dtype != KVC_BF16 || a.D != 128 || a.group > 64 || a.group % a.rot != 0)
      return KVC_E_UNSUPPORTED;
    if (a.base == KVC_BASE_CENTROID) {
      if (a.C > 512) return KVC_E_UNSUPPORTED;
    } else if (a.base == KVC_BASE_DPLR) {
      if (a.rank > 64) return KVC_E_UNSUPPORTED;
    } else if (a.base != KVC_BASE_NONE && a.base != KVC_BASE_TEMPORAL) {
      return KVC_E_UNSUPPORTED;
    }
  }
  a.code_words = a.vec_len * a.bits / 32;
  a.groups = a.vec_len / a.group;
  a.index_bytes = (a.base == KVC_BASE_CENTROID || a.base == KVC_BASE_COEFF) ? (a.C <= 256 ? 1 : 2) : 0;
  *out = a;
  return KVC_OK;
}

kvc_status resolve_store(const kvc_store* s, const CodecArgs& c, StoreArgs* out) {
  if (!s) return KVC_E_NULL;
  if (!s->codes || (c.groups && !s->scale_zero)) return KVC_E_NULL;
  if (c.index_bytes && !s->index) return KVC_E_NULL;
  if (!aligned16(s->codes) || (c.groups && !aligned16(s->scale_zero))) return KVC_E_ALIGN;
  if (c.index_bytes && !aligned16(s->index)) return KVC_E_ALIGN;
  if (s->capacity < 0) return KVC_E_SHAPE;
  out->codes = s->codes;
  out->sz = s->scale_zero;
  out->index = s->index;
  out->capacity = s->capacity;
  return KVC_OK;
}

kvc_status resolve_base(const kvc_base_params* b, const CodecArgs& c, BaseArgs* out, bool need_prev) {
  if (c.base == KVC_BASE_NONE) return KVC_OK;
  if (!b) return KVC_E_NULL;
  BaseArgs a;
  a.centroids = b->centroids;
  a.basis = b->basis;
  a.prev0 = b->prev0;
  a.prev1 = b->prev1;
  a.aux = b->aux;
  a.w_block = b->w_block;
  a.u = b->u;
  a.v_lr = b->v_lr;
  a.coef_a = b->coef_a;
  a.coef_b = b->coef_b;
  a.centroid_tables = b->centroid_tables;
  a.prev_stride = b->prev_token_stride ? b->prev_token_stride : (int64_t)c.H * c.D;
  if (a.prev_stride < (int64_t)c.H * c.D) return KVC_E_SHAPE;
  switch (c.base) {
    case KVC_BASE_CENTROID:
      if (!a.centroids) return KVC_E_NULL;
      if (!aligned16(a.centroids)) return KVC_E_ALIGN;
      break;
    case KVC_BASE_COEFF:
      if (!a.centroids || !a.basis) return KVC_E_NULL;
      if (!aligned16(a.centroids) || !aligned16(a.basis)) return KVC_E_ALIGN;
      break;
    case KVC_BASE_TEMPORAL:
      if (!need_prev) break;
      if (!a.prev0 || !a.coef_a) return KVC_E_NULL;
      if (a.prev_stride % 8) return KVC_E_ALIGN;   // 16-byte row pieces of the inputs
      if (a.w_block) {   // values: M aux + beta prev0
        if (!predict_available()) return KVC_E_UNSUPPORTED;
        if (!a.aux) return KVC_E_NULL;
        if (a.coef_b) return KVC_E_SHAPE;
      } else {           // keys: a prev0 + b prev1
        if (!a.prev1 || !a.coef_b) return KVC_E_NULL;
      }
      break;
    case KVC_BASE_DPLR:
      if (!need_prev) break;
      if (!a.prev0 || !a.w_block || !a.u || !a.v_lr) return KVC_E_NULL;
      if (a.prev_stride % 8) return KVC_E_ALIGN;
      if (c.n_inputs == 2 && !a.prev1) return KVC_E_NULL;
      break;
    default: break;
  }
  const void* ptrs[] = {a.prev0, a.prev1, a.aux, a.w_block, a.u, a.v_lr, a.coef_a, a.coef_b};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KVC_E_ALIGN;
  *out = a;
  return KVC_OK;
}

kvc_status from_hip(hipError_t e) { return e == hipSuccess ? KVC_OK : KVC_E_DEVICE; }

// Matrix-product bases need a buffer for the fp32 prediction (pred_out or the
// workspace) and, for DPLR, the workspace for the rank-r intermediate.
kvc_status check_predict_workspace(const CodecArgs& c, const BaseArgs& b, int64_t n_tokens,
                                   const float* pred_out, const void* workspace,
                                   size_t workspace_bytes) {
  const bool matrix = c.base == KVC_BASE_DPLR || (c.base == KVC_BASE_TEMPORAL && b.w_block);
  if (!matrix || n_tokens == 0) return KVC_OK;
  if (b.prev_stride % 8) return KVC_E_ALIGN;   // 16-byte fragments of the inputs
  const size_t need = encode_workspace_bytes(c, n_tokens);
  if (c.base == KVC_BASE_DPLR || !pred_out) {
    if (!workspace || workspace_bytes < need) return KVC_E_WORKSPACE;
    if (!aligned16(workspace)) return KVC_E_ALIGN;
  }
  return KVC_OK;
}

}  // namespace

extern "C" {

int32_t kvc_abi_version(void) { return KVC_ABI_VERSION; }

const char* kvc_status_str(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_E_NULL: return "a required pointer is NULL";
    case KVC_E_SHAPE: return "sizes inconsistent or out of range";
    case KVC_E_UNSUPPORTED: return "unsupported codec, dtype or size";
    case KVC_E_ALIGN: return "device pointer not 16-byte aligned";
    case KVC_E_WORKSPACE: return "workspace too small";
    case KVC_E_DEVICE: return "HIP runtime error";
  }
  return "unknown status";
}

kvc_status kvc_store_bytes(const kvc_codec* codec, int64_t capacity, size_t* codes_bytes,
                           size_t* scale_zero_bytes, size_t* index_bytes) {
  CodecArgs c;
  kvc_status st = resolve_codec(codec, &c);
  if (st != KVC_OK) return st;
  if (capacity < 0) return KVC_E_SHAPE;
  const size_t rows = (size_t)c.H * (size_t)capacity;
  if (codes_bytes) *codes_bytes = rows * c.code_words * 4u;   // bits 16: the bf16 cache
  if (scale_zero_bytes) *scale_zero_bytes = rows * c.groups * 4u;
  if (index_bytes) *index_bytes = rows * c.index_bytes;
  return KVC_OK;
}

size_t kvc_workspace_bytes(int32_t op, const kvc_codec* codec, int64_t n_tokens, int64_t n_queries) {
  CodecArgs c;
  if (resolve_codec(codec, &c) != KVC_OK || n_tokens < 0) return 0;
  if (op == KVC_OP_ENCODE || op == KVC_OP_DECODE) return encode_workspace_bytes(c, n_tokens);
  if (op == KVC_OP_ATTEND) return attend_workspace_bytes(c, n_tokens, n_queries);
  if (op == KVC_OP_ATTEND_MIXED) return attend_mixed_workspace_bytes(c, n_tokens, n_queries);
  if (op == KVC_OP_ATTEND_CHUNK) return attend_chunk_workspace_bytes(c, n_tokens, n_queries);
  if (op == KVC_OP_FIT) return fit_workspace_bytes(c, n_tokens);
  return 0;
}

// Validation shared by kvc_encode and kvc_encode_noalloc: everything but the workspace.
static kvc_status prepare_encode(const kvc_codec* codec, const void* x, int64_t n_tokens,
                                 int64_t x_token_stride, const kvc_base_params* base,
                                 const kvc_store* dst, int64_t token_offset, void* recon_out,
                                 float* pred_out, EncodeLaunch* out) {
  EncodeLaunch& a = *out;
  kvc_status st = resolve_codec(codec, &a.c);
  if (st != KVC_OK) return st;
  if (a.c.bits == 16) return KVC_E_UNSUPPORTED;
  if (n_tokens < 0 || token_offset < 0) return KVC_E_SHAPE;
  if (!x && n_tokens > 0) return KVC_E_NULL;   // an empty call may pass NULL buffers
  if (!aligned16(x) || (recon_out && !aligned16(recon_out)) || (pred_out && !aligned16(pred_out)))
    return KVC_E_ALIGN;
  const int64_t hd = (int64_t)a.c.H * a.c.D;
  const int64_t stride = x_token_stride ? x_token_stride : hd;
  if (stride < hd) return KVC_E_SHAPE;
  st = resolve_store(dst, a.c, &a.st);
  if (st != KVC_OK) return st;
  if (token_offset + n_tokens > a.st.capacity) return KVC_E_SHAPE;
  st = resolve_base(base, a.c, &a.b, true);
  if (st != KVC_OK) return st;
  if (a.c.base == KVC_BASE_COEFF && recon_out) return KVC_E_UNSUPPORTED;
  // rotated codecs: strides of 8 elements; the centroid encoder returns the store only
  if (a.c.rot != 0 && (stride % 8 != 0 || (a.c.base == KVC_BASE_CENTROID && (recon_out || pred_out))))
    return KVC_E_UNSUPPORTED;
  a.x = x;
  a.n_tokens = n_tokens;
  a.x_stride = stride;
  a.token_offset = token_offset;
  a.recon = recon_out;
  a.pred = pred_out;
  return KVC_OK;
}

kvc_status kvc_encode(const kvc_codec* codec, const void* x, int64_t n_tokens,
                      int64_t x_token_stride, const kvc_base_params* base, const kvc_store* dst,
                      int64_t token_offset, void* recon_out, float* pred_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  EncodeLaunch a;
  kvc_status st = prepare_encode(codec, x, n_tokens, x_token_stride, base, dst, token_offset,
                                 recon_out, pred_out, &a);
  if (st != KVC_OK) return st;
  st = check_predict_workspace(a.c, a.b, n_tokens, pred_out, workspace, workspace_bytes);
  if (st != KVC_OK) return st;
  a.workspace = workspace;
  return from_hip(launch_encode(a, reinterpret_cast<hipStream_t>(stream)));
}

kvc_status kvc_encode_kv(const kvc_codec* codec, const void* xk, const void* xv, int64_t n_tokens,
                         int64_t x_token_stride, const kvc_base_params* kbase,
                         const kvc_base_params* vbase, const kvc_store* kdst, const kvc_store* vdst,
                         int64_t token_offset, void* stream) {
  EncodeLaunch a, b;
  kvc_status st = prepare_encode(codec, xk, n_tokens, x_token_stride, kbase, kdst, token_offset,
                                 nullptr, nullptr, &a);
  if (st != KVC_OK) return st;
  st = prepare_encode(codec, xv, n_tokens, x_token_stride, vbase, vdst, token_offset, nullptr,
                      nullptr, &b);
  if (st != KVC_OK) return st;
  // bases that need a workspace (block-DPLR, temporal values) are not taken here
  if (check_predict_workspace(a.c, a.b, n_tokens, nullptr, nullptr, 0) != KVC_OK ||
      check_predict_workspace(b.c, b.b, n_tokens, nullptr, nullptr, 0) != KVC_OK)
    return KVC_E_UNSUPPORTED;
  if (n_tokens > 0 && (kdst->codes == vdst->codes || kdst->scale_zero == vdst->scale_zero ||
                       (a.c.index_bytes && kdst->index == vdst->index)))
    return KVC_E_SHAPE;   // the two stores overlap
  return from_hip(launch_encode_pair(a, b, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Scratch of kvc_encode_noalloc (the cross-layer predictor's rank-r intermediate), one
// copy per GPU, held by the loaded library until the process ends.  In host code
// `scratch` is only a handle: its device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and that pointer is what kernels receive.
static __device__ __align__(256) unsigned char scratch[KVC_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES];

hipError_t scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

kvc_status kvc_encode_noalloc(const kvc_codec* codec, const void* x, int64_t n_tokens,
                              int64_t x_token_stride, const kvc_base_params* base,
                              const kvc_store* dst, int64_t token_offset, void* recon_out,
                              float* pred_out, void* stream) {
  EncodeLaunch a;
  kvc_status st = prepare_encode(codec, x, n_tokens, x_token_stride, base, dst, token_offset,
                                 recon_out, pred_out, &a);
  if (st != KVC_OK) return st;
  const bool matrix = a.c.base == KVC_BASE_DPLR || (a.c.base == KVC_BASE_TEMPORAL && a.b.w_block);
  if (matrix && n_tokens > 0) {
    // outside the fused kernel's shapes the prediction goes through an fp32 buffer, which
    // only pred_out can provide here
    if (!encode_fused_shape(a) && !pred_out) return KVC_E_UNSUPPORTED;
    if (a.c.base == KVC_BASE_DPLR) {
      const size_t need = (size_t)n_tokens * a.c.rank * sizeof(float);
      if (need > (size_t)KVC_NOALLOC_SCRATCH_BYTES) return KVC_E_WORKSPACE;
      void* ptr = nullptr;
      st = from_hip(scratch_for_current_device(&ptr));
      if (st != KVC_OK) return st;
      a.rank_buf = reinterpret_cast<float*>(ptr);   // fully written by the rank kernel first
    }
  }
  return from_hip(launch_encode(a, reinterpret_cast<hipStream_t>(stream)));
}

kvc_status kvc_fit_centroids(const kvc_codec* codec, const void* x, int64_t n_tokens,
                             int64_t x_token_stride, void* centroids, int32_t iterations,
                             void* workspace, size_t workspace_bytes, void* stream) {
  EncodeLaunch a;
  kvc_status st = resolve_codec(codec, &a.c);
  if (st != KVC_OK) return st;
  if (a.c.base != KVC_BASE_CENTROID || a.c.x_dtype != KVC_BF16 || a.c.D != 128 || a.c.bits == 16)
    return KVC_E_UNSUPPORTED;
  if (n_tokens < 0 || iterations < 0) return KVC_E_SHAPE;
  const int64_t hd = (int64_t)a.c.H * a.c.D;
  const int64_t stride = x_token_stride ? x_token_stride : hd;
  if (stride < hd || stride % 8) return KVC_E_SHAPE;
  if (n_tokens == 0 || iterations == 0) return KVC_OK;
  if (!x || !centroids) return KVC_E_NULL;
  if (!aligned16(x) || !aligned16(centroids) || (workspace && !aligned16(workspace))) return KVC_E_ALIGN;
  if (!workspace || workspace_bytes < fit_workspace_bytes(a.c, n_tokens)) return KVC_E_WORKSPACE;
  a.x = x;
  a.n_tokens = n_tokens;
  a.x_stride = stride;
  a.b.centroids = centroids;
  a.b.prev_stride = hd;
  a.workspace = workspace;
  return from_hip(launch_fit(a, iterations, reinterpret_cast<hipStream_t>(stream)));
}

size_t kvc_centroid_tables_bytes(const kvc_codec* codec) {
  CodecArgs c;
  if (resolve_codec(codec, &c) != KVC_OK) return 0;
  if ((c.base != KVC_BASE_CENTROID && c.base != KVC_BASE_COEFF) || c.x_dtype != KVC_BF16 ||
      c.D != 128)
    return 0;
  return centroid_tables_header_bytes(c.H) + (size_t)c.H * c.C * c.D * 2;
}

kvc_status kvc_centroid_tables(const kvc_codec* codec, const void* centroids, void* tables,
                               size_t tables_bytes, void* stream) {
  CodecArgs c;
  kvc_status st = resolve_codec(codec, &c);
  if (st != KVC_OK) return st;
  if ((c.base != KVC_BASE_CENTROID && c.base != KVC_BASE_COEFF) || c.x_dtype != KVC_BF16 ||
      c.D != 128)
    return KVC_E_UNSUPPORTED;
  if (!centroids || !tables) return KVC_E_NULL;
  if (!aligned16(centroids) || !aligned16(tables)) return KVC_E_ALIGN;
  if (tables_bytes < kvc_centroid_tables_bytes(codec)) return KVC_E_SHAPE;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_centroid_tables(centroids, c.H, c.C, c.D, tables, s);
  if (e != hipSuccess) return KVC_E_DEVICE;
  std::vector<int32_t> exact((size_t)c.H);
  e = hipMemcpyAsync(exact.data(), reinterpret_cast<const int32_t*>(tables) + c.H,
                     sizeof(int32_t) * c.H, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return KVC_E_DEVICE;
  for (int32_t v : exact)
    if (v != 1) return KVC_E_UNSUPPORTED;
  return KVC_OK;
}

kvc_status kvc_decode(const kvc_codec* codec, const kvc_store* src, int64_t token_offset,
                      int64_t n_tokens, const kvc_base_params* base, void* out, int32_t out_dtype,
                      float* pred_out, void* workspace, size_t workspace_bytes, void* stream) {
  DecodeLaunch a;
  kvc_status st = resolve_codec(codec, &a.c);
  if (st != KVC_OK) return st;
  if (a.c.base == KVC_BASE_COEFF || a.c.bits == 16) return KVC_E_UNSUPPORTED;
  if (n_tokens < 0 || token_offset < 0) return KVC_E_SHAPE;
  if (!out && n_tokens > 0) return KVC_E_NULL;
  if (!aligned16(out) || (pred_out && !aligned16(pred_out))) return KVC_E_ALIGN;
  if (out_dtype != KVC_F32 && out_dtype != KVC_BF16) return KVC_E_UNSUPPORTED;
  st = resolve_store(src, a.c, &a.st);
  if (st != KVC_OK) return st;
  if (token_offset + n_tokens > a.st.capacity) return KVC_E_SHAPE;
  st = resolve_base(base, a.c, &a.b, true);
  if (st != KVC_OK) return st;
  st = check_predict_workspace(a.c, a.b, n_tokens, pred_out, workspace, workspace_bytes);
  if (st != KVC_OK) return st;
  a.workspace = workspace;
  a.n_tokens = n_tokens;
  a.token_offset = token_offset;
  a.out = out;
  a.out_dtype = out_dtype;
  a.pred = pred_out;
  return from_hip(launch_decode(a, reinterpret_cast<hipStream_t>(stream)));
}

// The bf16 attention kernels address each head's code and scale/zero rows (and a dense
// cache as a whole) through buffer resources with 32-bit byte ranges.
static bool attend_ranges_fit(const CodecArgs& c, const StoreArgs& s) {
  const int64_t lim = (int64_t)1 << 31;
  if (c.bits == 16) return (int64_t)s.capacity * c.H * c.D * 2 < lim;
  return (int64_t)s.capacity * c.code_words * 4 < lim && (int64_t)s.capacity * c.groups * 4 < lim &&
         (int64_t)s.capacity * c.index_bytes < lim;
}

static kvc_status check_attend(const kvc_codec* kc, const kvc_store* k, const kvc_base_params* kp,
                               const kvc_codec* vc, const kvc_store* v, const kvc_base_params* vp,
                               int64_t n_keys, const void* q, int64_t n_queries, float scale,
                               float* out, float* lse, AttendLaunch* a) {
  // the softmax scale must be finite and positive: the bf16 kernels' lazy running max
  // assumes that larger raw scores give larger logits
  if (!(scale > 0.0f) || !(scale < __builtin_inff())) return KVC_E_SHAPE;
  kvc_status st = resolve_codec(kc, &a->kc);
  if (st != KVC_OK) return st;
  st = resolve_codec(vc, &a->vc);
  if (st != KVC_OK) return st;
  if (n_keys < 1 || n_queries < 0) return KVC_E_SHAPE;
  if ((!q || !out) && n_queries > 0) return KVC_E_NULL;
  if (!aligned16(q) || !aligned16(out) || (lse && !aligned16(lse))) return KVC_E_ALIGN;
  if (a->kc.H != a->vc.H || a->kc.D != a->vc.D || a->kc.x_dtype != a->vc.x_dtype) return KVC_E_SHAPE;
  st = resolve_store(k, a->kc, &a->ks);
  if (st != KVC_OK) return st;
  st = resolve_store(v, a->vc, &a->vs);
  if (st != KVC_OK) return st;
  if (n_keys > a->ks.capacity || n_keys > a->vs.capacity) return KVC_E_SHAPE;
  st = resolve_base(kp, a->kc, &a->kb, false);
  if (st != KVC_OK) return st;
  st = resolve_base(vp, a->vc, &a->vb, false);
  if (st != KVC_OK) return st;
  if ((a->kb.centroid_tables && !aligned16(a->kb.centroid_tables)) ||
      (a->vb.centroid_tables && !aligned16(a->vb.centroid_tables)))
    return KVC_E_ALIGN;
  a->n_keys = n_keys;
  a->n_queries = n_queries;
  a->q = q;
  a->out = out;
  a->lse = lse;
  return KVC_OK;
}

// Attention flags: the Jensen correction needs the bf16 path with centroid K and V.
static kvc_status check_attend_flags(uint32_t flags, const AttendLaunch& a) {
  if (flags & ~(uint32_t)KVC_ATTEND_JENSEN) return KVC_E_UNSUPPORTED;
  if ((flags & KVC_ATTEND_JENSEN) &&
      (a.kc.x_dtype != KVC_BF16 || a.kc.bits == 16 || a.kc.base != KVC_BASE_CENTROID ||
       a.vc.base != KVC_BASE_CENTROID))
    return KVC_E_UNSUPPORTED;
  return KVC_OK;
}

kvc_status kvc_attend_compressed(const kvc_codec* kc, const kvc_store* k,
                                 const kvc_base_params* kp, const kvc_codec* vc,
                                 const kvc_store* v, const kvc_base_params* vp, int64_t n_keys,
                                 const void* q, int64_t n_queries, float softmax_scale,
                                 uint32_t flags, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  AttendLaunch a;
  kvc_status st = check_attend(kc, k, kp, vc, v, vp, n_keys, q, n_queries, softmax_scale, out, lse, &a);
  if (st != KVC_OK) return st;
  if (workspace && !aligned16(workspace)) return KVC_E_ALIGN;
  a.workspace = workspace;
  a.workspace_bytes = workspace ? workspace_bytes : 0;
  for (const CodecArgs* c : {&a.kc, &a.vc})
    if (c->base != KVC_BASE_NONE && c->base != KVC_BASE_CENTROID) return KVC_E_UNSUPPORTED;
  if (a.kc.x_dtype == KVC_BF16 && a.kc.D != 128) return KVC_E_UNSUPPORTED;
  if ((a.kc.bits == 16) != (a.vc.bits == 16)) return KVC_E_UNSUPPORTED;   // both dense or neither
  if (a.kc.x_dtype == KVC_BF16 &&
      (!attend_ranges_fit(a.kc, a.ks) || !attend_ranges_fit(a.vc, a.vs)))
    return KVC_E_SHAPE;
  // rotated residuals are undone in the tile decode of the centroid-K-and-V kernels
  if ((a.kc.rot || a.vc.rot) && (a.kc.base != KVC_BASE_CENTROID || a.vc.base != KVC_BASE_CENTROID))
    return KVC_E_UNSUPPORTED;
  st = check_attend_flags(flags, a);
  if (st != KVC_OK) return st;
  a.jensen = (flags & KVC_ATTEND_JENSEN) != 0;
  a.scale = softmax_scale;
  return from_hip(launch_attend(a, reinterpret_cast<hipStream_t>(stream)));
}

kvc_status kvc_attend_compressed_chunk(const kvc_codec* kc, const kvc_store* k,
                                       const kvc_base_params* kp, const kvc_codec* vc,
                                       const kvc_store* v, const kvc_base_params* vp,
                                       int64_t n_keys, const void* chunk_k, const void* chunk_v,
                                       int64_t n_chunk, const void* q, int64_t n_queries,
                                       float softmax_scale, uint32_t flags, float* out, float* lse,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  AttendLaunch a;
  kvc_status st = check_attend(kc, k, kp, vc, v, vp, n_keys, q, n_queries, softmax_scale, out, lse, &a);
  if (st != KVC_OK) return st;
  for (const CodecArgs* c : {&a.kc, &a.vc})
    if (c->base != KVC_BASE_NONE && c->base != KVC_BASE_CENTROID) return KVC_E_UNSUPPORTED;
  if (a.kc.x_dtype != KVC_BF16 || a.kc.D != 128 || a.kc.bits == 16 || a.vc.bits == 16)
    return KVC_E_UNSUPPORTED;
  if ((a.kc.rot || a.vc.rot) && (a.kc.base != KVC_BASE_CENTROID || a.vc.base != KVC_BASE_CENTROID))
    return KVC_E_UNSUPPORTED;
  st = check_attend_flags(flags, a);
  if (st != KVC_OK) return st;
  a.jensen = (flags & KVC_ATTEND_JENSEN) != 0;
  if (n_chunk < 1) return KVC_E_SHAPE;
  if (!chunk_k || !chunk_v) return KVC_E_NULL;
  if (!aligned16(chunk_k) || !aligned16(chunk_v) || (workspace && !aligned16(workspace)))
    return KVC_E_ALIGN;
  if (!attend_ranges_fit(a.kc, a.ks) || !attend_ranges_fit(a.vc, a.vs) ||
      n_chunk * a.kc.H * a.kc.D * 2 >= ((int64_t)1 << 31))
    return KVC_E_SHAPE;
  if (n_queries > 0 &&
      (!workspace || workspace_bytes < attend_chunk_workspace_bytes(a.kc, n_keys, n_queries)))
    return KVC_E_WORKSPACE;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.scale = softmax_scale;
  return from_hip(launch_attend_chunk(a, chunk_k, chunk_v, n_chunk, reinterpret_cast<hipStream_t>(stream)));
}

kvc_status kvc_attend_mixed_dim(const kvc_codec* kc, const kvc_store* k,
                                const kvc_base_params* kp, const kvc_codec* vc,
                                const kvc_store* v, const kvc_base_params* vp, int64_t n_keys,
                                const void* q, int64_t n_queries, float softmax_scale,
                                float* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
  AttendLaunch a;
  kvc_status st = check_attend(kc, k, kp, vc, v, vp, n_keys, q, n_queries, softmax_scale, out, lse, &a);
  if (st != KVC_OK) return st;
  if (workspace && !aligned16(workspace)) return KVC_E_ALIGN;
  a.workspace = workspace;
  a.workspace_bytes = workspace ? workspace_bytes : 0;
  if (a.kc.base != KVC_BASE_COEFF || a.vc.base != KVC_BASE_CENTROID) return KVC_E_UNSUPPORTED;
  if (a.vc.rot != 0) return KVC_E_UNSUPPORTED;
  if (a.kc.x_dtype != KVC_BF16 || a.kc.D != 128 || a.kc.m != 16 || a.kc.groups != 1)
    return KVC_E_UNSUPPORTED;
  if (!a.kb.basis) return KVC_E_NULL;
  if (!attend_ranges_fit(a.kc, a.ks) || !attend_ranges_fit(a.vc, a.vs)) return KVC_E_SHAPE;
  a.scale = softmax_scale;
  return from_hip(launch_attend_mixed(a, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
