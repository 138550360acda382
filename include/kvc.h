/*
 * kvc.h - C ABI of the compressed KV-cache codec and attention library (libkvc.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (pages: NanoKV project page and arXiv 2611.06377; Coral-KV arXiv
 * 2610.12514; TempoKV arXiv 2610.15324): every cached key/value vector gets a
 * base - its nearest cluster centroid (Coral-KV abstract, Fig. 2c; NanoKV
 * abstract), a block-diagonal-plus-low-rank prediction from the reconstructed
 * previous layer (Coral-KV Fig. 3), or a temporal prediction from the
 * reconstructed previous frames (TempoKV Fig. 2b) - and only the residual is
 * stored, quantized group-wise to INT2/INT4 with a shared scale per group
 * (Coral-KV Fig. 5c) and bit-packed (Coral-KV Table 9 caption lists the stored
 * state: residual codes and scales, assignments, codebooks or predictors).
 * Attention then runs over the compressed history (NanoKV abstract), either by
 * decoding K/V tiles on the fly or, NanoKV-Fast style, by scoring queries on the
 * stored low-dimensional coefficients (NanoKV page, '03 / Measured results').
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Ownership: every buffer is owned by the caller.  The library never
 *   allocates or frees device memory and keeps no mutable global state, with one
 *   exception: kvc_encode_noalloc's fixed scratch array (one per GPU, part of the
 *   loaded library) and the cached device address of that array.
 * - Pointers: all tensor pointers are DEVICE pointers and must be 16-byte
 *   aligned; descriptors (kvc_codec, kvc_store, kvc_base_params) are HOST
 *   structs read during the call only.  A call with nothing to process
 *   (n_tokens == 0, n_queries == 0) may pass NULL for the empty tensors and
 *   returns KVC_OK without launching anything.
 * - Streams: `stream` is a hipStream_t (NULL = the default stream).  Every call
 *   is asynchronous on that stream and never synchronizes.  Outputs must not
 *   alias inputs.
 * - Errors: arguments are validated on the host before anything is launched;
 *   on failure the call returns a kvc_status and touches no output.  A launch
 *   failure reported by the HIP runtime returns KVC_E_DEVICE.  Inputs must be
 *   finite (not checked).
 * - Layouts (element = x_dtype unless stated):
 *     x, reconstructions, queries, outputs   [N][H][d], token-major; consecutive
 *                                            tokens `token_stride` elements apart
 *     store.codes        uint32 [H][capacity][d*bits/32]   (m*bits/32 for COEFF)
 *     store.scale_zero   uint32 [H][capacity][d/group]     (m/group for COEFF)
 *     store.index        uint8 (<= 256 centroids) or uint16, [H][capacity]
 *     centroids          [H][C][d]
 *   Code i of a vector sits in word floor(i*bits/32) at bit bits*(i mod 32/bits)
 *   (little-endian).  A scale/zero word holds the fp16 bits of the scale in its
 *   low half and those of the zero in its high half.
 * - Arithmetic of the codec (bit-exact contract): residual r = x - base in fp32;
 *   per group of `group` consecutive values: z = fp16(min r),
 *   s = fp16(fp32(max r - min r) / (2^bits - 1)), code = clamp(rint((r - z)/s),
 *   0, 2^bits - 1) (all codes 0 when s == 0), fp32 IEEE division, ties to even;
 *   reconstruction = base + ((code * s) + z).  Groups whose scale or zero
 *   overflows fp16 are outside the contract.  Nearest-centroid distances are
 *   sum_i (x_i - c_i)^2 in fp32 in ascending channel order, ties to the lowest
 *   index.
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 4

typedef enum {
  KVC_OK = 0,
  KVC_E_NULL = 1,        /* a required pointer is NULL                          */
  KVC_E_SHAPE = 2,       /* sizes inconsistent or out of range                  */
  KVC_E_UNSUPPORTED = 3, /* valid request this build does not implement         */
  KVC_E_ALIGN = 4,       /* a device pointer is not 16-byte aligned             */
  KVC_E_WORKSPACE = 5,   /* workspace smaller than kvc_workspace_bytes()        */
  KVC_E_DEVICE = 6       /* the HIP runtime reported an error                   */
} kvc_status;

typedef enum { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype;

typedef enum {
  KVC_BASE_NONE = 0,     /* base 0: anchors and plain group quantization          */
  KVC_BASE_CENTROID = 1, /* base = C[h][a], a = nearest centroid                  */
  KVC_BASE_DPLR = 2,     /* cross-layer block-diagonal + rank-r prediction        */
  KVC_BASE_TEMPORAL = 3, /* per-channel AR(2) keys / key->value cross prediction  */
  KVC_BASE_COEFF = 4     /* C[h][a] + B c: m coefficients of the centroid residual */
} kvc_base_kind;

/* Codec description (plain data). */
typedef struct {
  int32_t heads;       /* H >= 1                                                 */
  int32_t head_dim;    /* d: 64 or 128                                           */
  int32_t bits;        /* residual code width: 2 or 4; 16 with KVC_BASE_NONE and
                          bf16 marks an uncompressed cache (attention input only:
                          store.codes then points to bf16 [capacity][H][d],
                          token-major, and scale_zero / index are unused)       */
  int32_t group;       /* values per scale/zero group: 16, 32, 64 or 128; must
                          divide d (or coeff_dim for KVC_BASE_COEFF)             */
  int32_t base;        /* kvc_base_kind                                          */
  int32_t n_centroids; /* CENTROID / COEFF: 1..65535                             */
  int32_t rank;        /* DPLR: r, a multiple of 16, <= 256                      */
  int32_t n_inputs;    /* DPLR: 1 (keys from K_{l-1}) or 2 (values from
                          [K_l ; V_{l-1}])                                       */
  int32_t coeff_dim;   /* COEFF: m = 16                                          */
  int32_t x_dtype;     /* kvc_dtype of x, centroids, queries, reconstructions    */
  int32_t rotation;    /* Hn residual transform (Coral-KV Fig. 5, Fig. 9b-c):
                          0 = none; n = 16 or 64 = the residual of every group of
                          n consecutive channels is multiplied by H_n / sqrt(n)
                          (H_n the Sylvester Hadamard matrix) before it is
                          quantized, and the dequantized vector is multiplied by
                          the same matrix (its own inverse) before the base is
                          added (Coral-KV rotates the prediction residuals).
                          Needs bf16, d = 128 and a group that n divides, with
                          group <= 64, and KVC_BASE_CENTROID (at most 512
                          centroids), KVC_BASE_NONE, KVC_BASE_TEMPORAL or
                          KVC_BASE_DPLR (rank <= 64).  The rounded transform is the Sylvester
                          recursion H_2m [a; b] = [H_m a + H_m b; H_m a - H_m b]
                          in fp32 (pairs at distance 1 combined first, then 2,
                          4, ..., n/2), then the exact 1/sqrt(n) scaling.        */
} kvc_codec;

/* A compressed store (device buffers owned by the caller). */
typedef struct {
  uint32_t* codes;      /* [H][capacity][code words]                     */
  uint32_t* scale_zero; /* [H][capacity][groups]                         */
  void* index;          /* [H][capacity]; NULL unless CENTROID / COEFF   */
  int64_t capacity;     /* tokens per head row                           */
} kvc_store;

/* Base parameters (device pointers; unused members may be NULL).
 *   CENTROID: centroids.
 *   COEFF:    centroids, basis [d][m] bf16 (orthonormal columns, shared by heads).
 *   DPLR:     prev0 = first input reconstruction (K_{l-1} for keys, K_l for values),
 *             prev1 = second input (V_{l-1}, values only), both bf16 [N][H][d];
 *             w_block [H][d][n_inputs*d], u [H*d][r], v_lr [r][n_inputs*H*d], bf16
 *             (every matrix is stored with its contraction index contiguous).
 *             prediction[h] = W_h [prev0_h ; prev1_h] + U (v_lr [prev0 ; prev1])[h],
 *             where [prev0 ; prev1] stacks all heads of prev0, then all of prev1.
 *   TEMPORAL: keys:   prediction = (coef_a * prev0) + (coef_b * prev1) per channel,
 *                     prev0 = K_{t-1}, prev1 = K_{t-2}, bf16 [N][H][d]; coef fp32 [H][d].
 *             values: prediction = M_h aux + (coef_a * prev0), aux = aligned K_t,
 *                     prev0 = V_{t-1}; M = w_block [H][d][d] bf16; coef_b = NULL.
 *   prev_token_stride: elements between consecutive tokens of prev0/prev1/aux
 *   (0 = H*d; a multiple of 8, else KVC_E_ALIGN: the inputs are read in 16-byte pieces).
 * Matrix-product bases (DPLR, temporal values) compute an fp32 prediction first: it
 * goes to pred_out when given, else to the workspace; DPLR always needs the workspace
 * (kvc_workspace_bytes) for its rank-r intermediate.
 *   centroid_tables: optional, attention only (NULL elsewhere is fine, and ignored by
 *   every other call): the buffer a successful kvc_centroid_tables call filled from
 *   these same centroids.  The bf16 decode-fused attention then adds the centroid rows
 *   from that fp16 image (identical results, fewer instructions per decoded value). */
typedef struct {
  const void* centroids;
  const void* basis;
  const void* prev0;
  const void* prev1;
  const void* aux;
  const void* w_block;
  const void* u;
  const void* v_lr;
  const float* coef_a;
  const float* coef_b;
  int64_t prev_token_stride;
  const void* centroid_tables;
} kvc_base_params;

/* Device bytes a store of `capacity` tokens needs (host-side helper). */
kvc_status kvc_store_bytes(const kvc_codec* codec, int64_t capacity, size_t* codes_bytes,
                           size_t* scale_zero_bytes, size_t* index_bytes);

/* kvc_encode - compress n_tokens vectors x [n][H][d] into dst at token rows
 * [token_offset, token_offset + n_tokens).
 * Computes, per (token, head): the base (per codec->base), the residual, the
 * group scale/zero, codes, and packs them (Coral-KV Fig. 3 and Fig. 5c; TempoKV
 * Fig. 2b; NanoKV abstract).  For KVC_BASE_COEFF the quantized vector is the m
 * coefficients B^T (x - C[a]).
 *   x_token_stride: elements between consecutive tokens of x (0 = H*d).
 *   recon_out: optional [n][H][d] x_dtype reconstruction (base + dequantized
 *              residual, rounded to x_dtype) - the input of the next predictor step.
 *   pred_out:  optional [n][H][d] fp32 copy of the base used (prediction).
 *   workspace: device scratch of kvc_workspace_bytes(KVC_OP_ENCODE, ...) bytes for
 *              the matrix-product bases (DPLR; temporal values without pred_out); the
 *              contents on return are unspecified.  NULL, 0 otherwise.
 * A rotated codec (codec->rotation != 0) quantizes the rotated residual and needs
 * x_token_stride to be a multiple of 8; recon_out then holds base + the dequantized
 * residual rotated back (what kvc_decode returns).  The rotated centroid codec takes no
 * recon_out or pred_out (decode the store instead).
 * Errors: KVC_E_NULL, KVC_E_SHAPE (token_offset + n_tokens > capacity, bad
 * codec), KVC_E_UNSUPPORTED, KVC_E_ALIGN, KVC_E_WORKSPACE, KVC_E_DEVICE. */
kvc_status kvc_encode(const kvc_codec* codec, const void* x, int64_t n_tokens,
                      int64_t x_token_stride, const kvc_base_params* base, const kvc_store* dst,
                      int64_t token_offset, void* recon_out, float* pred_out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* kvc_encode_kv - kvc_encode of the keys xk into kdst and of the values xv into vdst,
 * the two tensors of one chunk (Coral-KV Fig. 2c: a cache block is encoded when it
 * fills), with one codec, token count, stride and offset, and each its own base
 * parameters.  The stores are exactly what two kvc_encode calls write; where the codec
 * allows (KVC_BASE_CENTROID, bf16, d = 128, <= 512 centroids, group 16/32/64) both
 * tensors are encoded by a single launch, otherwise one after the other.  No
 * reconstruction, prediction or workspace: bases that need a workspace (block-DPLR,
 * temporal values) return KVC_E_UNSUPPORTED.  kdst and vdst must not overlap
 * (KVC_E_SHAPE when they share a buffer).
 * Errors: as kvc_encode. */
kvc_status kvc_encode_kv(const kvc_codec* codec, const void* xk, const void* xv, int64_t n_tokens,
                         int64_t x_token_stride, const kvc_base_params* kbase,
                         const kvc_base_params* vbase, const kvc_store* kdst, const kvc_store* vdst,
                         int64_t token_offset, void* stream);

/* Bytes of the device scratch array that kvc_encode_noalloc uses: one copy per GPU the
 * library runs on, held until the process ends. */
#define KVC_NOALLOC_SCRATCH_BYTES (16u << 20)

/* kvc_encode_noalloc - kvc_encode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments without the workspace, the same results bit for bit, and no
 * allocation of any kind.  Where kvc_encode needs a workspace, this call uses a fixed
 * scratch array of KVC_NOALLOC_SCRATCH_BYTES inside the library instead:
 *   - KVC_BASE_DPLR on the fused predictor + quantizer (bf16, d = 128, group <= 64,
 *     rank <= 64, x and input strides multiples of 8): the rank-r intermediate, n_tokens *
 *     rank * 4 bytes, which must fit the scratch (else KVC_E_WORKSPACE; 65536 tokens at
 *     rank 64);
 *   - other shapes of the matrix-product bases (DPLR, temporal values) route the
 *     prediction through an fp32 buffer: pred_out must then be given (else
 *     KVC_E_UNSUPPORTED); DPLR keeps its rank-r intermediate in the scratch as above;
 *   - every other base needs no scratch.
 * The scratch belongs to the current device (`stream` must be on it) and is shared by
 * every call on that device, which leaves it holding the last call's contents: calls
 * that overlap on one GPU (two streams, two host threads) race and must not be issued.
 * Nothing in it has to start at zero - the rank kernel writes every value before it is
 * read.  The first call on a device looks up the array's device address
 * (hipGetSymbolAddress) and keeps it.
 * Errors: as kvc_encode, and KVC_E_WORKSPACE / KVC_E_UNSUPPORTED as above. */
kvc_status kvc_encode_noalloc(const kvc_codec* codec, const void* x, int64_t n_tokens,
                              int64_t x_token_stride, const kvc_base_params* base,
                              const kvc_store* dst, int64_t token_offset, void* recon_out,
                              float* pred_out, void* stream);

/* kvc_fit_centroids - online centroid fitting at block fill (Coral-KV Fig. 2c: QVG
 * fits video-specific centroids when a cache block reaches its token limit): `iterations`
 * Lloyd steps on the n_tokens vectors x [n][H][d], per head, updating the centroid table
 * in place.  Each step assigns every vector to its nearest centroid exactly as
 * kvc_encode does (fp32 squared distance, ascending channels, ties to the lowest
 * index), then sets every centroid that received vectors to their mean - the fp32 sum
 * in ascending token order divided by the count, rounded to bf16 (nearest even) - and
 * leaves the others unchanged.
 *   codec: KVC_BASE_CENTROID, bf16, d = 128 (bits, group and rotation only shape the
 *          scratch encode; the fit does not depend on them).
 *   x_token_stride: elements between tokens of x (0 = H*d; a multiple of 8).
 *   centroids: [H][C][d] bf16, the initial table on entry, the fitted one on return.
 *   workspace: kvc_workspace_bytes(KVC_OP_FIT, codec, n_tokens, 0) bytes (a scratch
 *              store of n_tokens rows); the contents on return are unspecified.
 * n_tokens == 0 or iterations == 0 returns KVC_OK without launching anything.
 * Errors: KVC_E_NULL, KVC_E_SHAPE (negative sizes, bad stride), KVC_E_UNSUPPORTED,
 * KVC_E_ALIGN, KVC_E_WORKSPACE, KVC_E_DEVICE. */
kvc_status kvc_fit_centroids(const kvc_codec* codec, const void* x, int64_t n_tokens,
                             int64_t x_token_stride, void* centroids, int32_t iterations,
                             void* workspace, size_t workspace_bytes, void* stream);

/* kvc_decode - reconstruct rows [token_offset, token_offset + n_tokens) of a store:
 * out = base + ((code * s) + z), written as out_dtype [n][H][d] (bf16 output is the
 * fp32 value rounded to nearest even).  Predictor bases read `base` exactly as
 * kvc_encode did (so a chain decodes in the order it was encoded); pred_out:
 * optional fp32 base; workspace: as kvc_encode.
 * Errors: as kvc_encode; KVC_E_UNSUPPORTED for KVC_BASE_COEFF (those keys are only
 * read by kvc_attend_mixed_dim). */
kvc_status kvc_decode(const kvc_codec* codec, const kvc_store* src, int64_t token_offset,
                      int64_t n_tokens, const kvc_base_params* base, void* out, int32_t out_dtype,
                      float* pred_out, void* workspace, size_t workspace_bytes, void* stream);

/* Attention flags.
 * KVC_ATTEND_JENSEN: Jensen-bias correction (the INT2 Jensen-bias abstract on the
 *   Coral-KV listing page: rounding noise in quantized keys inflates their softmax
 *   weight through the convexity of exp, which a per-score correction from the step
 *   sizes and the query removes in expectation, by a second-order Taylor expansion).
 *   The logit of a compressed key becomes softmax_scale * q . k_hat -
 *   (softmax_scale^2 / 24) * sum_g s_g^2 * |q_g|^2 over its scale groups g (s_g = the
 *   group's stored fp16 scale, the quantization step; q_g = the query's channels of
 *   group g): the second-order term of log E[exp] for noise uniform on
 *   [-s_g/2, s_g/2].  Keys of an uncompressed current chunk are not corrected.  The
 *   correction enters the scores through one more bf16 MFMA per key block (s_g^2 and the
 *   query term rounded to bf16).  Needs the bf16 path with centroid K and V. */
enum { KVC_ATTEND_JENSEN = 1 };

/* kvc_centroid_tables - the fp16 image of a bf16 centroid table [H][C][d] that the
 * decode-fused attention reads in place of the table (kvc_base_params.centroid_tables).
 * The tile decode adds a key's centroid row to its dequantized residual in fp32; from a
 * bf16 table that takes an unpack and an add per value, from fp16 one mixed-precision
 * FMA, c16 * 2^-k + r with a single rounding, i.e. exactly the fp32 sum c + r.  Each
 * head h gets the power of two 2^k_h that brings its largest |c| closest below 65504,
 * and every c * 2^k_h must be an fp16 value exactly; then attention with the image
 * returns bit for bit what it returns with the bf16 table.
 *   codec: KVC_BASE_CENTROID or KVC_BASE_COEFF, bf16, d = 128 (the layout is that of
 *     the bf16 attention path; other codecs: KVC_E_UNSUPPORTED).
 *   centroids: [H][C][d] bf16 (C = codec->n_centroids).
 *   tables: device buffer of kvc_centroid_tables_bytes(codec) bytes, 16-byte aligned:
 *     [H] int32 k_h, [H] int32 exact flags, padding to 256 bytes, then [H][C][d] fp16.
 *   Synchronous: the call waits for `stream` to read the per-head checks back.
 * Returns KVC_OK when every head's image is exact; KVC_E_UNSUPPORTED when some entry is
 * not a finite value that fits (a table whose nonzero magnitudes span more than fp16's
 * range, about 2^30); the buffer must then not be passed to attention.  Errors:
 * KVC_E_NULL, KVC_E_SHAPE (tables_bytes too small), KVC_E_ALIGN, KVC_E_DEVICE. */
size_t kvc_centroid_tables_bytes(const kvc_codec* codec);
kvc_status kvc_centroid_tables(const kvc_codec* codec, const void* centroids, void* tables,
                               size_t tables_bytes, void* stream);

/* kvc_attend_compressed - O = softmax(Q K^T * softmax_scale) V per head, no mask,
 * over n_keys keys held compressed in stores k and v (rows 0..n_keys-1); K and V
 * tiles are decoded on the fly (NanoKV abstract: repeated attention over the
 * compressed history).  K and V codecs: KVC_BASE_CENTROID or KVC_BASE_NONE with
 * d = 128 and bf16 x_dtype (bf16 MFMA path; decoded values are rounded to bf16, as
 * a bf16 cache would hold them), or any d in {64, 128} with f32 x_dtype (fp32 path).
 * bits = 16 on both K and V attends over uncompressed bf16 caches (for example the
 * reconstructions a predictor chain decodes; each cache below 2 GiB).
 *   Only rows 0..n_keys-1 are read: rows beyond (a store sized for a longer history,
 *     not yet written) never reach the result.
 *   q:   [n_queries][H][d] x_dtype, token stride H*d.
 *   softmax_scale: finite and > 0 (else KVC_E_SHAPE).
 *   Range of the bf16 path: decoded values are held as fp16 for the P V product, so
 *     every decoded value (and every value of an uncompressed cache or chunk) must lie
 *     within fp16's range, |v| <= 65504; larger values are outside the contract.
 *   flags: 0 or KVC_ATTEND_JENSEN (other bits: KVC_E_UNSUPPORTED).
 *   out: [n_queries][H][d] fp32.
 *   lse: optional [H][n_queries] fp32 natural-log sum-exp of the scaled scores.
 *   workspace: optional device scratch.  With kvc_workspace_bytes(KVC_OP_ATTEND, kc,
 *     n_keys, n_queries) bytes (when that is nonzero) the bf16 path splits the keys
 *     across workgroups and merges the partial results by their log-sum-exp (the
 *     same softmax, summed in another order); NULL, or a smaller workspace, runs one
 *     pass over the keys.  The contents are overwritten.
 *   Rotated codecs (kc->rotation or vc->rotation nonzero; Coral-KV Fig. 5): each
 *     decoded tile rotates its dequantized residuals back before the centroid is added,
 *     with the decoder's arithmetic, so the tiles hold exactly what kvc_decode returns
 *     (rounded to bf16).  K and V must then both use KVC_BASE_CENTROID.
 *   kp->centroid_tables and vp->centroid_tables (both given, centroid K and V): the
 *     tile decode reads the fp16 images (kvc_centroid_tables); same results.  One of
 *     them alone is ignored.
 * Errors: KVC_E_NULL, KVC_E_SHAPE (n_keys > capacity, n_keys < 1, mismatched
 * heads/d, softmax_scale not finite and positive; bf16 path: a store whose per-head
 * code or scale/zero rows span 2 GiB or more, or a dense cache of 2 GiB or more - the
 * kernels address them with 32-bit byte offsets), KVC_E_UNSUPPORTED, KVC_E_ALIGN,
 * KVC_E_DEVICE. */
kvc_status kvc_attend_compressed(const kvc_codec* kc, const kvc_store* k,
                                 const kvc_base_params* kp, const kvc_codec* vc,
                                 const kvc_store* v, const kvc_base_params* vp, int64_t n_keys,
                                 const void* q, int64_t n_queries, float softmax_scale,
                                 uint32_t flags, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* kvc_attend_compressed_chunk - attention over the compressed history plus an
 * uncompressed current chunk: O = softmax(Q [K_hist ; K_chunk]^T * softmax_scale)
 * [V_hist ; V_chunk] per head, no mask, where the first n_keys keys and values are
 * decoded from stores k and v exactly as in kvc_attend_compressed and the last n_chunk
 * are read as they are.  (The TempoKV page keeps the most recent frames uncompressed,
 * and quantized keys take attention mass from the unquantized current chunk; this is
 * that layout.)  The two parts are attended separately and merged by their
 * log-sum-exp, the same softmax summed in another order.
 *   kc, vc, k, v, kp, vp, n_keys, q, flags, out, lse: as kvc_attend_compressed (bf16
 *     path only: d = 128, compressed K and V with centroid or no base); with
 *     KVC_ATTEND_JENSEN only the history keys' logits are corrected.
 *   chunk_k, chunk_v: [n_chunk][H][d] bf16, token stride H*d, n_chunk >= 1.
 *   workspace: required, kvc_workspace_bytes(KVC_OP_ATTEND_CHUNK, kc, n_keys,
 *     n_queries) bytes; the contents are overwritten.
 * Errors: as kvc_attend_compressed; KVC_E_SHAPE also for a chunk of 2 GiB or more,
 *   KVC_E_WORKSPACE for a missing or smaller workspace. */
kvc_status kvc_attend_compressed_chunk(const kvc_codec* kc, const kvc_store* k,
                                       const kvc_base_params* kp, const kvc_codec* vc,
                                       const kvc_store* v, const kvc_base_params* vp,
                                       int64_t n_keys, const void* chunk_k, const void* chunk_v,
                                       int64_t n_chunk, const void* q, int64_t n_queries,
                                       float softmax_scale, uint32_t flags, float* out, float* lse,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* kvc_attend_mixed_dim - NanoKV-Fast style attention from the stored representation
 * without rebuilding keys (NanoKV page, '03 / Measured results'): the score of key n
 * is (q . C_k[a_n] + (B^T q) . c_n) * softmax_scale, c_n = dequantized coefficients;
 * softmax over all n_keys keys; values decoded from their centroid store.
 *   kc: KVC_BASE_COEFF (bf16, d = 128, m = 16); kp: centroids + basis.
 *   vc: KVC_BASE_CENTROID (bf16, d = 128, not rotated); vp: centroids (and optionally
 *     centroid_tables, the fp16 image kvc_centroid_tables made of them: the ordered path
 *     then decodes V through it, same results).
 *   q, out, lse: as kvc_attend_compressed.
 *   workspace: optional.  With kvc_workspace_bytes(KVC_OP_ATTEND_MIXED, kc, n_keys,
 *     n_queries) bytes (and kc->n_centroids <= 4096) the call first copies the history
 *     into centroid-block order - keys whose centroids lie in one block of 32
 *     consecutive centroids become contiguous, each head's blocks in ascending order,
 *     token order kept inside a block, every value row moving with its key - and
 *     forms q . C_k[a] once per block and query instead of once per key; the order
 *     changes only the summation order of the softmax.  The size covers those copies
 *     (value rows sized for the widest value codec), their tables and the key splits'
 *     partial results; the contents on return are unspecified.  With less or none the
 *     centroid rows are gathered per key (and the keys split only when the workspace
 *     holds kvc_attend_compressed's split partials).
 * Errors: as kvc_attend_compressed. */
kvc_status kvc_attend_mixed_dim(const kvc_codec* kc, const kvc_store* k,
                                const kvc_base_params* kp, const kvc_codec* vc,
                                const kvc_store* v, const kvc_base_params* vp, int64_t n_keys,
                                const void* q, int64_t n_queries, float softmax_scale,
                                float* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Workspace bytes of an entry point (op: KVC_OP_*) for n_tokens tokens (the keys for
 * the attention ops; the history keys for KVC_OP_ATTEND_CHUNK) and n_queries queries.
 * Encode / decode: required by the DPLR and temporal-value bases, 0 otherwise.
 * Attention: the optional workspace that enables key splitting (0 when a single pass is
 * used anyway); with a current chunk: the required partial results; mixed-dimensional
 * (codec = the key codec): the cluster-ordered copies of the history, their tables and
 * the split partials.  Centroid fitting:
 * the scratch store of n_tokens rows. */
enum { KVC_OP_ENCODE = 0, KVC_OP_DECODE = 1, KVC_OP_ATTEND = 2, KVC_OP_ATTEND_MIXED = 3,
       KVC_OP_ATTEND_CHUNK = 4, KVC_OP_FIT = 5 };
size_t kvc_workspace_bytes(int32_t op, const kvc_codec* codec, int64_t n_tokens,
                           int64_t n_queries);

const char* kvc_status_str(kvc_status status);
int32_t kvc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H_ */
