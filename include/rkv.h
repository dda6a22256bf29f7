/*
 * rkv.h -- C ABI of librkv, the MI355X (gfx950) ResidualKV hot path.
 *
 * ResidualKV (also called DeltaKV) keeps a KV cache as two parts: a small set
 * of uncompressed reference tokens, and, for every position, the residual of
 * its K and V against the mean of its k nearest references, stored as
 * quantised codes.  Attention rebuilds each token as reference mean plus
 * residual while it reads the cache.
 *
 * Sources: "ResidualKV: Residual-Based KV Cache Compression for Efficient
 * Long-Context Inference" (paper page), section "DeltaKV Framework
 * Architecture" (strided reference selection, top-k nearest by L2 distance,
 * mean reference KV_R, residual, reconstruction KV^ = KV^_delta + KV_R) and
 * section "Practical Deployment via Sparse-vLLM" (a batched L2-distance
 * search and a fused gather / mean / residual-add reconstruction);
 * "New KV Cache Compression Method Cuts Long-Context Inference Costs by 85%",
 * section "How ResidualKV Works" (quantised residual codes, on-the-fly
 * reconstruction, dynamic-stride schedule).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them.  Scratch memory is the caller's
 *     workspace, sized by the matching *_workspace query.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  The returned status reports argument validation and launch
 *     errors only; a kernel fault shows up at the caller's next sync.
 *   - Errors come back as rkv_status; nothing throws across the ABI.  After
 *     RKV_ERR_HIP, rkv_last_hip_error() (thread-local) holds the hipError_t.
 *   - Layouts are dense and row-major, innermost dimension last.
 *     "inst" is an independent sequence-layer instance (batch x layers):
 *     every instance has its own cache and its own references.
 */
#ifndef RKV_H
#define RKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RKV_OK = 0,
  RKV_ERR_INVALID_ARG = 1,  /* NULL pointer, bad shape, bad stride, ...    */
  RKV_ERR_UNSUPPORTED = 2,  /* valid but not implemented (head_dim != 128)  */
  RKV_ERR_WORKSPACE = 3,    /* workspace smaller than the query returned    */
  RKV_ERR_HIP = 4,          /* a HIP call failed; see rkv_last_hip_error()  */
  RKV_ERR_RANGE = 5         /* more than 65535 references (uint16 slots)    */
} rkv_status;

typedef enum { RKV_F32 = 0, RKV_BF16 = 1 } rkv_dtype;

/* Reference schedule.  Position j is a reference iff j mod s(j) == 0, where
 * s(j) = base for j < double_after (or everywhere when double_after == 0),
 * and for j >= double_after the stride doubles each time the position
 * doubles: s = 2*base on [A, 2A), 4*base on [2A, 4A), ... (A = double_after).
 * The fixed schedule is the paper page's strided reference selection; the
 * doubling one is the news page's dynamic-stride schedule, whose reference
 * count grows about logarithmically.  Requires base >= 1 and, when
 * double_after > 0, double_after a multiple of 2*base. */
typedef struct {
  int32_t base;
  int64_t double_after;
} rkv_stride;

/* Alignment: every device buffer handed to the library (K, V, q, outputs,
 * workspaces, codes_k, codes_v, ref_kv) must be 16-byte aligned; ref_idx
 * must be aligned to 2k bytes when k is 4, 8 or 16 (16 at most), scales to
 * 4 and ref_scales to 2.  Any allocation from hipMalloc or torch satisfies
 * this.  Misaligned buffers give RKV_ERR_INVALID_ARG. */

/* Shape of a compressed cache and its device buffers (all caller-owned).
 *
 *   ref_idx  uint16 [inst][H][N][k]     slots (rank in the reference list) of
 *                                       the k_eff nearest references of each
 *                                       position, ascending, 0xFFFF padding
 *                                       (k_eff = min(k, #references <= pos)).
 *   codes_k  uint8  [inst][H][N][D*bits/8]
 *                                       K residual codes, token-major: code of
 *                                       dim t is a two's-complement field at
 *                                       bits [t*bits, (t+1)*bits) of the row.
 *            bits == 0: double [inst][H][N][D], the exact residual.
 *   codes_v  uint8  [inst][H][ceil(N/32)][D][32*bits/8]
 *                                       V residual codes, transposed per tile
 *                                       of 32 positions: for each dim, the 32
 *                                       codes of the tile form one bit string,
 *                                       position u at bits [u*bits,(u+1)*bits);
 *                                       positions past N are 0.
 *            bits == 0: double [inst][H][N][D], the exact residual.
 *   scales   uint16 [inst][H][N][2][D/group]   fp16 bit patterns, plane 0 = K,
 *                                       1 = V.  Unused (may be NULL) when
 *                                       bits == 0.
 *   ref_kv   dtype  [inst][H][2][n_refs][D]    the uncompressed references
 *                                       (plane 0 = K rows, 1 = V rows).
 *
 * Every position, references included, gets a record; decode and
 * reconstruction read a reference position from ref_kv. */
typedef struct {
  rkv_dtype dtype;       /* K/V/q element type                                 */
  int64_t n_inst;        /* independent instances (batch x layers)             */
  int32_t n_kv_heads;    /* H                                                  */
  int64_t seq_len;       /* N, positions per instance, at most 2^22            */
  int32_t head_dim;      /* D; 128 is the supported value                      */
  rkv_stride stride;     /* reference schedule                                 */
  int32_t k;             /* nearest references averaged per token, 1..16       */
  int32_t bits;          /* residual code width: 2, 4, 8, or 0 = no quantising */
  int32_t group;         /* dims per fp16 scale: 32, 64 or 128 (divides D)     */
  int64_t n_refs;        /* written by rkv_cache_init                          */
  uint16_t *ref_idx;
  uint8_t *codes_k;
  uint8_t *codes_v;
  uint16_t *scales;
  void *ref_kv;
  /* Full-pipeline quantisation (paper page, sections "Impact and Future
   * Directions" and "Improvements for AI systems": 4-bit quantisation applied
   * to the uncompressed reference tokens too).  ref_bits = 0: ref_kv holds the
   * raw rows (layout above), ref_scales unused.  ref_bits = 4 (needs
   * bits > 0): every reference row is quantised like a residual -- per group
   * of `group` dims an fp16 scale nearest to max|x|/7 and codes nearest to
   * x/scale, clamped to +-7 -- and
   *   ref_kv      uint8  [inst][H][2][n_refs][D/2]  two's-complement nibbles,
   *                                                  dim t in bits [4t, 4t+4)
   *   ref_scales  uint16 [inst][H][2][n_refs][D/group]  fp16 bit patterns.
   * Everything downstream then uses the dequantised references: the means
   * the residuals are taken against, reference positions in reconstruction
   * and decode, the QK table and W . Vref.  Selection still compares the
   * original keys. */
  int32_t ref_bits;
  uint16_t *ref_scales;
  /* Latent residuals (paper page, section "DeltaKV Framework Architecture":
   * the residual is taken between compressor outputs f_c(KV) - f_c(KV_R) and
   * rebuilt through a decompressor f_d).  The pages' pair is trained; a
   * fixed orthogonal pair stands in for it here.  latent = 1 (needs bits > 0) stores the codes and scales
   * of f_c(KV - KV_R) instead of KV - KV_R, with the fixed orthogonal pair
   *   f_c(x) = H D x / 16,   f_d(y) = D H y / 8   (f_d(f_c(x)) = x),
   * H the 128-point Walsh-Hadamard matrix (entry (i, t) = (-1)^popcount(i&t))
   * and D = diag(+-1), dim t negated iff the top bit of the (t+1)-th output
   * of SplitMix64 seeded with latent_seed is set.  f_c is linear, so this is
   * the pages' difference of projections.  Reconstruction adds f_d of the
   * dequantised codes to KV_R; decode scores the codes against H D q / 8 and
   * applies f_d to the merged residual output.  latent = 0: plain residuals,
   * latent_seed unused. */
  int32_t latent;
  uint64_t latent_seed;
} rkv_cache;

/* Number of references below seq_len; -1 if the schedule is invalid. */
int64_t rkv_num_refs(int64_t seq_len, rkv_stride stride);

/* Position of reference `slot`; -1 if out of range or invalid. */
int64_t rkv_ref_position(int64_t slot, rkv_stride stride);

/* Validates the shape fields of *c and fills c->n_refs.  Pointers are not
 * inspected.  RKV_ERR_RANGE if the schedule yields more than 65535
 * references; RKV_ERR_UNSUPPORTED for head_dim != 128. */
rkv_status rkv_cache_init(rkv_cache *c);

/* Bytes of each cache buffer for the shape in *c (after rkv_cache_init):
 * sizes[0..5] = ref_idx, codes_k, codes_v, scales, ref_kv, ref_scales. */
rkv_status rkv_cache_sizes(const rkv_cache *c, size_t sizes[6]);

/* Workspace bytes for rkv_encode / rkv_select_refs / rkv_quantize. */
rkv_status rkv_encode_workspace(const rkv_cache *c, size_t *bytes);

/* Encode (paper page, section "DeltaKV Framework Architecture": strided
 * references, the k nearest by L2 distance, their mean KV_R and the
 * residual; news page, section "How ResidualKV Works": residuals kept as
 * quantised codes): K, V dtype [inst][H][N][D] -> the compressed cache in *c.
 * = rkv_select_refs followed by rkv_quantize on the same stream. */
rkv_status rkv_encode(const void *K, const void *V, const rkv_cache *c,
                      void *ws, size_t ws_bytes, void *stream);

/* Streaming encode (decode-time append; the references are historical
 * tokens, paper page section "DeltaKV Framework Architecture"): encodes the
 * n_new positions pos0 .. pos0+n_new-1 from their rows only,
 *   K_new, V_new  dtype [inst][H][n_new][D]  (device),
 * writing their ref_idx rows, codes, scales and, for reference positions,
 * their ref_kv rows.  The result is bit-identical to rkv_encode over the
 * whole sequence: a position's candidates are the references at or before
 * it, so positions before pos0 must already be encoded -- by rkv_encode or
 * earlier rkv_append calls -- with this same workspace `ws`, which carries
 * the reference keys and norms from call to call (rkv_encode_workspace
 * bytes).  Positions from pos0 + n_new on are not touched; codes of other
 * positions sharing a 32-position V tile keep their bits.
 * RKV_ERR_INVALID_ARG unless 0 <= pos0 and pos0 + n_new <= seq_len, n_new >= 1. */
rkv_status rkv_append(const void *K_new, const void *V_new, int64_t n_new, const rkv_cache *c,
                      int64_t pos0, void *ws, size_t ws_bytes, void *stream);

/* Reference selection ("Batch L2 distance" search of the paper page):
 * writes ref_kv, and ref_idx as the k_eff references with the smallest
 * squared L2 distance between bf16-rounded keys (ties: lower slot), found
 * among the references at positions <= the token's own.  The distances are
 * |k|^2 + |r|^2 - 2 k.r with bf16 products and fp32 accumulation; they never
 * leave the chip.  Fills ws. */
rkv_status rkv_select_refs(const void *K, const void *V, const rkv_cache *c,
                           void *ws, size_t ws_bytes, void *stream);

/* Residual quantisation (paper page, sections "DeltaKV Framework
 * Architecture" -- KV_R is the mean of the selected references and the
 * residual is KV - KV_R -- and "Practical Deployment via Sparse-vLLM" -- the
 * gather, mean and residual are one fused kernel; news page, section "How
 * ResidualKV Works": compact quantised residual codes) with the indices
 * already in c->ref_idx and the references in c->ref_kv (as rkv_select_refs
 * leaves them): for each position and each of K and V, KV_R = the mean of
 * its selected references and residual = x - KV_R, both formed in fp32 (an
 * fp32 sum of the selected rows, divided by k_eff; the result is within
 * 2^-21 (sum of |selected rows| + |x|) of the exact residual), and per group
 * of `group` dims an fp16 scale nearest to max|residual|/qmax (qmax =
 * 2^(bits-1)-1, saturating at 65504) and codes nearest to residual/scale
 * (ties to even), clamped to +-qmax; both roundings are exact for that fp32
 * residual.  bits == 0 stores x - KV_R exactly, in double.  Writes codes_k,
 * codes_v, scales.  ws is unused. */
rkv_status rkv_quantize(const void *K, const void *V, const rkv_cache *c,
                        void *ws, size_t ws_bytes, void *stream);

/* Rebuild the cache (paper page, section "DeltaKV Framework Architecture":
 * KV^ = KV^_delta + KV_R): K_hat, V_hat float [inst][H][N][D].  Reference
 * positions come back from ref_kv; others as KV_R + scale*code (or + the
 * exact residual when bits == 0, which gives the input rows back bit for
 * bit).  For parity checks and debugging; decode never materialises it. */
rkv_status rkv_reconstruct(const rkv_cache *c, float *K_hat, float *V_hat,
                           void *stream);

/* Workspace bytes for rkv_decode_attn* with n_q_heads query heads and
 * n_split partitions of the sequence per (instance, KV head): a QK table
 * and one partial record per (instance, query head, split). */
rkv_status rkv_decode_workspace(const rkv_cache *c, int32_t n_q_heads,
                                int32_t n_split, size_t *bytes);

/* A split count for rkv_decode_attn* on the current device: about three
 * decode blocks per compute unit over all (instance, KV head) pairs, at
 * least 1, at most ceil(seq_len / 32) and 4096.  Host-only (queries the
 * device's CU count); the result is a hint, any n_split >= 1 is valid. */
rkv_status rkv_decode_split_hint(const rkv_cache *c, int32_t n_q_heads, int32_t *n_split);

/* Decode attention straight from the compressed cache (news page, section
 * "How ResidualKV Works": tokens are rebuilt on the fly when attention needs
 * them; paper page, section "Practical Deployment via Sparse-vLLM": the
 * reconstruction is fused to save memory bandwidth): one query per
 * instance, q dtype [inst][n_q_heads][D]; query head h reads KV head
 * h / (n_q_heads / H).  out float [inst][n_q_heads][D] =
 * softmax(softmax_scale * q . K^) . V^ over all N positions, where K^, V^
 * are the reconstructed cache.  The reference mean is folded into the dot
 * products (q . KV_R is the mean of q . K_ref over the selected slots), so
 * no K^/V^ is materialised.  n_split >= 1 partitions each sequence; the
 * result does not depend on it beyond rounding.
 *
 * Arithmetic: q enters fp16 matrix products with a power-of-two pre-scale
 * (the largest |q| of a KV head's query heads moved to [2^8, 2^9)) and the
 * products p * scale_V with a power-of-two exponent per 1024 positions of a
 * split (the largest V scale there moved below 1), so no magnitude of q or
 * V overflows or flushes them; each keeps fp16's 11 bits for values within
 * 2^14 of that largest one, and degrades gradually below (fp16 subnormals).
 * Softmax, scales and merges run in fp32.
 *
 * Limits (RKV_ERR_UNSUPPORTED, checked before any device work): with
 * bits > 0 the query heads of one KV head times the scale groups per row,
 * G * (D / group), must not exceed 16 (e.g. GQA 4 with 32-dim groups, GQA
 * 16 with 128-dim groups); the QK table and the reference weights of every
 * reference are held on chip, (2G + 2 ceil(G/2)) (n_refs + 8) + 1040 G
 * floats of LDS, which must fit 160 KiB (GQA 4: about 3000 references).
 * bits == 0 (exact residuals) rebuilds every attended position from KV_R
 * plus its stored residual and runs plain softmax attention: G <= 16, no
 * per-reference LDS.  A query head whose KV head attends no position (an
 * empty tile selection) gets a zero row. */
rkv_status rkv_decode_attn(const void *q, int32_t n_q_heads,
                           const rkv_cache *c, float softmax_scale,
                           float *out, int32_t n_split, void *ws,
                           size_t ws_bytes, void *stream);

/* rkv_decode_attn over the first `length` positions only (1 <= length <=
 * seq_len), for a cache filled up to there by rkv_append: positions and
 * references beyond are never read.  RKV_ERR_INVALID_ARG for another length. */
rkv_status rkv_decode_attn_len(const void *q, int32_t n_q_heads, const rkv_cache *c,
                               int64_t length, float softmax_scale, float *out, int32_t n_split,
                               void *ws, size_t ws_bytes, void *stream);

/* Selective decompression under a block-sparse attention mask (paper page,
 * section "Training and Inference Integration": only the KV pairs that the
 * sparse attention mask needs are rebuilt; news page, section "Performance
 * Results": about 30% of the attention computation).  Same as
 * rkv_decode_attn, but each (instance, KV head) attends only to the
 * positions of its selected 32-position tiles:
 *   tiles  int32 device [inst][H][n_tiles], tile indices t (positions
 *          32t .. 32t+31, those >= seq_len excluded), distinct; an entry
 *          outside [0, ceil(seq_len/32)) selects nothing.  The order is
 *          free.  Every query head of a KV head uses its KV head's list.
 * The reference rows (QK table, W . Vref) are read as in rkv_decode_attn;
 * only the selected tiles' records are streamed.  Workspace as for
 * rkv_decode_attn.  RKV_ERR_INVALID_ARG if n_tiles < 1 or tiles is NULL. */
rkv_status rkv_decode_attn_tiles(const void *q, int32_t n_q_heads, const rkv_cache *c,
                                 float softmax_scale, const int32_t *tiles, int32_t n_tiles,
                                 float *out, int32_t n_split, void *ws, size_t ws_bytes,
                                 void *stream);

/* Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): rkv_decode_attn with its workspace taken from a fixed device
 * array of RKV_SCRATCH_BYTES inside the library instead of a caller buffer.
 * Each GPU the library runs on holds its own copy of that array until the
 * process ends; the first call on a device looks up its address there (a
 * host-side query).  The call allocates nothing and launches the same
 * kernels as rkv_decode_attn, so the results are the same bits.
 * RKV_ERR_WORKSPACE when rkv_decode_workspace(c, n_q_heads, n_split) exceeds
 * RKV_SCRATCH_BYTES (checked before any device work); other errors as for
 * rkv_decode_attn.  All calls on one GPU share the array and nothing in it
 * is kept between calls: calls that overlap on one GPU (other streams, other
 * host threads) race and must be serialised by the caller. */
#define RKV_SCRATCH_BYTES (32u << 20)
rkv_status rkv_decode_attn_noalloc(const void *q, int32_t n_q_heads, const rkv_cache *c,
                                   float softmax_scale, float *out, int32_t n_split,
                                   void *stream);

const char *rkv_status_string(rkv_status s);
int32_t rkv_last_hip_error(void);
int32_t rkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RKV_H */
