// Host side of librkv: argument checks, buffer sizes and kernel dispatch.
// The entry points are declared (and documented) in include/rkv.h.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/rkv.h"
#include "rkv_common.h"

namespace rkv {
// Encode kernels work on positions [p0, p0 + n_in) whose K/V rows are the
// input [inst][H][n_in][128]; the cache keeps its full [.][.][N] layout.
hipError_t launch_refstore(int dtype, const void* K, const void* V, void* ref_kv,
                           uint16_t* ref_scales, int ref_bits, int group, void* refkey,
                           float* refnorm, int64_t n_inst, int H, int64_t p0, int64_t n_in,
                           int64_t n_refs, Sched sc, hipStream_t st);
hipError_t launch_dist_topk(int dtype, const void* K, const void* refkey, const float* refnorm,
                            uint16_t* idx, int64_t n_inst, int H, int64_t N, int64_t n_refs,
                            Sched sc, int k, int64_t p0, int64_t n_in, hipStream_t st);
hipError_t launch_quantize(int dtype, int bits, const void* K, const void* V,
                           const uint16_t* idx, const void* ref_kv, const uint16_t* ref_scales,
                           int ref_bits, uint8_t* ck, uint8_t* cv,
                           uint16_t* sc16, int64_t n_inst, int H, int64_t N, int64_t n_refs,
                           Sched sc, int k, int group, int64_t p0, int64_t n_in,
                           const LatMask* lm, hipStream_t st);
hipError_t launch_reconstruct(int dtype, int bits, const uint16_t* idx, const void* ref_kv,
                              const uint16_t* ref_scales, int ref_bits, const uint8_t* ck, const uint8_t* cv, const uint16_t* sc16,
                              float* Kh, float* Vh, int64_t n_inst, int H, int64_t N,
                              int64_t n_refs, Sched sc, int k, int group, const LatMask* lm,
                              hipStream_t st);
hipError_t launch_decode(int dtype, int bits, const void* q, int n_q_heads, const uint16_t* idx,
                         const void* ref_kv, const uint16_t* ref_scales, int ref_bits,
                         const uint8_t* ck, const uint8_t* cv,
                         const uint16_t* sc16, float softmax_scale, float* out, int n_split,
                         void* ws, int64_t n_inst, int H, int64_t N, int64_t len,
                         int64_t n_refs, Sched sc, int k, int group, const int32_t* tile_list,
                         int32_t n_list, const LatMask* lm, hipStream_t st);
size_t decode_ws_bytes(int64_t n_inst, int H, int n_q_heads, int n_split, int64_t n_refs,
                       bool latent);
bool decode_fits(int G, int group, int64_t n_refs, int n_split, bool exact);
}  // namespace rkv

using rkv::Sched;

namespace {

thread_local int32_t g_last_hip = 0;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

constexpr int64_t kMaxPos = int64_t(1) << 30;  // positions must stay below 2^30
// Positions per sequence in a cache: the kernels address one head's rows,
// codes and slots with 32-bit byte offsets and buffer ranges (an fp32 row is
// 512 bytes, so 2^22 rows are 2^31 bytes).
constexpr int64_t kMaxSeqLen = int64_t(1) << 22;

bool sched_ok(rkv_stride s) {
  if (s.base < 1 || s.base > (1 << 20)) return false;
  if (s.double_after < 0 || s.double_after > kMaxPos) return false;
  if (s.double_after > 0 && s.double_after % (2 * (int64_t)s.base) != 0) return false;
  return true;
}

Sched to_sched(rkv_stride s) { return rkv::make_sched(s.base, s.double_after); }

rkv_status hip_status(hipError_t e) {
  if (e == hipSuccess) return RKV_OK;
  g_last_hip = (int32_t)e;
  return RKV_ERR_HIP;
}

size_t elt_bytes(rkv_dtype d) { return d == RKV_F32 ? 4 : 2; }

// The kernels read rows with 16-byte (index rows: 2k-byte, at most 16)
// vector loads; misaligned buffers are rejected up front.
inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline bool al16(const void* p) { return aligned(p, 16); }

// The dtype field as the integer a C caller stored: C++ may not load a value
// outside the enumerators' range through the enum type, so the field is
// validated on its bytes before anything reads it as rkv_dtype.
static_assert(sizeof(rkv_dtype) == sizeof(int32_t), "rkv_dtype is stored as a C int");
inline int32_t dtype_code(const rkv_cache* c) {
  int32_t v;
  memcpy(&v, &c->dtype, sizeof v);
  return v;
}

rkv_status check_shape(const rkv_cache* c) {
  if (!c) return RKV_ERR_INVALID_ARG;
  const int32_t dt = dtype_code(c);
  if (dt != RKV_F32 && dt != RKV_BF16) return RKV_ERR_INVALID_ARG;
  if (c->n_inst < 0 || c->n_kv_heads < 1 || c->seq_len < 0) return RKV_ERR_INVALID_ARG;
  if (c->seq_len > kMaxSeqLen) return RKV_ERR_INVALID_ARG;
  if (c->n_inst > 65535 || c->n_kv_heads > 65535) return RKV_ERR_INVALID_ARG;
  if (!sched_ok(c->stride)) return RKV_ERR_INVALID_ARG;
  if (c->k < 1 || c->k > 16) return RKV_ERR_INVALID_ARG;
  if (c->bits != 0 && c->bits != 2 && c->bits != 4 && c->bits != 8) return RKV_ERR_INVALID_ARG;
  if (c->head_dim != 128) return c->head_dim > 0 ? RKV_ERR_UNSUPPORTED : RKV_ERR_INVALID_ARG;
  if (c->bits != 0) {
    if (c->group != 32 && c->group != 64 && c->group != 128) return RKV_ERR_INVALID_ARG;
  }
  if (c->ref_bits != 0 && c->ref_bits != 4) return RKV_ERR_INVALID_ARG;
  if (c->ref_bits != 0 && c->bits == 0) return RKV_ERR_INVALID_ARG;
  if (c->latent != 0 && c->latent != 1) return RKV_ERR_INVALID_ARG;
  if (c->latent != 0 && c->bits == 0) return RKV_ERR_INVALID_ARG;
  const int64_t nr = rkv::sched_count((int32_t)c->seq_len, to_sched(c->stride));
  if (nr > 65535) return RKV_ERR_RANGE;
  return RKV_OK;
}

rkv_status check_ready(const rkv_cache* c) {
  rkv_status s = check_shape(c);
  if (s != RKV_OK) return s;
  if (c->n_refs != rkv::sched_count((int32_t)c->seq_len, to_sched(c->stride))) return RKV_ERR_INVALID_ARG;
  if (c->n_inst == 0 || c->seq_len == 0) return RKV_OK;
  if (!c->ref_idx || !c->codes_k || !c->codes_v || !c->ref_kv) return RKV_ERR_INVALID_ARG;
  if (c->bits != 0 && !c->scales) return RKV_ERR_INVALID_ARG;
  if (c->ref_bits != 0 && !c->ref_scales) return RKV_ERR_INVALID_ARG;
  const uintptr_t idx_align = (c->k & (c->k - 1)) == 0 ? (c->k >= 8 ? 16 : 2 * c->k) : 2;
  if (!al16(c->codes_k) || !al16(c->codes_v) || !al16(c->ref_kv) ||
      !aligned(c->ref_idx, idx_align) || !aligned(c->scales, 4) || !aligned(c->ref_scales, 2))
    return RKV_ERR_INVALID_ARG;
  return RKV_OK;
}

void sizes_of(const rkv_cache* c, size_t out[6]) {
  const size_t ih = (size_t)c->n_inst * c->n_kv_heads;
  const size_t N = (size_t)c->seq_len;
  const size_t D = (size_t)c->head_dim;
  out[0] = ih * N * c->k * 2;
  if (c->bits == 0) {
    out[1] = ih * N * D * 8;
    out[2] = ih * N * D * 8;
    out[3] = 0;
  } else {
    out[1] = ih * N * D * c->bits / 8;
    out[2] = ih * ((N + 31) / 32) * D * (32 * c->bits / 8);
    out[3] = ih * N * 2 * (D / c->group) * 2;
  }
  if (c->ref_bits == 4) {
    out[4] = ih * 2 * (size_t)c->n_refs * D / 2;
    out[5] = ih * 2 * (size_t)c->n_refs * (D / c->group) * 2;
  } else {
    out[4] = ih * 2 * (size_t)c->n_refs * D * elt_bytes(c->dtype);
    out[5] = 0;
  }
}

// The latent sign mask of a cache, or NULL when latent codes are off.
struct LatArg {
  rkv::LatMask m;
  const rkv::LatMask* p;
  explicit LatArg(const rkv_cache* c) : m(rkv::make_latmask(c->latent_seed)), p(c->latent ? &m : nullptr) {}
};

size_t encode_ws(const rkv_cache* c) {
  const size_t nr = (size_t)c->n_inst * c->n_kv_heads * c->n_refs;
  return align_up(nr * 128 * 2) + align_up(nr * 4);
}

}  // namespace

extern "C" {

int64_t rkv_num_refs(int64_t seq_len, rkv_stride stride) {
  if (!sched_ok(stride) || seq_len < 0 || seq_len > kMaxPos) return -1;
  return rkv::sched_count((int32_t)seq_len, to_sched(stride));
}

int64_t rkv_ref_position(int64_t slot, rkv_stride stride) {
  if (!sched_ok(stride) || slot < 0) return -1;
  const Sched sc = to_sched(stride);
  if (slot >= rkv::sched_count((int32_t)kMaxPos, sc)) return -1;  // position beyond 2^30
  return rkv::sched_pos((int32_t)slot, sc);
}

rkv_status rkv_cache_init(rkv_cache* c) {
  rkv_status s = check_shape(c);
  if (s != RKV_OK) return s;
  c->n_refs = rkv::sched_count((int32_t)c->seq_len, to_sched(c->stride));
  return RKV_OK;
}

rkv_status rkv_cache_sizes(const rkv_cache* c, size_t sizes[6]) {
  if (!sizes) return RKV_ERR_INVALID_ARG;
  rkv_status s = check_shape(c);
  if (s != RKV_OK) return s;
  if (c->n_refs != rkv::sched_count((int32_t)c->seq_len, to_sched(c->stride))) return RKV_ERR_INVALID_ARG;
  sizes_of(c, sizes);
  return RKV_OK;
}

rkv_status rkv_encode_workspace(const rkv_cache* c, size_t* bytes) {
  if (!bytes) return RKV_ERR_INVALID_ARG;
  rkv_status s = check_shape(c);
  if (s != RKV_OK) return s;
  if (c->n_refs != rkv::sched_count((int32_t)c->seq_len, to_sched(c->stride))) return RKV_ERR_INVALID_ARG;
  *bytes = encode_ws(c);
  return RKV_OK;
}

// Reference store + selection for positions [p0, p0 + n_in).
static rkv_status select_range(const void* K, const void* V, const rkv_cache* c, int64_t p0,
                               int64_t n_in, void* ws, size_t ws_bytes, hipStream_t st) {
  const size_t need = encode_ws(c);
  if (!ws || ws_bytes < need) return RKV_ERR_WORKSPACE;
  if (!al16(ws)) return RKV_ERR_INVALID_ARG;
  const size_t nr = (size_t)c->n_inst * c->n_kv_heads * c->n_refs;
  char* refkey = (char*)ws;
  float* refnorm = (float*)((char*)ws + align_up(nr * 128 * 2));
  const Sched sc = to_sched(c->stride);
  hipError_t e = rkv::launch_refstore((int)c->dtype, K, V, c->ref_kv, c->ref_scales, c->ref_bits,
                                      c->group, refkey, refnorm, c->n_inst,
                                      c->n_kv_heads, p0, n_in, c->n_refs, sc, st);
  if (e != hipSuccess) return hip_status(e);
  e = rkv::launch_dist_topk((int)c->dtype, K, refkey, refnorm, c->ref_idx, c->n_inst,
                            c->n_kv_heads, c->seq_len, c->n_refs, sc, c->k, p0, n_in, st);
  return hip_status(e);
}

static rkv_status quantize_range(const void* K, const void* V, const rkv_cache* c, int64_t p0,
                                 int64_t n_in, hipStream_t st) {
  const LatArg lat(c);
  hipError_t e = rkv::launch_quantize((int)c->dtype, c->bits, K, V, c->ref_idx, c->ref_kv,
                                      c->ref_scales, c->ref_bits, c->codes_k, c->codes_v, c->scales, c->n_inst,
                                      c->n_kv_heads, c->seq_len, c->n_refs,
                                      to_sched(c->stride), c->k, c->group, p0, n_in,
                                      lat.p, st);
  return hip_status(e);
}

rkv_status rkv_select_refs(const void* K, const void* V, const rkv_cache* c, void* ws,
                           size_t ws_bytes, void* stream) {
  rkv_status s = check_ready(c);
  if (s != RKV_OK) return s;
  if (c->n_inst == 0 || c->seq_len == 0) return RKV_OK;
  if (!K || !V || !al16(K) || !al16(V)) return RKV_ERR_INVALID_ARG;
  return select_range(K, V, c, 0, c->seq_len, ws, ws_bytes, (hipStream_t)stream);
}

rkv_status rkv_quantize(const void* K, const void* V, const rkv_cache* c, void* ws,
                        size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  rkv_status s = check_ready(c);
  if (s != RKV_OK) return s;
  if (c->n_inst == 0 || c->seq_len == 0) return RKV_OK;
  if (!K || !V || !al16(K) || !al16(V)) return RKV_ERR_INVALID_ARG;
  return quantize_range(K, V, c, 0, c->seq_len, (hipStream_t)stream);
}

rkv_status rkv_encode(const void* K, const void* V, const rkv_cache* c, void* ws,
                      size_t ws_bytes, void* stream) {
  rkv_status s = rkv_select_refs(K, V, c, ws, ws_bytes, stream);
  if (s != RKV_OK) return s;
  return rkv_quantize(K, V, c, ws, ws_bytes, stream);
}

rkv_status rkv_append(const void* K_new, const void* V_new, int64_t n_new, const rkv_cache* c,
                      int64_t pos0, void* ws, size_t ws_bytes, void* stream) {
  rkv_status s = check_ready(c);
  if (s != RKV_OK) return s;
  if (n_new < 1 || pos0 < 0 || pos0 + n_new > c->seq_len) return RKV_ERR_INVALID_ARG;
  if (c->n_inst == 0) return RKV_OK;
  if (!K_new || !V_new || !al16(K_new) || !al16(V_new)) return RKV_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  s = select_range(K_new, V_new, c, pos0, n_new, ws, ws_bytes, st);
  if (s != RKV_OK) return s;
  return quantize_range(K_new, V_new, c, pos0, n_new, st);
}

rkv_status rkv_reconstruct(const rkv_cache* c, float* K_hat, float* V_hat, void* stream) {
  rkv_status s = check_ready(c);
  if (s != RKV_OK) return s;
  if (c->n_inst == 0 || c->seq_len == 0) return RKV_OK;
  if (!K_hat || !V_hat || !al16(K_hat) || !al16(V_hat)) return RKV_ERR_INVALID_ARG;
  const LatArg lat(c);
  hipError_t e = rkv::launch_reconstruct((int)c->dtype, c->bits, c->ref_idx, c->ref_kv,
                                         c->ref_scales, c->ref_bits,
                                         c->codes_k, c->codes_v, c->scales, K_hat, V_hat,
                                         c->n_inst, c->n_kv_heads, c->seq_len, c->n_refs,
                                         to_sched(c->stride), c->k, c->group, lat.p,
                                         (hipStream_t)stream);
  return hip_status(e);
}

rkv_status rkv_decode_workspace(const rkv_cache* c, int32_t n_q_heads, int32_t n_split,
                                size_t* bytes) {
  if (!bytes) return RKV_ERR_INVALID_ARG;
  rkv_status s = check_shape(c);
  if (s != RKV_OK) return s;
  if (n_q_heads < 1 || n_q_heads % c->n_kv_heads != 0 || n_split < 1 || n_split > 4096)
    return RKV_ERR_INVALID_ARG;
  *bytes = rkv::decode_ws_bytes(c->n_inst, c->n_kv_heads, n_q_heads, n_split,
                                rkv::sched_count((int32_t)c->seq_len, to_sched(c->stride)),
                                c->latent != 0);
  return RKV_OK;
}

rkv_status rkv_decode_split_hint(const rkv_cache* c, int32_t n_q_heads, int32_t* n_split) {
  if (!n_split) return RKV_ERR_INVALID_ARG;
  rkv_status s = check_shape(c);
  if (s != RKV_OK) return s;
  if (n_q_heads < 1 || n_q_heads % c->n_kv_heads != 0) return RKV_ERR_INVALID_ARG;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  // about three decode blocks per compute unit: the kernel holds three per
  // CU, and more splits only add partial records to merge
  const int64_t heads = c->n_inst * (int64_t)c->n_kv_heads;
  const int64_t tiles = (c->seq_len + 31) / 32;
  int64_t ns = heads > 0 ? (3 * (int64_t)cus + heads - 1) / heads : 1;
  if (ns > tiles) ns = tiles;
  if (ns > 4096) ns = 4096;
  *n_split = (int32_t)(ns < 1 ? 1 : ns);
  return RKV_OK;
}

static rkv_status decode_common(const void* q, int32_t n_q_heads, const rkv_cache* c,
                                int64_t length, float softmax_scale, float* out,
                                const int32_t* tiles, int32_t n_tiles, int32_t n_split, void* ws,
                                size_t ws_bytes, void* stream) {
  if (length < 1 || length > c->seq_len) return RKV_ERR_INVALID_ARG;
  rkv_status s = check_ready(c);
  if (s != RKV_OK) return s;
  if (n_q_heads < 1 || n_q_heads % c->n_kv_heads != 0 || n_split < 1 || n_split > 4096)
    return RKV_ERR_INVALID_ARG;
  const int G = n_q_heads / c->n_kv_heads;
  // The quantised decode holds one MFMA row per (query head, scale group) of
  // a KV head: at most 16.  Exact residuals (bits = 0) take one row per
  // query head.
  const int rows = c->bits == 0 ? G : G * (c->head_dim / c->group);
  if (rows > 16) return RKV_ERR_UNSUPPORTED;
  // LDS holds the QK table and reference weights of every reference
  if (!rkv::decode_fits(G, c->bits == 0 ? 128 : c->group, c->n_refs, n_split, c->bits == 0))
    return RKV_ERR_UNSUPPORTED;
  if (c->n_inst == 0) return RKV_OK;
  if (!q || !out || !al16(q) || !al16(out)) return RKV_ERR_INVALID_ARG;
  if (c->seq_len == 0) return RKV_ERR_INVALID_ARG;
  const size_t need = rkv::decode_ws_bytes(c->n_inst, c->n_kv_heads, n_q_heads, n_split, c->n_refs,
                                           c->latent != 0);
  if (!ws || ws_bytes < need) return RKV_ERR_WORKSPACE;
  if (!al16(ws)) return RKV_ERR_INVALID_ARG;
  const LatArg lat(c);
  hipError_t e = rkv::launch_decode((int)c->dtype, c->bits, q, n_q_heads, c->ref_idx, c->ref_kv,
                                    c->ref_scales, c->ref_bits,
                                    c->codes_k, c->codes_v, c->scales, softmax_scale, out,
                                    n_split, ws, c->n_inst, c->n_kv_heads, c->seq_len, length,
                                    c->n_refs, to_sched(c->stride), c->k, c->group, tiles,
                                    n_tiles, lat.p, (hipStream_t)stream);
  return hip_status(e);
}

rkv_status rkv_decode_attn(const void* q, int32_t n_q_heads, const rkv_cache* c,
                           float softmax_scale, float* out, int32_t n_split, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!c) return RKV_ERR_INVALID_ARG;
  return decode_common(q, n_q_heads, c, c->seq_len, softmax_scale, out, nullptr, 0, n_split, ws,
                       ws_bytes, stream);
}

rkv_status rkv_decode_attn_len(const void* q, int32_t n_q_heads, const rkv_cache* c,
                               int64_t length, float softmax_scale, float* out, int32_t n_split,
                               void* ws, size_t ws_bytes, void* stream) {
  if (!c) return RKV_ERR_INVALID_ARG;
  return decode_common(q, n_q_heads, c, length, softmax_scale, out, nullptr, 0, n_split, ws,
                       ws_bytes, stream);
}

rkv_status rkv_decode_attn_tiles(const void* q, int32_t n_q_heads, const rkv_cache* c,
                                 float softmax_scale, const int32_t* tiles, int32_t n_tiles,
                                 float* out, int32_t n_split, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (n_tiles < 0 || (n_tiles > 0 && !tiles)) return RKV_ERR_INVALID_ARG;
  if (n_tiles == 0) return RKV_ERR_INVALID_ARG;  // attention over no position is undefined
  if (!c) return RKV_ERR_INVALID_ARG;
  return decode_common(q, n_q_heads, c, c->seq_len, softmax_scale, out, tiles, n_tiles, n_split,
                       ws, ws_bytes, stream);
}

}  // extern "C"

// Fixed device scratch of rkv_decode_attn_noalloc (each GPU the library runs
// on holds its own copy until the process ends).  In host code this name is
// only a stand-in: the kernels get the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[RKV_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, resolved once per device.
rkv_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return RKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return RKV_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RKV_OK;
}

}  // namespace

extern "C" {

rkv_status rkv_decode_attn_noalloc(const void* q, int32_t n_q_heads, const rkv_cache* c,
                                   float softmax_scale, float* out, int32_t n_split,
                                   void* stream) {
  size_t need = 0;
  rkv_status s = rkv_decode_workspace(c, n_q_heads, n_split, &need);
  if (s != RKV_OK) return s;
  if (need > (size_t)RKV_SCRATCH_BYTES) return RKV_ERR_WORKSPACE;
  s = check_ready(c);
  if (s != RKV_OK) return s;
  void* ws = nullptr;
  s = scratch_address(&ws);
  if (s != RKV_OK) return s;
  // Every kernel of the decode writes the parts of the scratch it later
  // reads (QK table, partial records, rotated rows): nothing needs clearing.
  return decode_common(q, n_q_heads, c, c->seq_len, softmax_scale, out, nullptr, 0, n_split, ws,
                       (size_t)RKV_SCRATCH_BYTES, stream);
}

const char* rkv_status_string(rkv_status s) {
  switch (s) {
    case RKV_OK: return "ok";
    case RKV_ERR_INVALID_ARG: return "invalid argument";
    case RKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case RKV_ERR_WORKSPACE: return "workspace too small";
    case RKV_ERR_HIP: return "HIP error";
    case RKV_ERR_RANGE: return "more than 65535 references";
  }
  return "unknown status";
}

int32_t rkv_last_hip_error(void) { return g_last_hip; }

int32_t rkv_version(void) { return 1; }

}  // extern "C"
