"""Host-side checks of librkv's C ABI: it loads, exports every entry point the
header declares, and its host logic (schedule, shape checks, sizes, error
codes) is right.  No GPU work is launched: every call here either is pure
host arithmetic or fails validation before touching the device."""

import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
from conftest import ROOT

from long_context_attention_rkv_amd import _lib as L

HEADER = os.path.join(ROOT, "include", "rkv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from long_context_attention_rkv_amd.build import build
        build(verbose=False)
    return L.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rkv_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.SIGNATURES, f"{n} has no ctypes signature"


def _st(b, a=0):
    return L.RkvStride(b, a)


@pytest.mark.parametrize("n,base,A", [(1024, 16, 0), (1000, 7, 0), (1, 1, 0), (0, 4, 0),
                                      (131072, 16, 4096), (9000, 16, 4096), (5000, 16, 512),
                                      (4097, 16, 4096), (777, 32, 0), (100, 3, 12)])
def test_num_refs_and_positions_match_the_oracle_schedule(lib, n, base, A):
    T = oracle.ref_positions(n, base, A)
    assert lib.rkv_num_refs(n, _st(base, A)) == T.shape[0]
    for s, p in enumerate(T):
        assert lib.rkv_ref_position(s, _st(base, A)) == p


@pytest.mark.parametrize("n,base,A", [(1_000_003, 7, 0), (1 << 20, 3, 3072), (600_000, 16, 4096),
                                      (300_000, 5, 40), (262_144, 1, 2), (131072, 16, 4096)])
def test_num_refs_and_positions_at_scale(lib, n, base, A):
    """The library's constant-division schedule against a plain walk."""
    T = oracle.ref_positions(n, base, A) if n <= 300_000 else None
    if T is None:
        pos, j = [], 0
        while j < n:
            s = base
            if A and j >= A:
                b = 0
                while j >= A << b:
                    b += 1
                s = base << b
            if j % s == 0:
                pos.append(j)
            j += 1 if (A and j >= A) or base > 1 else 1
        T = np.array(pos)
    assert lib.rkv_num_refs(n, _st(base, A)) == T.shape[0]
    for s in list(range(0, T.shape[0], max(1, T.shape[0] // 2000))) + [T.shape[0] - 1]:
        assert lib.rkv_ref_position(s, _st(base, A)) == T[s]


def test_schedule_rejects_bad_strides(lib):
    assert lib.rkv_num_refs(100, _st(0)) == -1
    assert lib.rkv_num_refs(100, _st(16, 100)) == -1      # not a multiple of 2*base
    assert lib.rkv_num_refs(-1, _st(16)) == -1


def _cache(**kw):
    c = L.RkvCache()
    c.dtype = kw.get("dtype", L.RKV_BF16)
    c.n_inst = kw.get("n_inst", 2)
    c.n_kv_heads = kw.get("H", 8)
    c.seq_len = kw.get("N", 8192)
    c.head_dim = kw.get("D", 128)
    c.stride = _st(kw.get("base", 32), kw.get("A", 0))
    c.k = kw.get("k", 8)
    c.bits = kw.get("bits", 4)
    c.group = kw.get("group", 32)
    c.ref_bits = kw.get("ref_bits", 0)
    c.latent = kw.get("latent", 0)
    c.latent_seed = kw.get("latent_seed", 0)
    return c


def test_cache_init_and_sizes(lib):
    c = _cache()
    assert lib.rkv_cache_init(C.byref(c)) == L.RKV_OK
    assert c.n_refs == 256
    sz = (C.c_size_t * 6)()
    assert lib.rkv_cache_sizes(C.byref(c), sz) == L.RKV_OK
    ih, N = 16, 8192
    assert list(sz) == [ih * N * 8 * 2, ih * N * 64, ih * (N // 32) * 128 * 16,
                        ih * N * 2 * 4 * 2, ih * 2 * 256 * 128 * 2, 0]
    # per head-token record: 64 + 64 code bytes, 16 scale bytes, 16 index bytes
    assert (sz[0] + sz[1] + sz[2] + sz[3]) // (ih * N) == 160
    # full-pipeline quantisation: the reference rows as int4 + fp16 scales
    c.ref_bits = 4
    assert lib.rkv_cache_sizes(C.byref(c), sz) == L.RKV_OK
    assert (sz[4], sz[5]) == (ih * 2 * 256 * 64, ih * 2 * 256 * 4 * 2)


@pytest.mark.parametrize("bad,status", [
    (dict(k=0), L.RKV_ERR_INVALID_ARG), (dict(k=17), L.RKV_ERR_INVALID_ARG),
    (dict(bits=3), L.RKV_ERR_INVALID_ARG), (dict(group=48), L.RKV_ERR_INVALID_ARG),
    (dict(D=64), L.RKV_ERR_UNSUPPORTED), (dict(base=0), L.RKV_ERR_INVALID_ARG),
    (dict(dtype=7), L.RKV_ERR_INVALID_ARG), (dict(H=0), L.RKV_ERR_INVALID_ARG),
    (dict(N=65536 * 2, base=2), L.RKV_ERR_RANGE), (dict(A=100, base=16), L.RKV_ERR_INVALID_ARG),
    (dict(ref_bits=2), L.RKV_ERR_INVALID_ARG), (dict(ref_bits=4, bits=0), L.RKV_ERR_INVALID_ARG),
    (dict(latent=2), L.RKV_ERR_INVALID_ARG), (dict(latent=1, bits=0), L.RKV_ERR_INVALID_ARG),
    # more positions than the kernels' 32-bit row offsets reach
    (dict(N=(1 << 22) + 32, base=1 << 16), L.RKV_ERR_INVALID_ARG),
])
def test_cache_init_rejects(lib, bad, status):
    c = _cache(**bad)
    assert lib.rkv_cache_init(C.byref(c)) == status


def test_longest_sequence_is_accepted(lib):
    c = _cache(n_inst=1, H=1, N=1 << 22, base=1 << 16)
    assert lib.rkv_cache_init(C.byref(c)) == L.RKV_OK
    assert c.n_refs == 64


def test_entry_points_validate_before_touching_the_device(lib):
    c = _cache()
    assert lib.rkv_cache_init(C.byref(c)) == L.RKV_OK
    null = C.c_void_p(0)
    # buffers unset -> invalid argument, no launch
    assert lib.rkv_encode(null, null, C.byref(c), null, 0, null) == L.RKV_ERR_INVALID_ARG
    for name in ("ref_idx", "codes_k", "codes_v", "scales", "ref_kv"):
        setattr(c, name, 0x1000)
    # K/V missing
    assert lib.rkv_select_refs(null, null, C.byref(c), null, 0, null) == L.RKV_ERR_INVALID_ARG
    # workspace too small
    ws = C.c_size_t()
    assert lib.rkv_encode_workspace(C.byref(c), C.byref(ws)) == L.RKV_OK
    assert ws.value >= 16 * 256 * (256 + 4)
    assert lib.rkv_select_refs(C.c_void_p(0x2000), C.c_void_p(0x3000), C.byref(c),
                               C.c_void_p(0x4000), ws.value - 1, null) == L.RKV_ERR_WORKSPACE
    # decode: GQA groups must divide, workspace checked, quantisation required
    assert lib.rkv_decode_workspace(C.byref(c), 30, 4, C.byref(ws)) == L.RKV_ERR_INVALID_ARG
    assert lib.rkv_decode_workspace(C.byref(c), 32, 4, C.byref(ws)) == L.RKV_OK
    out = C.c_void_p(0x5000)
    assert lib.rkv_decode_attn(C.c_void_p(0x6000), 32, C.byref(c), 0.1, out, 4,
                               C.c_void_p(0x7000), ws.value - 1, null) == L.RKV_ERR_WORKSPACE
    # streaming encode: the range must lie inside the cache
    for pos0, n_new in ((-1, 1), (0, 0), (8190, 3), (8192, 1)):
        assert lib.rkv_append(C.c_void_p(0x2000), C.c_void_p(0x3000), n_new, C.byref(c), pos0,
                              C.c_void_p(0x4000), 1 << 40, null) == L.RKV_ERR_INVALID_ARG
    assert lib.rkv_append(C.c_void_p(0x2000), C.c_void_p(0x3000), 1, C.byref(c), 100,
                          C.c_void_p(0x4000), 16, null) == L.RKV_ERR_WORKSPACE
    # decode over a prefix: 1 <= length <= seq_len
    for length in (0, 8193):
        assert lib.rkv_decode_attn_len(C.c_void_p(0x6000), 32, C.byref(c), length, 0.1, out, 4,
                                       C.c_void_p(0x7000), ws.value, null) == L.RKV_ERR_INVALID_ARG
    # block-sparse decode: a tile list is required, and must not be empty
    assert lib.rkv_decode_attn_tiles(C.c_void_p(0x6000), 32, C.byref(c), 0.1, null, 4, out, 4,
                                     C.c_void_p(0x7000), ws.value, null) == L.RKV_ERR_INVALID_ARG
    assert lib.rkv_decode_attn_tiles(C.c_void_p(0x6000), 32, C.byref(c), 0.1,
                                     C.c_void_p(0x8000), 0, out, 4, C.c_void_p(0x7000),
                                     ws.value, null) == L.RKV_ERR_INVALID_ARG
    assert lib.rkv_decode_attn_tiles(C.c_void_p(0x6000), 32, C.byref(c), 0.1,
                                     C.c_void_p(0x8000), 4, out, 4, C.c_void_p(0x7000),
                                     ws.value - 1, null) == L.RKV_ERR_WORKSPACE
    # exact residuals (bits = 0) decode too; the workspace is still checked
    c.bits = 0
    assert lib.rkv_decode_workspace(C.byref(c), 32, 4, C.byref(ws)) == L.RKV_OK
    assert lib.rkv_decode_attn(C.c_void_p(0x6000), 32, C.byref(c), 0.1, out, 4,
                               C.c_void_p(0x7000), ws.value - 1, null) == L.RKV_ERR_WORKSPACE
    # n_refs not initialised for this shape
    c2 = _cache()
    assert lib.rkv_encode(C.c_void_p(1), C.c_void_p(1), C.byref(c2), null, 0, null) == \
        L.RKV_ERR_INVALID_ARG


def test_status_strings(lib):
    for s in range(6):
        assert lib.rkv_status_string(s)
    assert lib.rkv_version() >= 1


def test_latent_decode_workspace_holds_two_rows_per_query_head(lib):
    c = _cache()
    assert lib.rkv_cache_init(C.byref(c)) == L.RKV_OK
    plain, lat = C.c_size_t(), C.c_size_t()
    assert lib.rkv_decode_workspace(C.byref(c), 32, 4, C.byref(plain)) == L.RKV_OK
    c.latent, c.latent_seed = 1, 0xFFFFFFFFFFFFFFFF
    assert lib.rkv_cache_init(C.byref(c)) == L.RKV_OK
    assert lib.rkv_decode_workspace(C.byref(c), 32, 4, C.byref(lat)) == L.RKV_OK
    # rotated queries and rotated residual outputs, fp32 [inst][n_q_heads][128] each
    assert lat.value - plain.value >= 2 * 2 * 32 * 128 * 4
    # the code sizes do not change
    sz_p, sz_l = (C.c_size_t * 6)(), (C.c_size_t * 6)()
    c.latent = 0
    lib.rkv_cache_sizes(C.byref(c), sz_p)
    c.latent = 1
    lib.rkv_cache_sizes(C.byref(c), sz_l)
    assert list(sz_p) == list(sz_l)


def test_misaligned_buffers_are_rejected(lib):
    c = _cache()
    assert lib.rkv_cache_init(C.byref(c)) == L.RKV_OK
    for name in ("ref_idx", "codes_k", "codes_v", "scales", "ref_kv"):
        setattr(c, name, 0x10000)
    null = C.c_void_p(0)
    ws = C.c_void_p(0x40000)
    big = 1 << 40
    K, V = C.c_void_p(0x20000), C.c_void_p(0x30000)
    # aligned pointers pass validation up to the workspace check
    assert lib.rkv_select_refs(K, V, C.byref(c), ws, 16, null) == L.RKV_ERR_WORKSPACE
    # K, V, workspace off by 8 bytes
    assert lib.rkv_select_refs(C.c_void_p(0x20008), V, C.byref(c), ws, big, null) == L.RKV_ERR_INVALID_ARG
    assert lib.rkv_quantize(K, C.c_void_p(0x30008), C.byref(c), ws, big, null) == L.RKV_ERR_INVALID_ARG
    assert lib.rkv_select_refs(K, V, C.byref(c), C.c_void_p(0x40008), big, null) == L.RKV_ERR_INVALID_ARG
    assert lib.rkv_append(C.c_void_p(0x20004), V, 1, C.byref(c), 5, ws, big, null) == L.RKV_ERR_INVALID_ARG
    # a cache buffer off by 8 bytes
    for name in ("codes_k", "codes_v", "ref_kv", "ref_idx"):
        setattr(c, name, 0x10008)
        assert lib.rkv_quantize(K, V, C.byref(c), ws, big, null) == L.RKV_ERR_INVALID_ARG, name
        setattr(c, name, 0x10000)
    # decode: q and out
    out = C.c_void_p(0x50000)
    assert lib.rkv_decode_attn(C.c_void_p(0x60004), 32, C.byref(c), 0.1, out, 4, ws, big,
                               null) == L.RKV_ERR_INVALID_ARG
    assert lib.rkv_decode_attn(C.c_void_p(0x60000), 32, C.byref(c), 0.1, C.c_void_p(0x50004), 4,
                               ws, big, null) == L.RKV_ERR_INVALID_ARG
    # reconstruct outputs
    assert lib.rkv_reconstruct(C.byref(c), C.c_void_p(0x70002), C.c_void_p(0x80000),
                               null) == L.RKV_ERR_INVALID_ARG


def test_decode_split_hint(lib):
    ns = C.c_int32()
    # 8 sequences x 8 KV heads of 32K: about three blocks per CU (256 CUs
    # when the device cannot be queried, as on a host without a GPU)
    c = _cache(n_inst=8, H=8, N=32768, base=64)
    assert lib.rkv_cache_init(C.byref(c)) == L.RKV_OK
    assert lib.rkv_decode_split_hint(C.byref(c), 32, C.byref(ns)) == L.RKV_OK
    assert ns.value == 12  # 64 heads x 12 = 768 blocks: three per CU
    # more heads than three blocks per CU: one split each
    many = _cache(n_inst=256, H=8, N=32768, base=64)
    assert lib.rkv_cache_init(C.byref(many)) == L.RKV_OK
    assert lib.rkv_decode_split_hint(C.byref(many), 32, C.byref(ns)) == L.RKV_OK
    assert ns.value == 1
    short = _cache(n_inst=1, H=1, N=100, base=16)
    assert lib.rkv_cache_init(C.byref(short)) == L.RKV_OK
    assert lib.rkv_decode_split_hint(C.byref(short), 4, C.byref(ns)) == L.RKV_OK
    assert ns.value == 4   # capped at ceil(100 / 32) tiles
    two = _cache(n_inst=1, H=2, N=100, base=16)
    assert lib.rkv_cache_init(C.byref(two)) == L.RKV_OK
    assert lib.rkv_decode_split_hint(C.byref(two), 3, C.byref(ns)) == L.RKV_ERR_INVALID_ARG


def test_noalloc_decode_checks_the_scratch_limit_before_the_device(lib):
    null = C.c_void_p(0)
    q, out = C.c_void_p(0x6000), C.c_void_p(0x5000)
    ws = C.c_size_t()
    # a whole 32-layer batch of 8 x 32K sequences needs more than the fixed
    # scratch: refused before any device call
    big = _cache(n_inst=256, H=8, N=32768, base=64)
    assert lib.rkv_cache_init(C.byref(big)) == L.RKV_OK
    assert lib.rkv_decode_workspace(C.byref(big), 32, 12, C.byref(ws)) == L.RKV_OK
    assert ws.value > L.RKV_SCRATCH_BYTES
    assert lib.rkv_decode_attn_noalloc(q, 32, C.byref(big), 0.1, out, 12, null) == \
        L.RKV_ERR_WORKSPACE
    # one layer of it fits; with the cache buffers unset the call fails
    # validation, still before the device
    layer = _cache(n_inst=8, H=8, N=32768, base=64)
    assert lib.rkv_cache_init(C.byref(layer)) == L.RKV_OK
    assert lib.rkv_decode_workspace(C.byref(layer), 32, 12, C.byref(ws)) == L.RKV_OK
    assert ws.value <= L.RKV_SCRATCH_BYTES
    assert lib.rkv_decode_attn_noalloc(q, 32, C.byref(layer), 0.1, out, 12, null) == \
        L.RKV_ERR_INVALID_ARG
    assert lib.rkv_decode_attn_noalloc(q, 30, C.byref(layer), 0.1, out, 12, null) == \
        L.RKV_ERR_INVALID_ARG


def test_decode_refuses_what_its_layout_cannot_hold(lib):
    """Decode holds one MFMA row per (query head, scale group) of a KV head
    (at most 16), and keeps the QK table and reference weights of every
    reference in LDS; both limits come back as RKV_ERR_UNSUPPORTED before
    any device work."""
    null = C.c_void_p(0)
    q, out, ws = C.c_void_p(0x6000), C.c_void_p(0x5000), C.c_void_p(0x7000)
    big = 1 << 40

    def ready(c):
        assert lib.rkv_cache_init(C.byref(c)) == L.RKV_OK
        for name in ("ref_idx", "codes_k", "codes_v", "scales", "ref_kv"):
            setattr(c, name, 0x10000)
        return c

    # GQA 8 with 32-dim groups: 8 x 4 = 32 rows
    c = ready(_cache(n_inst=1, H=1, N=4096, base=64))
    assert lib.rkv_decode_attn(q, 8, C.byref(c), 0.1, out, 2, ws, big, null) == L.RKV_ERR_UNSUPPORTED
    # the same with 128-dim groups fits (8 rows) up to the workspace check
    c.group = 128
    assert lib.rkv_decode_attn(q, 8, C.byref(c), 0.1, out, 2, ws, 16, null) == L.RKV_ERR_WORKSPACE
    # exact residuals: one row per query head, 17 heads are too many
    c0 = ready(_cache(n_inst=1, H=1, N=4096, base=64))
    c0.bits = 0
    assert lib.rkv_decode_attn(q, 17, C.byref(c0), 0.1, out, 2, ws, big, null) == L.RKV_ERR_UNSUPPORTED
    assert lib.rkv_decode_attn(q, 16, C.byref(c0), 0.1, out, 2, ws, 16, null) == L.RKV_ERR_WORKSPACE
    # 4096 references with GQA 4: the per-reference LDS state does not fit
    many = ready(_cache(n_inst=1, H=1, N=16384, base=4))
    assert many.n_refs == 4096
    assert lib.rkv_decode_attn(q, 4, C.byref(many), 0.1, out, 2, ws, big, null) == \
        L.RKV_ERR_UNSUPPORTED
    # 2048 references fit
    fits = ready(_cache(n_inst=1, H=1, N=8192, base=4))
    assert lib.rkv_decode_attn(q, 4, C.byref(fits), 0.1, out, 2, ws, 16, null) == L.RKV_ERR_WORKSPACE
