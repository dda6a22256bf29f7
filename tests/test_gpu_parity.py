"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars (from the method's contract):
  * reference sets bit-exact except counted near-ties (exact distance gap
    within 1e-5 relative, floored at |k_i|^2);
  * codes and scales bit-exact on every token whose set matches;
  * reference store bit-exact;
  * reconstruction within 1e-5 relative L2 (fp32 arithmetic);
  * decode attention within 2e-3 relative L2.
Inputs are the seeded prototype-mixture caches of the workloads (or smaller
slices of them); the oracle reads the very tensors the GPU consumed.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from rkv_testlib import GpuCache, attn_err, compare_encode, rel_l2, to_np_f32
from synth import gen_head_kv, gen_queries, get_config

pytestmark = pytest.mark.gpu

if gpu_available():
    import long_context_attention_rkv_amd as rkv


def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def say(*a):
    print(*a, flush=True)


def make_kv(cfg, n_inst, seq_len, device="cuda"):
    """[n_inst, H, N, D] K and V; instance i = (layer i // batch, seq i % batch)."""
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    K = torch.empty(n_inst, cfg.n_kv_heads, seq_len, cfg.head_dim, dtype=dt, device=device)
    V = torch.empty_like(K)
    for i in range(n_inst):
        layer, seq = divmod(i, max(cfg.batch, 1))
        for h in range(cfg.n_kv_heads):
            k, v = gen_head_kv(cfg, layer, seq, h, device=device, seq_len=seq_len)
            K[i, h].copy_(k)
            V[i, h].copy_(v)
    return K, V


def make_q(cfg, n_inst, device="cuda"):
    return torch.stack([gen_queries(cfg, *divmod(i, max(cfg.batch, 1)), device=device)
                        for i in range(n_inst)])


def _latent_kw(latent_seed):
    return dict(latent=0, latent_seed=0) if latent_seed is None else \
        dict(latent=1, latent_seed=latent_seed)


def encode(cfg, K, V, bits, n_inst, seq_len, ref_bits=0, latent_seed=None):
    cache = rkv.Cache(n_inst, cfg.n_kv_heads, seq_len, cfg.dtype, cfg.stride_base, cfg.k,
                      bits, cfg.group, double_after=cfg.double_after, ref_bits=ref_bits,
                      **_latent_kw(latent_seed))
    rkv.rkv_encode(K, V, cache)
    torch.cuda.synchronize()
    return cache


def _cfg(index, **kw):
    return dataclasses.replace(get_config(index), **kw)


# (id, config, bits, n_inst, seq_len)
SMALL = [
    ("tiny_int8_f32", get_config(0), 8, 1, 1024),
    ("tiny_int4_f32_ragged", _cfg(0, n_kv_heads=2), 4, 2, 999),
    ("llama_int4_bf16_ragged", _cfg(1, n_kv_heads=2), 4, 1, 1000),
    ("stress_int2_k16", _cfg(4, n_kv_heads=2, batch=2), 2, 2, 777),
    ("stress_int4_k16", _cfg(4, n_kv_heads=2, batch=2), 4, 2, 777),
    ("dynamic_int4", _cfg(3, n_kv_heads=2, double_after=512, drift_block=128), 4, 1, 2600),
    ("bf16_int8_g128", _cfg(1, n_kv_heads=1, group=128), 8, 1, 600),
    ("edge_k_exceeds_refs", _cfg(1, n_kv_heads=1, stride_base=64, k=16), 4, 1, 200),
    ("edge_one_token", _cfg(1, n_kv_heads=1), 4, 1, 1),
    ("edge_33_tokens", _cfg(0, n_kv_heads=1, stride_base=5, k=3), 8, 1, 33),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_encode_parity_small(case):
    _need_gpu()
    name, cfg, bits, n_inst, N = case
    say(f"[encode parity] {name}: N={N} H={cfg.n_kv_heads} inst={n_inst} bits={bits}")
    K, V = make_kv(cfg, n_inst, N)
    cache = encode(cfg, K, V, bits, n_inst, N)
    gc = GpuCache(cache)
    Kn, Vn = to_np_f32(K), to_np_f32(V)
    near = 0
    for i in range(n_inst):
        for h in range(cfg.n_kv_heads):
            r = compare_encode(gc, i * cfg.n_kv_heads + h, Kn[i, h], Vn[i, h],
                               cfg.stride_base, cfg.double_after)
            near += r["near_ties"]
    say(f"  near-ties: {near} of {n_inst * cfg.n_kv_heads * N} tokens")


# (dtype, bits, log2 of the input scaling): residual scales in the fp16
# subnormal range, rounded to zero, or saturated at 65504.  Those scales are
# not the plain rounding of a normal-range estimate, so every code of their
# groups is decided exactly and clamped.
EXTREME = [("bf16", 4, -20), ("bf16", 2, -22), ("f32", 4, -30), ("bf16", 4, 20), ("f32", 8, 24)]


@pytest.mark.parametrize("case", EXTREME, ids=[f"{d}_int{b}_2^{e}" for d, b, e in EXTREME])
def test_encode_parity_extreme_magnitudes(case):
    _need_gpu()
    dtype, bits, e = case
    cfg = _cfg(1, n_kv_heads=1, dtype=dtype)
    N = 800
    say(f"[encode parity, inputs x 2^{e}] {dtype} bits={bits}")
    K, V = make_kv(cfg, 1, N)
    K.mul_(2.0 ** e)  # a power of two: exact at these magnitudes
    V.mul_(2.0 ** e)
    cache = encode(cfg, K, V, bits, 1, N)
    gc = GpuCache(cache)
    r = compare_encode(gc, 0, to_np_f32(K[0, 0]), to_np_f32(V[0, 0]), cfg.stride_base,
                       cfg.double_after)
    say(f"  near-ties: {r['near_ties']}")


@pytest.mark.parametrize("case", SMALL[:6], ids=[c[0] for c in SMALL[:6]])
def test_reconstruct_parity_small(case):
    _need_gpu()
    name, cfg, bits, n_inst, N = case
    say(f"[reconstruct parity] {name}")
    K, V = make_kv(cfg, n_inst, N)
    cache = encode(cfg, K, V, bits, n_inst, N)
    Kh, Vh = rkv.rkv_reconstruct(cache)
    torch.cuda.synchronize()
    Khn, Vhn = Kh.cpu().numpy(), Vh.cpu().numpy()
    gc = GpuCache(cache)
    Kn, Vn = to_np_f32(K), to_np_f32(V)
    for i in range(n_inst):
        for h in range(cfg.n_kv_heads):
            r = compare_encode(gc, i * cfg.n_kv_heads + h, Kn[i, h], Vn[i, h],
                               cfg.stride_base, cfg.double_after)
            kv = oracle.reconstruct(r["enc_gpu_codes"], Kn[i, h], Vn[i, h], bits)
            m = r["matched"]
            assert rel_l2(Khn[i, h][m], kv[m, 0]) <= 1e-5
            assert rel_l2(Vhn[i, h][m], kv[m, 1]) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_no_quantisation_is_lossless(dtype):
    _need_gpu()
    cfg = _cfg(1, n_kv_heads=2, dtype=dtype)
    say(f"[bits=0] {dtype}")
    K, V = make_kv(cfg, 1, 700)
    cache = encode(cfg, K, V, 0, 1, 700)
    gc = GpuCache(cache)
    Kn, Vn = to_np_f32(K), to_np_f32(V)
    for h in range(2):
        compare_encode(gc, h, Kn[0, h], Vn[0, h], cfg.stride_base, 0)
    Kh, Vh = rkv.rkv_reconstruct(cache)
    torch.cuda.synchronize()
    # the exact residual rebuilds every position bit for bit
    assert torch.equal(Kh, K.float()) and torch.equal(Vh, V.float())


def test_stride1_k1_gives_zero_residuals():
    _need_gpu()
    cfg = _cfg(1, n_kv_heads=2, stride_base=1, k=1)
    say("[stride 1, k 1]")
    K, V = make_kv(cfg, 1, 300)
    cache = encode(cfg, K, V, 4, 1, 300)
    gc = GpuCache(cache)
    assert np.array_equal(gc.idx[:, :, 0], np.tile(np.arange(300), (2, 1)))
    for ih in range(2):
        assert np.all(gc.codes(ih) == 0)
    assert np.all(gc.scales.view(np.uint16) == 0)


def test_encode_is_deterministic():
    _need_gpu()
    cfg = _cfg(1, n_kv_heads=4)
    say("[determinism]")
    K, V = make_kv(cfg, 1, 2048)
    c1 = encode(cfg, K, V, 4, 1, 2048)
    c2 = encode(cfg, K, V, 4, 1, 2048)
    for name in rkv.Cache.BUFFERS:
        assert torch.equal(c1.buffers[name], c2.buffers[name]), name


# ------------------------------------------------------------------ decode

DECODE = [
    ("tiny", get_config(0), 8, 1, 1024),
    ("llama_ragged", _cfg(1, n_kv_heads=2, n_q_heads=8), 4, 1, 1000),
    ("llama_int8", _cfg(1, n_kv_heads=2, n_q_heads=8), 8, 1, 640),
    ("gqa7_g64_int2", _cfg(4, n_kv_heads=2, n_q_heads=14, batch=1), 2, 2, 500),
    ("gqa7_g64_int4", _cfg(4, n_kv_heads=2, n_q_heads=14, batch=1), 4, 1, 500),
    ("g128_gqa4", _cfg(1, n_kv_heads=1, n_q_heads=4, group=128), 4, 1, 300),
    # an odd number of query heads per KV head with 32-dim groups: the last
    # head pair of the reference weights has no partner
    ("gqa3_g32", _cfg(1, n_kv_heads=2, n_q_heads=6), 4, 1, 700),
    ("gqa2_g32", _cfg(1, n_kv_heads=2, n_q_heads=4), 4, 1, 600),
    # more than 8 query heads per KV head
    ("g128_gqa16_bf16", _cfg(1, n_kv_heads=2, n_q_heads=32, group=128), 4, 1, 700),
    ("g128_gqa12_f32_int8", _cfg(0, n_kv_heads=1, n_q_heads=12, group=128), 8, 1, 500),
    # more references than the combine requests up front per thread (512 bf16
    # rows, 256 fp32 rows): the rest of W . Vref is read in its tail loop
    ("many_refs_bf16", _cfg(1, n_kv_heads=1, n_q_heads=4, stride_base=4), 4, 1, 3000),
    ("many_refs_f32", _cfg(0, n_kv_heads=1, n_q_heads=4, stride_base=4), 4, 1, 1500),
]


def _oracle_decode(cfg, K, V, q, bits, scale, ref_bits=0, latent_seed=None):
    n_inst, H = K.shape[0], K.shape[1]
    out = np.zeros((n_inst, q.shape[1], q.shape[2]))
    for i in range(n_inst):
        kh, vh = [], []
        for h in range(H):
            enc = oracle.encode(K[i, h], V[i, h], cfg.stride_base, cfg.double_after, cfg.k,
                                bits, cfg.group, ref_bits=ref_bits, latent_seed=latent_seed)
            kv = oracle.reconstruct(enc, K[i, h], V[i, h], bits)
            kh.append(kv[:, 0])
            vh.append(kv[:, 1])
        out[i] = oracle.decode_attn(q[i], np.stack(kh), np.stack(vh), scale)
    return out


def test_decode_parity_many_blocks():
    """More than 512 (instance, query head) pairs: the combine runs as
    256-thread blocks instead of 1024-thread ones."""
    _need_gpu()
    cfg = _cfg(1, n_kv_heads=8, n_q_heads=32, batch=17)
    n_inst, N, bits = 17, 300, 4
    say(f"[decode parity, many blocks] inst={n_inst} Hkv=8 Hq=32 N={N}")
    K, V = make_kv(cfg, n_inst, N)
    q = make_q(cfg, n_inst)
    cache = encode(cfg, K, V, bits, n_inst, N)
    Kn, Vn, qn = to_np_f32(K), to_np_f32(V), to_np_f32(q)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    got = rkv.rkv_decode_attn(q, cfg.n_q_heads, cache, scale, n_split=3).cpu().numpy()
    want = _oracle_decode(cfg, Kn, Vn, qn, bits, scale)
    err = attn_err(got, want)
    say(f"  worst per-head rel L2 = {err:.2e}")
    assert err <= 2e-3


@pytest.mark.parametrize("case", DECODE, ids=[c[0] for c in DECODE])
def test_decode_parity(case):
    _need_gpu()
    name, cfg, bits, n_inst, N = case
    say(f"[decode parity] {name}: N={N} Hkv={cfg.n_kv_heads} Hq={cfg.n_q_heads} bits={bits}")
    K, V = make_kv(cfg, n_inst, N)
    q = make_q(cfg, n_inst)
    cache = encode(cfg, K, V, bits, n_inst, N)
    Kn, Vn, qn = to_np_f32(K), to_np_f32(V), to_np_f32(q)
    for scale in (1.0 / math.sqrt(cfg.head_dim), 1.0):
        got = rkv.rkv_decode_attn(q, cfg.n_q_heads, cache, scale, n_split=3)
        torch.cuda.synchronize()
        want = _oracle_decode(cfg, Kn, Vn, qn, bits, scale)
        err = attn_err(got.cpu().numpy(), want)
        say(f"  scale={scale:.4f} worst per-head rel L2 = {err:.2e}")
        assert err <= 2e-3


# (log2 of the q scaling, log2 of the V scaling, code bits): the query enters
# the f16 score MFMA with a power-of-two pre-scale and the P.V operand with a
# power-of-two exponent per softmax chunk, so decode holds its bar whatever
# the magnitudes (fp16 would otherwise overflow or flush these).
SCALED = [(8, 0, 4), (-8, 0, 4), (16, 0, 4), (-20, 0, 4), (0, -8, 4), (0, -12, 4), (0, -20, 4),
          (0, 12, 4), (-8, -20, 8), (0, -20, 2)]


@pytest.mark.parametrize("case", SCALED, ids=[f"q2^{a}_v2^{b}_int{c}" for a, b, c in SCALED])
def test_decode_parity_scaled_inputs(case):
    _need_gpu()
    eq, ev, bits = case
    cfg = _cfg(1, n_kv_heads=2, n_q_heads=8)
    N = 1000
    say(f"[decode parity, q x 2^{eq}, V x 2^{ev}] int{bits}")
    K, V = make_kv(cfg, 1, N)
    V.mul_(2.0 ** ev)
    q = make_q(cfg, 1)
    q.mul_(2.0 ** eq)
    cache = encode(cfg, K, V, bits, 1, N)
    Kn, Vn, qn = to_np_f32(K), to_np_f32(V), to_np_f32(q)
    for scale in (1.0 / math.sqrt(cfg.head_dim), 1.0):
        got = rkv.rkv_decode_attn(q, cfg.n_q_heads, cache, scale, n_split=3).cpu().numpy()
        want = _oracle_decode(cfg, Kn, Vn, qn, bits, scale)
        err = attn_err(got, want)
        say(f"  scale={scale:.4f} worst per-head rel L2 = {err:.2e}")
        assert err <= 2e-3


EXACT = [("tiny_f32", get_config(0), 1, 1024, 1e-5), ("llama_bf16_gqa4", _cfg(1, n_kv_heads=2, n_q_heads=8), 2, 700, 1e-5),
         ("stress_bf16_k16", _cfg(4, n_kv_heads=2, n_q_heads=14, batch=1), 1, 600, 1e-5)]


@pytest.mark.parametrize("case", EXACT, ids=[c[0] for c in EXACT])
def test_decode_without_quantisation_is_full_attention(case):
    """bits = 0 keeps exact residuals: decode over the rebuilt cache is
    textbook softmax attention over the raw K, V (dense, over a prefix, and
    over listed tiles)."""
    _need_gpu()
    name, cfg, n_inst, N, tol = case
    say(f"[exact decode] {name}: N={N}")
    K, V = make_kv(cfg, n_inst, N)
    q = make_q(cfg, n_inst)
    cache = encode(cfg, K, V, 0, n_inst, N)
    Kn, Vn, qn = to_np_f32(K), to_np_f32(V), to_np_f32(q)
    G = cfg.n_q_heads // cfg.n_kv_heads
    L = N - 77
    lists = _tile_lists(n_inst, cfg.n_kv_heads, N, 0.4, seed=5)
    tiles = torch.from_numpy(lists).cuda()
    for scale in (1.0 / math.sqrt(cfg.head_dim), 1.0):
        want = np.stack([oracle.decode_attn(qn[i], Kn[i].astype(np.float64), Vn[i].astype(np.float64), scale)
                         for i in range(n_inst)])
        got = rkv.rkv_decode_attn(q, cfg.n_q_heads, cache, scale, n_split=3).cpu().numpy()
        err = attn_err(got, want)
        want_l = np.stack([oracle.decode_attn(qn[i], Kn[i, :, :L].astype(np.float64),
                                              Vn[i, :, :L].astype(np.float64), scale)
                           for i in range(n_inst)])
        got_l = rkv.rkv_decode_attn_len(q, cfg.n_q_heads, cache, L, scale, n_split=2).cpu().numpy()
        err_l = attn_err(got_l, want_l)
        want_t = np.zeros_like(want)
        for i in range(n_inst):
            for h in range(cfg.n_kv_heads):
                pos = oracle.tile_positions(lists[i, h], N)
                want_t[i, h * G:(h + 1) * G] = oracle.decode_attn(
                    qn[i, h * G:(h + 1) * G], Kn[i, h][None, pos].astype(np.float64),
                    Vn[i, h][None, pos].astype(np.float64), scale)
        got_t = rkv.rkv_decode_attn_tiles(q, cfg.n_q_heads, cache, scale, tiles, n_split=3).cpu().numpy()
        err_t = attn_err(got_t, want_t)
        say(f"  scale={scale:.4f} worst per-head rel L2: dense {err:.2e}, prefix {err_l:.2e}, "
            f"tiles {err_t:.2e}")
        assert max(err, err_l, err_t) <= tol


def test_decode_tiles_empty_selection_gives_zero_rows():
    """A KV head whose list selects no position attends nothing: its query
    heads get zero rows, the other heads are unaffected."""
    _need_gpu()
    cfg = _cfg(1, n_kv_heads=2, n_q_heads=8)
    N = 640
    say("[decode tiles] empty selection")
    K, V = make_kv(cfg, 1, N)
    q = make_q(cfg, 1)
    cache = encode(cfg, K, V, 4, 1, N)
    n_tiles = N // 32
    lists = np.array([[[3, 7, 11], [-1, n_tiles, n_tiles + 5]]], dtype=np.int32)
    got = rkv.rkv_decode_attn_tiles(q, 8, cache, 1.0, torch.from_numpy(lists).cuda(),
                                    n_split=2).cpu().numpy()
    assert np.all(got[0, 4:] == 0)
    Kn, Vn, qn = to_np_f32(K), to_np_f32(V), to_np_f32(q)
    enc = oracle.encode(Kn[0, 0], Vn[0, 0], cfg.stride_base, 0, cfg.k, 4, cfg.group)
    kv = oracle.reconstruct(enc, Kn[0, 0], Vn[0, 0], 4)
    pos = oracle.tile_positions(lists[0, 0], N)
    want = oracle.decode_attn(qn[0, :4], kv[None, pos, 0], kv[None, pos, 1], 1.0)
    assert attn_err(got[0, :4], want) <= 2e-3


def test_decode_split_invariance():
    _need_gpu()
    cfg = _cfg(1, n_kv_heads=2, n_q_heads=8)
    say("[decode split invariance]")
    K, V = make_kv(cfg, 2, 3000)
    q = make_q(cfg, 2)
    cache = encode(cfg, K, V, 4, 2, 3000)
    outs = [rkv.rkv_decode_attn(q, 8, cache, 1.0, n_split=s).cpu().numpy()
            for s in (1, 2, 7, 40, 200)]
    # The P.V product rounds each p*scale operand to fp16 (relative error
    # <= 2^-11) against a running maximum that depends on the split, so two
    # split counts may differ by up to 2 * 2^-11 relative in the worst
    # (fully aligned) case; random rounding keeps it near 1e-4.
    for o in outs[1:]:
        assert rel_l2(o, outs[0]) <= 2 * 2.0 ** -11


# ------------------------------------------------------------------ selective decode

TILE_CASES = [
    ("tiny_30pct", get_config(0), 8, 1, 1024, 0.3),
    ("llama_ragged_30pct", _cfg(1, n_kv_heads=2, n_q_heads=8), 4, 2, 1000, 0.3),
    ("gqa7_int2_half", _cfg(4, n_kv_heads=2, n_q_heads=14, batch=1), 2, 1, 500, 0.5),
    ("llama_one_tile", _cfg(1, n_kv_heads=2, n_q_heads=8), 4, 1, 640, 0.0),
    # 130 list entries: a split walks two softmax chunks of the list
    ("llama_two_chunks_half", _cfg(1, n_kv_heads=2, n_q_heads=8), 4, 1, 8192, 0.5),
]


def _tile_lists(n_inst, H, N, frac, seed):
    """Random distinct tiles per (instance, KV head) in shuffled order, the
    ragged last tile forced into one list, plus two entries that select
    nothing (-1 and one past the end)."""
    rng = np.random.default_rng(seed)
    n_tiles = -(-N // 32)
    n_sel = max(1, int(round(frac * n_tiles)))
    lists = np.empty((n_inst, H, n_sel + 2), dtype=np.int32)
    for i in range(n_inst):
        for h in range(H):
            sel = rng.choice(n_tiles, n_sel, replace=False)
            if i == 0 and h == 0:
                sel[0] = n_tiles - 1 if (n_tiles - 1) not in sel[1:] else sel[0]
            row = np.concatenate([sel, [-1, n_tiles + 3]])
            rng.shuffle(row)
            lists[i, h] = row
    return lists


@pytest.mark.parametrize("case", TILE_CASES, ids=[c[0] for c in TILE_CASES])
def test_decode_tiles_parity(case):
    _need_gpu()
    name, cfg, bits, n_inst, N, frac = case
    say(f"[decode tiles] {name}: N={N} frac={frac}")
    K, V = make_kv(cfg, n_inst, N)
    q = make_q(cfg, n_inst)
    cache = encode(cfg, K, V, bits, n_inst, N)
    lists = _tile_lists(n_inst, cfg.n_kv_heads, N, frac, seed=11)
    tiles = torch.from_numpy(lists).cuda()
    Kn, Vn, qn = to_np_f32(K), to_np_f32(V), to_np_f32(q)
    G = cfg.n_q_heads // cfg.n_kv_heads
    for scale in (1.0 / math.sqrt(cfg.head_dim), 1.0):
        got = rkv.rkv_decode_attn_tiles(q, cfg.n_q_heads, cache, scale, tiles, n_split=3)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        want = np.zeros_like(got, dtype=np.float64)
        for i in range(n_inst):
            for h in range(cfg.n_kv_heads):
                enc = oracle.encode(Kn[i, h], Vn[i, h], cfg.stride_base, cfg.double_after,
                                    cfg.k, bits, cfg.group)
                kv = oracle.reconstruct(enc, Kn[i, h], Vn[i, h], bits)
                pos = oracle.tile_positions(lists[i, h], N)
                want[i, h * G:(h + 1) * G] = oracle.decode_attn(
                    qn[i, h * G:(h + 1) * G], kv[None, pos, 0], kv[None, pos, 1], scale)
        err = attn_err(got, want)
        say(f"  scale={scale:.4f} worst per-head rel L2 = {err:.2e}")
        assert err <= 2e-3


def test_decode_all_tiles_equals_dense():
    _need_gpu()
    cfg = _cfg(1, n_kv_heads=2, n_q_heads=8)
    say("[decode tiles] all tiles == dense")
    N = 1500
    K, V = make_kv(cfg, 2, N)
    q = make_q(cfg, 2)
    cache = encode(cfg, K, V, 4, 2, N)
    n_tiles = -(-N // 32)
    tiles = torch.arange(n_tiles, dtype=torch.int32, device="cuda").expand(2, 2, n_tiles).contiguous()
    dense = rkv.rkv_decode_attn(q, 8, cache, 1.0, n_split=5).cpu().numpy()
    sparse = rkv.rkv_decode_attn_tiles(q, 8, cache, 1.0, tiles, n_split=5).cpu().numpy()
    # identical streams and a fixed merge order: the same bits
    assert np.array_equal(sparse, dense)


# ------------------------------------------------------------------ quantised reference store

REFQ_CASES = [
    ("tiny_f32_int8", get_config(0), 8, 1, 1024),
    ("llama_bf16_int4_gqa4", _cfg(1, n_kv_heads=2, n_q_heads=8), 4, 1, 1000),
    ("stress_int2_k16_g64", _cfg(4, n_kv_heads=2, n_q_heads=14, batch=2), 2, 2, 500),
    ("gqa16_g128_f32", _cfg(0, n_kv_heads=1, n_q_heads=16, group=128), 4, 1, 800),
]


@pytest.mark.parametrize("case", REFQ_CASES, ids=[c[0] for c in REFQ_CASES])
def test_quantized_refs_parity(case):
    """Full-pipeline quantisation: reference codes/scales bit-exact, residual
    codes bit-exact against the dequantised references, reconstruction and
    decode against the oracle."""
    _need_gpu()
    name, cfg, bits, n_inst, N = case
    say(f"[quantised refs] {name}: N={N} bits={bits}")
    K, V = make_kv(cfg, n_inst, N)
    q = make_q(cfg, n_inst)
    cache = encode(cfg, K, V, bits, n_inst, N, ref_bits=4)
    gc = GpuCache(cache)
    Kn, Vn, qn = to_np_f32(K), to_np_f32(V), to_np_f32(q)
    Kh, Vh = rkv.rkv_reconstruct(cache)
    Khn, Vhn = Kh.cpu().numpy(), Vh.cpu().numpy()
    near = 0
    for i in range(n_inst):
        for h in range(cfg.n_kv_heads):
            r = compare_encode(gc, i * cfg.n_kv_heads + h, Kn[i, h], Vn[i, h],
                               cfg.stride_base, cfg.double_after)
            near += r["near_ties"]
            kv = oracle.reconstruct(r["enc_gpu_codes"], Kn[i, h], Vn[i, h], bits)
            m = r["matched"]
            assert rel_l2(Khn[i, h][m], kv[m, 0]) <= 1e-5
            assert rel_l2(Vhn[i, h][m], kv[m, 1]) <= 1e-5
    say(f"  near-ties: {near}")
    for scale in (1.0 / math.sqrt(cfg.head_dim), 1.0):
        got = rkv.rkv_decode_attn(q, cfg.n_q_heads, cache, scale, n_split=3).cpu().numpy()
        want = _oracle_decode(cfg, Kn, Vn, qn, bits, scale, ref_bits=4)
        err = attn_err(got, want)
        say(f"  decode scale={scale:.4f} worst per-head rel L2 = {err:.2e}")
        assert err <= 2e-3


# ------------------------------------------------------------------ latent residuals

LATENT_CASES = [
    # (id, config, bits, n_inst, N, ref_bits, seed)
    ("tiny_f32_int8", get_config(0), 8, 1, 1024, 0, 0),
    ("llama_bf16_int4_gqa4_ragged", _cfg(1, n_kv_heads=2, n_q_heads=8), 4, 1, 1000, 0, 1234567),
    ("stress_int2_k16_g64", _cfg(4, n_kv_heads=2, n_q_heads=14, batch=2), 2, 2, 500, 0,
     0xFFFFFFFFFFFFFFFF),
    ("dynamic_int4_g128", _cfg(3, n_kv_heads=1, n_q_heads=4, group=128, double_after=512,
                                drift_block=128), 4, 1, 1300, 0, 99),
    ("llama_int4_quantised_refs", _cfg(1, n_kv_heads=2, n_q_heads=8), 4, 1, 700, 4, 7),
    ("gqa16_g128_quantised_refs", _cfg(1, n_kv_heads=1, n_q_heads=16, group=128), 4, 1, 600, 4, 3),
]


@pytest.mark.parametrize("case", LATENT_CASES, ids=[c[0] for c in LATENT_CASES])
def test_latent_parity(case):
    """Latent residuals f_c(KV - KV_R): codes and scales bit-exact (both sides
    rotate the fp32 residual with the same butterfly order), reconstruction
    through f_d and decode through the rotated query against the oracle."""
    _need_gpu()
    name, cfg, bits, n_inst, N, ref_bits, seed = case
    say(f"[latent] {name}: N={N} bits={bits} ref_bits={ref_bits} seed={seed:#x}")
    K, V = make_kv(cfg, n_inst, N)
    q = make_q(cfg, n_inst)
    cache = encode(cfg, K, V, bits, n_inst, N, ref_bits=ref_bits, latent_seed=seed)
    gc = GpuCache(cache)
    assert gc.latent_seed == seed
    Kn, Vn, qn = to_np_f32(K), to_np_f32(V), to_np_f32(q)
    Kh, Vh = rkv.rkv_reconstruct(cache)
    Khn, Vhn = Kh.cpu().numpy(), Vh.cpu().numpy()
    near = 0
    for i in range(n_inst):
        for h in range(cfg.n_kv_heads):
            r = compare_encode(gc, i * cfg.n_kv_heads + h, Kn[i, h], Vn[i, h],
                               cfg.stride_base, cfg.double_after)
            near += r["near_ties"]
            kv = oracle.reconstruct(r["enc_gpu_codes"], Kn[i, h], Vn[i, h], bits)
            m = r["matched"]
            assert rel_l2(Khn[i, h][m], kv[m, 0]) <= 1e-5
            assert rel_l2(Vhn[i, h][m], kv[m, 1]) <= 1e-5
    say(f"  near-ties: {near}")
    for scale in (1.0 / math.sqrt(cfg.head_dim), 1.0):
        got = rkv.rkv_decode_attn(q, cfg.n_q_heads, cache, scale, n_split=3).cpu().numpy()
        want = _oracle_decode(cfg, Kn, Vn, qn, bits, scale, ref_bits=ref_bits, latent_seed=seed)
        err = attn_err(got, want)
        say(f"  decode scale={scale:.4f} worst per-head rel L2 = {err:.2e}")
        assert err <= 2e-3


def test_latent_changes_codes_not_the_rebuilt_cache():
    """Two seeds give different codes; both rebuild K, V about as well as the
    plain residual codes (the rotation is orthogonal up to scaling)."""
    _need_gpu()
    cfg = _cfg(1, n_kv_heads=2)
    N = 900
    say(f"[latent seeds] N={N}")
    K, V = make_kv(cfg, 1, N)
    plain = encode(cfg, K, V, 4, 1, N)
    a = encode(cfg, K, V, 4, 1, N, latent_seed=1)
    b = encode(cfg, K, V, 4, 1, N, latent_seed=2)
    assert not torch.equal(a.buffers["codes_k"], b.buffers["codes_k"])
    assert torch.equal(a.buffers["ref_idx"], plain.buffers["ref_idx"])
    Kn = to_np_f32(K)
    errs = []
    for c in (plain, a, b):
        Kh, _ = rkv.rkv_reconstruct(c)
        errs.append(rel_l2(Kh.cpu().numpy(), Kn))
    say(f"  rel L2 of K^: plain {errs[0]:.3e}, latent {errs[1]:.3e} / {errs[2]:.3e}")
    assert max(errs[1:]) <= 2 * errs[0]


# ------------------------------------------------------------------ streaming encode

APPEND_CASES = [
    # (id, config, bits, n_inst, N, prefill, chunk sizes cycled after it)
    ("tiny_int8_f32", get_config(0), 8, 1, 1024, 200, (1,)),
    ("llama_int4_from_zero", _cfg(1, n_kv_heads=2), 4, 1, 700, 0, (1, 7, 33)),
    ("stress_int2_k16", _cfg(4, n_kv_heads=2, batch=2), 2, 2, 777, 100, (1, 5, 64)),
    ("dynamic_int4", _cfg(3, n_kv_heads=2, double_after=512, drift_block=128), 4, 1, 1500, 450,
     (3, 1, 40)),
    ("bf16_nobits", _cfg(1, n_kv_heads=1), 0, 1, 300, 37, (1, 2)),
    ("llama_int4_quantised_refs", _cfg(1, n_kv_heads=2), 4, 1, 700, 100, (1, 9)),
    ("stress_int2_latent", _cfg(4, n_kv_heads=2, batch=2), 2, 2, 500, 77, (1, 40)),
]


def _stream_encode(cfg, K, V, bits, n_inst, N, prefill, chunks, ref_bits=0, latent_seed=None):
    cache = rkv.Cache(n_inst, cfg.n_kv_heads, N, cfg.dtype, cfg.stride_base, cfg.k, bits,
                      cfg.group, double_after=cfg.double_after, ref_bits=ref_bits,
                      **_latent_kw(latent_seed))
    ws = torch.empty(rkv.rkv_encode_workspace(cache), dtype=torch.uint8, device="cuda")
    pos = 0
    if prefill:
        rkv.rkv_append(K[:, :, :prefill].contiguous(), V[:, :, :prefill].contiguous(), cache, 0, ws)
        pos = prefill
    i = 0
    while pos < N:
        n = min(chunks[i % len(chunks)], N - pos)
        rkv.rkv_append(K[:, :, pos:pos + n].contiguous(), V[:, :, pos:pos + n].contiguous(),
                       cache, pos, ws)
        pos += n
        i += 1
    torch.cuda.synchronize()
    return cache


@pytest.mark.parametrize("case", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_append_equals_batch_encode(case):
    """Appending positions (prefill, then chunks of a few positions) gives the
    batch encode byte for byte: same arithmetic, causal candidate sets."""
    _need_gpu()
    name, cfg, bits, n_inst, N, prefill, chunks = case
    say(f"[append] {name}: N={N} prefill={prefill} chunks={chunks}")
    K, V = make_kv(cfg, n_inst, N)
    ref_bits = 4 if "quantised_refs" in name else 0
    seed = 0x5EED if "latent" in name else None
    whole = encode(cfg, K, V, bits, n_inst, N, ref_bits=ref_bits, latent_seed=seed)
    streamed = _stream_encode(cfg, K, V, bits, n_inst, N, prefill, chunks, ref_bits=ref_bits,
                              latent_seed=seed)
    for buf in rkv.Cache.BUFFERS:
        if (bits == 0 and buf == "scales") or (ref_bits == 0 and buf == "ref_scales"):
            continue
        assert torch.equal(whole.buffers[buf], streamed.buffers[buf]), buf
    # and the streamed cache against the oracle directly
    gc = GpuCache(streamed)
    Kn, Vn = to_np_f32(K), to_np_f32(V)
    for i in range(n_inst):
        for h in range(cfg.n_kv_heads):
            compare_encode(gc, i * cfg.n_kv_heads + h, Kn[i, h], Vn[i, h], cfg.stride_base,
                           cfg.double_after)


def test_decode_len_reads_only_the_prefix():
    """A cache of capacity N filled to L by appends, every other byte garbage
    (NaN patterns included): decode over length L matches the oracle on the
    first L positions."""
    _need_gpu()
    cfg = _cfg(1, n_kv_heads=2, n_q_heads=8)
    N, L = 1000, 643
    say(f"[decode len] N={N} L={L}")
    K, V = make_kv(cfg, 1, N)
    q = make_q(cfg, 1)
    cache = rkv.Cache(1, 2, N, cfg.dtype, cfg.stride_base, cfg.k, 4, cfg.group)
    for buf in rkv.Cache.BUFFERS:
        cache.buffers[buf].fill_(0xFF)   # fp16/bf16 NaN, slot 65535, code -1
    ws = torch.empty(rkv.rkv_encode_workspace(cache), dtype=torch.uint8, device="cuda")
    rkv.rkv_append(K[:, :, :400].contiguous(), V[:, :, :400].contiguous(), cache, 0, ws)
    rkv.rkv_append(K[:, :, 400:L].contiguous(), V[:, :, 400:L].contiguous(), cache, 400, ws)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    got = rkv.rkv_decode_attn_len(q, 8, cache, L, scale, n_split=4).cpu().numpy()
    Kn, Vn, qn = to_np_f32(K[:, :, :L]), to_np_f32(V[:, :, :L]), to_np_f32(q)
    want = _oracle_decode(cfg, Kn, Vn, qn, 4, scale)
    err = attn_err(got, want)
    say(f"  worst per-head rel L2 = {err:.2e}")
    assert np.isfinite(got).all()
    assert err <= 2e-3


# ------------------------------------------------------------------ full sizes
# The workloads at their real per-instance shapes, in the launch
# configuration the benchmark times; the oracle checks sampled tokens.

FULL = [
    ("llama3_8b_layer", 1, 4, 1),
    ("llama3_8b_32k_one_instance", 2, 4, 1),
    ("dynamic_131k", 3, 4, 1),
    ("prefill_stress_int4", 4, 4, 1),
    ("prefill_stress_int2", 4, 2, 1),
]


def _sample_rows(N, n, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 31, 32, 63, 64, 127, 128, N // 2, N - 129, N - 65, N - 33, N - 2, N - 1]
    rows = set(r for r in fixed if 0 <= r < N)
    rows.update(rng.integers(0, N, n).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("case", FULL, ids=[c[0] for c in FULL])
def test_full_size_sampled_encode(case):
    _need_gpu()
    name, index, bits, n_inst = case
    cfg = get_config(index)
    N = cfg.seq_len
    say(f"[full-size encode] {name}: N={N} H={cfg.n_kv_heads} inst={n_inst} bits={bits}")
    K, V = make_kv(cfg, n_inst, N)
    cache = encode(cfg, K, V, bits, n_inst, N)
    gc = GpuCache(cache)
    near = 0
    for h in range(cfg.n_kv_heads):
        Kn = to_np_f32(K[0, h])
        Vn = to_np_f32(V[0, h])
        rows = _sample_rows(N, 40, h)
        near += compare_encode(gc, h, Kn, Vn, cfg.stride_base, cfg.double_after,
                               rows=rows)["near_ties"]
    say(f"  near-ties: {near}")


# The longest sequence a cache accepts (2^22 positions), where the kernels'
# 32-bit per-head byte offsets and buffer ranges are largest: 512 references
# (the quantiser keeps them in LDS and reads the token rows through one
# 2^30-byte range) and 32768 references (gathers from memory, and the
# largest distance/top-k launch of the suite).
LONGEST = [("longest_512_refs", 8192), ("longest_32768_refs", 128)]


@pytest.mark.parametrize("name,base", LONGEST, ids=[c[0] for c in LONGEST])
def test_longest_sequence_sampled_encode(name, base):
    _need_gpu()
    cfg = _cfg(1, n_kv_heads=1, stride_base=base)
    N = 1 << 22
    say(f"[longest encode] {name}: N={N} stride={base}")
    K, V = make_kv(cfg, 1, N)
    cache = encode(cfg, K, V, 4, 1, N)
    assert cache.c.n_refs == N // base
    gc = GpuCache(cache)
    Kn, Vn = to_np_f32(K[0, 0]), to_np_f32(V[0, 0])
    del K, V, cache
    torch.cuda.empty_cache()
    near = compare_encode(gc, 0, Kn, Vn, cfg.stride_base, cfg.double_after,
                          rows=_sample_rows(N, 40, 11))["near_ties"]
    say(f"  near-ties: {near}")


def test_longest_sequence_decode():
    """Decode over a 2^22-position head (512 references, GQA 4) against the
    oracle's softmax attention over the library's own reconstruction (whose
    parity with the oracle is checked at smaller sizes): the property holds at
    any length, and here one split walks 4096 softmax chunks, so the
    per-reference weight totals reach their largest values."""
    _need_gpu()
    cfg = _cfg(1, n_kv_heads=1, n_q_heads=4, stride_base=8192)
    N = 1 << 22
    say(f"[longest decode] N={N} stride={cfg.stride_base}")
    K, V = make_kv(cfg, 1, N)
    q = make_q(cfg, 1)
    cache = encode(cfg, K, V, 4, 1, N)
    del K, V
    Kh, Vh = rkv.rkv_reconstruct(cache)
    torch.cuda.synchronize()
    Khn, Vhn = Kh[0].cpu().numpy(), Vh[0].cpu().numpy()
    del Kh, Vh
    torch.cuda.empty_cache()
    qn = to_np_f32(q[0])
    splits = sorted({rkv.rkv_decode_split_hint(cache, cfg.n_q_heads), 1}, reverse=True)
    for scale in (1.0 / math.sqrt(cfg.head_dim), 1.0):
        want = oracle.decode_attn(qn, Khn, Vhn, scale)
        for n_split in splits:
            got = rkv.rkv_decode_attn(q, cfg.n_q_heads, cache, scale,
                                      n_split=n_split).cpu().numpy()
            err = attn_err(got[0], want)
            say(f"  scale={scale:.4f} n_split={n_split} worst per-head rel L2 = {err:.2e}")
            assert np.isfinite(got).all()
            assert err <= 2e-3


@pytest.mark.parametrize("index", [1, 2, 3])
def test_full_size_decode_one_kv_head(index):
    """Decode at the full context of the workload for all query heads of KV
    head 0 (the oracle rebuilds that head completely).  Index 3 is the
    dynamic-stride 131072-position workload (896 references: the largest
    oracle encode of the suite)."""
    _need_gpu()
    cfg = get_config(index)
    N = cfg.seq_len
    say(f"[full-size decode] {cfg.name}: N={N}")
    K, V = make_kv(cfg, 1, N)
    q = make_q(cfg, 1)
    cache = encode(cfg, K, V, 4, 1, N)
    G = cfg.n_q_heads // cfg.n_kv_heads
    Kn, Vn = to_np_f32(K[0, 0]), to_np_f32(V[0, 0])
    enc = oracle.encode(Kn, Vn, cfg.stride_base, cfg.double_after, cfg.k, 4, cfg.group)
    kv = oracle.reconstruct(enc, Kn, Vn, 4)
    # the flat 1/sqrt(d) query and the sharp alpha = 1 one; the split count
    # the library suggests for this cache, 16 splits, and one split that walks the whole context
    # (N / 1024 softmax chunks, each folding its fixed-point reference
    # weights into the totals)
    splits = sorted({rkv.rkv_decode_split_hint(cache, cfg.n_q_heads), 16, 1}, reverse=True)
    for scale in (1.0 / math.sqrt(cfg.head_dim), 1.0):
        want = oracle.decode_attn(to_np_f32(q[0, :G]), kv[None, :, 0], kv[None, :, 1], scale)
        for n_split in splits:
            got = rkv.rkv_decode_attn(q, cfg.n_q_heads, cache, scale,
                                      n_split=n_split).cpu().numpy()
            err = attn_err(got[0, :G], want)
            say(f"  scale={scale:.4f} n_split={n_split} worst per-head rel L2 = {err:.2e}")
            assert err <= 2e-3
