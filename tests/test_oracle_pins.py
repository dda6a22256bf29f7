"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against something other than itself: values
derived by hand from the definitions (tests/golden), brute force on tiny
integer inputs, closed forms, invariants of the method, or library routines
for the special cases that reduce to one.  A plausible slip in the oracle (a
dropped term, a wrong sign or index, a transposed operand, the wrong rounding
or summation order) fails at least one of them.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- rounding

def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    normal = rng.standard_normal(20000).astype(np.float32)
    tiny = (rng.standard_normal(2000) * 1e-30).astype(np.float32)
    # exact ties between two bf16 neighbours: the dropped 16 bits are 0x8000
    hi = rng.integers(0x0080, 0x7F00, 4000).astype(np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    x = np.concatenate([normal, tiny, ties, -ties])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _nearest_fp16_exact(x: Fraction) -> float:
    """Nearest fp16 to a non-negative rational, ties to even, saturating at
    65504, by exhaustive comparison with the fp16 grid (independent of
    numpy's conversion)."""
    grid = _FP16_GRID
    lo, hi = 0, len(grid) - 1
    if x >= grid[-1][0]:
        return 65504.0 if x < Fraction(65520) else 65504.0
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if grid[mid][0] <= x:
            lo = mid
        else:
            hi = mid
    a, b = grid[lo], grid[hi]
    da, db = x - a[0], b[0] - x
    if da < db:
        return float(a[0])
    if db < da:
        return float(b[0])
    return float(a[0]) if a[1] % 2 == 0 else float(b[0])


def _fp16_grid():
    out = []
    for bits in range(0, 0x7C00):          # all finite non-negative fp16
        v = np.array([bits], dtype=np.uint16).view(np.float16)[0]
        out.append((Fraction(float(v)), bits))
    return out


_FP16_GRID = _fp16_grid()


def test_fp16_scale_is_exact_nearest_even():
    rng = np.random.default_rng(2)
    vals = []
    # random magnitudes over the whole fp16 range incl. subnormals
    for e in range(-26, 17):
        vals.extend((rng.random(30) + 0.5) * 2.0 ** e)
    # exact midpoints and their fp64 neighbours
    for bits in rng.integers(1, 0x7BFF, 300):
        a = float(np.array([bits], np.uint16).view(np.float16)[0])
        b = float(np.array([bits + 1], np.uint16).view(np.float16)[0])
        m = (a + b) / 2
        vals.extend([m, np.nextafter(m, 0), np.nextafter(m, 1e9)])
    vals.extend([65504.0, 65519.99, 65520.0, 1e6, 0.0, 2.0 ** -25, 2.0 ** -24 * 1.5])
    vals = np.array(vals, dtype=np.float64)
    got = oracle.fp16_scale(vals).astype(np.float64)
    want = np.array([_nearest_fp16_exact(Fraction(float(v))) for v in vals])
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- schedule

def test_schedule_counts_golden():
    for c in _golden("schedule.json")["cases"]:
        T = oracle.ref_positions(c["n"], c["base"], c["double_after"])
        assert T.shape[0] == c["n_refs"], c
        assert T[0] == 0 and np.all(np.diff(T) > 0)
        if "sum_candidates" in c:
            tot = sum(oracle.candidate_count(i, T) for i in range(c["n"]))
            assert tot == c["sum_candidates"]


def test_schedule_fixed_closed_form():
    for n in (1, 2, 15, 16, 17, 100, 1000):
        for s in (1, 2, 3, 5, 16, 64):
            T = oracle.ref_positions(n, s)
            assert T.shape[0] == -(-n // s)
            assert np.array_equal(T, np.arange(0, n, s))


def test_schedule_dynamic_bands():
    T = oracle.ref_positions(40000, 16, 4096)
    gaps = {}
    for a, b in zip(T[:-1], T[1:]):
        gaps.setdefault(int(a).bit_length(), set()).add(int(b - a))
    assert np.all(np.diff(T[T < 4096]) == 16)
    assert np.all(np.diff(T[(T >= 4096) & (T < 8192)]) == 32)
    assert np.all(np.diff(T[(T >= 8192) & (T < 16384)]) == 64)
    assert np.all(np.diff(T[(T >= 16384) & (T < 32768)]) == 128)
    assert np.all(np.diff(T[T >= 32768]) == 256)


# ---------------------------------------------------------------- top-k

def _brute_topk(keys_int, T, i, k):
    """All candidates sorted by (squared distance, position) with Python ints."""
    cand = [(sum((a - b) ** 2 for a, b in zip(keys_int[i], keys_int[j])), slot)
            for slot, j in enumerate(T) if j <= i]
    cand.sort()
    return sorted(s for _, s in cand[:k])


@pytest.mark.parametrize("d", [4, 8])
@pytest.mark.parametrize("s", [1, 2, 3, 5])
def test_topk_brute_force_with_exact_ties(d, s):
    rng = np.random.default_rng(100 + d * 10 + s)
    n = 96
    # small integers force many exact distance ties
    keys_int = rng.integers(-3, 4, size=(n, d)).tolist()
    K = np.array(keys_int, dtype=np.float32)
    V = rng.standard_normal((n, d)).astype(np.float32)
    T = oracle.ref_positions(n, s)
    for k in range(1, 7):
        enc = oracle.encode(K, V, s, 0, k, 0, d)
        for i in range(n):
            want = _brute_topk(keys_int, T.tolist(), i, k)
            got = [int(x) for x in enc["idx"][i] if x != oracle.IDX_PAD]
            assert got == want, (i, k)
            assert enc["k_eff"][i] == min(k, oracle.candidate_count(i, T))
            assert np.all(enc["idx"][i, len(want):] == oracle.IDX_PAD)


def test_topk_uses_bf16_rounded_keys():
    # Two references whose fp32 keys differ only below bf16 precision from
    # the query: after rounding they tie, and the lower position must win.
    d = 4
    K = np.zeros((3, d), dtype=np.float32)
    K[0] = [1.0, 0, 0, 0]
    K[1] = [1.0 + 2.0 ** -12, 0, 0, 0]    # rounds to 1.0 in bf16
    K[2] = [1.0 + 2.0 ** -13, 0, 0, 0]    # the query, also 1.0 in bf16
    V = np.zeros_like(K)
    enc = oracle.encode(K, V, 1, 0, 1, 0, d)
    # with stride 1 the query's own slot (distance 0) ties with slot 0 and 1;
    # the lowest slot wins.
    assert list(enc["idx"][2]) == [0]


# ---------------------------------------------------------------- mean

def test_mean_fp64_golden():
    for c in _golden("mean_f64.json")["cases"]:
        rows = np.array(c["rows"], dtype=np.float32).reshape(-1, 1)
        m = oracle.ref_mean(rows)
        assert m.dtype == np.float64
        assert hex(int(m.view(np.uint64)[0])) == c["mean_hex"], c


def test_mean_and_residual_are_exact_rationals_on_short_inputs():
    # fp64 holds the sum of a few fp32 values exactly when their exponents
    # are close; then the mean is the correctly rounded rational and the
    # residual's error is below 2^-52 relative (checked with Fractions).
    rng = np.random.default_rng(21)
    for k in (1, 2, 3, 5, 7, 8):
        rows = rng.standard_normal((k, 64)).astype(np.float32)
        x = rng.standard_normal(64).astype(np.float32)
        m = oracle.ref_mean(rows)
        z = oracle.residual(x, m)
        for t in (0, 17, 63):
            want_m = sum(Fraction(float(r)) for r in rows[:, t]) / k
            assert m[t] == float(want_m)
            want_z = Fraction(float(x[t])) - want_m
            assert abs(Fraction(float(z[t])) - want_z) <= \
                (abs(want_z) + abs(want_m)) * Fraction(1, 2 ** 52)


# ---------------------------------------------------------------- quantiser

@pytest.mark.parametrize("bits", [2, 4, 8])
def test_quantizer_closed_form_bounds(bits):
    rng = np.random.default_rng(bits)
    qmax = 2 ** (bits - 1) - 1
    for trial in range(300):
        g = 32
        z = (rng.standard_normal(128) * 10.0 ** rng.uniform(-6, 2)).astype(np.float32)
        z[rng.random(128) < 0.05] = 0
        if trial % 17 == 0:
            z[:g] = 0                       # an all-zero group
        s, c = oracle.quantize_residual(z, bits, g)
        assert np.all(np.abs(c) <= qmax)
        for gi in range(128 // g):
            zz = z[gi * g:(gi + 1) * g].astype(np.float64)
            cc = c[gi * g:(gi + 1) * g]
            sc = float(s[gi])
            a = np.abs(zz).max()
            if a == 0:
                assert sc == 0 and np.all(cc == 0)
                continue
            if sc == 0:                     # a / qmax below half the least fp16
                assert a / qmax <= 2.0 ** -25 and np.all(cc == 0)
                continue
            assert abs(sc - a / qmax) <= 2.0 ** -11 * (a / qmax) + 2.0 ** -25
            unclamped = np.abs(zz / sc) <= qmax + 0.5
            assert np.all(np.abs(zz - sc * cc)[unclamped] <= sc / 2 * (1 + 1e-12))
            if a / qmax < 2.0 ** -14:
                continue                    # subnormal scale: coarse grid
            j = int(np.argmax(np.abs(zz)))
            # the largest element maps to +-qmax, or +-(qmax-1) when the
            # scale rounded up
            allowed = (qmax,) if sc <= a / qmax else (qmax - 1, qmax)
            assert abs(cc[j]) in allowed, (cc[j], allowed)
            assert np.sign(cc[j]) == np.sign(zz[j])


def test_quantizer_ties_round_to_even():
    s = np.float16(0.125)
    z = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 7.0 * 8 / 8] + [0.0] * 24,
                 dtype=np.float64) * float(s)
    z[7] = 7 * float(s)                   # the group max: scale = 7s/7 = s
    s_got, c = oracle.quantize_residual(z.astype(np.float32), 4, 32)
    assert float(s_got[0]) == float(s)
    assert list(c[:8]) == [0, 2, 2, 0, -2, -2, 4, 7]


def test_quantizer_scale_saturates():
    z = np.zeros(32, np.float32)
    z[0] = 1e9
    s, c = oracle.quantize_residual(z, 8, 32)
    assert float(s[0]) == 65504.0 and c[0] == 127


# ---------------------------------------------------------------- packing

def test_pack_codes_golden():
    for c in _golden("pack_codes.json")["cases"]:
        got = oracle.pack_codes(np.array(c["codes"]), c["bits"])
        assert got.tolist() == c["bytes"], c


def test_pack_v_tile_is_transposed_token_major():
    rng = np.random.default_rng(5)
    tile = rng.integers(-7, 8, size=(32, 8))
    packed = oracle.pack_v_tile(tile, 4)
    assert packed.shape == (8, 16)
    for t in range(8):
        # byte u//2 of dim t holds tokens 2*(u//2) (low) and +1 (high)
        for u in range(32):
            nib = (int(packed[t, u // 2]) >> (4 * (u % 2))) & 0xF
            val = nib - 16 if nib >= 8 else nib
            assert val == tile[u, t]


# ---------------------------------------------------------------- invariants

def _mixture(n, d, protos, sigma, seed, dtype=np.float32):
    rng = np.random.default_rng(seed)
    P = rng.standard_normal((protos, d))
    ids = rng.integers(0, protos, n)
    K = P[ids] + sigma * rng.standard_normal((n, d))
    V = rng.standard_normal((protos, d))[ids] + sigma * rng.standard_normal((n, d))
    K = K.astype(np.float32)
    V = V.astype(np.float32)
    if dtype == "bf16":
        K, V = oracle.bf16_round(K), oracle.bf16_round(V)
    return K, V


@pytest.mark.parametrize("bits", [0, 4, 8])
def test_invariant_stride1_k1_zero_residual(bits):
    K, V = _mixture(200, 32, 8, 0.1, 7)
    enc = oracle.encode(K, V, 1, 0, 1, bits, 32)
    assert np.array_equal(enc["idx"][:, 0], np.arange(200))
    assert np.all(enc["delta"] == 0)
    if bits:
        assert np.all(enc["codes"] == 0)
        assert np.all(enc["scales"] == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("s,k", [(4, 2), (16, 4), (7, 3)])
def test_invariant_no_quantisation_reconstructs_exactly(dtype, s, k):
    K, V = _mixture(300, 64, 16, 0.2, 11, dtype)
    enc = oracle.encode(K, V, s, 0, k, 0, 32)
    kv = oracle.reconstruct(enc, K, V, 0)
    # KV_R + (KV - KV_R) = KV: exact after rounding to the input precision,
    # and within fp64 round-off before it
    assert np.array_equal(kv[:, 0].astype(np.float32), K)
    assert np.array_equal(kv[:, 1].astype(np.float32), V)
    assert np.all(np.abs(kv[:, 0] - K) <= 2.0 ** -52 * (np.abs(K) + np.abs(enc["mean"][:, 0])))


def test_invariant_no_quantisation_decode_is_full_attention():
    K, V = _mixture(257, 64, 16, 0.2, 13)
    enc = oracle.encode(K, V, 8, 0, 3, 0, 32)
    kv = oracle.reconstruct(enc, K, V, 0)
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 64))
    out = oracle.decode_attn(q, kv[None, :, 0], kv[None, :, 1], 0.3)
    # textbook attention from the library routine on the raw cache
    qt = torch.from_numpy(q).view(1, 4, 1, 64)
    kt = torch.from_numpy(K.astype(np.float64)).view(1, 1, 257, 64).expand(1, 4, 257, 64)
    vt = torch.from_numpy(V.astype(np.float64)).view(1, 1, 257, 64).expand(1, 4, 257, 64)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.3)
    np.testing.assert_allclose(out, ref.view(4, 64).numpy(), rtol=0, atol=1e-13)


def test_reconstruction_error_within_half_scale():
    K, V = _mixture(400, 128, 32, 0.1, 17)
    enc = oracle.encode(K, V, 16, 0, 4, 8, 32)
    kv = oracle.reconstruct(enc, K, V, 8)
    T = enc["T"]
    for r, i in enumerate(enc["rows"]):
        if i in T:
            assert np.array_equal(kv[r, 0], K[i].astype(np.float64))
            continue
        for p, X in enumerate((K, V)):
            sc = np.repeat(enc["scales"][r, p].astype(np.float64), 32)
            err = np.abs(kv[r, p] - X[i].astype(np.float64))
            # |z - s c| <= s/2, up to fp64 round-off
            assert np.all(err <= sc / 2 * (1 + 1e-12) + 1e-15 * (np.abs(X[i]) + 1))


def test_reconstruction_mean_is_reference_average():
    # k = 2 with references chosen by hand: KV_R must be their average and a
    # reference position must come back uncompressed.
    d = 4
    K = np.array([[0, 0, 0, 0], [9, 9, 9, 9], [2, 0, 0, 0], [1, 0, 0, 0],
                  [0, 2, 0, 0]], dtype=np.float32)
    V = np.arange(20, dtype=np.float32).reshape(5, 4)
    enc = oracle.encode(K, V, 2, 0, 2, 0, 4)    # T = {0, 2, 4}
    # row 3: candidates slots 0 (pos 0, dist 1), 1 (pos 2, dist 1) -> both
    assert list(enc["idx"][3]) == [0, 1]
    np.testing.assert_array_equal(enc["mean"][3, 0], [1, 0, 0, 0])
    np.testing.assert_array_equal(enc["mean"][3, 1], (V[0].astype(np.float64) + V[2]) / 2)
    np.testing.assert_array_equal(enc["delta"][3, 0], K[3] - [1, 0, 0, 0])
    # row 1: candidates slot 0 only -> k_eff = 1, KV_R is that reference
    assert list(enc["idx"][1]) == [0, oracle.IDX_PAD]
    np.testing.assert_array_equal(enc["mean"][1, 0], K[0])
    np.testing.assert_array_equal(enc["delta"][1, 1], V[1] - V[0])
    kv = oracle.reconstruct(enc, K, V, 0)
    np.testing.assert_array_equal(kv[4, 0], K[4])


# ---------------------------------------------------------------- decode

def test_decode_uniform_logits_give_mean_value():
    rng = np.random.default_rng(4)
    kh = rng.standard_normal((2, 50, 8))
    vh = rng.standard_normal((2, 50, 8))
    q = np.zeros((4, 8))
    out = oracle.decode_attn(q, kh, vh, 1.0)
    np.testing.assert_allclose(out[0], vh[0].mean(0), atol=1e-14)
    np.testing.assert_allclose(out[3], vh[1].mean(0), atol=1e-14)   # GQA: head 3 -> kv 1


def test_decode_dominant_key_selects_its_value():
    kh = np.zeros((1, 10, 4))
    kh[0, 6] = [50, 0, 0, 0]
    vh = np.arange(40, dtype=np.float64).reshape(1, 10, 4)
    out = oracle.decode_attn(np.array([[1.0, 0, 0, 0]]), kh, vh, 1.0)
    np.testing.assert_allclose(out[0], vh[0, 6], atol=1e-15)


def test_tile_positions_golden():
    # n = 70: three tiles, the last one ragged (64..69); -1 and 9 select nothing
    got = oracle.tile_positions([2, -1, 0, 9], 70)
    assert got.tolist() == list(range(0, 32)) + list(range(64, 70))
    assert oracle.tile_positions([1], 32).tolist() == []
    assert oracle.tile_positions(range(3), 70).tolist() == list(range(70))


def test_quantized_refs_dequantise_exactly_and_within_half_scale():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((300, 128)).astype(np.float32)
    V = (3.0 * rng.standard_normal((300, 128))).astype(np.float32)
    T = oracle.ref_positions(300, 16)
    q = oracle.quantize_refs(K, V, T, 32)
    assert q["codes"].shape == (2, T.shape[0], 128)
    assert np.abs(q["codes"]).max() <= 7
    for p, X in enumerate((K, V)):
        sc = np.repeat(q["scales"][p].astype(np.float64), 32, axis=-1)
        # dequantised value = code * scale exactly (checked in rationals)
        for s_, t in ((0, 0), (3, 77), (T.shape[0] - 1, 127)):
            want = Fraction(int(q["codes"][p][s_, t])) * Fraction(float(sc[s_, t]))
            assert Fraction(float(q["deq"][p][s_, t])) == want
        err = np.abs(X[T].astype(np.float64) - q["deq"][p].astype(np.float64))
        assert np.all(err <= sc / 2 + 1e-12)


def test_encode_with_quantized_refs_uses_the_dequantised_rows():
    rng = np.random.default_rng(6)
    K = rng.standard_normal((96, 16)).astype(np.float32)
    V = rng.standard_normal((96, 16)).astype(np.float32)
    enc = oracle.encode(K, V, 8, 0, 3, 4, 8, ref_bits=4)
    deq = enc["ref_q"]["deq"]
    for r in (5, 40, 95):
        sel = enc["idx"][r][enc["idx"][r] != oracle.IDX_PAD].astype(np.int64)
        # the library mean of the dequantised (not the raw) rows
        np.testing.assert_allclose(enc["mean"][r, 0], deq[0][sel].astype(np.float64).mean(0),
                                   rtol=0, atol=1e-15)
        assert not np.allclose(enc["mean"][r, 0], K[enc["T"][sel]].astype(np.float64).mean(0),
                               rtol=0, atol=1e-6)
    kv = oracle.reconstruct(enc, K, V, 4)
    T = enc["T"]
    np.testing.assert_array_equal(kv[T, 0], deq[0].astype(np.float64))


def test_splitmix64_published_vectors():
    assert oracle.splitmix64(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert oracle.splitmix64(1234567, 1) == [0x599ED017FB08FC85]
    sg = oracle.latent_signs(0)
    assert sg.shape == (128,) and set(np.unique(sg)) == {-1.0, 1.0}
    assert sg[0] == -1.0 and sg[1] == 1.0 and sg[2] == 1.0   # top bits of the vector above


def test_hadamard_and_latent_fc():
    import scipy.linalg
    Hm = oracle.hadamard(128)
    # the Sylvester construction of the library routine
    np.testing.assert_array_equal(Hm, scipy.linalg.hadamard(128).astype(np.float64))
    np.testing.assert_array_equal(Hm @ Hm, 128 * np.eye(128))
    sg = oracle.latent_signs(5)
    # f_c of a unit vector e_t is column t of H times the sign of dim t, / 16
    for t in (0, 1, 77, 127):
        e = np.zeros(128)
        e[t] = 1.0
        np.testing.assert_array_equal(oracle.latent_fc64(e, sg),
                                      sg[t] * scipy.linalg.hadamard(128)[:, t] / 16.0)
    # linear: f_c(a x + y) = a f_c(x) + f_c(y) (non-integer data)
    rng = np.random.default_rng(3)
    x, y = rng.standard_normal((2, 128))
    np.testing.assert_allclose(oracle.latent_fc64(2.5 * x + y, sg),
                               2.5 * oracle.latent_fc64(x, sg) + oracle.latent_fc64(y, sg),
                               rtol=0, atol=1e-13)
    # the norm shrinks by sqrt(128) / 16 = 1/sqrt(2)
    assert abs(np.linalg.norm(oracle.latent_fc64(x, sg)) - np.linalg.norm(x) / np.sqrt(2)) <= \
        1e-13 * np.linalg.norm(x)


def test_latent_pair_inverts():
    rng = np.random.default_rng(4)
    sg = oracle.latent_signs(99)
    x = rng.standard_normal(128)
    back = oracle.latent_fd64(oracle.latent_fc64(x, sg), sg)
    assert np.max(np.abs(back - x)) <= 1e-13 * np.max(np.abs(x))
    # exact on integer data (no rounding anywhere)
    xi = rng.integers(-8, 8, 128).astype(np.float64)
    np.testing.assert_array_equal(oracle.latent_fd64(oracle.latent_fc64(xi, sg), sg), xi)


def test_latent_encode_reconstruct_within_bound():
    rng = np.random.default_rng(8)
    K = rng.standard_normal((200, 128)).astype(np.float32)
    V = rng.standard_normal((200, 128)).astype(np.float32)
    enc = oracle.encode(K, V, 16, 0, 4, 4, 32, latent_seed=7)
    kv = oracle.reconstruct(enc, K, V, 4)
    T = enc["T"]
    nonref = np.setdiff1d(np.arange(200), T)
    # error of the rotated codes is <= scale/2 per element; f_d scales norms by 1/sqrt(2)
    sc = np.repeat(enc["scales"].astype(np.float64), 32, axis=-1)
    err = kv[nonref, 0] - K[nonref].astype(np.float64)
    bound = np.linalg.norm(sc[nonref, 0] / 2, axis=-1) * np.sqrt(128) / 8 + 1e-9
    assert np.all(np.linalg.norm(err, axis=-1) <= bound)
