"""Pins of the rounding-boundary classifier (tests/boundary.py).

The oracle decides scales and codes from the fp64 residual; a GPU forms the
residual in fp32.  These tests feed the classifier with a model of fp32
arithmetic written here (an ascending-slot fp32 sum, an fp32 division, an
fp32 subtraction, fp32 Walsh-Hadamard butterflies, then exact decisions) --
a stand-in for any fp32 implementation, not the HIP library's output -- and
check that:
  * every difference between that model and the oracle is accepted, and is
    counted as a boundary case;
  * such differences really occur (a constructed k_eff = 3 case, the tiny
    workload's data, latent int2 scales), so the acceptance is exercised;
  * planted mistakes away from a boundary (a code off by one, a scale one
    fp16 step off) are rejected.
"""

import dataclasses
from fractions import Fraction

import numpy as np

import oracle
from boundary import classify_codes, fp16_nearest, latent_bound, residual_bound
from synth import gen_head_kv, get_config


# ------------------------------------------------------------ fp32 model

def fp32_mean_residual(rows, x):
    """KV_R and z in fp32: rows added one after another, / k_eff, x - KV_R."""
    rows = np.asarray(rows, np.float32)
    s = rows[0].copy()
    for r in rows[1:]:
        s = (s + r).astype(np.float32)
    m = (s / np.float32(rows.shape[0])).astype(np.float32)
    return (np.asarray(x, np.float32) - m).astype(np.float32)


def fwht_f32(x):
    """Unnormalised Walsh-Hadamard transform in fp32 (butterflies on index
    bit 0, 1, ..., each rounded to fp32)."""
    y = np.asarray(x, np.float32).copy()
    n = y.shape[0]
    h = 1
    while h < n:
        y = y.reshape(-1, 2, h)
        a, b = y[:, 0, :].copy(), y[:, 1, :].copy()
        y[:, 0, :] = (a + b).astype(np.float32)
        y[:, 1, :] = (a - b).astype(np.float32)
        y = y.reshape(n)
        h *= 2
    return y


def exact_decisions(z32, bits, group):
    """Scale and codes decided exactly from fp32 values (fp64 is exact
    enough for fp32 operands: no fp32 value lies within 2^-53 relative of a
    rounding boundary unless it sits on one)."""
    return oracle.quantize_residual(np.asarray(z32, np.float64), bits, group)


def model_encode(K, V, enc, bits, group, signs=None):
    """Scales/codes [R, 2, ...] of the fp32 model for the oracle's rows and
    selections."""
    T = enc["T"]
    R = enc["rows"].shape[0]
    d = K.shape[1]
    sc = np.zeros((R, 2, d // group), np.float16)
    cd = np.zeros((R, 2, d), np.int64)
    for r, i in enumerate(enc["rows"]):
        sel = enc["idx"][r][enc["idx"][r] != oracle.IDX_PAD].astype(np.int64)
        for p, X in enumerate((K, V)):
            z32 = fp32_mean_residual(X[T[sel]], X[i])
            if signs is not None:
                z32 = (fwht_f32(z32 * signs) * np.float32(0.0625)).astype(np.float32)
            sc[r, p], cd[r, p] = exact_decisions(z32, bits, group)
    return sc, cd


def bounds(K, V, enc, p, latent=False):
    T = enc["T"]
    X = (K, V)[p]
    S = np.zeros((enc["rows"].shape[0], K.shape[1]))
    for r in range(S.shape[0]):
        sel = enc["idx"][r][enc["idx"][r] != oracle.IDX_PAD].astype(np.int64)
        S[r] = np.abs(X[T[sel]].astype(np.float64)).sum(0)
    e = residual_bound(S, X[enc["rows"]])
    return latent_bound(e, enc["delta"][:, p]) if latent else e


def classify(K, V, enc, sc, cd, bits, group, latent=False):
    out = []
    for p in range(2):
        out.append(classify_codes(enc["z"][:, p], bounds(K, V, enc, p, latent),
                                  enc["scales"][:, p], enc["codes"][:, p],
                                  sc[:, p], cd[:, p], bits, group))
    return out


# ------------------------------------------------------------ constructed case

def _k3_case():
    """Three fp32 references with an exact sum S and one fp32 token whose
    exact residual x - S/3 lies just above the half-integer 2.5 * 0.125,
    while fp32's rounded mean pushes it below (search over a small grid,
    verified with exact rationals)."""
    sigma = Fraction(1, 8)
    for num in range(1, 400):
        S = Fraction(num, 64)
        r = [float(S / 4), float(S / 4), float(S / 2)]          # exact in fp32
        target = S / 3 + Fraction(5, 2) * sigma                 # boundary of codes 2 and 3
        x = np.float32(float(target))
        for cand in (x, np.nextafter(x, np.float32(2)), np.nextafter(x, np.float32(0))):
            zx = Fraction(float(cand)) - S / 3
            if not (Fraction(5, 2) * sigma + Fraction(1, 2 ** 45) < zx <
                    Fraction(5, 2) * sigma + Fraction(1, 2 ** 26)):
                continue
            rows = np.zeros((3, 32), np.float32)
            rows[:, 0] = r
            xr = np.zeros(32, np.float32)
            xr[0] = cand
            xr[1] = 7 * 0.125                                    # group max -> scale 1/8
            z32 = fp32_mean_residual(rows, xr)
            if np.rint(float(z32[0]) / 0.125) == 2:              # fp32 lands below
                return rows, xr
    raise AssertionError("no constructed case found")


def test_constructed_keff3_fp32_case_is_a_counted_boundary_case():
    rows, x = _k3_case()
    m = oracle.ref_mean(rows)
    z = oracle.residual(x, m)
    s_o, c_o = oracle.quantize_residual(z, 4, 32)
    assert float(s_o[0]) == 0.125 and c_o[0] == 3                # exact: above 2.5
    s_g, c_g = exact_decisions(fp32_mean_residual(rows, x), 4, 32)
    assert float(s_g[0]) == 0.125 and c_g[0] == 2                # fp32: below
    e = residual_bound(np.abs(rows.astype(np.float64)).sum(0), x)
    res = classify_codes(z[None], e[None], s_o[None], c_o[None], s_g[None], c_g[None], 4, 32)
    assert res["ok_rows"].all() and res["code_cases"] == 1 and res["scale_cases"] == 0
    # a code two steps from the oracle's, or off by one away from a boundary
    for bad in ((0, 1), (1, c_o[1] - 1)):
        c_b = c_g.copy()
        c_b[bad[0]] = bad[1]
        res = classify_codes(z[None], e[None], s_o[None], c_o[None], s_g[None], c_b[None], 4, 32)
        assert not res["ok_rows"].any(), bad


# ------------------------------------------------------------ workload data

def _tiny(**kw):
    cfg = dataclasses.replace(get_config(0), **kw)
    k, v = gen_head_kv(cfg, 0, 0, 0, device="cpu")
    return cfg, k.float().numpy(), v.float().numpy()


def test_tiny_workload_fp32_differences_are_boundary_cases():
    cfg, K, V = _tiny()
    enc = oracle.encode(K, V, cfg.stride_base, 0, cfg.k, 8, cfg.group)
    sc, cd = model_encode(K, V, enc, 8, cfg.group)
    res = classify(K, V, enc, sc, cd, 8, cfg.group)
    assert all(r["ok_rows"].all() for r in res)
    n_code = sum(r["code_cases"] for r in res)
    n_scale = sum(r["scale_cases"] for r in res)
    n_diff = int(np.sum(cd != enc["codes"])) + int(np.sum(sc.view(np.uint16) != enc["scales"].view(np.uint16)))
    # every difference of the fp32 model is one of the counted cases, and
    # this data has some (the fp64 definition and fp32 disagree)
    assert n_code + n_scale >= 1
    assert np.sum(cd != enc["codes"]) >= n_code
    assert n_diff >= 1
    # planted: a code one step off where the oracle's value is far from a
    # half-integer, and a scale one fp16 step up, are both rejected
    rng = np.random.default_rng(0)
    s_el = np.repeat(enc["scales"].astype(np.float64), cfg.group, axis=-1)
    frac = np.abs(enc["z"] / np.where(s_el > 0, s_el, 1) - np.rint(enc["z"] / np.where(s_el > 0, s_el, 1)))
    far = np.argwhere((frac < 0.3) & (np.abs(enc["codes"]) < 100) & (s_el > 0))
    r, p, t = far[rng.integers(len(far))]
    cd_b = cd.copy()
    cd_b[r, p, t] += 1
    assert not classify(K, V, enc, sc, cd_b, 8, cfg.group)[p]["ok_rows"][r]
    sc_b = sc.copy()
    sc_b[r, p, 0] = np.nextafter(sc_b[r, p, 0], np.float16(np.inf))
    assert not classify(K, V, enc, sc_b, cd, 8, cfg.group)[p]["ok_rows"][r]


def test_latent_int2_scale_differences_are_boundary_cases():
    cfg, K, V = _tiny(group=64)
    seed = 0        # this seed's rotation puts one group's max next to an fp16 midpoint
    enc = oracle.encode(K, V, cfg.stride_base, 0, cfg.k, 2, 64, latent_seed=seed)
    sc, cd = model_encode(K, V, enc, 2, 64, signs=enc["signs"])
    res = classify(K, V, enc, sc, cd, 2, 64, latent=True)
    assert all(r["ok_rows"].all() for r in res)
    n_scale = sum(r["scale_cases"] for r in res)
    assert n_scale == int(np.sum(sc.view(np.uint16) != enc["scales"].view(np.uint16)))
    assert n_scale >= 1
    # with a zero error bound the same differences are rejected: the
    # acceptance comes from the bound alone
    tight = [classify_codes(enc["z"][:, p], bounds(K, V, enc, p, latent=False) * 0,
                            enc["scales"][:, p], enc["codes"][:, p], sc[:, p], cd[:, p], 2, 64)
             for p in range(2)]
    assert not all(r["ok_rows"].all() for r in tight)


def test_fp16_nearest_matches_the_oracle_scale_rounding():
    rng = np.random.default_rng(9)
    x = np.concatenate([(rng.random(2000) + 0.5) * 2.0 ** rng.integers(-26, 17, 2000),
                        [0.0, 65504.0, 65519.0, 65520.0, 1e9]])
    np.testing.assert_array_equal(fp16_nearest(x), oracle.fp16_scale(x).astype(np.float64))
