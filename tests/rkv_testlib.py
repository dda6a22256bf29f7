"""Helpers shared by the test files: reading the library's output buffers
back into plain arrays (following the layouts documented in include/rkv.h),
the parity comparisons against the oracle, and the record of near-ties and
rounding-boundary cases the comparisons accepted."""

import numpy as np
import torch

import oracle
from boundary import classify_codes, latent_bound, residual_bound

# Accepted near-ties and boundary cases per test, written to a JSON record at
# the end of the session (see conftest.py).
REPORT = {}


def record(test: str, **counts):
    """Add counts to the record of `test` (summed over calls)."""
    r = REPORT.setdefault(test, {})
    for key, v in counts.items():
        r[key] = r.get(key, 0) + int(v)


def current_test() -> str:
    import os
    return os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]


def to_np_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy()


def buf_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


def sign_extend(v: np.ndarray, bits: int) -> np.ndarray:
    v = v.astype(np.int64)
    return np.where(v >= (1 << (bits - 1)), v - (1 << bits), v)


def unpack_rows(b: np.ndarray, bits: int) -> np.ndarray:
    """uint8 [..., nbytes] token-major bit strings -> int [..., nbytes*8/bits]."""
    b = b.astype(np.int64)
    per = 8 // bits
    fields = [(b >> (bits * j)) & ((1 << bits) - 1) for j in range(per)]
    out = np.stack(fields, axis=-1).reshape(*b.shape[:-1], b.shape[-1] * per)
    return sign_extend(out, bits)


class GpuCache:
    """Host copy of a library cache, one (instance, head) at a time."""

    def __init__(self, cache):
        c = cache.c
        self.n_inst, self.H, self.N, self.D = c.n_inst, c.n_kv_heads, c.seq_len, c.head_dim
        self.k, self.bits, self.group, self.n_refs = c.k, c.bits, c.group, c.n_refs
        self.dtype = cache.dtype
        ih = self.n_inst * self.H
        self.idx = buf_u16(cache.ref_idx)[: ih * self.N * self.k].reshape(ih, self.N, self.k)
        self.tiles = (self.N + 31) // 32
        if self.bits:
            ck = cache.codes_k.cpu().numpy()[: cache.sizes["codes_k"]]
            self.codes_k_bytes = ck.reshape(ih, self.N, 16 * self.bits)
            cv = cache.codes_v.cpu().numpy()[: cache.sizes["codes_v"]]
            self.codes_v_bytes = cv.reshape(ih, self.tiles, self.D, 4 * self.bits)
            ng = self.D // self.group
            self.scales = buf_u16(cache.scales)[: ih * self.N * 2 * ng].reshape(
                ih, self.N, 2, ng).view(np.float16)
        else:
            ck = cache.codes_k.cpu().numpy()[: cache.sizes["codes_k"]].view(np.float64)
            cv = cache.codes_v.cpu().numpy()[: cache.sizes["codes_v"]].view(np.float64)
            self.resid = np.stack([ck.reshape(ih, self.N, self.D),
                                   cv.reshape(ih, self.N, self.D)], axis=2)
        self.ref_bits = c.ref_bits
        self.latent_seed = int(c.latent_seed) if c.latent else None
        rk = cache.ref_kv.cpu()
        if self.ref_bits == 4:
            rb = rk[: cache.sizes["ref_kv"]].numpy().reshape(ih, 2, self.n_refs, self.D // 2)
            self.ref_codes = unpack_rows(rb, 4)
            ng = self.D // self.group
            self.ref_scales = buf_u16(cache.ref_scales)[: cache.sizes["ref_scales"] // 2].reshape(
                ih, 2, self.n_refs, ng).view(np.float16)
            self.ref_kv = (self.ref_codes.astype(np.float64) *
                           np.repeat(self.ref_scales.astype(np.float64), self.group, axis=-1))
        elif self.dtype == "bf16":
            rk = rk[: cache.sizes["ref_kv"]].view(torch.bfloat16).float().numpy()
            self.ref_kv = rk.reshape(ih, 2, self.n_refs, self.D)
        else:
            rk = rk[: cache.sizes["ref_kv"]].view(torch.float32).numpy()
            self.ref_kv = rk.reshape(ih, 2, self.n_refs, self.D)

    def codes(self, ih: int) -> np.ndarray:
        """int [N, 2, D] codes of one (instance, head)."""
        k = unpack_rows(self.codes_k_bytes[ih], self.bits)               # [N, D]
        v = unpack_rows(self.codes_v_bytes[ih], self.bits)               # [tiles, D, 32]
        v = v.transpose(0, 2, 1).reshape(self.tiles * 32, self.D)[: self.N]
        return np.stack([k, v], axis=1)


def near_tie_ok(keys_bf16, T, i, gpu_sel, ora_sel, rel=1e-5):
    """Mismatched reference sets of token i are acceptable only as near-ties:
    the extra GPU picks and the missed oracle picks, matched by rank, have
    exact distances within rel * max(D_a, D_b, |k_i|^2)."""
    ki = keys_bf16[i].astype(np.float64)
    d = lambda s: float(((keys_bf16[T[s]].astype(np.float64) - ki) ** 2).sum())
    extra = sorted(set(gpu_sel) - set(ora_sel), key=d)
    missed = sorted(set(ora_sel) - set(gpu_sel), key=d)
    if len(extra) != len(missed):
        return False
    floor = float((ki * ki).sum())
    for a, b in zip(extra, missed):
        da, db = d(a), d(b)
        if abs(da - db) > rel * max(da, db, floor):
            return False
    return True


def _abs_ref_sums(refs_abs: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """S[r, t] = sum over the selected slots of |reference row|[t]."""
    valid = idx != 0xFFFF
    rows = refs_abs[np.where(valid, idx, 0).astype(np.int64)]        # [R, k, d]
    return (rows * valid[..., None]).sum(axis=1)


def compare_encode(gc: GpuCache, ih: int, K: np.ndarray, V: np.ndarray, stride_base,
                   double_after, rows=None):
    """Compare one (instance, head) of a GPU cache with the oracle on `rows`.

    Reference sets must match except near-ties.  On matching rows every
    scale and code must equal the oracle's, except where the oracle's fp64
    pre-rounding value lies within the GPU's fp32 error bound of a rounding
    boundary (boundary.classify_codes); those are counted.  Returns a dict
    of counts plus the oracle record ``enc``, ``enc_gpu_codes`` (the same
    with the GPU's accepted scales and codes on matching rows), and masks
    ``matched`` (reference sets equal) and ``exact`` (also every scale and
    code equal); raises AssertionError on any failure."""
    enc = oracle.encode(K, V, stride_base, double_after, gc.k, gc.bits, gc.group, rows=rows,
                        ref_bits=gc.ref_bits, latent_seed=gc.latent_seed)
    T = enc["T"]
    assert T.shape[0] == gc.n_refs
    if gc.ref_bits == 4:
        # the quantised reference store: codes and scales bit-exact (decided
        # from the exact input values on both sides)
        np.testing.assert_array_equal(gc.ref_codes[ih], enc["ref_q"]["codes"])
        np.testing.assert_array_equal(gc.ref_scales[ih].view(np.uint16),
                                      enc["ref_q"]["scales"].view(np.uint16))
        refs = enc["ref_q"]["deq"].astype(np.float64)
    else:
        # the reference store is an exact copy
        np.testing.assert_array_equal(gc.ref_kv[ih, 0], K[T])
        np.testing.assert_array_equal(gc.ref_kv[ih, 1], V[T])
        refs = np.stack([K[T], V[T]]).astype(np.float64)
    keys = oracle.bf16_round(K)
    rows_ = enc["rows"]
    gidx = gc.idx[ih][rows_]
    match = np.all(gidx == enc["idx"], axis=1)
    near = 0
    for r in np.nonzero(~match)[0]:
        i = int(rows_[r])
        gsel = [int(x) for x in gidx[r] if x != 0xFFFF]
        osel = [int(x) for x in enc["idx"][r] if x != 0xFFFF]
        assert gidx[r].tolist()[len(gsel):] == [0xFFFF] * (gc.k - len(gsel)), (i, gidx[r])
        assert gsel == sorted(gsel) and len(gsel) == len(osel), (i, gsel, osel)
        assert near_tie_ok(keys, T, i, gsel, osel), (i, gsel, osel)
        near += 1
    m = np.nonzero(match)[0]
    counts = {"rows": len(rows_), "near_ties": near, "scale_cases": 0, "code_cases": 0,
              "elements": 0}
    X = (K, V)
    # the oracle's record with the GPU's accepted scales and codes on matching
    # rows: reconstruction is then compared value by value
    enc_g = dict(enc)
    exact = match.copy()
    if gc.bits:
        enc_g["scales"] = enc["scales"].copy()
        enc_g["codes"] = enc["codes"].copy()
        g_codes = gc.codes(ih)[rows_[m]]
        g_scales = gc.scales[ih][rows_[m]]
        enc_g["codes"][m] = g_codes
        enc_g["scales"][m] = g_scales
        same = np.all(g_codes == enc["codes"][m], axis=(1, 2)) & \
            np.all(g_scales.view(np.uint16) == enc["scales"][m].view(np.uint16), axis=(1, 2))
        exact[m] = same
    for p in range(2):
        S = _abs_ref_sums(np.abs(refs[p]), enc["idx"][m])
        x = np.asarray(X[p], np.float64)[rows_[m]]
        e = residual_bound(S, x)
        if gc.bits:
            z = enc["z"][m, p]
            if gc.latent_seed is not None:
                e = latent_bound(e, enc["delta"][m, p])
            res = classify_codes(z, e, enc["scales"][m, p], enc["codes"][m, p],
                                 gc.scales[ih][rows_[m], p], gc.codes(ih)[rows_[m], p],
                                 gc.bits, gc.group)
            bad = np.nonzero(~res["ok_rows"])[0]
            assert bad.size == 0, (
                f"plane {p}: scale or code outside the fp32 error bound at rows "
                f"{rows_[m][bad][:10]}")
            counts["scale_cases"] += res["scale_cases"]
            counts["code_cases"] += res["code_cases"]
            counts["elements"] += z.size
        else:
            # no quantisation: the stored residual is x - KV_R within the bound
            res = gc.resid[ih][rows_[m], p]
            d = enc["delta"][m, p]
            assert np.all(np.abs(res - d) <= e + 2.0 ** -40 * np.abs(d)), f"plane {p}"
            counts["elements"] += d.size
    record(current_test(), **counts)
    counts.update(enc=enc, enc_gpu_codes=enc_g, matched=match, exact=exact)
    return counts


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def attn_err(got, want) -> float:
    """Worst relative L2 error over the rows (one per instance and query
    head) of attention outputs [..., d]; the bar applies to every head, so
    one bad head cannot hide behind the others."""
    g = np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    g = g.reshape(-1, g.shape[-1])
    w = w.reshape(-1, w.shape[-1])
    num = np.linalg.norm(g - w, axis=1)
    den = np.maximum(np.linalg.norm(w, axis=1), 1e-300)
    return float(np.max(num / den))
