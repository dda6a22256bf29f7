"""Rounding-boundary classifier for quantised scales and codes.

The oracle decides every scale and code from the fp64 residual
z = KV_i - KV_R (paper page "DeltaKV Framework Architecture": KV_R is the
mean of the selected references, the residual is KV_i - KV_R).  The GPU forms
the same residual in fp32, so its z differs from the oracle's by at most a
rounding error bound e.  Where the oracle's value sits within e of a
rounding boundary -- a half-integer for a code, the midpoint of two fp16
neighbours for a scale -- either side of the boundary is a correct fp32
result.  Only those differences are accepted; they are counted and reported.
Any other difference fails.

Error model of the GPU's residual (u = 2^-24, the fp32 unit roundoff; each
operation is allowed 2u so that any summation order and a non-RNE hardware
add still fit):
  * KV_R = (sum of k_eff rows) / k_eff: k_eff - 1 additions and one division
    or multiplication, |KV_R32 - KV_R| <= 2u S + u S / k_eff <= 3u S, with
    S the sum of |row| over the selected rows;
  * z32 = fl(x - KV_R32): a further u (|x| + S);
so |z32 - z| <= 4u (S + |x|) = 2^-22 (S + |x|); the bound used, 2^-21 (S + |x|),
doubles it.  Scales and codes are then the exact roundings of the GPU's own
z32 (ties to even decided exactly).  In latent mode z = H D (x - KV_R) / 16 is formed by seven fp32
butterfly stages on z32; each output is a signed sum of all 128 inputs, so
the bound is (sum_t e_t + 14u sum_t (|z_t| + e_t)) / 16 for every element.
"""

import numpy as np

U = 2.0 ** -24          # fp32 unit roundoff
REL = 2.0 ** -40        # the oracle's own fp64 rounding, with a wide margin


def residual_bound(S, x):
    """Bound on |z32 - z| per element: S = sum of |selected reference rows|,
    x = the token's row (same shape)."""
    return 2.0 ** -21 * (np.asarray(S, np.float64) + np.abs(np.asarray(x, np.float64)))


def latent_bound(e, delta):
    """Bound on the rotated residual's error per element from the plain
    bound e and the fp64 residual delta ([..., d] each)."""
    e = np.asarray(e, np.float64)
    tot = (e.sum(-1) + 14 * U * (np.abs(delta).sum(-1) + e.sum(-1))) / 16
    return np.broadcast_to(tot[..., None], e.shape).copy()


def fp16_nearest(x):
    """Nearest fp16 (ties to even) of non-negative fp64 values, saturating at
    65504, as fp64."""
    with np.errstate(over="ignore"):
        h = np.asarray(x, np.float64).astype(np.float16)
    return np.where(np.isinf(h), 65504.0, h.astype(np.float64))


def classify_codes(z, e, s_oracle, c_oracle, s_gpu, c_gpu, bits, group):
    """Check GPU scales and codes of rows against the oracle's.

    z, e: fp64 [R, d] -- the oracle's pre-rounding values and the GPU's
    error bound on them; s_*: fp16 [R, d/group]; c_*: int [R, d].

    A group's GPU scale is accepted when it is the fp16 rounding of
    max|z'| / qmax for some z' within e of z (the rounding is monotone, so
    the accepted scales are those between the roundings of (a - e_a)/qmax and
    (a + e_a)/qmax).  Its codes are then checked against the GPU's own scale
    s: a code is accepted when it is the clamped nearest integer of some
    value within e/s of z/s.  Returns a dict:
      ok_rows      bool [R]  every scale and code of the row accepted
      scale_cases  groups whose GPU scale differs from the oracle's (accepted)
      code_cases   elements of groups with equal scales whose GPU code
                   differs from the oracle's (accepted)
    """
    qmax = (1 << (bits - 1)) - 1
    z = np.asarray(z, np.float64)
    e = np.asarray(e, np.float64)
    R, d = z.shape
    ng = d // group
    a = np.abs(z).reshape(R, ng, group).max(-1)
    ea = e.reshape(R, ng, group).max(-1) + REL * a
    s_lo = fp16_nearest(np.maximum(a - ea, 0.0) / qmax)
    s_hi = fp16_nearest((a + ea) / qmax)
    sg = np.asarray(s_gpu, np.float16).astype(np.float64)
    so = np.asarray(s_oracle, np.float16).astype(np.float64)
    scale_ok = (sg >= s_lo) & (sg <= s_hi)
    s_el = np.repeat(sg, group, axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s_el > 0, z / np.where(s_el > 0, s_el, 1.0), 0.0)
        ev = np.where(s_el > 0, e / np.where(s_el > 0, s_el, 1.0), 0.0) + REL * np.abs(v)
    c_lo = np.clip(np.rint(v - ev), -qmax, qmax)
    c_hi = np.clip(np.rint(v + ev), -qmax, qmax)
    cg = np.asarray(c_gpu, np.int64)
    code_ok = (cg >= c_lo) & (cg <= c_hi)
    same_scale = np.repeat(sg == so, group, axis=-1)
    code_cases = int(np.sum(same_scale & (cg != np.asarray(c_oracle, np.int64))))
    ok_rows = scale_ok.all(-1) & code_ok.all(-1)
    return {"ok_rows": ok_rows, "scale_cases": int(np.sum(sg != so)),
            "code_cases": code_cases}
