"""CPU oracle for the ResidualKV hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library and does
not import it.

It is a plain, slow, step-by-step statement of what the path computes, for
one (instance, KV head) at a time, on NumPy arrays, in fp64 throughout:
the reference mean KV_R and the residual KV - KV_R are formed in fp64 from
the original-precision rows, and every quantised scale and code is the
round-to-nearest-even of that fp64 value.  Distances are taken on keys
rounded to bf16 (the one place the method's own precision enters), exactly.

Sources (the method's pages):
  [P1] "ResidualKV: Residual-Based KV Cache Compression for Efficient
       Long-Context Inference" (paper page with summary and transcript):
       section "DeltaKV Framework Architecture" -- strided reference
       selection, top-k nearest by L2 distance, mean reference KV_R,
       residual z = f(KV) - f(KV_R), reconstruction KV^ = KV^_delta + KV_R;
       section "Key concepts" -- residual computation;
       section "Performance Results" -- residuals suit token-wise
       quantisation; transcript -- the cache is split into uncompressed
       reference tokens and compressed tokens.
  [P3] "New KV Cache Compression Method Cuts Long-Context Inference Costs by
       85%", section "How ResidualKV Works" -- global reference tokens plus
       compact quantised residual codes, reconstruction on the fly, and a
       dynamic-stride schedule with roughly logarithmic reference growth.

Readings where the pages are silent (each is the plainest one the rest
supports):
  * position j is a reference iff j mod s(j) == 0 (so position 0 always is);
  * token i's candidates are the references at positions <= i (itself
    included when i is a reference);
  * fewer than k candidates: k_eff = |candidates|, slots padded with 0xFFFF;
  * distances use keys rounded to bf16 (RNE) in every input precision;
  * ties in distance go to the lower position;
  * the compressor/decompressor pair is the identity; the residual is stored
    as symmetric absmax group-quantised codes with an fp16 scale;
  * bits == 0 means no quantisation: the residual is kept as is.
"""

import numpy as np

IDX_PAD = 0xFFFF
V_TILE = 32          # tokens per tile of the transposed V-code layout


# ---------------------------------------------------------------------------
# Reference schedule  ([P1] "DeltaKV Framework Architecture", strided
# reference selection; [P3] "How ResidualKV Works", dynamic-stride schedule)
# ---------------------------------------------------------------------------

def stride_at(j: int, base: int, double_after: int) -> int:
    """Stride in force at position j.

    Fixed schedule (double_after == 0): ``base`` everywhere.  Dynamic
    schedule: ``base`` below ``double_after``; from there the stride doubles
    each time the position doubles, so [A, 2A) uses 2*base, [2A, 4A) uses
    4*base, and so on (A = double_after).
    """
    if double_after == 0 or j < double_after:
        return base
    band = 0
    while j >= double_after << band:
        band += 1
    return base << band


def ref_positions(n: int, base: int, double_after: int = 0) -> np.ndarray:
    """Sorted reference positions T in [0, n): j is in T iff j mod s(j) == 0."""
    return np.array([j for j in range(n) if j % stride_at(j, base, double_after) == 0],
                    dtype=np.int64)


# ---------------------------------------------------------------------------
# Rounding helpers (IEEE 754 round-to-nearest-even)
# ---------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32.

    bf16 keeps the top 16 bits of an fp32 word; adding 0x7FFF plus the lowest
    kept bit before truncating implements round-half-to-even on the dropped
    16 bits.  (Inputs here are finite.)
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def fp16_scale(x64: np.ndarray) -> np.ndarray:
    """Nearest fp16 to fp64 values x (ties to even), saturating at 65504."""
    with np.errstate(over="ignore"):
        h = np.asarray(x64, dtype=np.float64).astype(np.float16)
    return np.where(np.isinf(h), np.float16(65504.0), h)


# ---------------------------------------------------------------------------
# Encode, one token row at a time ([P1] "DeltaKV Framework Architecture")
# ---------------------------------------------------------------------------

def candidate_count(i: int, T: np.ndarray) -> int:
    """|C_i|: references at positions <= i."""
    return int(np.searchsorted(T, i, side="right"))


def distances(key_i: np.ndarray, ref_keys: np.ndarray) -> np.ndarray:
    """Squared L2 distance from one key to each candidate key, fp64, summed
    directly over (a - b)^2 (exact for bf16-valued inputs)."""
    diff = ref_keys.astype(np.float64) - key_i.astype(np.float64)[None, :]
    return (diff * diff).sum(axis=1)


def select_topk(dist: np.ndarray, k: int) -> np.ndarray:
    """Slots of the k_eff nearest candidates, lowest slot first among equal
    distances; returned in ascending slot order."""
    k_eff = min(k, dist.shape[0])
    order = np.argsort(dist, kind="stable")[:k_eff]
    return np.sort(order)


def ref_mean(ref_rows: np.ndarray) -> np.ndarray:
    """KV_R: the mean of the selected reference rows (the rows in ascending
    slot order), in fp64 on the rows' original values."""
    rows = np.asarray(ref_rows, dtype=np.float64)
    s = rows[0].copy()
    for m in range(1, rows.shape[0]):
        s = s + rows[m]
    return s / rows.shape[0]


def residual(x: np.ndarray, mean64: np.ndarray) -> np.ndarray:
    """z = KV_i - KV_R in fp64 (compressor = identity)."""
    return np.asarray(x, dtype=np.float64) - np.asarray(mean64, dtype=np.float64)


def quantize_residual(z: np.ndarray, bits: int, group: int):
    """Symmetric absmax group quantisation of one residual row (fp64).

    For each run of ``group`` contiguous elements: a = max |z|, the scale is
    the fp16 nearest to a / qmax (qmax = 2^(bits-1) - 1), and each code is
    the integer nearest to z / scale (ties to even) clamped to [-qmax, qmax];
    a zero scale gives zero codes.  Returns (scales fp16 [d/group],
    codes int64 [d]).
    """
    qmax = (1 << (bits - 1)) - 1
    zg = np.asarray(z, dtype=np.float64).reshape(-1, group)
    a = np.abs(zg).max(axis=1)
    scale = fp16_scale(a / qmax)
    s64 = scale.astype(np.float64)
    codes = np.zeros_like(zg)
    nz = s64 > 0
    codes[nz] = np.rint(zg[nz] / s64[nz, None])
    codes = np.clip(codes, -qmax, qmax)
    return scale, codes.reshape(-1).astype(np.int64)


def quantize_refs(K, V, T, group, bits=4):
    """Full-pipeline quantisation of the reference store ([P1] "Impact and
    Future Directions" and "Improvements for AI systems": 4-bit applied to
    the uncompressed components as well).  Every reference row of K and V is
    quantised like a residual row (quantize_residual).  Returns a dict:
      scales  fp16 [2, |T|, d/group]
      codes   int64 [2, |T|, d]
      deq     fp32 [2, |T|, d]   code * scale (exact in fp32: a 4-bit
                                 integer times an fp16 value)
    """
    out = {"scales": [], "codes": [], "deq": []}
    for X in (K, V):
        sc_p, c_p, d_p = [], [], []
        for pos in T:
            sc, c = quantize_residual(np.asarray(X[pos], dtype=np.float64), bits, group)
            deq = c.astype(np.float64) * np.repeat(sc.astype(np.float64), group)
            sc_p.append(sc)
            c_p.append(c)
            d_p.append(deq.astype(np.float32))
        out["scales"].append(np.stack(sc_p))
        out["codes"].append(np.stack(c_p))
        out["deq"].append(np.stack(d_p))
    return {key: np.stack(v) for key, v in out.items()}


# ---------------------------------------------------------------------------
# Latent variant ([P1] "DeltaKV Framework Architecture": the residual is taken
# between compressed projections, z = f_c(KV) - f_c(KV_R), and decoded by f_d;
# [P1] "Improvements for AI systems": f_c and f_d are a compressor /
# decompressor pair).  Untrained stand-in: a fixed, seeded sign flip D
# followed by the Walsh-Hadamard transform H (H[i][t] = (-1)^popcount(i&t)):
#     f_c(x) = H D x / 16,     f_d(y) = D H y / 8,     f_d(f_c(x)) = x
# (H H = 128 I, D D = I; both scalings are powers of two).  f_c is linear, so
# z = f_c(KV - KV_R) is the rotated residual; it is quantised as usual.  Both
# maps are taken here as fp64 matrix products.
# ---------------------------------------------------------------------------

_M64 = (1 << 64) - 1


def splitmix64(seed: int, n: int):
    """First n outputs of SplitMix64 (Steele, Lea and Flood; Vigna's public
    reference): the state advances by 0x9E3779B97F4A7C15 and each output is
    the state mixed by two xor-shift-multiply rounds and a final xor-shift."""
    out, st = [], seed & _M64
    for _ in range(n):
        st = (st + 0x9E3779B97F4A7C15) & _M64
        z = st
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        out.append(z ^ (z >> 31))
    return out


def latent_signs(seed: int, d: int = 128) -> np.ndarray:
    """D: sign of dim t is -1 when the top bit of the t-th SplitMix64 output
    is set, else +1."""
    return np.array([-1.0 if (x >> 63) else 1.0 for x in splitmix64(seed, d)], dtype=np.float32)


def latent_fc64(z, signs) -> np.ndarray:
    """f_c in fp64: H D z / 16 (a matrix product with the Hadamard matrix)."""
    z = np.asarray(z, dtype=np.float64)
    return (hadamard(z.shape[-1]) @ (z * signs.astype(np.float64))) / 16.0


def latent_fd64(y, signs) -> np.ndarray:
    """f_d in fp64: D H y / 8."""
    y = np.asarray(y, dtype=np.float64)
    n = y.shape[-1]
    Hm = hadamard(n)
    return (y @ Hm.T) * signs.astype(np.float64) / 8.0


def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix, entries (-1)^popcount(i & t), fp64."""
    i = np.arange(n)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def encode(K, V, base, double_after, k, bits, group, rows=None, ref_bits=0, latent_seed=None):
    """Encode one (instance, KV head).

    K, V: [N, d] arrays holding the input values (bf16 inputs widened to
    fp32 exactly).  Returns a dict with, for the requested rows (all by
    default):
      rows      int64 [R]
      idx       uint16 [R, k]   ascending reference slots, 0xFFFF padding
      k_eff     int64 [R]
      mean      fp64 [R, 2, d]  KV_R for K and V
      delta     fp64 [R, 2, d]  residual KV_i - KV_R
      z         fp64 [R, 2, d]  the quantised quantity: delta, or
                                f_c(delta) in latent mode     (bits > 0)
      scales    fp16 [R, 2, d/group]                          (bits > 0)
      codes     int64 [R, 2, d]                               (bits > 0)
    plus ``T`` (reference positions), and with ref_bits = 4 ``ref_q`` (the
    quantised reference store of quantize_refs), whose dequantised rows
    then stand in for the references in the means.  With latent_seed set
    (bits > 0) ``signs`` holds D.  With bits == 0 the residual itself is
    the stored record.
    """
    K = np.asarray(K, dtype=np.float32)
    V = np.asarray(V, dtype=np.float32)
    n, d = K.shape
    T = ref_positions(n, base, double_after)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = bf16_round(K)
    ref_q = quantize_refs(K, V, T, group) if ref_bits == 4 else None
    R = rows.shape[0]
    out = {
        "T": T, "rows": rows,
        "idx": np.full((R, k), IDX_PAD, dtype=np.uint16),
        "k_eff": np.zeros(R, dtype=np.int64),
        "mean": np.zeros((R, 2, d), dtype=np.float64),
        "delta": np.zeros((R, 2, d), dtype=np.float64),
    }
    if ref_q is not None:
        out["ref_q"] = ref_q
    signs = None
    if latent_seed is not None:
        assert bits > 0
        signs = latent_signs(latent_seed, d)
        out["signs"] = signs
    if bits > 0:
        out["z"] = np.zeros((R, 2, d), dtype=np.float64)
        out["scales"] = np.zeros((R, 2, d // group), dtype=np.float16)
        out["codes"] = np.zeros((R, 2, d), dtype=np.int64)
    for r, i in enumerate(rows):
        c = candidate_count(int(i), T)
        dist = distances(keys[i], keys[T[:c]])
        sel = select_topk(dist, k)
        out["idx"][r, :sel.shape[0]] = sel
        out["k_eff"][r] = sel.shape[0]
        pos = T[sel]
        for p, X in enumerate((K, V)):
            m = ref_mean(ref_q["deq"][p][sel] if ref_q is not None else X[pos])
            z = residual(X[i], m)
            out["mean"][r, p] = m
            out["delta"][r, p] = z
            if bits > 0:
                zq = latent_fc64(z, signs) if signs is not None else z
                s, q = quantize_residual(zq, bits, group)
                out["z"][r, p] = zq
                out["scales"][r, p] = s
                out["codes"][r, p] = q
    return out


# ---------------------------------------------------------------------------
# Storage formats of the compressed cache
# ---------------------------------------------------------------------------

def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Token-major packing of one row of codes: element t occupies bits
    [t*bits, (t+1)*bits) of the row's little-endian bit string, as a
    two's-complement field.  Returns uint8 [d*bits/8]."""
    c = np.asarray(codes, dtype=np.int64)
    field = c & ((1 << bits) - 1)
    nbytes = c.shape[0] * bits // 8
    out = np.zeros(nbytes, dtype=np.uint8)
    for t, f in enumerate(field):
        bit = t * bits
        out[bit // 8] |= np.uint8((int(f) << (bit % 8)) & 0xFF)
    return out


def pack_v_tile(codes_tile: np.ndarray, bits: int) -> np.ndarray:
    """Transposed packing of a tile of V codes: codes_tile is int [32, d]
    (tokens x dims; missing tokens are zero).  For each dim t the 32 codes of
    the tile form one little-endian bit string, token u at bits
    [u*bits, (u+1)*bits).  Returns uint8 [d, 32*bits/8]."""
    ct = np.asarray(codes_tile, dtype=np.int64)
    return np.stack([pack_codes(ct[:, t], bits) for t in range(ct.shape[1])])


def ref_store(K, V, T) -> np.ndarray:
    """The uncompressed reference tokens: [2, |T|, d] (K plane, V plane)."""
    return np.stack([np.asarray(K)[T], np.asarray(V)[T]])


# ---------------------------------------------------------------------------
# Reconstruction and decode attention ([P1] "DeltaKV Framework
# Architecture", reconstruction; [P3] on-the-fly reconstruction)
# ---------------------------------------------------------------------------

def reconstruct(enc, K, V, bits):
    """KV^_i for the encoded rows, fp64 [R, 2, d].

    Reference positions come back as stored: raw, or dequantised when the
    reference store is quantised (enc has ``ref_q``).  Every other position
    is KV_R plus the dequantised residual: scale * code (through f_d in
    latent mode) for bits > 0, the residual itself for bits == 0.
    """
    T = enc["T"]
    is_ref = np.isin(enc["rows"], T)
    out = enc["mean"].copy()
    if bits > 0:
        g = enc["codes"].shape[-1] // enc["scales"].shape[-1]
        sc = np.repeat(enc["scales"].astype(np.float64), g, axis=-1)
        y = sc * enc["codes"].astype(np.float64)
        out += latent_fd64(y, enc["signs"]) if "signs" in enc else y
    else:
        out += enc["delta"]
    if "ref_q" in enc:
        slot = np.searchsorted(T, enc["rows"])
        deq = enc["ref_q"]["deq"].astype(np.float64)
        raw = np.stack([deq[0][np.minimum(slot, T.shape[0] - 1)],
                        deq[1][np.minimum(slot, T.shape[0] - 1)]], axis=1)
    else:
        raw = np.stack([np.asarray(K, np.float64)[enc["rows"]],
                        np.asarray(V, np.float64)[enc["rows"]]], axis=1)
    out[is_ref] = raw[is_ref]
    return out


def decode_attn(q, k_hat, v_hat, scale):
    """Single-query attention over a reconstructed cache, fp64.

    q: [Hq, d]; k_hat, v_hat: [Hkv, N, d].  Query head h reads KV head
    h // (Hq / Hkv).  logits = scale * q . k, softmax over all N positions,
    output = sum_i p_i v_i.  Returns [Hq, d].
    """
    q = np.asarray(q, dtype=np.float64)
    hq = q.shape[0]
    hkv = k_hat.shape[0]
    grp = hq // hkv
    out = np.zeros((hq, q.shape[1]), dtype=np.float64)
    for h in range(hq):
        kh = k_hat[h // grp]
        logits = scale * (kh @ q[h])
        m = logits.max()
        w = np.exp(logits - m)
        p = w / w.sum()
        out[h] = p @ v_hat[h // grp]
    return out


# ---------------------------------------------------------------------------
# Selective decompression ([P1] "Training and Inference Integration": only
# the KV pairs the sparse attention mask needs are rebuilt)
# ---------------------------------------------------------------------------

def tile_positions(tiles, n: int, tile: int = 32) -> np.ndarray:
    """Sorted positions covered by a block-sparse selection: tile t covers
    positions [t*tile, (t+1)*tile) below n; entries outside
    [0, ceil(n/tile)) select nothing.  Attention under the selection is
    decode_attn over k_hat[:, positions], v_hat[:, positions]."""
    n_tiles = -(-n // tile)
    pos = []
    for t in sorted(set(int(x) for x in tiles)):
        if 0 <= t < n_tiles:
            pos.extend(range(t * tile, min((t + 1) * tile, n)))
    return np.array(pos, dtype=np.int64)
