"""Seeded prototype-mixture K/V caches and decode queries.

Recipe (one table of prototypes per (layer, KV head), shared by every
sequence of that layer):

* A prototype is a (K, V) pair of independent N(0, I) vectors of length
  head_dim; there are ``n_protos`` of them.
* Every position draws a prototype id i.i.d. uniformly, so tokens sharing a
  prototype are scattered over the whole sequence (long-range similarity).
  K and V of a position use the same id with independent noise.
* Noise is ``sigma * N(0, 1)`` per element.  With ``heavy_frac > 0`` a
  Bernoulli(heavy_frac) draw per position switches that position to
  ``sigma * t_nu`` noise (Student t with ``heavy_nu`` degrees of freedom,
  drawn as Z / sqrt(chi2_nu / nu)).
* With ``drift > 0`` prototypes move as random walks: in drift block b
  (positions [b*drift_block, (b+1)*drift_block)) the table is the initial
  table plus ``drift * sum_{b' <= b, b' >= 1} Z_b'``.
* bf16 workloads round the fp32 draw to bf16 with round-to-nearest-even.
* A decode query is N(0, 1)/sqrt(head_dim) per element, from its own stream.

Every stream is a ``torch.Generator`` seeded from a hash of the workload
index, the stream name and the (layer, sequence, head) it belongs to, so the
same call gives the same tensor on a given device type.  CPU and GPU
generators differ; callers that compare the GPU path against the oracle copy
the very tensors the GPU consumed to the host.
"""

import hashlib
import math

import torch

from .configs import Config

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(cfg_or_name) -> torch.dtype:
    name = cfg_or_name.dtype if isinstance(cfg_or_name, Config) else cfg_or_name
    return _DTYPES[name]


def seed_for(*parts) -> int:
    """A stable 63-bit seed from any tuple of ints and strings."""
    h = hashlib.blake2b(repr(("rkv-synth",) + tuple(parts)).encode(),
                        digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(*parts))
    return g


def _prototypes(cfg: Config, layer: int, head: int, device):
    """(P_K, P_V), each [n_protos, head_dim] fp32 (drift-free table)."""
    g = _gen(device, cfg.index, "proto", layer, head)
    pk = torch.randn(cfg.n_protos, cfg.head_dim, generator=g, device=device)
    pv = torch.randn(cfg.n_protos, cfg.head_dim, generator=g, device=device)
    return pk, pv


def _drifted(cfg: Config, base: torch.Tensor, layer: int, head: int,
             which: str, n_blocks: int, device) -> torch.Tensor:
    """[n_blocks, n_protos, head_dim]: the random-walk table per drift block."""
    g = _gen(device, cfg.index, "drift", which, layer, head)
    steps = torch.randn(n_blocks, cfg.n_protos, cfg.head_dim, generator=g,
                        device=device) * cfg.drift
    steps[0].zero_()
    return base.unsqueeze(0) + torch.cumsum(steps, dim=0)


def gen_head_kv(cfg: Config, layer: int, seq: int, head: int, device="cpu",
                seq_len: int = None, return_ids: bool = False):
    """K, V of one (layer, sequence, KV head): two [seq_len, head_dim] tensors
    in the workload dtype (and the positions' prototype ids when
    ``return_ids``)."""
    n = cfg.seq_len if seq_len is None else seq_len
    d = cfg.head_dim
    pk, pv = _prototypes(cfg, layer, head, device)
    g = _gen(device, cfg.index, "tok", layer, seq, head)
    ids = torch.randint(0, cfg.n_protos, (n,), generator=g, device=device)
    nk = torch.randn(n, d, generator=g, device=device)
    nv = torch.randn(n, d, generator=g, device=device)
    if cfg.heavy_frac > 0:
        heavy = torch.rand(n, generator=g, device=device) < cfg.heavy_frac
        nu = cfg.heavy_nu
        for noise in (nk, nv):
            chi2 = torch.randn(n, d, nu, generator=g, device=device).pow(2).sum(-1)
            t = torch.randn(n, d, generator=g, device=device) / torch.sqrt(chi2 / nu)
            noise.copy_(torch.where(heavy[:, None], t, noise))
    if cfg.drift > 0:
        n_blocks = (n + cfg.drift_block - 1) // cfg.drift_block
        blk = torch.arange(n, device=device) // cfg.drift_block
        tk = _drifted(cfg, pk, layer, head, "k", n_blocks, device)
        tv = _drifted(cfg, pv, layer, head, "v", n_blocks, device)
        base_k = tk[blk, ids]
        base_v = tv[blk, ids]
        del tk, tv
    else:
        base_k = pk[ids]
        base_v = pv[ids]
    k = base_k + cfg.sigma * nk
    v = base_v + cfg.sigma * nv
    dt = torch_dtype(cfg)
    if return_ids:
        return k.to(dt), v.to(dt), ids
    return k.to(dt), v.to(dt)


def gen_instance_kv(cfg: Config, layer: int, seq: int, device="cpu",
                    seq_len: int = None, out_k=None, out_v=None):
    """K, V of one instance (layer, sequence): [n_kv_heads, seq_len, head_dim].

    ``out_k``/``out_v`` may be preallocated views to fill in place."""
    n = cfg.seq_len if seq_len is None else seq_len
    dt = torch_dtype(cfg)
    if out_k is None:
        out_k = torch.empty(cfg.n_kv_heads, n, cfg.head_dim, dtype=dt, device=device)
        out_v = torch.empty_like(out_k)
    for h in range(cfg.n_kv_heads):
        k, v = gen_head_kv(cfg, layer, seq, h, device=device, seq_len=n)
        out_k[h].copy_(k)
        out_v[h].copy_(v)
    return out_k, out_v


def gen_queries(cfg: Config, layer: int, seq: int, device="cpu"):
    """Decode queries of one instance: [n_q_heads, head_dim], N(0,1)/sqrt(d)."""
    g = _gen(device, cfg.index, "query", layer, seq)
    q = torch.randn(cfg.n_q_heads, cfg.head_dim, generator=g, device=device)
    q = q / math.sqrt(cfg.head_dim)
    return q.to(torch_dtype(cfg))
