"""Statistics of the seeded prototype-mixture generator (synth/).

A token is a prototype (a pair of independent N(0, I) vectors) plus
sigma * N(0, 1) noise per element, so for two tokens i, j
  E |K_i - K_j|^2 = 2 sigma^2 d          (same prototype)
  E |K_i - K_j|^2 = 2 (1 + sigma^2) d    (different prototypes)
and a decode query is N(0, 1)/sqrt(d) per element (variance 1/d).
"""

import dataclasses

import numpy as np
import torch

from synth import gen_head_kv, gen_queries, get_config


def _same_pairs(ids):
    """Every pair (a < b) of positions that drew the same prototype."""
    order = np.argsort(ids, kind="stable")
    a, b = [], []
    start = 0
    for end in range(1, len(order) + 1):
        if end == len(order) or ids[order[end]] != ids[order[start]]:
            grp = order[start:end]
            ia, ib = np.triu_indices(len(grp), 1)
            a.append(grp[ia])
            b.append(grp[ib])
            start = end
    return np.concatenate(a), np.concatenate(b)


def _diff_pairs(ids, n, rng):
    a = rng.integers(0, len(ids), n)
    b = rng.integers(0, len(ids), n)
    keep = ids[a] != ids[b]
    return a[keep], b[keep]


def test_distance_statistics_same_and_different_prototype():
    cfg = dataclasses.replace(get_config(1), dtype="f32")
    d = cfg.head_dim
    k, v, ids = gen_head_kv(cfg, 0, 0, 0, device="cpu", seq_len=8192, return_ids=True)
    K = k.double().numpy()
    V = v.double().numpy()
    ids = ids.numpy()
    rng = np.random.default_rng(0)
    for X in (K, V):
        a, b = _same_pairs(ids)
        assert len(a) > 30000
        same = ((X[a] - X[b]) ** 2).sum(1).mean()
        assert abs(same / (2 * cfg.sigma ** 2 * d) - 1) < 0.02, same
        a, b = _diff_pairs(ids, 40000, rng)
        diff = ((X[a] - X[b]) ** 2).sum(1).mean()
        assert abs(diff / (2 * (1 + cfg.sigma ** 2) * d) - 1) < 0.03, diff


def test_prototype_ids_are_uniform_and_bf16_rounds_the_draw():
    cfg = get_config(1)
    k, v, ids = gen_head_kv(cfg, 0, 0, 1, device="cpu", seq_len=8192, return_ids=True)
    counts = np.bincount(ids.numpy(), minlength=cfg.n_protos)
    # 16 tokens per prototype on average: chi-square within a wide band
    chi2 = ((counts - 16.0) ** 2 / 16.0).sum()
    assert 0.7 * cfg.n_protos < chi2 < 1.3 * cfg.n_protos
    assert k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16


def test_query_variance():
    cfg = get_config(2)
    q = torch.cat([gen_queries(cfg, layer, 0).float() for layer in range(8)]).numpy()
    assert abs(q.var() * cfg.head_dim - 1) < 0.05
    assert abs(q.mean()) < 0.01
