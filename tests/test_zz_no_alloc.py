"""The allocation-free decode entry point against rkv_decode_attn.

rkv_decode_attn_noalloc takes its workspace from the library's fixed device
scratch.  Two calls in a row (the second on a smaller cache, so the scratch
still holds the first call's data) must each give exactly what
rkv_decode_attn gives with a caller workspace, and meet the attention bar
against the oracle.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from rkv_testlib import attn_err, to_np_f32
from synth import gen_head_kv, gen_queries, get_config

pytestmark = pytest.mark.gpu

if gpu_available():
    import long_context_attention_rkv_amd as rkv


def _case(n_inst, H, Hq, N, seed_layer):
    cfg = dataclasses.replace(get_config(1), n_kv_heads=H, n_q_heads=Hq)
    K = torch.empty(n_inst, H, N, 128, dtype=torch.bfloat16, device="cuda")
    V = torch.empty_like(K)
    for i in range(n_inst):
        for h in range(H):
            k, v = gen_head_kv(cfg, seed_layer + i, 0, h, device="cuda", seq_len=N)
            K[i, h].copy_(k)
            V[i, h].copy_(v)
    q = torch.stack([gen_queries(cfg, seed_layer + i, 0, device="cuda")
                     for i in range(n_inst)]).contiguous()
    cache = rkv.Cache(n_inst, H, N, "bf16", cfg.stride_base, cfg.k, 4, cfg.group)
    rkv.rkv_encode(K, V, cache)
    return cfg, K, V, q, cache


def test_noalloc_decode_equals_decode_with_workspace():
    if not gpu_available():
        pytest.skip("no GPU")
    scale = 1.0 / math.sqrt(128)
    # the second call is smaller: fewer instances, heads and positions
    for n_inst, H, Hq, N, n_split in ((3, 4, 16, 3000, 7), (1, 2, 8, 700, 3)):
        print(f"[noalloc] inst={n_inst} H={H} Hq={Hq} N={N} n_split={n_split}", flush=True)
        cfg, K, V, q, cache = _case(n_inst, H, Hq, N, seed_layer=10 * n_inst)
        want_ws = rkv.rkv_decode_attn(q, Hq, cache, scale, n_split=n_split)
        got = torch.full_like(want_ws, float("nan"))
        rkv.rkv_decode_attn_noalloc(q, Hq, cache, scale, got, n_split=n_split)
        torch.cuda.synchronize()
        assert torch.equal(got, want_ws)
        # and the oracle's attention bar on the first instance
        Kn, Vn, qn = to_np_f32(K[0]), to_np_f32(V[0]), to_np_f32(q[0])
        kh, vh = [], []
        for h in range(H):
            enc = oracle.encode(Kn[h], Vn[h], cfg.stride_base, 0, cfg.k, 4, cfg.group)
            kv = oracle.reconstruct(enc, Kn[h], Vn[h], 4)
            kh.append(kv[:, 0])
            vh.append(kv[:, 1])
        want = oracle.decode_attn(qn, np.stack(kh), np.stack(vh), scale)
        err = attn_err(got[0].cpu().numpy(), want)
        print(f"  worst per-head rel L2 = {err:.2e}", flush=True)
        assert err <= 2e-3
