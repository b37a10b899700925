"""Sparse attention at large decode batches: the launches with at least 512
(query, 16-head group) pairs, which the library runs with 4-wave workgroups
of 32 heads (two MFMA column blocks per wave) when H is a multiple of 32, and
of 16 heads otherwise.  Compared with the oracle row by row
(max |o - o_ref| / max |o_ref| <= 2e-3, lse within 2e-3), including the
softmax and number-format edge cases of test_gpu_attn_edges."""
import math

import numpy as np
import pytest
import torch

from gpu_util import dev, host, row_rel_err
from test_gpu_attn_edges import build_decode_case, check, upload_cache

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128.0)


def say(msg):
    print(f"[attn-large-batch] {msg}", flush=True)


@pytest.mark.parametrize("B,cap,H,topk", [(160, 2048, 64, 512), (80, 1024, 128, 100),
                                          (128, 4096, 64, 2048), (176, 1024, 48, 512),
                                          (136, 512, 32, 300)])
def test_attn_large_batch_decode(gpu, oracle_mod, B, cap, H, topk):
    say(f"decode B={B} cap={cap} H={H} topk={topk}")
    g = np.random.default_rng(9300 + B)
    k = g.standard_normal((B * cap, 128)).astype(np.float32)
    v = g.standard_normal((B * cap, 128)).astype(np.float32)
    codes, scales = oracle_mod.quant_fp4(k, v)
    codes, scales = codes.reshape(B, cap, 128), scales.reshape(B, cap, 16)
    sk, sks = oracle_mod.quant_fp8_rows(g.standard_normal((B, 128, 128)).astype(np.float32))
    sv, svs = oracle_mod.quant_fp8_rows(g.standard_normal((B, 128, 128)).astype(np.float32))
    idx = np.full((B, topk), -1, np.int32)
    n_sel = g.integers(0, topk + 1, B)
    n_sel[:4] = [topk, topk - 1, 1, 0]
    for b in range(B):
        idx[b, :n_sel[b]] = np.sort(g.choice(cap, n_sel[b], replace=False))
    sl = g.integers(0, 129, B).astype(np.int32)
    sl[:4] = [128, 0, 1, 0]
    q = g.standard_normal((B, H, 128)).astype(np.float32)
    ref_out, ref_lse = oracle_mod.attn_decode_batch(q, codes, scales, idx, sk, sv, sks, svs, sl, SM)
    cache = gpu.Cache(B, cap)
    cache.kv_codes.copy_(dev(codes.reshape(-1, 128)))
    cache.kv_scales.copy_(dev(scales.reshape(-1, 16)))
    out = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    gpu.sparse_attn_decode(dev(q), cache, dev(idx), dev(sk), dev(sv), dev(sks), dev(svs), dev(sl),
                           out, lse)
    o, l = host(out), host(lse)
    empty = (n_sel == 0) & (sl == 0)
    assert np.all(o[empty] == 0) and np.all(np.isneginf(l[empty]))
    err = row_rel_err(o[~empty], ref_out[~empty])
    say(f"max row error {err.max():.2e}")
    assert err.max() <= 2e-3
    np.testing.assert_allclose(l[~empty], ref_lse[~empty], rtol=2e-3, atol=2e-3)


@pytest.mark.parametrize("B,H", [(128, 64), (176, 48)])  # 32-head, then 16-head workgroups
@pytest.mark.parametrize("name", ["peaked_x32", "dominant_global_first_then_later",
                                  "dominant_window", "all_extremes",
                                  "window_sigmas_2^-20_to_2^4"])
def test_attn_large_batch_edges(gpu, oracle_mod, name, B, H):
    say(f"edges {name} B={B} H={H}")
    c = build_decode_case(oracle_mod, name, B=B, cap=1024, H=H, seed=40)
    cache = upload_cache(gpu, c)
    ref_out, ref_lse = oracle_mod.attn_decode_batch(c["q"], c["codes"], c["scales"], c["idx"],
                                                    c["sk"], c["sv"], c["sks"], c["svs"], c["sl"],
                                                    SM)
    out = torch.empty((c["B"], c["H"], 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((c["B"], c["H"]), dtype=torch.float32, device="cuda")
    win = (dev(c["sk"]), dev(c["sv"]), dev(c["sks"]), dev(c["svs"]), dev(c["sl"]))
    gpu.sparse_attn_decode(dev(c["q"]), cache, dev(c["idx"]), *win, out, lse)
    check(out, lse, ref_out, ref_lse, f"large batch {name}")
