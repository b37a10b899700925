"""csa2_index_full_noalloc (no workspace, the library's fixed scratch) against
csa2_index_full with a caller workspace, on the GPU: bit-identical top-K and
pool rows on two calls in a row, the second with a smaller input."""
import numpy as np
import pytest
import torch

from gpu_util import dev, host

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[noalloc] {msg}", flush=True)


def case(gpu, B, cap, seed):
    from compressed_kv_cache_decode_amd import synth
    gen = synth.device_generator(seed)
    cache = gpu.Cache(B, cap)
    CH = 1 << 18
    for r0 in range(0, B * cap, CH):
        n = min(CH, B * cap - r0)
        gpu.quant_fp8(synth.device_normal(gen, (n, 64)), cache.ik_codes, cache.ik_sigma,
                      layout=gpu.FP8_IDX_TILED,
                      dst_rows=torch.arange(r0, r0 + n, dtype=torch.int64, device="cuda"))
    iq = synth.device_normal(gen, (B, 1, 4, 64))
    iw = torch.rand((B, 1, 4), generator=gen, device="cuda")
    return cache, iq, iw


@pytest.mark.parametrize("B,cap,topk,pool,nvis", [
    (16, 131072, 512, 2048, None),                 # the decode stack's Full layer
    (3, 8192, 100, 200, [8192, 5000, 37]),         # smaller, ragged visibility
])
def test_noalloc_matches_workspace_call(gpu, B, cap, topk, pool, nvis):
    say(f"B={B} cap={cap} topk={topk} pool={pool}")
    cache, iq, iw = case(gpu, B, cap, 500 + B)
    nv = dev(np.array(nvis if nvis else [cap] * B, np.int32).reshape(B, 1))
    tk_ref = torch.full((B, 1, topk), -9, dtype=torch.int32, device="cuda")
    pl_ref = torch.full((B, 1, pool), -9, dtype=torch.int32, device="cuda")
    gpu.index_full(cache, iq, iw, nv, tk_ref, pl_ref, topk=topk, pool_blocks=pool)
    tk = torch.full_like(tk_ref, -7)
    pl = torch.full_like(pl_ref, -7)
    gpu.index_full_noalloc(cache, iq, iw, nv, tk, pl, topk=topk, pool_blocks=pool)
    np.testing.assert_array_equal(host(tk), host(tk_ref))
    np.testing.assert_array_equal(host(pl), host(pl_ref))
    assert (host(tk) >= -1).all() and (host(tk)[:, :, 0] >= 0).all()


def test_noalloc_twice_in_a_row_second_smaller(gpu, oracle_mod):
    """Two calls back to back on one stream, the second over a smaller input:
    the scratch holds the first call's contents when the second starts."""
    big = case(gpu, 8, 65536, 610)
    small = case(gpu, 2, 4096, 611)
    outs = []
    for (cache, iq, iw), topk, pool in ((big, 512, 2048), (small, 64, 128)):
        B = cache.B
        nv = dev(np.full((B, 1), cache.cap - 3, np.int32))
        tk = torch.empty((B, 1, topk), dtype=torch.int32, device="cuda")
        pl = torch.empty((B, 1, pool), dtype=torch.int32, device="cuda")
        gpu.index_full_noalloc(cache, iq, iw, nv, tk, pl, topk=topk, pool_blocks=pool)
        outs.append((cache, iq, iw, nv, tk, pl, topk, pool))
    for cache, iq, iw, nv, tk, pl, topk, pool in outs:
        tk_ref = torch.empty_like(tk)
        pl_ref = torch.empty_like(pl)
        gpu.index_full(cache, iq, iw, nv, tk_ref, pl_ref, topk=topk, pool_blocks=pool)
        np.testing.assert_array_equal(host(tk), host(tk_ref))
        np.testing.assert_array_equal(host(pl), host(pl_ref))
    # the smaller call also against the oracle
    cache, iq, iw, nv, tk, pl, topk, pool = outs[1]
    from gpu_util import untile_ik
    ikc = untile_ik(host(cache.ik_codes), cache.B, cache.cap)
    iks = host(cache.ik_sigma).reshape(cache.B, cache.cap)
    tk_o, pl_o = oracle_mod.index_full_batch(ikc, iks, host(iq), host(iw), host(nv), topk, pool)
    np.testing.assert_array_equal(host(tk), tk_o)
    np.testing.assert_array_equal(host(pl), pl_o)
