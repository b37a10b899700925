"""Cross-path and determinism checks on the GPU (no oracle needed): the
multi-query MFMA indexer path against one single-query exact call per query,
the chunk attention against per-query decode attention with the same window,
and identical bytes across reruns and streams."""
import numpy as np
import pytest
import torch

from gpu_util import dev, host, row_rel_err, tile_ik, tile_ik4

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def idx_cache(gpu, oracle_mod, B, cap, seed, fp4):
    g = np.random.default_rng(seed)
    x = g.standard_normal((B, cap, 64)).astype(np.float32)
    cache = gpu.Cache(B, cap, idx_fp4=fp4)
    if fp4:
        kc, ks = oracle_mod.idx4_quant_rows(x)
        cache.ik_codes.copy_(dev(tile_ik4(kc)))
        cache.ik_scales4.copy_(dev(ks.reshape(-1, 4)))
    else:
        kc, ks = oracle_mod.quant_fp8_rows(x)
        cache.ik_codes.copy_(dev(tile_ik(kc)))
        cache.ik_sigma.copy_(dev(ks.reshape(-1)))
    return cache


@pytest.mark.parametrize("fp4", [False, True])
@pytest.mark.parametrize("pool", [0, 2048])
def test_mma_chunk_path_equals_single_query_calls(gpu, oracle_mod, fp4, pool):
    """csa2_index_full with 128 queries of a replay chunk (MFMA bounds, exact
    rescore) gives, query by query, the indices and pools of 128 separate
    single-query calls (the exact scan), at 131072 entries."""
    say(f"cross-path index fp4={fp4} pool={pool}")
    B, Q, cap = 1, 128, 131072
    cache = idx_cache(gpu, oracle_mod, B, cap, 900 + pool, fp4)
    g = np.random.default_rng(901)
    iq = dev(g.standard_normal((B, Q, 4, 64)).astype(np.float32))
    iw = dev(g.random((B, Q, 4)).astype(np.float32))
    nv = dev(np.arange(cap - Q + 1, cap + 1, dtype=np.int32)[None])
    tk = torch.empty((B, Q, 512), dtype=torch.int32, device="cuda")
    pl = torch.empty((B, Q, max(pool, 1)), dtype=torch.int32, device="cuda")
    gpu.index_full(cache, iq, iw, nv, tk, pl if pool else None, topk=512, pool_blocks=pool)
    tk1 = torch.empty((B, 1, 512), dtype=torch.int32, device="cuda")
    pl1 = torch.empty((B, 1, max(pool, 1)), dtype=torch.int32, device="cuda")
    ws = gpu.alloc_workspace(gpu.workspace_size(gpu.OP_INDEX_FULL, B, 1, cap, 512, pool, 0),
                             "cuda")
    for i in range(Q):
        gpu.index_full(cache, iq[:, i:i + 1].contiguous(), iw[:, i:i + 1].contiguous(),
                       nv[:, i:i + 1].contiguous(), tk1, pl1 if pool else None, topk=512,
                       pool_blocks=pool, ws=ws)
        np.testing.assert_array_equal(host(tk1)[0, 0], host(tk)[0, i], err_msg=f"query {i}")
        if pool:
            np.testing.assert_array_equal(host(pl1)[0, 0], host(pl)[0, i], err_msg=f"pool {i}")


def test_chunk_attention_equals_decode_attention(gpu, oracle_mod):
    """Each query of a 200-token chunk against a decode call whose window holds
    the same chunk tokens [max(0, i - 127), i]."""
    say("cross-path attention")
    B, Q, H, cap = 1, 200, 32, 4096
    g = np.random.default_rng(902)
    k = g.standard_normal((cap, 128)).astype(np.float32)
    v = g.standard_normal((cap, 128)).astype(np.float32)
    cache = gpu.Cache(B, cap)
    gpu.quant_fp4(dev(k), dev(v), cache.kv_codes, cache.kv_scales)
    q = dev(g.standard_normal((B, Q, H, 128)).astype(np.float32))
    idx = np.sort(np.stack([g.choice(cap - Q + i + 1, 512, replace=False) for i in range(Q)]),
                  axis=-1).astype(np.int32)[None]
    swk = torch.empty((B, Q, 128), dtype=torch.uint8, device="cuda")
    swv = torch.empty_like(swk)
    sks = torch.empty((B, Q), dtype=torch.float32, device="cuda")
    svs = torch.empty_like(sks)
    gpu.quant_fp8(dev(g.standard_normal((Q, 128)).astype(np.float32)), swk, sks)
    gpu.quant_fp8(dev(g.standard_normal((Q, 128)).astype(np.float32)), swv, svs)
    out = torch.empty((B, Q, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Q, H), dtype=torch.float32, device="cuda")
    gpu.sparse_attn_chunk(q, cache, dev(idx), swk, swv, sks, svs, out, lse)
    out_c, lse_c = host(out), host(lse)
    o1 = torch.empty((1, H, 128), dtype=torch.float32, device="cuda")
    l1 = torch.empty((1, H), dtype=torch.float32, device="cuda")
    for i in (0, 1, 63, 127, 128, 150, 199):
        lo = max(0, i - 127)
        n = i + 1 - lo
        wk = torch.zeros((1, 128, 128), dtype=torch.uint8, device="cuda")
        wv = torch.zeros_like(wk)
        wks = torch.zeros((1, 128), dtype=torch.float32, device="cuda")
        wvs = torch.zeros_like(wks)
        wk[0, :n], wv[0, :n] = swk[0, lo:i + 1], swv[0, lo:i + 1]
        wks[0, :n], wvs[0, :n] = sks[0, lo:i + 1], svs[0, lo:i + 1]
        gpu.sparse_attn_decode(q[:, i].contiguous(), cache, dev(idx[:, i]), wk, wv, wks, wvs,
                               dev(np.array([n], np.int32)), o1, l1)
        assert row_rel_err(host(o1)[0], out_c[0, i]).max() <= 1e-5, i
        np.testing.assert_allclose(host(l1)[0], lse_c[0, i], rtol=1e-5, atol=1e-5)


def test_stack_bytes_identical_across_reruns_and_streams(gpu, oracle_mod):
    """The same decode stack step, three times on each of two streams:
    identical indices, outputs and lse every time."""
    from compressed_kv_cache_decode_amd import synth
    from compressed_kv_cache_decode_amd.stack import DecodeStack
    say("determinism")
    wl = synth.WORKLOADS["decoder_stack_128k"]
    inp = synth.decode_inputs(wl, n_ent=16000, B=2, layers=9)
    cap = 16000
    cache = gpu.Cache(2, cap)
    for b in range(2):
        rows = cache.rows(b, np.arange(cap))
        gpu.quant_fp4(dev(inp.k_tok[b]), dev(inp.v_tok[b]), cache.kv_codes, cache.kv_scales,
                      dst_rows=rows)
        gpu.quant_fp8(dev(inp.idx_k[b]), cache.ik_codes, cache.ik_sigma,
                      layout=gpu.FP8_IDX_TILED, dst_rows=rows)
    wins = []
    for x in (inp.swa_k, inp.swa_v):
        codes = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
        sig = torch.empty(x.shape[:-1], dtype=torch.float32, device="cuda")
        gpu.quant_fp8(dev(x.reshape(-1, 128)), codes, sig)
        wins += [codes, sig]
    st = DecodeStack(cache, wl.plan[:9], 2, wl.H, topk=512, pool_blocks=1024)
    args = (dev(inp.iq[:, :, None]), dev(inp.iw[:, :, None]), dev(np.full((2, 1), cap, np.int32)),
            dev(inp.q), wins[0], wins[2], wins[1], wins[3], dev(inp.swa_len))
    ref = None
    for s in (torch.cuda.Stream(), torch.cuda.Stream()):
        for rep in range(3):
            st.out.zero_()
            st.topk_bufs.fill_(-9)
            torch.cuda.synchronize()
            with torch.cuda.stream(s):
                st.step(*args)
            torch.cuda.synchronize()
            got = (host(st.topk_bufs).copy(), host(st.out).copy(), host(st.lse).copy())
            if ref is None:
                ref = got
            for a, b in zip(got, ref):
                np.testing.assert_array_equal(a, b)
