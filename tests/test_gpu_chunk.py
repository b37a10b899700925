"""GPU parity of the bounded-replay chunk: the last 128 prompt tokens re-run
the decoder over a 128K-entry FP4 cache.  The chunk's 128 new entries are
quantised after RoPE by the library; each of the 128 queries takes its own
top-512 over positions [0, N-128+i] and attends to the chunk's window tokens
[0, i].  The oracle checks sampled queries one by one."""
import math
import time

import numpy as np
import pytest
import torch

from compressed_kv_cache_decode_amd import synth
from gpu_util import dev, host, row_rel_err, untile_ik

pytestmark = pytest.mark.gpu
SM = 1.0 / math.sqrt(128.0)


def say(msg):
    print(f"[gpu-case] {time.strftime('%H:%M:%S')} {msg}", flush=True)


def run_chunk(gpu, oracle_mod, n_ent, Q, H, sample, seed=None):
    wl = synth.WORKLOADS["replay_chunk_128k"]
    inp = synth.chunk_inputs(wl, n_ent=n_ent, Q=Q, H=H, seed=seed)
    B = wl.B
    cap = (n_ent + 63) // 64 * 64
    say(f"chunk: n_ent={n_ent} Q={Q} H={H}: writing caches")
    cache = gpu.Cache(B, cap)
    for b in range(B):
        # prefix entries, then the chunk's Q new entries, all quantised after RoPE
        for lo, hi in ((0, n_ent - Q), (n_ent - Q, n_ent)):
            pos = np.arange(lo, hi)
            rows = cache.rows(b, pos)
            gpu.quant_fp4(dev(inp.k_tok[b, lo:hi]), dev(inp.v_tok[b, lo:hi]), cache.kv_codes,
                          cache.kv_scales, rope_cs=dev(gpu.rope_table(pos)), dst_rows=rows)
        gpu.quant_fp8(dev(inp.idx_k[b]), cache.ik_codes, cache.ik_sigma,
                      layout=gpu.FP8_IDX_TILED, dst_rows=cache.rows(b, np.arange(n_ent)))
    swk = torch.empty((B, Q, 128), dtype=torch.uint8, device="cuda")
    swv = torch.empty_like(swk)
    sks = torch.empty((B, Q), dtype=torch.float32, device="cuda")
    svs = torch.empty_like(sks)
    gpu.quant_fp8(dev(inp.swa_k.reshape(-1, 128)), swk, sks)
    gpu.quant_fp8(dev(inp.swa_v.reshape(-1, 128)), swv, svs)
    n_vis = np.tile(np.arange(n_ent - Q + 1, n_ent + 1, dtype=np.int32), (B, 1))
    tk = torch.empty((B, Q, 512), dtype=torch.int32, device="cuda")
    say("chunk: index_full with Q queries")
    gpu.index_full(cache, dev(inp.iq), dev(inp.iw), dev(n_vis), tk, None, topk=512, pool_blocks=0)
    out = torch.empty((B, Q, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Q, H), dtype=torch.float32, device="cuda")
    say("chunk: attention")
    gpu.sparse_attn_chunk(dev(inp.q), cache, tk, swk, swv, sks, svs, out, lse)
    tk_h, out_h, lse_h = host(tk), host(out), host(lse)
    kvc, kvs = host(cache.kv_codes), host(cache.kv_scales)
    ikc = untile_ik(host(cache.ik_codes), B, cap)

    say("chunk: oracle")
    cs = oracle_mod.rope_table(np.arange(n_ent))
    b = 0
    codes, scales = oracle_mod.quant_fp4(inp.k_tok[b], inp.v_tok[b], 1, cs)
    np.testing.assert_array_equal(kvc[:n_ent], codes)
    np.testing.assert_array_equal(kvs[:n_ent], scales)
    ik_ref, iks_ref = oracle_mod.quant_fp8_rows(inp.idx_k[b])
    np.testing.assert_array_equal(ikc[b, :n_ent], ik_ref)
    sk, sks_r = oracle_mod.quant_fp8_rows(inp.swa_k[b])
    sv, svs_r = oracle_mod.quant_fp8_rows(inp.swa_v[b])
    for i in sample:
        ref_tk, _ = oracle_mod.index_full(ik_ref, iks_ref, n_ent - Q + i + 1, inp.iq[b, i],
                                          inp.iw[b, i], 512, 0)
        np.testing.assert_array_equal(tk_h[b, i], ref_tk, err_msg=f"query {i}")
        o, l = oracle_mod.attn(inp.q[b, i], codes, scales, ref_tk, sk, sv, sks_r, svs_r, i + 1, SM)
        assert row_rel_err(out_h[b, i], o).max() <= 2e-3, i
        np.testing.assert_allclose(lse_h[b, i], l, rtol=2e-3, atol=2e-3)


def test_chunk_small(gpu, oracle_mod):
    run_chunk(gpu, oracle_mod, n_ent=3000, Q=128, H=16, sample=range(128), seed=9)


def test_chunk_128k_full_size(gpu, oracle_mod):
    run_chunk(gpu, oracle_mod, n_ent=131072, Q=128, H=64, sample=[0, 1, 2, 63, 100, 127])


def run_chunk_stack(gpu, oracle_mod, n_ent, Q, H, layers, sample, B=1):
    """A replay chunk through a layer stack: the chunk's entries, indexer keys
    and every layer's window written in one call, then per layer the Full /
    Reindex selection of each chunk token (per-token pools) and the chunk
    attention; sampled tokens are checked against the oracle layer by layer
    (indices and pools bit for bit)."""
    from compressed_kv_cache_decode_amd.stack import ChunkStack
    wl = synth.WORKLOADS["replay_stack_128k"]
    inp = synth.chunk_stack_inputs(wl, n_ent=n_ent, Q=Q, H=H, B=B, layers=layers)
    plan = inp.plan
    L = len(plan)
    cap = (n_ent + 63) // 64 * 64
    say(f"chunk stack: n_ent={n_ent} Q={Q} H={H} plan={plan}: writing caches")
    cache = gpu.Cache(B, cap)
    swk = torch.empty((L, B, Q, 128), dtype=torch.uint8, device="cuda")
    swv = torch.empty_like(swk)
    sks = torch.empty((L, B, Q), dtype=torch.float32, device="cuda")
    svs = torch.empty_like(sks)
    for b in range(B):
        pre = np.arange(n_ent - Q)
        gpu.quant_fp4(dev(inp.k_tok[b, :n_ent - Q]), dev(inp.v_tok[b, :n_ent - Q]), cache.kv_codes,
                      cache.kv_scales, rope_cs=dev(gpu.rope_table(pre)), dst_rows=cache.rows(b, pre))
        gpu.quant_fp8(dev(inp.idx_k[b, :n_ent - Q]), cache.ik_codes, cache.ik_sigma,
                      layout=gpu.FP8_IDX_TILED, dst_rows=cache.rows(b, pre))
        rows = cache.rows(b, inp.positions)
        jobs = [dict(x=dev(inp.idx_k[b, n_ent - Q:]), codes=cache.ik_codes, sigma=cache.ik_sigma,
                     layout=gpu.FP8_IDX_TILED, dst_rows=rows)]
        if b == 0:   # every layer's window of every sequence, in the same launch
            jobs += [dict(x=dev(inp.swa_k.reshape(-1, 128)), codes=swk, sigma=sks),
                     dict(x=dev(inp.swa_v.reshape(-1, 128)), codes=swv, sigma=svs)]
        gpu.write_entries(dev(inp.k_tok[b, n_ent - Q:]), dev(inp.v_tok[b, n_ent - Q:]),
                          cache.kv_codes, cache.kv_scales, rope_cs=dev(gpu.rope_table(inp.positions)),
                          dst_rows=rows, fp8_jobs=jobs)
    st = ChunkStack(cache, plan, B, Q, H, topk=512, pool_blocks=2048)
    n_vis = np.tile(np.arange(n_ent - Q + 1, n_ent + 1, dtype=np.int32), (B, 1))
    say("chunk stack: step")
    used = st.step(dev(inp.iq), dev(inp.iw), dev(n_vis), dev(inp.q), swk, swv, sks, svs)
    torch.cuda.synchronize()
    for layer, src in enumerate(st.sources):
        assert used[layer].data_ptr() == used[src].data_ptr()
    tk_all = [host(t) for t in used]
    pool_h = host(st.pool)
    out_h, lse_h = host(st.out), host(st.lse)
    kvc, kvs = host(cache.kv_codes), host(cache.kv_scales)
    ikc = untile_ik(host(cache.ik_codes), B, cap)
    for b in range(B):
        say(f"chunk stack: oracle, sequence {b}")
        codes, scales = oracle_mod.quant_fp4(inp.k_tok[b], inp.v_tok[b], 1,
                                             oracle_mod.rope_table(np.arange(n_ent)))
        np.testing.assert_array_equal(kvc[b * cap:b * cap + n_ent], codes)
        np.testing.assert_array_equal(kvs[b * cap:b * cap + n_ent], scales)
        ik_ref, iks_ref = oracle_mod.quant_fp8_rows(inp.idx_k[b])
        np.testing.assert_array_equal(ikc[b, :n_ent], ik_ref)
        wins = [(oracle_mod.quant_fp8_rows(inp.swa_k[layer, b]),
                 oracle_mod.quant_fp8_rows(inp.swa_v[layer, b])) for layer in range(L)]
        for i in sample:
            nv = n_ent - Q + i + 1
            cur, pool, k = None, None, 0
            for layer, mode in enumerate(plan):
                if mode == "F":
                    cur, pool = oracle_mod.index_full(ik_ref, iks_ref, nv, inp.iq[k, b, i],
                                                      inp.iw[k, b, i], 512, 2048)
                    np.testing.assert_array_equal(pool_h[b, i], pool, err_msg=f"pool, token {i}")
                    k += 1
                elif mode == "X":
                    cur = oracle_mod.index_reindex(ik_ref, iks_ref, nv, inp.iq[k, b, i],
                                                   inp.iw[k, b, i], pool, 512)
                    k += 1
                np.testing.assert_array_equal(tk_all[layer][b, i], cur,
                                              err_msg=f"layer {layer} ({mode}), token {i}")
                (sk, sks_r), (sv, svs_r) = wins[layer]
                lo = max(0, i - 127)  # the window: the last 128 chunk tokens up to i
                o, l = oracle_mod.attn(inp.q[layer, b, i], codes, scales, cur, sk[lo:], sv[lo:],
                                       sks_r[lo:], svs_r[lo:], i + 1 - lo, SM)
                assert row_rel_err(out_h[layer, b, i], o).max() <= 2e-3, (layer, i)
                np.testing.assert_allclose(lse_h[layer, b, i], l, rtol=2e-3, atol=2e-3)


def test_chunk_stack_small(gpu, oracle_mod):
    # 2500 blocks: more than the pool's 2048, so each token's pool is a real choice
    run_chunk_stack(gpu, oracle_mod, n_ent=20000, Q=16, H=16, layers=8, sample=range(16), B=2)


def test_chunk_stack_128k_full_size(gpu, oracle_mod):
    run_chunk_stack(gpu, oracle_mod, n_ent=131072, Q=128, H=64, layers=20, sample=[0, 77, 127])


def test_chunk_stack_longer_than_the_window(gpu, oracle_mod):
    """A replay chunk of 300 tokens (the exact replay of several windows):
    tokens past the 128th attend to the last 128 chunk tokens up to themselves."""
    run_chunk_stack(gpu, oracle_mod, n_ent=20000, Q=300, H=16, layers=6,
                    sample=[0, 127, 128, 129, 250, 299], B=1)
