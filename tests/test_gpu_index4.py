"""GPU parity of the FP4 indexer-key calls against the CPU oracle: the key
quantiser (alone and in the projected write path), the Full-layer scan with
its pool and top-K, Reindex, and a decoder stack over FP4 keys.  Codes,
scales and indices bit-exact; attention rows within 2e-3."""
import math

import numpy as np
import pytest
import torch

from compressed_kv_cache_decode_amd import synth
from gpu_util import dev, host, row_rel_err, tile_ik4, untile_ik4

pytestmark = pytest.mark.gpu
SM = 1.0 / math.sqrt(128.0)


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def make_idx4_cache(gpu, oracle_mod, B, cap, seed, dup_frac=0.0):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((B, cap, 64)) * np.exp2(g.integers(-3, 3, (B, cap, 1)))).astype(np.float32)
    if dup_frac:
        n = int(dup_frac * cap)
        for b in range(B):
            x[b, g.integers(0, cap, n)] = x[b, g.integers(0, cap, n)]
    kc4, ks4 = oracle_mod.idx4_quant_rows(x)
    cache = gpu.Cache(B, cap, idx_fp4=True)
    cache.ik_codes.copy_(dev(tile_ik4(kc4)))
    cache.ik_scales4.copy_(dev(ks4.reshape(-1, 4)))
    return cache, kc4, ks4


def test_quant_idx_fp4_bit_exact(gpu, oracle_mod):
    say("quant_idx_fp4")
    g = np.random.default_rng(60)
    n, cap = 300, 704
    x = (g.standard_normal((n, 64)) * np.exp2(g.integers(-12, 12, (n, 1)))).astype(np.float32)
    x[0] = 0.0
    x[1, 16:32] = -0.0
    x[2, :16] = 1e30  # saturating scale
    rows = (np.arange(n)[::-1] * 2 + 3).astype(np.int64)
    assert rows.max() < cap
    codes = torch.full((cap * 32,), 0x77, dtype=torch.uint8, device="cuda")
    scales = torch.full((cap, 4), 0x66, dtype=torch.uint8, device="cuda")
    gpu.quant_idx_fp4(dev(x), codes, scales, dst_rows=dev(rows))
    cref, sref = oracle_mod.idx4_quant_rows(x)
    got = untile_ik4(host(codes), 1, cap)[0]
    np.testing.assert_array_equal(got[rows], cref)
    np.testing.assert_array_equal(host(scales)[rows], sref)
    untouched = np.setdiff1d(np.arange(cap), rows)
    assert (got[untouched] == 0x77).all() and (host(scales)[untouched] == 0x66).all()


@pytest.mark.parametrize("n_tok,ratio,rope", [(128, 1, True), (10, 2, False)])
def test_write_entries_proj_fp4_bit_exact(gpu, oracle_mod, n_tok, ratio, rope):
    say(f"write_entries_proj_fp4 n_tok={n_tok} ratio={ratio}")
    g = np.random.default_rng(61 + n_tok)
    n_ent = n_tok // ratio
    k = (g.standard_normal((n_tok, 128)) * np.exp2(g.integers(-8, 8, (n_tok, 1)))).astype(np.float32)
    v = g.standard_normal((n_tok, 128)).astype(np.float32)
    W = (g.standard_normal((64, 128)) / np.sqrt(128)).astype(np.float32)
    rows = (np.arange(n_ent)[::-1] + 9).astype(np.int64)
    cap = 64 * ((int(rows.max()) + 1 + 63) // 64)
    assert rows.max() < cap
    pos = np.arange(700, 700 + n_ent)
    cs = oracle_mod.rope_table(pos) if rope else None
    kvc = torch.zeros((cap, 128), dtype=torch.uint8, device="cuda")
    kvs = torch.zeros((cap, 16), dtype=torch.uint8, device="cuda")
    codes = torch.zeros(cap * 32, dtype=torch.uint8, device="cuda")
    scales = torch.zeros((cap, 4), dtype=torch.uint8, device="cuda")
    gpu.write_entries(dev(k), dev(v), kvc, kvs, ratio=ratio,
                      rope_cs=dev(gpu.rope_table(pos)) if rope else None, dst_rows=dev(rows),
                      idx_proj=dev(W), ik_codes=codes, ik_scales4=scales)
    c_ref, s_ref = oracle_mod.quant_fp4(k, v, ratio, cs)
    kc4, ks4 = oracle_mod.idx4_quant_rows(
        oracle_mod.project_idx(oracle_mod.entry_k(k, ratio, cs), W))
    np.testing.assert_array_equal(host(kvc)[rows], c_ref)
    np.testing.assert_array_equal(host(kvs)[rows], s_ref)
    np.testing.assert_array_equal(untile_ik4(host(codes), 1, cap)[0][rows], kc4)
    np.testing.assert_array_equal(host(scales)[rows], ks4)


@pytest.mark.parametrize("B,Q,cap,nvis,topk,pool", [
    (1, 1, 1024, [1024], 512, 0),
    (2, 1, 4096, [4093, 1500], 512, 2048),        # pool larger than the visible blocks
    (3, 1, 8192, [8192, 8000, 13], 64, 128),      # ragged tails, fewer visible than K
    (2, 3, 2048, [[2048, 2047, 1], [0, 999, 1024]], 40, 40),
    (16, 1, 16384, [16384 - 37 * b for b in range(16)], 512, 2048),
    (1, 1, 131072, [131072], 512, 2048),
    (1, 1, 262144, [262141], 512, 2048),          # more than 16384 blocks: streaming blocks
    (1, 1, 65536, [65533], 2048, 4096),           # the largest top-K and pool
    # many queries per sequence: the MFMA bounds path with FP4 keys (guard
    # band for |k| <= 6 x 448), ragged visibility down to none, a capacity
    # that partly fills the last workgroup, more than 128 queries (two
    # staging passes), and pools decided from the bounds
    (1, 130, 8192, [[8192 - 37 * i if i % 5 else (97 * i) % 600 for i in range(130)]], 512, 0),
    (2, 16, 16384, [[0, 1, 5, 300, 511, 512, 513, 4096, 8191, 8192, 12000, 16383, 16384,
                     16384, 7, 9000], [16384 - 1000 * i for i in range(16)]], 512, 0),
    (1, 5, 1088, [[1088, 1087, 1000, 700, 64]], 64, 0),
    (2, 16, 16384, [[0, 1, 5, 300, 511, 512, 513, 4096, 8191, 8192, 12000, 16383, 16384,
                     16384, 7, 9000], [16384 - 1000 * i for i in range(16)]], 512, 2048),
    (1, 8, 131072, [[131072, 131000, 100001, 65536, 20000, 16385, 2048, 9]], 512, 2048),
    (1, 6, 8192, [[8192, 8191, 4000, 1030, 1024, 1017]], 64, 128),
])
def test_index_full_fp4_bit_exact(gpu, oracle_mod, B, Q, cap, nvis, topk, pool):
    say(f"index_full_fp4 B={B} Q={Q} cap={cap} topk={topk} pool={pool}")
    cache, kc4, ks4 = make_idx4_cache(gpu, oracle_mod, B, cap, 600 + cap + B, dup_frac=0.2)
    g = np.random.default_rng(601)
    iq = g.standard_normal((B, Q, 4, 64)).astype(np.float32)
    iw = g.random((B, Q, 4)).astype(np.float32)
    nv = np.array(nvis, np.int32).reshape(B, Q)
    tk_ref, pl_ref = oracle_mod.index_full4_batch(kc4, ks4, iq, iw, nv, topk, pool)
    tk = torch.full((B, Q, topk), -7, dtype=torch.int32, device="cuda")
    pl = torch.full((B, Q, max(pool, 1)), -7, dtype=torch.int32, device="cuda")
    gpu.index_full(cache, dev(iq), dev(iw), dev(nv), tk, pl if pool else None, topk=topk,
                   pool_blocks=pool)
    np.testing.assert_array_equal(host(tk), tk_ref)
    if pool:
        np.testing.assert_array_equal(host(pl), pl_ref)


def test_index_full_fp4_all_ties(gpu, oracle_mod):
    """Every key identical: the lowest positions and blocks win."""
    say("index_full_fp4 all ties")
    B, cap = 1, 8192
    x = np.tile(np.random.default_rng(62).standard_normal(64).astype(np.float32), (B, cap, 1))
    kc4, ks4 = oracle_mod.idx4_quant_rows(x)
    cache = gpu.Cache(B, cap, idx_fp4=True)
    cache.ik_codes.copy_(dev(tile_ik4(kc4)))
    cache.ik_scales4.copy_(dev(ks4.reshape(-1, 4)))
    iq = np.abs(np.random.default_rng(63).standard_normal((B, 1, 4, 64))).astype(np.float32)
    iw = np.ones((B, 1, 4), np.float32)
    nv = np.full((B, 1), 8000, np.int32)
    tk_ref, pl_ref = oracle_mod.index_full4_batch(kc4, ks4, iq, iw, nv, 512, 1024)
    tk = torch.empty((B, 1, 512), dtype=torch.int32, device="cuda")
    pl = torch.empty((B, 1, 1024), dtype=torch.int32, device="cuda")
    gpu.index_full(cache, dev(iq), dev(iw), dev(nv), tk, pl, topk=512, pool_blocks=1024)
    np.testing.assert_array_equal(host(tk), tk_ref)
    np.testing.assert_array_equal(host(pl), pl_ref)
    assert tk_ref[0, 0, 0] == 0 and tk_ref[0, 0, -1] == 511


@pytest.mark.parametrize("B,cap,nvis,pool,topk", [
    (2, 8192, [8192, 5000], 512, 512),
    (3, 32768, [32768, 30001, 9], 2048, 512),
    (1, 65536, [65536], 4096, 2048),
])
def test_index_reindex_fp4_bit_exact(gpu, oracle_mod, B, cap, nvis, pool, topk):
    say(f"index_reindex_fp4 B={B} cap={cap} pool={pool} topk={topk}")
    cache, kc4, ks4 = make_idx4_cache(gpu, oracle_mod, B, cap, 700 + cap, dup_frac=0.1)
    g = np.random.default_rng(701)
    iq0 = g.standard_normal((B, 1, 4, 64)).astype(np.float32)
    iw0 = g.random((B, 1, 4)).astype(np.float32)
    iq = g.standard_normal((B, 1, 4, 64)).astype(np.float32)
    iw = g.random((B, 1, 4)).astype(np.float32)
    nv = np.array(nvis, np.int32).reshape(B, 1)
    _, pl_ref = oracle_mod.index_full4_batch(kc4, ks4, iq0, iw0, nv, min(topk, pool), pool)
    rk_ref = oracle_mod.index_reindex4_batch(kc4, ks4, iq, iw, nv, pl_ref, topk)
    tk = torch.full((B, 1, topk), -7, dtype=torch.int32, device="cuda")
    gpu.index_reindex(cache, dev(iq), dev(iw), dev(nv), dev(pl_ref), tk, topk=topk)
    np.testing.assert_array_equal(host(tk), rk_ref)


def test_decoder_stack_fp4_keys(gpu, oracle_mod):
    """A 9-layer decoder stack (F R R R X R R R X) whose indexer keys are FP4,
    written by the library from the fixture's fp32 keys: indices of every layer
    bit-exact, outputs within 2e-3."""
    from compressed_kv_cache_decode_amd.stack import DecodeStack
    wl = synth.WORKLOADS["decoder_stack_128k"]
    B, n_ent, L = 3, 20000, 9
    inp = synth.decode_inputs(wl, n_ent=n_ent, B=B, layers=L)
    plan = wl.plan[:L]
    cap = (n_ent + 63) // 64 * 64
    say("fp4-key stack: writing the cache")
    cache = gpu.Cache(B, cap, idx_fp4=True)
    for b in range(B):
        rows = cache.rows(b, np.arange(n_ent))
        gpu.quant_fp4(dev(inp.k_tok[b]), dev(inp.v_tok[b]), cache.kv_codes, cache.kv_scales,
                      dst_rows=rows)
        gpu.quant_idx_fp4(dev(inp.idx_k[b]), cache.ik_codes, cache.ik_scales4, dst_rows=rows)
    wins = []
    for x in (inp.swa_k, inp.swa_v):
        codes = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
        sig = torch.empty(x.shape[:-1], dtype=torch.float32, device="cuda")
        gpu.quant_fp8(dev(x.reshape(-1, 128)), codes, sig)
        wins += [codes, sig]
    swk, sks, swv, svs = wins
    st = DecodeStack(cache, plan, B, wl.H, topk=256, pool_blocks=512)
    used = st.step(dev(inp.iq[:, :, None]), dev(inp.iw[:, :, None]),
                   dev(np.full((B, 1), n_ent, np.int32)), dev(inp.q), swk, swv, sks, svs,
                   dev(inp.swa_len))
    torch.cuda.synchronize()
    for b in range(B):
        say(f"fp4-key stack: oracle for sequence {b}")
        codes, scales = oracle_mod.quant_fp4(inp.k_tok[b], inp.v_tok[b], 1, None)
        kc4, ks4 = oracle_mod.idx4_quant_rows(inp.idx_k[b])
        cur, pool, k = None, None, 0
        for layer, mode in enumerate(plan):
            if mode == "F":
                cur, pool = oracle_mod.index_full4(kc4, ks4, n_ent, inp.iq[k, b], inp.iw[k, b],
                                                   256, 512)
                k += 1
            elif mode == "X":
                cur = oracle_mod.index_reindex4(kc4, ks4, n_ent, inp.iq[k, b], inp.iw[k, b],
                                                pool, 256)
                k += 1
            np.testing.assert_array_equal(host(used[layer])[b, 0], cur, err_msg=f"layer {layer}")
            sk, sks_ = oracle_mod.quant_fp8_rows(inp.swa_k[layer, b])
            sv, svs_ = oracle_mod.quant_fp8_rows(inp.swa_v[layer, b])
            o, _ = oracle_mod.attn(inp.q[layer, b], codes, scales, cur, sk, sv, sks_, svs_,
                                   int(inp.swa_len[b]), SM)
            err = row_rel_err(host(st.out)[layer, b], o)
            assert err.max() <= 2e-3, (layer, err.max())


@pytest.mark.parametrize("pool", [0, 1024])
def test_index_full_fp4_chunk_all_ties(gpu, oracle_mod, pool):
    """Many queries over identical FP4 keys: every bound ties, the candidate
    lists overflow, and each query falls back to its exact scan in the same
    workgroup; the lowest positions and blocks win."""
    say(f"index_full_fp4 chunk all ties pool={pool}")
    B, Q, cap = 1, 8, 8192
    x = np.tile(np.random.default_rng(64).standard_normal(64).astype(np.float32), (B, cap, 1))
    kc4, ks4 = oracle_mod.idx4_quant_rows(x)
    cache = gpu.Cache(B, cap, idx_fp4=True)
    cache.ik_codes.copy_(dev(tile_ik4(kc4)))
    cache.ik_scales4.copy_(dev(ks4.reshape(-1, 4)))
    g = np.random.default_rng(65)
    iq = np.abs(g.standard_normal((B, Q, 4, 64))).astype(np.float32)
    iw = g.random((B, Q, 4)).astype(np.float32)
    nv = np.array([[8192, 8000, 5000, 4097, 1024, 600, 100, 0]], np.int32)
    tk_ref, pl_ref = oracle_mod.index_full4_batch(kc4, ks4, iq, iw, nv, 512, pool)
    tk = torch.full((B, Q, 512), -7, dtype=torch.int32, device="cuda")
    pl = torch.full((B, Q, max(pool, 1)), -7, dtype=torch.int32, device="cuda")
    gpu.index_full(cache, dev(iq), dev(iw), dev(nv), tk, pl if pool else None, topk=512,
                   pool_blocks=pool)
    np.testing.assert_array_equal(host(tk), tk_ref)
    if pool:
        np.testing.assert_array_equal(host(pl), pl_ref)
