"""GPU parity of every entry point against the CPU oracle, on the same seeded
inputs, at sizes the oracle finishes in seconds that still span several tiles
and a ragged tail.

Bit-exact: FP4 codes, E4M3 scales, FP8 codes and sigmas, top-K and pool
indices.  Attention: per (query, head) row, max |o - o_ref| / max |o_ref|
<= 2e-3 against the fp64 oracle.
"""
import math

import numpy as np
import pytest
import torch

from gpu_util import dev, host, row_rel_err, tile_ik, untile_ik

pytestmark = pytest.mark.gpu
ATOL_ROW = 2e-3
SM = 1.0 / math.sqrt(128.0)


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


# --------------------------------------------------------------------------- codecs
def test_codec_probe_matches_oracle(gpu, oracle_mod):
    say("codec probe")
    g = np.random.default_rng(100)
    finite = np.array([oracle_mod.e4m3_decode(c) for c in range(0x7F)], np.float32)
    mids = ((finite[1:] + finite[:-1]) / 2).astype(np.float32)
    x = np.concatenate([finite, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        np.exp2(g.uniform(-24, 10, 20000)).astype(np.float32),
                        np.array([0.0, 1e-45, 1e-40, 447.99, 448, 464, 480, 1e30, 0.25, 0.75,
                                  1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0], np.float32)])
    x = np.concatenate([x, -x]).astype(np.float32)
    e4, e4h, fp4, enc4, enc2 = [host(t) for t in gpu.codec_probe(dev(x))]
    for c in range(256):
        ref = oracle_mod.e4m3_decode(c)
        if c & 0x7F == 0x7F:
            continue  # NaN codes are never produced by the encoders
        assert e4[c] == ref, (hex(c), e4[c], ref)
        assert e4h[c] == ref, (hex(c), e4h[c], ref)
        for code in range(16):  # the attention's FP4 path: code x scale, exact
            assert fp4[c, code] == oracle_mod.e2m1_decode(code) * ref, (hex(c), code)
    ref4 = np.array([oracle_mod.e4m3_encode(float(v)) for v in x], np.uint8)
    ref2 = np.array([oracle_mod.e2m1_encode(float(v)) for v in x], np.uint8)
    np.testing.assert_array_equal(enc4, ref4)
    np.testing.assert_array_equal(enc2, ref2)


# --------------------------------------------------------------------------- write path
@pytest.mark.parametrize("ratio,rope,n_tok", [(1, False, 1), (1, False, 203), (1, True, 131),
                                              (2, False, 2), (2, False, 390)])
def test_quant_fp4_bit_exact(gpu, oracle_mod, ratio, rope, n_tok):
    say(f"quant_fp4 ratio={ratio} rope={rope} n_tok={n_tok}")
    g = np.random.default_rng(200 + n_tok)
    k = (g.standard_normal((n_tok, 128)) * np.exp2(g.integers(-10, 10, (n_tok, 1)))).astype(np.float32)
    v = g.standard_normal((n_tok, 128)).astype(np.float32)
    k[0, :16] = 0.0          # a zero group
    k[0, 16] = -0.0
    if n_tok > 1:
        k[1, :] = 1e5        # saturated scale
    n_ent = n_tok // ratio
    cs = oracle_mod.rope_table(np.arange(5000, 5000 + n_ent)) if rope else None
    codes_ref, scales_ref = oracle_mod.quant_fp4(k, v, ratio, cs)
    # the binding's own table must equal the oracle's (both fp64 -> fp32)
    if rope:
        np.testing.assert_array_equal(gpu.rope_table(np.arange(5000, 5000 + n_ent)), cs)
    # scatter into a larger cache through dst_rows (reversed order)
    rows = np.arange(n_ent)[::-1].copy() + 7
    codes = torch.zeros((n_ent + 9, 128), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((n_ent + 9, 16), dtype=torch.uint8, device="cuda")
    gpu.quant_fp4(dev(k), dev(v), codes, scales, ratio=ratio,
                  rope_cs=dev(gpu.rope_table(np.arange(5000, 5000 + n_ent))) if rope else None,
                  dst_rows=dev(rows))
    c, s = host(codes), host(scales)
    np.testing.assert_array_equal(c[rows], codes_ref)
    np.testing.assert_array_equal(s[rows], scales_ref)
    untouched = np.setdiff1d(np.arange(n_ent + 9), rows)
    assert np.all(c[untouched] == 0) and np.all(s[untouched] == 0)


@pytest.mark.parametrize("dim,layout,n", [(128, 0, 1), (128, 0, 300), (64, 0, 77), (64, 1, 320)])
def test_quant_fp8_bit_exact(gpu, oracle_mod, dim, layout, n):
    say(f"quant_fp8 dim={dim} layout={layout} n={n}")
    g = np.random.default_rng(300 + n)
    x = (g.standard_normal((n, dim)) * np.exp2(g.integers(-30, 30, (n, 1)))).astype(np.float32)
    x[0] = 0.0
    x[0, 3] = -0.0
    codes_ref, sig_ref = oracle_mod.quant_fp8_rows(x)
    codes = torch.zeros(n * dim, dtype=torch.uint8, device="cuda")
    sigma = torch.zeros(n, dtype=torch.float32, device="cuda")
    gpu.quant_fp8(dev(x), codes, sigma, layout=layout)
    c = host(codes)
    if layout == 1:
        c = untile_ik(c, 1, n)[0]
    np.testing.assert_array_equal(c.reshape(n, dim), codes_ref)
    np.testing.assert_array_equal(host(sigma), sig_ref)


@pytest.mark.parametrize("n_tok,ratio,rope,n_rows", [(128, 1, True, 128), (16, 1, False, 16),
                                                     (10, 2, False, 3), (0, 1, False, 200)])
def test_write_entries_bit_exact(gpu, oracle_mod, n_tok, ratio, rope, n_rows):
    """One launch writes what quant_fp4 and three quant_fp8 calls write: the
    entries' FP4 records (scattered rows), their tiled indexer keys, and two
    FP8 row sets (window K and V), each equal to the oracle's codes."""
    say(f"write_entries n_tok={n_tok} ratio={ratio} rope={rope} n_rows={n_rows}")
    g = np.random.default_rng(700 + n_tok + n_rows)
    n_ent = n_tok // ratio
    k = (g.standard_normal((n_tok, 128)) * np.exp2(g.integers(-8, 8, (n_tok, 1)))).astype(np.float32)
    v = g.standard_normal((n_tok, 128)).astype(np.float32)
    ik = g.standard_normal((n_rows, 64)).astype(np.float32)
    wk = (g.standard_normal((n_rows, 128)) * 3).astype(np.float32)
    wv = g.standard_normal((n_rows, 128)).astype(np.float32)
    if n_rows:
        wk[0] = 0.0
    cap = 64 * ((max(n_ent, n_rows) + 9 + 63) // 64)
    rows = (np.arange(n_ent)[::-1] + 5).astype(np.int64)
    irows = (np.arange(n_rows)[::-1] + 3).astype(np.int64)
    pos = np.arange(900, 900 + n_ent)
    cs = oracle_mod.rope_table(pos) if rope else None
    codes = torch.zeros((cap, 128), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((cap, 16), dtype=torch.uint8, device="cuda")
    ikc = torch.zeros(cap * 64, dtype=torch.uint8, device="cuda")
    iks = torch.zeros(cap, dtype=torch.float32, device="cuda")
    wkc = torch.zeros((max(n_rows, 1), 128), dtype=torch.uint8, device="cuda")
    wks = torch.zeros(max(n_rows, 1), dtype=torch.float32, device="cuda")
    wvc, wvs = torch.zeros_like(wkc), torch.zeros_like(wks)
    gpu.write_entries(dev(k), dev(v), codes, scales, ratio=ratio,
                      rope_cs=dev(gpu.rope_table(pos)) if rope else None, dst_rows=dev(rows),
                      fp8_jobs=[dict(x=dev(ik), codes=ikc, sigma=iks, layout=gpu.FP8_IDX_TILED,
                                     dst_rows=dev(irows)),
                                dict(x=dev(wk), codes=wkc, sigma=wks),
                                dict(x=dev(wv), codes=wvc, sigma=wvs)])
    if n_ent:
        cref, sref = oracle_mod.quant_fp4(k, v, ratio, cs)
        np.testing.assert_array_equal(host(codes)[rows], cref)
        np.testing.assert_array_equal(host(scales)[rows], sref)
    untouched = np.setdiff1d(np.arange(cap), rows)
    assert np.all(host(codes)[untouched] == 0) and np.all(host(scales)[untouched] == 0)
    if n_rows:
        ic_ref, is_ref = oracle_mod.quant_fp8_rows(ik)
        np.testing.assert_array_equal(untile_ik(host(ikc), 1, cap)[0][irows], ic_ref)
        np.testing.assert_array_equal(host(iks)[irows], is_ref)
        for x, c, sg in ((wk, wkc, wks), (wv, wvc, wvs)):
            c_ref, s_ref = oracle_mod.quant_fp8_rows(x)
            np.testing.assert_array_equal(host(c), c_ref)
            np.testing.assert_array_equal(host(sg), s_ref)


@pytest.mark.parametrize("n_tok,ratio,rope,n_rows", [(128, 1, True, 128), (16, 1, True, 0),
                                                     (21, 1, False, 5), (10, 2, False, 3)])
def test_write_entries_proj_bit_exact(gpu, oracle_mod, n_tok, ratio, rope, n_rows):
    """The write path with the indexer key projected on the device: FP4
    records, the projected keys' FP8 codes and sigmas at the entries' rows
    (tile layout) and the window rows of the FP8 jobs, each equal to the
    oracle's bytes; rows not addressed stay untouched."""
    say(f"write_entries_proj n_tok={n_tok} ratio={ratio} rope={rope} n_rows={n_rows}")
    g = np.random.default_rng(900 + n_tok + n_rows)
    n_ent = n_tok // ratio
    k = (g.standard_normal((n_tok, 128)) * np.exp2(g.integers(-8, 8, (n_tok, 1)))).astype(np.float32)
    v = g.standard_normal((n_tok, 128)).astype(np.float32)
    k[-ratio:] = 0.0  # an all-zero entry: zero key, zero sigma
    W = (g.standard_normal((64, 128)) / np.sqrt(128)).astype(np.float32)
    wk = (g.standard_normal((max(n_rows, 1), 128)) * 3).astype(np.float32)[:n_rows]
    wv = g.standard_normal((max(n_rows, 1), 128)).astype(np.float32)[:n_rows]
    rows = (np.arange(n_ent)[::-1] * 2 + 7).astype(np.int64)
    cap = 64 * ((int(rows.max()) + 1 + 63) // 64)
    assert rows.max() < cap  # every destination row inside the arrays
    pos = np.arange(5000, 5000 + n_ent)
    cs = oracle_mod.rope_table(pos) if rope else None
    codes = torch.zeros((cap, 128), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((cap, 16), dtype=torch.uint8, device="cuda")
    ikc = torch.full((cap * 64,), 0x5A, dtype=torch.uint8, device="cuda")
    iks = torch.full((cap,), -1.0, dtype=torch.float32, device="cuda")
    wkc = torch.zeros((max(n_rows, 1), 128), dtype=torch.uint8, device="cuda")
    wks = torch.zeros(max(n_rows, 1), dtype=torch.float32, device="cuda")
    wvc, wvs = torch.zeros_like(wkc), torch.zeros_like(wks)
    jobs = [dict(x=dev(wk), codes=wkc, sigma=wks), dict(x=dev(wv), codes=wvc, sigma=wvs)]
    gpu.write_entries(dev(k), dev(v), codes, scales, ratio=ratio,
                      rope_cs=dev(gpu.rope_table(pos)) if rope else None, dst_rows=dev(rows),
                      fp8_jobs=jobs if n_rows else (), idx_proj=dev(W), ik_codes=ikc,
                      ik_sigma=iks)
    cref, sref, ikref, isref = oracle_mod.write_entries_proj(k, v, W, ratio, cs)
    np.testing.assert_array_equal(host(codes)[rows], cref)
    np.testing.assert_array_equal(host(scales)[rows], sref)
    ik_rows = untile_ik(host(ikc), 1, cap)[0]
    np.testing.assert_array_equal(ik_rows[rows], ikref)
    np.testing.assert_array_equal(host(iks)[rows], isref)
    assert isref[-1] == 0.0 and not ikref[-1].any()  # the all-zero last entry
    untouched = np.setdiff1d(np.arange(cap), rows)
    assert (ik_rows[untouched] == 0x5A).all() and (host(iks)[untouched] == -1.0).all()
    if n_rows:
        for (xc, xs), x in (((wkc, wks), wk), ((wvc, wvs), wv)):
            c_ref, s_ref = oracle_mod.quant_fp8_rows(x)
            np.testing.assert_array_equal(host(xc), c_ref)
            np.testing.assert_array_equal(host(xs), s_ref)


# --------------------------------------------------------------------------- indexer
def make_idx_cache(gpu, oracle_mod, B, cap, seed, dup_frac=0.0):
    g = np.random.default_rng(seed)
    x = g.standard_normal((B, cap, 64)).astype(np.float32)
    if dup_frac:
        n = int(dup_frac * cap)
        for b in range(B):
            x[b, g.integers(0, cap, n)] = x[b, g.integers(0, cap, n)]
    ikc, iks = oracle_mod.quant_fp8_rows(x)
    cache = gpu.Cache(B, cap)
    cache.ik_codes.copy_(dev(tile_ik(ikc)))
    cache.ik_sigma.copy_(dev(iks.reshape(-1)))
    return cache, ikc, iks


@pytest.mark.parametrize("B,Q,cap,nvis,topk,pool", [
    (1, 1, 1024, [1024], 512, 0),                 # the 1K single Full layer
    (2, 1, 4096, [4093, 1500], 512, 2048),        # pool larger than the visible blocks
    (3, 1, 8192, [8192, 8000, 13], 64, 128),      # ragged tails, fewer visible than K
    (2, 3, 2048, [[2048, 2047, 1], [0, 999, 1024]], 40, 40),
    (1, 1, 32768, [32765], 512, 2048),            # more blocks than the pool
    (4, 1, 16384, [16384, 16384, 16000, 8], 512, 0),
    # many queries per sequence (the multi-query scan), ragged visible counts
    (2, 37, 4096, [[4096 - 13 * i for i in range(37)], [1 + 97 * i for i in range(37)]], 64, 0),
    # multi-query Full layers without a pool take the MFMA guard-band path:
    # two staging passes of queries (130 > 128), queries seeing fewer than K
    # positions (down to none), duplicated key rows (ties)
    (1, 130, 8192, [[8192 - 37 * i if i % 5 else (97 * i) % 600 for i in range(130)]], 512, 0),
    (2, 16, 16384, [[0, 1, 5, 300, 511, 512, 513, 4096, 8191, 8192, 12000, 16383, 16384,
                     16384, 7, 9000], [16384 - 1000 * i for i in range(16)]], 512, 0),
    (1, 4, 1024, [[1024, 1024, 1000, 3]], 2048, 0),   # top-K larger than what is visible
    # a capacity that is not a multiple of 256: the scans' last workgroup is
    # partly past it (MFMA path with Q = 5, single-query scan with Q = 1)
    (1, 5, 1088, [[1088, 1087, 1000, 700, 64]], 64, 0),
    (2, 1, 1088, [1088, 1025], 64, 128),
    # top-K above 1024 takes the exact multi-query scan; at 1024 the MFMA
    # path's largest candidate list (3072 half-blocks, 12288 keys in LDS); more
    # than 16384 blocks: the candidate threshold streams
    (1, 5, 65536, [[65536, 65000, 40000, 20000, 9]], 2048, 0),
    (1, 5, 65536, [[65536, 65000, 40000, 20000, 9]], 1024, 0),
    (1, 4, 262144, [[262144, 262000, 131073, 70000]], 512, 0),
    # the largest top-K and pool the boundary accepts; 32768 pool positions take
    # the streaming selection path
    (1, 1, 65536, [65533], 2048, 4096),
    # more than 16384 blocks: the block selection streams too
    (1, 1, 262144, [262141], 512, 2048),
    # multi-query Full layers with a pool on the MFMA path (at most 16384
    # blocks): pools larger than the visible blocks, queries seeing nothing,
    # ragged tails, the full 16384 blocks, the largest pool and top-K, and a
    # small pool (P + 1 = 129 upper bounds) under duplicated keys
    (2, 16, 16384, [[0, 1, 5, 300, 511, 512, 513, 4096, 8191, 8192, 12000, 16383, 16384,
                     16384, 7, 9000], [16384 - 1000 * i for i in range(16)]], 512, 2048),
    (1, 8, 131072, [[131072, 131000, 100001, 65536, 20000, 16385, 2048, 9]], 512, 2048),
    (1, 5, 65536, [[65536, 65000, 40000, 20000, 9]], 1024, 4096),
    (1, 6, 8192, [[8192, 8191, 4000, 1030, 1024, 1017]], 64, 128),
    # more than 16384 blocks with a pool: the exact multi-query scan
    (1, 4, 262144, [[262144, 200000, 131080, 5]], 512, 2048),
])
def test_index_full_bit_exact(gpu, oracle_mod, B, Q, cap, nvis, topk, pool):
    say(f"index_full B={B} Q={Q} cap={cap} topk={topk} pool={pool}")
    cache, ikc, iks = make_idx_cache(gpu, oracle_mod, B, cap, 400 + cap + B, dup_frac=0.2)
    g = np.random.default_rng(401)
    iq = g.standard_normal((B, Q, 4, 64)).astype(np.float32)
    iw = g.random((B, Q, 4)).astype(np.float32)
    nv = np.array(nvis, np.int32).reshape(B, Q)
    tk_ref, pl_ref = oracle_mod.index_full_batch(ikc, iks, iq, iw, nv, topk, pool)
    tk = torch.full((B, Q, topk), -7, dtype=torch.int32, device="cuda")
    pl = torch.full((B, Q, max(pool, 1)), -7, dtype=torch.int32, device="cuda")
    gpu.index_full(cache, dev(iq), dev(iw), dev(nv), tk, pl if pool else None, topk=topk,
                   pool_blocks=pool)
    np.testing.assert_array_equal(host(tk), tk_ref)
    if pool:
        np.testing.assert_array_equal(host(pl), pl_ref)


def test_index_full_chunk_candidate_overflow(gpu, oracle_mod):
    """Identical key rows tie every score of a query, so every visible block is
    a candidate of the MFMA path and the candidates overflow its pool: the
    flagged queries are rescored exactly by their selection workgroup and
    must come out unchanged (the lowest positions, by the tie rule)."""
    say("index_full multi-query, all-equal scores (candidate overflow)")
    B, Q, cap = 1, 8, 16384
    x = np.tile(np.random.default_rng(9).standard_normal((1, 1, 64)), (B, cap, 1)).astype(np.float32)
    ikc, iks = oracle_mod.quant_fp8_rows(x)
    cache = gpu.Cache(B, cap)
    cache.ik_codes.copy_(dev(tile_ik(ikc)))
    cache.ik_sigma.copy_(dev(iks.reshape(-1)))
    g = np.random.default_rng(10)
    iq = g.standard_normal((B, Q, 4, 64)).astype(np.float32)
    iw = g.random((B, Q, 4)).astype(np.float32)
    # ragged visible counts (not multiples of 8) among the overflowing queries
    nv = np.array([[16384, 16001, 9003, 8200, 600, 512, 100, 16384]], np.int32)
    tk_ref, _ = oracle_mod.index_full_batch(ikc.reshape(B, cap, 64), iks.reshape(B, cap), iq, iw,
                                            nv, 512, 0)
    tk = torch.full((B, Q, 512), -7, dtype=torch.int32, device="cuda")
    gpu.index_full(cache, dev(iq), dev(iw), dev(nv), tk, None, topk=512, pool_blocks=0)
    np.testing.assert_array_equal(host(tk), tk_ref)


def test_index_full_chunk_pool_overflow(gpu, oracle_mod):
    """All scores equal, with a pool: no block is decided by the bounds and
    all the visible ones stay undecided, more than the MFMA path's list holds,
    so each query is rescored exactly and takes the Full selection (pool of
    the lowest blocks, then the lowest positions).  A query with 1013 visible
    blocks fits the list: they are scored exactly and the tie rule takes the
    lowest 1000; one with fewer visible blocks than the pool takes them all."""
    say("index_full multi-query with a pool, all-equal scores")
    B, Q, cap = 1, 6, 16384
    x = np.tile(np.random.default_rng(19).standard_normal((1, 1, 64)), (B, cap, 1)).astype(np.float32)
    ikc, iks = oracle_mod.quant_fp8_rows(x)
    cache = gpu.Cache(B, cap)
    cache.ik_codes.copy_(dev(tile_ik(ikc)))
    cache.ik_sigma.copy_(dev(iks.reshape(-1)))
    g = np.random.default_rng(20)
    iq = g.standard_normal((B, Q, 4, 64)).astype(np.float32)
    iw = g.random((B, Q, 4)).astype(np.float32)
    nv = np.array([[16384, 16001, 9003, 8200, 8100, 100]], np.int32)
    tk_ref, pl_ref = oracle_mod.index_full_batch(ikc.reshape(B, cap, 64), iks.reshape(B, cap), iq,
                                                 iw, nv, 512, 1000)
    tk = torch.full((B, Q, 512), -7, dtype=torch.int32, device="cuda")
    pl = torch.full((B, Q, 1000), -7, dtype=torch.int32, device="cuda")
    gpu.index_full(cache, dev(iq), dev(iw), dev(nv), tk, pl, topk=512, pool_blocks=1000)
    np.testing.assert_array_equal(host(tk), tk_ref)
    np.testing.assert_array_equal(host(pl), pl_ref)


def test_index_full_all_ties(gpu, oracle_mod):
    say("index_full all-equal scores")
    B, cap = 1, 4096
    x = np.tile(np.random.default_rng(5).standard_normal((1, 1, 64)), (B, cap, 1)).astype(np.float32)
    ikc, iks = oracle_mod.quant_fp8_rows(x)
    cache = gpu.Cache(B, cap)
    cache.ik_codes.copy_(dev(tile_ik(ikc)))
    cache.ik_sigma.copy_(dev(iks.reshape(-1)))
    iq = np.random.default_rng(6).standard_normal((B, 1, 4, 64)).astype(np.float32)
    iw = np.ones((B, 1, 4), np.float32)
    nv = np.array([[4000]], np.int32)
    tk = torch.empty((B, 1, 512), dtype=torch.int32, device="cuda")
    pl = torch.empty((B, 1, 2048), dtype=torch.int32, device="cuda")
    gpu.index_full(cache, dev(iq), dev(iw), dev(nv), tk, pl, topk=512, pool_blocks=2048)
    assert host(tk)[0, 0].tolist() == list(range(512))
    p = host(pl)[0, 0]
    assert p[:500].tolist() == list(range(500)) and np.all(p[500:] == -1)


def test_index_full_all_ties_streaming_blocks(gpu, oracle_mod):
    """More blocks than the register path holds, every score equal: all 4096
    superblocks tie, more than the two-level block selection takes, so the
    blocks are selected by streaming; ties go to the lowest blocks and
    positions."""
    say("index_full all-equal scores, 262144 positions")
    B, cap = 1, 262144
    x = np.tile(np.random.default_rng(15).standard_normal((1, 1, 64)), (B, cap, 1)).astype(np.float32)
    ikc, iks = oracle_mod.quant_fp8_rows(x)
    cache = gpu.Cache(B, cap)
    cache.ik_codes.copy_(dev(tile_ik(ikc)))
    cache.ik_sigma.copy_(dev(iks.reshape(-1)))
    iq = np.random.default_rng(16).standard_normal((B, 1, 4, 64)).astype(np.float32)
    iw = np.ones((B, 1, 4), np.float32)
    nv = np.array([[262141]], np.int32)
    tk = torch.empty((B, 1, 512), dtype=torch.int32, device="cuda")
    pl = torch.empty((B, 1, 2048), dtype=torch.int32, device="cuda")
    gpu.index_full(cache, dev(iq), dev(iw), dev(nv), tk, pl, topk=512, pool_blocks=2048)
    assert host(tk)[0, 0].tolist() == list(range(512))
    assert host(pl)[0, 0].tolist() == list(range(2048))


@pytest.mark.parametrize("B,cap,nvis,pool,topk", [(2, 8192, [8192, 5001], 512, 512),
                                                  (3, 32768, [32768, 30000, 77], 2048, 512),
                                                  # part of the pool past the visible blocks
                                                  (2, 16384, [16384, 14001], 2048, 256),
                                                  (1, 131072, [131067], 2048, 511),
                                                  (1, 4096, [4096], 64, 100),
                                                  (1, 65536, [65531], 4096, 2048)])
def test_index_reindex_bit_exact(gpu, oracle_mod, B, cap, nvis, pool, topk):
    say(f"index_reindex B={B} cap={cap} pool={pool} topk={topk}")
    cache, ikc, iks = make_idx_cache(gpu, oracle_mod, B, cap, 500 + cap, dup_frac=0.1)
    g = np.random.default_rng(501)
    iq = g.standard_normal((B, 1, 4, 64)).astype(np.float32)
    iw = g.random((B, 1, 4)).astype(np.float32)
    iq2 = g.standard_normal((B, 1, 4, 64)).astype(np.float32)
    iw2 = g.random((B, 1, 4)).astype(np.float32)
    nv = np.array(nvis, np.int32).reshape(B, 1)
    _, pool_ref = oracle_mod.index_full_batch(ikc, iks, iq, iw, nv, min(topk, pool), pool)
    tk_ref = oracle_mod.index_reindex_batch(ikc, iks, iq2, iw2, nv, pool_ref, topk)
    tk = torch.full((B, 1, topk), -7, dtype=torch.int32, device="cuda")
    gpu.index_reindex(cache, dev(iq2), dev(iw2), dev(nv), dev(pool_ref), tk, topk=topk)
    np.testing.assert_array_equal(host(tk), tk_ref)


def test_full_topk_equals_reindex_with_own_query(gpu, oracle_mod):
    say("Full top-K == Reindex(own query, own pool)")
    B, cap = 2, 16384
    cache, ikc, iks = make_idx_cache(gpu, oracle_mod, B, cap, 600, dup_frac=0.3)
    g = np.random.default_rng(601)
    iq = dev(g.standard_normal((B, 1, 4, 64)).astype(np.float32))
    iw = dev(g.random((B, 1, 4)).astype(np.float32))
    nv = dev(np.array([[16384], [12345]], np.int32))
    tk = torch.empty((B, 1, 512), dtype=torch.int32, device="cuda")
    pl = torch.empty((B, 1, 2048), dtype=torch.int32, device="cuda")
    tk2 = torch.empty_like(tk)
    gpu.index_full(cache, iq, iw, nv, tk, pl, topk=512, pool_blocks=2048)
    gpu.index_reindex(cache, iq, iw, nv, pl, tk2, topk=512)
    np.testing.assert_array_equal(host(tk), host(tk2))


@pytest.mark.parametrize("n_vals,topk", [(1, 512), (2, 512), (3, 511), (6, 512)])
def test_index_few_valued_scores(gpu, oracle_mod, n_vals, topk):
    """Key rows drawn from a few vectors, so every score takes one of a few
    values: the selections start from lower bounds of the cut (the block
    selection's group maxima for the Full layer's positions, the pool
    scoring's group maxima for Reindex) and meet heavy ties at and above it.
    4096 blocks, pool 2048, Full and Reindex against the oracle."""
    say(f"index_full / reindex with {n_vals}-valued scores, topk={topk}")
    B, cap = 2, 32768
    g = np.random.default_rng(70 + n_vals)
    base = g.standard_normal((n_vals, 64)).astype(np.float32)
    p = 0.5 ** np.arange(n_vals)
    x = base[g.choice(n_vals, size=(B, cap), p=p / p.sum())]
    ikc, iks = oracle_mod.quant_fp8_rows(x)
    cache = gpu.Cache(B, cap)
    cache.ik_codes.copy_(dev(tile_ik(ikc)))
    cache.ik_sigma.copy_(dev(iks.reshape(-1)))
    iq = g.standard_normal((B, 1, 4, 64)).astype(np.float32)
    iw = g.random((B, 1, 4)).astype(np.float32)
    iq2 = g.standard_normal((B, 1, 4, 64)).astype(np.float32)
    iw2 = g.random((B, 1, 4)).astype(np.float32)
    nv = np.array([[32765], [30001]], np.int32)
    tk_ref, pl_ref = oracle_mod.index_full_batch(ikc, iks, iq, iw, nv, topk, 2048)
    tk = torch.full((B, 1, topk), -7, dtype=torch.int32, device="cuda")
    pl = torch.full((B, 1, 2048), -7, dtype=torch.int32, device="cuda")
    gpu.index_full(cache, dev(iq), dev(iw), dev(nv), tk, pl, topk=topk, pool_blocks=2048)
    np.testing.assert_array_equal(host(pl), pl_ref)
    np.testing.assert_array_equal(host(tk), tk_ref)
    tk2_ref = oracle_mod.index_reindex_batch(ikc, iks, iq2, iw2, nv, pl_ref, topk)
    tk2 = torch.full((B, 1, topk), -7, dtype=torch.int32, device="cuda")
    gpu.index_reindex(cache, dev(iq2), dev(iw2), dev(nv), dev(pl_ref), tk2, topk=topk)
    np.testing.assert_array_equal(host(tk2), tk2_ref)


# --------------------------------------------------------------------------- attention
def make_attn_case(gpu, oracle_mod, B, cap, H, seed, Q=1):
    g = np.random.default_rng(seed)
    k = g.standard_normal((B, cap, 128)).astype(np.float32)
    v = g.standard_normal((B, cap, 128)).astype(np.float32)
    codes, scales = oracle_mod.quant_fp4(k.reshape(-1, 128), v.reshape(-1, 128))
    cache = gpu.Cache(B, cap)
    cache.kv_codes.copy_(dev(codes))
    cache.kv_scales.copy_(dev(scales))
    rows = 128 if Q == 1 else Q
    sk, sks = oracle_mod.quant_fp8_rows(g.standard_normal((B, rows, 128)).astype(np.float32))
    sv, svs = oracle_mod.quant_fp8_rows(g.standard_normal((B, rows, 128)).astype(np.float32))
    shape = (B, H, 128) if Q == 1 else (B, Q, H, 128)
    q = g.standard_normal(shape).astype(np.float32)
    return cache, codes.reshape(B, cap, 128), scales.reshape(B, cap, 16), sk, sv, sks, svs, q


@pytest.mark.parametrize("B,cap,H,topk,swa_len,n_sel", [
    (1, 1024, 16, 512, [128], [512]),
    (3, 4096, 64, 512, [128, 5, 0], [512, 300, 0]),
    (2, 2048, 32, 100, [77, 128], [100, 3]),
    (4, 1024, 128, 512, [128, 128, 1, 64], [512, 511, 512, 17]),
    (1, 640, 48, 0, [128], [0]),
    (2, 8192, 128, 2048, [128, 100], [2048, 1500]),   # the largest top-K and head count
])
def test_sparse_attn_decode(gpu, oracle_mod, B, cap, H, topk, swa_len, n_sel):
    say(f"attn_decode B={B} cap={cap} H={H} topk={topk}")
    cache, codes, scales, sk, sv, sks, svs, q = make_attn_case(gpu, oracle_mod, B, cap, H, 700 + H)
    g = np.random.default_rng(701)
    idx = np.full((B, max(topk, 1)), -1, np.int32)[:, :topk]
    for b in range(B):
        sel = np.sort(g.choice(cap, n_sel[b], replace=False))
        idx[b, :n_sel[b]] = sel
    sl = np.array(swa_len, np.int32)
    out_ref, lse_ref = oracle_mod.attn_decode_batch(q, codes, scales,
                                                    idx if topk else np.zeros((B, 0), np.int32),
                                                    sk, sv, sks, svs, sl, SM)
    out = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    idx_d = dev(idx) if topk else torch.empty((B, 0), dtype=torch.int32, device="cuda")
    gpu.sparse_attn_decode(dev(q), cache, idx_d, dev(sk), dev(sv), dev(sks), dev(svs), dev(sl),
                           out, lse)
    o, l = host(out), host(lse)
    empty = (np.array(n_sel) == 0) & (sl == 0)
    for b in range(B):
        if empty[b]:
            assert np.all(o[b] == 0) and np.all(np.isneginf(l[b]))
            continue
        err = row_rel_err(o[b], out_ref[b])
        assert err.max() <= ATOL_ROW, (b, err.max())
        np.testing.assert_allclose(l[b], lse_ref[b], rtol=2e-3, atol=2e-3)


@pytest.mark.parametrize("B,cap,H,topk,swa_len,n_sel", [
    (3, 4096, 64, 512, [128, 5, 0], [512, 300, 0]),
    (2, 2048, 32, 100, [77, 128], [100, 3]),
    (2, 8192, 128, 2048, [128, 100], [2048, 1500]),
])
def test_sparse_attn_decode_reuse_stage(gpu, oracle_mod, B, cap, H, topk, swa_len, n_sel):
    """A gathering call writes the stage; later calls with other queries and
    windows read it (no cache, no positions): every output equals the plain
    call's bit for bit, and the oracle's to the attention tolerance."""
    say(f"attn_decode_reuse B={B} cap={cap} H={H} topk={topk}")
    cache, codes, scales, sk, sv, sks, svs, q = make_attn_case(gpu, oracle_mod, B, cap, H, 740 + H)
    g = np.random.default_rng(741)
    idx = np.full((B, topk), -1, np.int32)
    for b in range(B):
        idx[b, :n_sel[b]] = np.sort(g.choice(cap, n_sel[b], replace=False))
    clean = idx.copy()
    clean[0, -1] = -1
    idx[0, -1] = cap + 3   # an out-of-range position is staged as absent (the oracle sees -1)
    sl = np.array(swa_len, np.int32)
    stage = gpu.alloc_workspace(gpu.workspace_size(gpu.OP_ATTN_STAGE, B, 1, cap, topk, 0, H))
    assert stage.numel() == B * ((topk + 31) // 32) * 4672
    stage.fill_(0xAB)  # no byte of a previous content may leak through
    for layer in range(3):
        ql = q if layer == 0 else g.standard_normal(q.shape).astype(np.float32)
        skl, svl = (sk, sv) if layer == 0 else (np.roll(sk, layer, axis=1), np.roll(sv, layer, axis=1))
        sksl, svsl = (sks, svs) if layer == 0 else (sks[:, ::-1].copy(), svs[:, ::-1].copy())
        args = (dev(skl), dev(svl), dev(sksl), dev(svsl), dev(sl))
        out_p = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
        lse_p = torch.empty((B, H), dtype=torch.float32, device="cuda")
        gpu.sparse_attn_decode(dev(ql), cache, dev(idx), *args, out_p, lse_p)
        out = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
        if layer == 0:
            gpu.sparse_attn_decode_reuse(dev(ql), cache, dev(idx), topk, stage, gpu.STAGE_WRITE,
                                         *args, out, lse)
        else:
            gpu.sparse_attn_decode_reuse(dev(ql), None, None, topk, stage, gpu.STAGE_READ,
                                         *args, out, lse)
        np.testing.assert_array_equal(host(out), host(out_p))
        np.testing.assert_array_equal(host(lse), host(lse_p))
        out_ref, _ = oracle_mod.attn_decode_batch(ql, codes, scales, clean, skl, svl, sksl, svsl,
                                                  sl, SM)
        for b in range(B):
            if n_sel[b] == 0 and sl[b] == 0:
                continue
            assert row_rel_err(host(out)[b], out_ref[b]).max() <= ATOL_ROW


def test_sparse_attn_decode_ignores_out_of_range_indices(gpu, oracle_mod):
    say("attn_decode with out-of-range indices")
    B, cap, H = 1, 1024, 16
    cache, codes, scales, sk, sv, sks, svs, q = make_attn_case(gpu, oracle_mod, B, cap, H, 720)
    idx = np.full((B, 64), -1, np.int32)
    idx[0, :10] = np.arange(10) * 7
    bad = idx.copy()
    bad[0, 10:20] = [cap, cap + 5, 1 << 30, -5, -100, cap * 2, 99999, 4096, 2048, 1025]
    sl = np.array([128], np.int32)
    out_ref, _ = oracle_mod.attn_decode_batch(q, codes, scales, idx, sk, sv, sks, svs, sl, SM)
    out = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    gpu.sparse_attn_decode(dev(q), cache, dev(bad), dev(sk), dev(sv), dev(sks), dev(svs), dev(sl),
                           out, lse)
    assert row_rel_err(host(out)[0], out_ref[0]).max() <= ATOL_ROW


@pytest.mark.parametrize("B,Q,cap,H", [(1, 128, 2048, 64), (2, 37, 1024, 16),
                                       (1, 300, 4096, 16)])   # window slides past 128 tokens
def test_sparse_attn_chunk(gpu, oracle_mod, B, Q, cap, H):
    say(f"attn_chunk B={B} Q={Q} cap={cap} H={H}")
    cache, codes, scales, sk, sv, sks, svs, q = make_attn_case(gpu, oracle_mod, B, cap, H, 800, Q=Q)
    g = np.random.default_rng(801)
    idx = np.full((B, Q, 512), -1, np.int32)
    for b in range(B):
        for i in range(Q):
            n = min(512, cap - Q + i + 1)
            idx[b, i, :n] = np.sort(g.choice(cap - Q + i + 1, n, replace=False))
    out_ref, lse_ref = oracle_mod.attn_chunk_batch(q, codes, scales, idx, sk, sv, sks, svs, SM)
    out = torch.empty((B, Q, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Q, H), dtype=torch.float32, device="cuda")
    gpu.sparse_attn_chunk(dev(q), cache, dev(idx), dev(sk), dev(sv), dev(sks), dev(svs), out, lse)
    err = row_rel_err(host(out), out_ref)
    assert err.max() <= ATOL_ROW, err.max()
    np.testing.assert_allclose(host(lse), lse_ref, rtol=2e-3, atol=2e-3)
