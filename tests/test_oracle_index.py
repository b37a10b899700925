"""Pins of the oracle's indexer: score arithmetic, ranking, pool, Reindex, Reuse.

References: exact integer arithmetic on hand-built inputs (closed forms), an
fp64 evaluation with the classical error bound of a length-64 fp32 sum, and
brute-force rankings written here with Python's sort.
"""
import json
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def e4m3_value(code):
    return torch.tensor(np.asarray(code, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e4m3_rne(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def brute_top(keys, cap):
    """Indices of the `cap` best (larger key first, lower index on ties), ascending, -1 padded."""
    order = sorted(range(len(keys)), key=lambda i: (-keys[i], i))[:cap]
    out = sorted(order)
    return np.array(out + [-1] * (cap - len(out)), np.int32)


def test_score_closed_form_small_integers(oracle_mod):
    # Each head holds one 448 (so sq = 1 and the query codes are the values
    # themselves) and small integers; K codes decode to small integers; sigma
    # and the head weights are powers of two: every step is exact.
    g = np.random.default_rng(10)
    iq = g.integers(-4, 5, (4, 64)).astype(np.float32)
    iq[:, 0] = 448.0
    iw = np.array([1.0, 0.5, 0.25, 2.0], np.float32)
    kvals = g.integers(-3, 4, 64).astype(np.float32)
    kc = e4m3_rne(kvals)
    assert np.array_equal(e4m3_value(kc), kvals)
    qc, wq = oracle_mod.quant_iq(iq, iw)
    np.testing.assert_array_equal(e4m3_value(qc), iq)
    np.testing.assert_array_equal(wq, iw)
    sigma = 0.125
    dots = [int(np.dot(iq[h].astype(np.int64), kvals.astype(np.int64))) for h in range(4)]
    expect = sigma * sum(w * max(d, 0) for w, d in zip(iw.tolist(), dots))
    assert oracle_mod.score(qc, wq, kc, sigma) == expect


def test_score_relu_and_weights(oracle_mod):
    qc = np.zeros((4, 64), np.uint8)
    qc[:, 0] = e4m3_rne(np.float32(1.0))
    kc = np.zeros(64, np.uint8)
    kc[0] = e4m3_rne(np.float32(-2.0))  # every dot is -2 -> ReLU -> 0
    assert oracle_mod.score(qc, np.ones(4, np.float32), kc, 1.0) == 0.0
    qc[1, 0] = e4m3_rne(np.float32(-1.0))  # head 1 dot = +2
    wq = np.array([1.0, 3.0, 5.0, 7.0], np.float32)
    assert oracle_mod.score(qc, wq, kc, 0.5) == 0.5 * 3.0 * 2.0


def test_score_channel_order_is_sequential_fp32(oracle_mod):
    # products: 448*448, then 2^-18 (subnormal x subnormal), then -448*448.
    # Summed left to right in fp32 the tiny product is absorbed: dot = 0.
    # (An exact or reordered sum would give 2^-18.)
    qc = np.zeros((4, 64), np.uint8)
    kc = np.zeros(64, np.uint8)
    qc[0, :3] = [0x7E, 0x01, 0xFE]
    kc[:3] = [0x7E, 0x01, 0x7E]
    wq = np.array([1.0, 0.0, 0.0, 0.0], np.float32)
    assert oracle_mod.score(qc, wq, kc, 1.0) == 0.0
    qc[0, :3] = [0x01, 0x7E, 0xFE]  # tiny first: 2^-18 + 200704 - 200704 = 0 as well
    assert oracle_mod.score(qc, wq, kc[[1, 0, 2] + list(range(3, 64))], 1.0) == 0.0
    qc[0, :3] = [0x7E, 0xFE, 0x01]  # cancellation first, tiny last: exact 2^-18
    kc2 = np.zeros(64, np.uint8)
    kc2[:3] = [0x7E, 0x7E, 0x01]
    assert oracle_mod.score(qc, wq, kc2, 1.0) == 2.0 ** -18


def test_score_random_within_fp32_sum_bound(oracle_mod):
    g = np.random.default_rng(11)
    u = 2.0 ** -24
    for _ in range(300):
        iq = g.standard_normal((4, 64)).astype(np.float32)
        iw = g.random(4).astype(np.float32)
        kc = e4m3_rne(g.standard_normal(64).astype(np.float32) * 100)
        sigma = np.float32(g.random() * 0.01)
        qc, wq = oracle_mod.quant_iq(iq, iw)
        got = oracle_mod.score(qc, wq, kc, sigma)
        qv, kv = e4m3_value(qc), e4m3_value(kc)
        prods = qv * kv[None, :]
        dots = prods.sum(axis=1)
        exact = float(sigma) * sum(float(wq[h]) * max(dots[h], 0.0) for h in range(4))
        # |fl-sum - sum| <= 63u sum|p| per head, then 4 products, 3 adds, 1 product
        bound = float(sigma) * sum(float(wq[h]) * 64 * u * np.abs(prods[h]).sum() for h in range(4))
        bound += 10 * u * abs(exact) + 1e-45
        assert abs(got - exact) <= bound, (got, exact, bound)


def make_index_case(oracle_mod, seed, n, dup_rows=0):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, 64)).astype(np.float32)
    if dup_rows:
        src = g.integers(0, n, dup_rows)
        dst = g.integers(0, n, dup_rows)
        x[dst] = x[src]  # identical rows -> identical scores -> ties
    ikc, iks = oracle_mod.quant_fp8_rows(x)
    iq = g.standard_normal((4, 64)).astype(np.float32)
    iw = g.random(4).astype(np.float32)
    return ikc, iks, iq, iw


@pytest.mark.parametrize("n_vis,topk,pool", [(1, 4, 0), (37, 5, 0), (100, 16, 3), (203, 9, 4),
                                             (64, 64, 8), (513, 40, 12), (300, 512, 0)])
def test_index_full_against_brute_force(oracle_mod, n_vis, topk, pool):
    if pool and pool < topk:
        pool = max(pool, 1)
    ikc, iks, iq, iw = make_index_case(oracle_mod, 20 + n_vis, n_vis + 17, dup_rows=n_vis // 3)
    tk, pl, sc = oracle_mod.index_full(ikc, iks, n_vis, iq, iw, topk, pool, want_scores=True)
    keys = sc.tolist()
    np.testing.assert_array_equal(tk, brute_top(keys, topk))
    if pool:
        nb = (n_vis + 7) // 8
        bmax = [max(keys[8 * b: min(8 * b + 8, n_vis)]) for b in range(nb)]
        np.testing.assert_array_equal(pl, brute_top(bmax, pool))
    # ties really occur in these cases
    if n_vis > 50:
        assert len(set(keys)) < len(keys)


def test_ties_go_to_lowest_position(oracle_mod):
    ikc, iks, iq, iw = make_index_case(oracle_mod, 30, 40)
    ikc[:] = ikc[5]
    iks[:] = iks[5]  # every position scores the same
    tk, pl = oracle_mod.index_full(ikc, iks, 40, iq, iw, 7, 2)
    assert tk.tolist() == list(range(7))
    assert pl.tolist() == [0, 1]


def test_fewer_visible_than_k_returns_all(oracle_mod):
    ikc, iks, iq, iw = make_index_case(oracle_mod, 31, 64)
    tk, pl = oracle_mod.index_full(ikc, iks, 13, iq, iw, 512, 2048)
    assert tk[:13].tolist() == list(range(13)) and np.all(tk[13:] == -1)
    assert pl[:2].tolist() == [0, 1] and np.all(pl[2:] == -1)
    tk0, _ = oracle_mod.index_full(ikc, iks, 0, iq, iw, 4, 0)
    assert np.all(tk0 == -1)


def test_reindex_against_brute_force(oracle_mod):
    ikc, iks, iq, iw = make_index_case(oracle_mod, 40, 800, dup_rows=200)
    n_vis = 795
    _, pool = oracle_mod.index_full(ikc, iks, n_vis, iq, iw, 16, 20)
    g = np.random.default_rng(41)
    iq2 = g.standard_normal((4, 64)).astype(np.float32)
    iw2 = g.random(4).astype(np.float32)
    tk = oracle_mod.index_reindex(ikc, iks, n_vis, iq2, iw2, pool, 30)
    _, _, sc2 = oracle_mod.index_full(ikc, iks, n_vis, iq2, iw2, 1, 0, want_scores=True)
    cand = [s for b in pool if b >= 0 for s in range(8 * b, min(8 * b + 8, n_vis))]
    order = sorted(cand, key=lambda s: (-sc2[s], s))[:30]
    np.testing.assert_array_equal(tk, np.array(sorted(order) + [-1] * (30 - len(order)), np.int32))


def test_full_topk_lies_in_its_pool(oracle_mod):
    # With pool >= topk blocks, the Full layer's own top-K over every visible
    # position equals the top-K inside its pool (Reindex with the same query).
    for seed in range(5):
        ikc, iks, iq, iw = make_index_case(oracle_mod, 50 + seed, 4000, dup_rows=1000)
        n_vis = 3999 - seed * 7
        tk, pool = oracle_mod.index_full(ikc, iks, n_vis, iq, iw, 64, 64)
        tk2 = oracle_mod.index_reindex(ikc, iks, n_vis, iq, iw, pool, 64)
        np.testing.assert_array_equal(tk, tk2)


def test_pool_bounds_from_pages(oracle_mod):
    gold = json.load(open(os.path.join(GOLD, "page_constants.json")))
    P = gold["pool_blocks_max"]["value"]
    bs = gold["positions_per_block"]["value"]
    assert P * bs == gold["pool_positions_max"]["value"]
    ikc, iks, iq, iw = make_index_case(oracle_mod, 60, 20000)
    tk, pool = oracle_mod.index_full(ikc, iks, 20000, iq, iw, gold["topk_max"]["value"], P)
    assert np.all(pool >= 0) and len(set(pool.tolist())) == P
    assert np.all(np.diff(pool) > 0) and np.all(np.diff(tk) > 0)
    covered = set((pool[:, None] * bs + np.arange(bs)[None, :]).ravel().tolist())
    assert len(covered) == P * bs and set(tk.tolist()) <= covered


def test_batch_equals_single(oracle_mod):
    g = np.random.default_rng(70)
    B, Q, cap = 2, 3, 128
    x = g.standard_normal((B, cap, 64)).astype(np.float32)
    ikc, iks = oracle_mod.quant_fp8_rows(x)
    iq = g.standard_normal((B, Q, 4, 64)).astype(np.float32)
    iw = g.random((B, Q, 4)).astype(np.float32)
    nv = np.array([[128, 77, 3], [1, 64, 100]], np.int32)
    tk, pl = oracle_mod.index_full_batch(ikc, iks, iq, iw, nv, 9, 10)
    for b in range(B):
        for q in range(Q):
            t1, p1 = oracle_mod.index_full(ikc[b], iks[b], nv[b, q], iq[b, q], iw[b, q], 9, 10)
            np.testing.assert_array_equal(tk[b, q], t1)
            np.testing.assert_array_equal(pl[b, q], p1)


def test_query_scale_fold_at_random_scales(oracle_mod):
    """The indexer query's per-head scale sq = fl(amax / 448) reaches the score
    only through the folded head weight w' = fl(w * sq).  Queries of random
    magnitude (sq far from 1) pin the fold: the codes are RNE_E4M3(fl(q / sq)),
    w' equals fl(w * sq) bit for bit with sq computed here, and every score of
    the Full scan lies within the fp32 rounding bound of an fp64 score computed
    from the dequantised query sq * E4M3(code), the unfolded weight w and the
    decoded key.  A dropped fold (w' = w) or an inverted one (w / sq) misses
    that bound by orders of magnitude."""
    g = np.random.default_rng(12)
    u = 2.0 ** -24
    for trial in range(40):
        # sq is about mag / 180: magnitudes on both sides of 180, away from it
        mag = 10.0 ** (g.uniform(-3.0, 1.3) if trial % 2 else g.uniform(3.0, 4.5))
        iq = (g.standard_normal((4, 64)) * mag).astype(np.float32)
        iw = g.random(4).astype(np.float32)
        qc, wq = oracle_mod.quant_iq(iq, iw)
        sq = np.abs(iq).max(axis=1) / np.float32(448.0)  # fp32 division, one rounding
        assert sq.dtype == np.float32 and np.all(np.abs(np.log2(sq)) > 1.0)
        np.testing.assert_array_equal(qc, e4m3_rne(iq / sq[:, None]))
        np.testing.assert_array_equal(wq.view(np.uint32), (iw * sq).view(np.uint32))

        n = 24
        x = g.standard_normal((n, 64)).astype(np.float32)
        ikc, iks = oracle_mod.quant_fp8_rows(x)
        _, _, sc = oracle_mod.index_full(ikc, iks, n, iq, iw, 4, 0, want_scores=True)
        qhat = e4m3_value(qc) * sq[:, None].astype(np.float64)
        for s in range(n):
            kv = e4m3_value(ikc[s])
            dots = qhat @ kv
            exact = float(iks[s]) * sum(float(iw[h]) * max(dots[h], 0.0) for h in range(4))
            absp = np.abs(qhat * kv[None, :]).sum(axis=1)
            # 63 roundings of the channel chain, the fold, the weight product,
            # 3 head adds and the sigma product, each at most u relative
            bound = float(iks[s]) * sum(float(iw[h]) * 70 * u * absp[h] for h in range(4))
            bound += 8 * u * abs(exact) + 1e-45
            assert abs(float(sc[s]) - exact) <= bound, (trial, s, sc[s], exact, bound)
            assert sc[s] == oracle_mod.score(qc, wq, ikc[s], iks[s])


def test_reindex_batch_equals_single(oracle_mod):
    g = np.random.default_rng(71)
    B, Q, cap, P = 2, 3, 256, 6
    x = g.standard_normal((B, cap, 64)).astype(np.float32)
    ikc, iks = oracle_mod.quant_fp8_rows(x)
    iq = g.standard_normal((B, Q, 4, 64)).astype(np.float32)
    iw = g.random((B, Q, 4)).astype(np.float32)
    nv = np.array([[256, 130, 9], [1, 64, 200]], np.int32)
    _, pl = oracle_mod.index_full_batch(ikc, iks, iq, iw, nv, 8, P)
    iq2 = (g.standard_normal((B, Q, 4, 64)) * 3.0).astype(np.float32)
    iw2 = g.random((B, Q, 4)).astype(np.float32)
    tk = oracle_mod.index_reindex_batch(ikc, iks, iq2, iw2, nv, pl, 11)
    for b in range(B):
        for q in range(Q):
            t1 = oracle_mod.index_reindex(ikc[b], iks[b], nv[b, q], iq2[b, q], iw2[b, q],
                                          pl[b, q], 11)
            np.testing.assert_array_equal(tk[b, q], t1)
