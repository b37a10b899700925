"""Pins of the oracle's FP4 indexer-key variant: the key format, the
block-scaled score and the selections over it.

References: the FP4 main-KV quantiser (pinned in test_oracle_quant.py) for the
key format, the pages' 4 + 8/16 bits per value, closed forms on hand-built
inputs, an fp64 evaluation within a rounding bound, and brute-force rankings
written here with Python's sort.
"""
import numpy as np
import pytest
import torch

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e4m3_value(code):
    return torch.tensor(np.asarray(code, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e4m3_rne(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e2m1_code(v):
    """E2M1 code of a value on the grid (sign in bit 3)."""
    mag = int(np.flatnonzero(E2M1 == abs(v))[0])
    return mag | (8 if v < 0 else 0)


def dequant4(kc4, ks4):
    """Independent decode of a 64-channel FP4 key: nibble table x E4M3 scale."""
    kc4 = np.asarray(kc4, np.uint8)
    nib = np.empty(64, np.uint8)
    nib[0::2], nib[1::2] = kc4 & 0xF, kc4 >> 4
    val = E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    return val * np.repeat(e4m3_value(ks4), 16)


def brute_top(keys, cap):
    order = sorted(range(len(keys)), key=lambda i: (-keys[i], i))[:cap]
    out = sorted(order)
    return np.array(out + [-1] * (cap - len(out)), np.int32)


def pack(codes64):
    codes64 = np.asarray(codes64, np.uint8)
    return (codes64[0::2] | (codes64[1::2] << 4)).astype(np.uint8)


def test_key_format_is_the_main_kv_fp4_of_64_channels(oracle_mod):
    """36 bytes per 64-channel key = 4.5 bits per value; codes and scales equal
    the first four groups of the main-KV quantiser applied to the same values."""
    g = np.random.default_rng(40)
    x = (g.standard_normal((9, 64)) * np.exp2(g.integers(-6, 6, (9, 1)))).astype(np.float32)
    x[0, 16:32] = 0.0
    codes, scales = oracle_mod.idx4_quant_rows(x)
    assert codes.shape == (9, 32) and scales.shape == (9, 4)
    assert (codes.shape[1] + scales.shape[1]) * 8 / 64 == 4.5
    for i in range(9):
        k = np.zeros((1, 128), np.float32)
        k[0, :64] = x[i]
        c128, s128 = oracle_mod.quant_fp4(k, np.zeros_like(k), 1, None)
        np.testing.assert_array_equal(codes[i], c128[0, :32])
        np.testing.assert_array_equal(scales[i], s128[0, :4])


@pytest.mark.parametrize("c", [0, 1, 14, 15, 16, 33, 47, 62, 63])
def test_score4_single_channel_closed_form(oracle_mod, c):
    """One nonzero key channel: score = w'_h * q_hc * e2m1 * scale of group
    c // 16, exactly (pins the nibble order and which scale a channel takes)."""
    qc = e4m3_rne(np.full((4, 64), 3.0, np.float32))
    wq = np.array([1.0, 0.5, 2.0, 0.25], np.float32)
    codes = np.zeros(64, np.uint8)
    codes[c] = e2m1_code(1.5)
    ks = e4m3_rne(np.array([1.0, 2.0, 0.5, 4.0], np.float32))
    expect = sum(float(w) for w in wq) * 3.0 * 1.5 * [1.0, 2.0, 0.5, 4.0][c // 16]
    assert oracle_mod.score4(qc, wq, pack(codes), ks) == np.float32(expect)


def test_score4_small_values_exact(oracle_mod):
    """Small-integer queries, grid keys, power-of-two scales and weights: every
    sum is exact, so the score equals the fp64 value exactly; a head with a
    negative dot contributes +0."""
    g = np.random.default_rng(41)
    qv = g.integers(-4, 5, (4, 64)).astype(np.float32)
    qc = e4m3_rne(qv)
    kv = g.choice(np.concatenate([E2M1, -E2M1]), 64)
    codes = np.array([e2m1_code(v) for v in kv], np.uint8)
    sv = np.array([1.0, 2.0, 0.25, 8.0])
    ks = e4m3_rne(sv.astype(np.float32))
    wq = np.array([1.0, 0.5, 0.25, 2.0], np.float32)
    k = kv * np.repeat(sv, 16)
    dots = qv.astype(np.float64) @ k
    expect = sum(float(w) * max(d, 0.0) for w, d in zip(wq, dots))
    assert oracle_mod.score4(qc, wq, pack(codes), ks) == expect
    qv[0] = -qv[0]  # flips head 0's dot
    dots0 = qv.astype(np.float64) @ k
    expect0 = sum(float(w) * max(d, 0.0) for w, d in zip(wq, dots0))
    assert oracle_mod.score4(e4m3_rne(qv), wq, pack(codes), ks) == expect0


def test_score4_random_within_rounding_bound(oracle_mod):
    """Random keys and queries: within 2^-18 * sum_h |w'_h| sum_c |q_hc k_c| of
    the fp64 score of the dequantised key (at most 21 roundings of unit 2^-24
    per head plus the head combine); a wrong nibble, scale or channel misses
    by far more."""
    g = np.random.default_rng(42)
    x = g.standard_normal((300, 64)).astype(np.float32)
    codes, scales = oracle_mod.idx4_quant_rows(x)
    worst = 0.0
    for i in range(300):
        iq = g.standard_normal((4, 64)).astype(np.float32)
        iw = g.random(4).astype(np.float32)
        qc, wq = oracle_mod.quant_iq(iq, iw)
        qv = e4m3_value(qc)
        k = dequant4(codes[i], scales[i])
        dots = qv @ k
        exact = sum(float(w) * max(d, 0.0) for w, d in zip(wq, dots))
        mag = sum(abs(float(w)) * float(np.abs(qv[h] * k).sum()) for h, w in enumerate(wq))
        got = oracle_mod.score4(qc, wq, codes[i], scales[i])
        assert abs(got - exact) <= 2.0 ** -18 * mag, (i, got, exact)
        worst = max(worst, abs(got - exact))
    assert worst > 0.0  # fp32 arithmetic, not fp64


@pytest.mark.parametrize("n_vis,topk,pool", [(100, 16, 4), (1000, 16, 64), (37, 64, 8)])
def test_index_full4_against_brute_force(oracle_mod, n_vis, topk, pool):
    g = np.random.default_rng(43 + n_vis)
    codes, scales = oracle_mod.idx4_quant_rows(g.standard_normal((n_vis, 64)).astype(np.float32))
    codes[5] = codes[9]  # a duplicated key: ties to the lower position
    scales[5] = scales[9]
    iq = g.standard_normal((4, 64)).astype(np.float32)
    iw = g.random(4).astype(np.float32)
    qc, wq = oracle_mod.quant_iq(iq, iw)
    sc = [oracle_mod.score4(qc, wq, codes[s], scales[s]) for s in range(n_vis)]
    tk, pl, got_sc = oracle_mod.index_full4(codes, scales, n_vis, iq, iw, topk, pool,
                                            want_scores=True)
    np.testing.assert_array_equal(got_sc, np.array(sc, np.float32))
    np.testing.assert_array_equal(tk, brute_top(sc, topk))
    bmax = [max(sc[b * 8:min(b * 8 + 8, n_vis)]) for b in range((n_vis + 7) // 8)]
    np.testing.assert_array_equal(pl, brute_top(bmax, pool))
    if topk <= pool:  # the Full top-K lies inside its pool of >= K blocks (ties to lower indices)
        blocks = set(pl[pl >= 0].tolist())
        assert all(p // 8 in blocks for p in tk if p >= 0)


def test_reindex4_against_brute_force_and_full(oracle_mod):
    g = np.random.default_rng(44)
    n_vis = 2000
    codes, scales = oracle_mod.idx4_quant_rows(g.standard_normal((n_vis, 64)).astype(np.float32))
    iq = g.standard_normal((4, 64)).astype(np.float32)
    iw = g.random(4).astype(np.float32)
    tk, pl = oracle_mod.index_full4(codes, scales, n_vis, iq, iw, 64, 64)
    # Reindex with the Full layer's own query over its pool gives its top-K
    np.testing.assert_array_equal(oracle_mod.index_reindex4(codes, scales, n_vis, iq, iw, pl, 64), tk)
    iq2 = g.standard_normal((4, 64)).astype(np.float32)
    iw2 = g.random(4).astype(np.float32)
    qc, wq = oracle_mod.quant_iq(iq2, iw2)
    cand = [p for b in pl if b >= 0 for p in range(b * 8, min(b * 8 + 8, n_vis))]
    sc = {p: oracle_mod.score4(qc, wq, codes[p], scales[p]) for p in cand}
    order = sorted(cand, key=lambda p: (-sc[p], p))[:64]
    expect = np.array(sorted(order) + [-1] * (64 - len(order)), np.int32)
    np.testing.assert_array_equal(oracle_mod.index_reindex4(codes, scales, n_vis, iq2, iw2, pl, 64),
                                  expect)


def test_batch4_equals_single(oracle_mod):
    g = np.random.default_rng(45)
    B, cap, Q = 2, 256, 2
    codes, scales = oracle_mod.idx4_quant_rows(g.standard_normal((B, cap, 64)).astype(np.float32))
    iq = g.standard_normal((B, Q, 4, 64)).astype(np.float32)
    iw = g.random((B, Q, 4)).astype(np.float32)
    nv = np.array([[256, 100], [7, 200]], np.int32)
    tk, pl = oracle_mod.index_full4_batch(codes, scales, iq, iw, nv, 32, 8)
    rk = oracle_mod.index_reindex4_batch(codes, scales, iq[:, ::-1].copy(), iw[:, ::-1].copy(), nv,
                                         pl, 16)
    for b in range(B):
        for q in range(Q):
            t1, p1 = oracle_mod.index_full4(codes[b], scales[b], nv[b, q], iq[b, q], iw[b, q], 32, 8)
            np.testing.assert_array_equal(tk[b, q], t1)
            np.testing.assert_array_equal(pl[b, q], p1)
            r1 = oracle_mod.index_reindex4(codes[b], scales[b], nv[b, q], iq[b, Q - 1 - q],
                                           iw[b, Q - 1 - q], pl[b, q], 16)
            np.testing.assert_array_equal(rk[b, q], r1)


def test_score4_query_scale_fold_at_random_scales(oracle_mod):
    """FP4 keys take the same folded weight w' = fl(w * sq): scores of queries
    with sq far from 1 lie within the rounding bound of the fp64 score over the
    dequantised query sq * E4M3(code) with the unfolded weight w."""
    g = np.random.default_rng(46)
    x = g.standard_normal((50, 64)).astype(np.float32)
    codes, scales = oracle_mod.idx4_quant_rows(x)
    for i in range(50):
        mag = 10.0 ** (g.uniform(-3.0, 1.3) if i % 2 else g.uniform(3.0, 4.5))
        iq = (g.standard_normal((4, 64)) * mag).astype(np.float32)
        iw = g.random(4).astype(np.float32)
        qc, wq = oracle_mod.quant_iq(iq, iw)
        sq = np.abs(iq).max(axis=1) / np.float32(448.0)
        assert np.all(np.abs(np.log2(sq)) > 1.0)
        qhat = e4m3_value(qc) * sq[:, None].astype(np.float64)
        k = dequant4(codes[i], scales[i])
        dots = qhat @ k
        exact = sum(float(w) * max(d, 0.0) for w, d in zip(iw, dots))
        mag = sum(float(w) * float(np.abs(qhat[h] * k).sum()) for h, w in enumerate(iw))
        got = oracle_mod.score4(qc, wq, codes[i], scales[i])
        assert abs(got - exact) <= 2.0 ** -18 * mag + 2.0 ** -21 * abs(exact) + 1e-45, (i, got, exact)
