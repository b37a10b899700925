"""Pins of the oracle's sparse attention.

References: a dense softmax attention written with numpy matrix products over
independently dequantised K/V (E2M1 table x torch E4M3 decode), and closed
forms (uniform keys -> mean of V; one dominant key -> its V; lse of equal
logits = logit + ln n).
"""
import numpy as np
import torch

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
SM = np.float32(1.0 / np.sqrt(128.0))


def e4m3_value(code):
    return torch.tensor(np.asarray(code, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def fp4_matrix(codes, scales):
    """[n][128] codes/[n][16] scales -> K [n][128], V [n][128] in float64."""
    nib = np.empty((codes.shape[0], 256), np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    val = E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    sc = np.repeat(e4m3_value(scales), 16, axis=1)
    full = val * sc
    return full[:, :128], full[:, 128:]


def dense_attention(q, k, v, sm):
    logits = (q.astype(np.float64) @ k.T) * float(sm)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    return (p @ v) / p.sum(axis=1, keepdims=True), (m[:, 0] + np.log(p.sum(axis=1)))


def make_case(oracle_mod, seed, n, H=16, swa_len=128):
    g = np.random.default_rng(seed)
    k = g.standard_normal((n, 128)).astype(np.float32)
    v = g.standard_normal((n, 128)).astype(np.float32)
    codes, scales = oracle_mod.quant_fp4(k, v)
    sk, sks = oracle_mod.quant_fp8_rows(g.standard_normal((128, 128)).astype(np.float32))
    sv, svs = oracle_mod.quant_fp8_rows(g.standard_normal((128, 128)).astype(np.float32))
    q = g.standard_normal((H, 128)).astype(np.float32)
    return q, codes, scales, sk, sv, sks, svs


def test_sparse_equals_dense_when_topk_covers_everything(oracle_mod):
    n_vis = 300
    q, codes, scales, sk, sv, sks, svs = make_case(oracle_mod, 1, 320)
    idx = np.array(list(range(n_vis)) + [-1] * (512 - n_vis), np.int32)
    out, lse = oracle_mod.attn(q, codes, scales, idx, sk, sv, sks, svs, 128, SM)
    K, V = fp4_matrix(codes[:n_vis], scales[:n_vis])
    Ks = e4m3_value(sk) * sks[:, None].astype(np.float64)
    Vs = e4m3_value(sv) * svs[:, None].astype(np.float64)
    ref, ref_lse = dense_attention(q, np.vstack([K, Ks]), np.vstack([V, Vs]), SM)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-6)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-6)


def test_selected_subset_equals_dense_over_subset(oracle_mod):
    q, codes, scales, sk, sv, sks, svs = make_case(oracle_mod, 2, 1000)
    g = np.random.default_rng(3)
    sel = np.sort(g.choice(1000, 512, replace=False)).astype(np.int32)
    out, _ = oracle_mod.attn(q, codes, scales, sel, sk, sv, sks, svs, 50, SM)
    K, V = fp4_matrix(codes[sel], scales[sel])
    Ks = e4m3_value(sk[:50]) * sks[:50, None].astype(np.float64)
    Vs = e4m3_value(sv[:50]) * svs[:50, None].astype(np.float64)
    ref, _ = dense_attention(q, np.vstack([K, Ks]), np.vstack([V, Vs]), SM)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-6)


def test_uniform_keys_give_mean_of_values(oracle_mod):
    q, codes, scales, sk, sv, sks, svs = make_case(oracle_mod, 4, 64)
    codes[:, :64] = codes[0, :64]
    scales[:, :8] = scales[0, :8]  # all global keys identical
    sk[:] = 0
    sks[:] = 0  # window keys zero
    K0, _ = fp4_matrix(codes[:1], scales[:1])
    # make the global logit equal to the window logit (0): q orthogonal to K0
    q = q - (q @ K0[0])[:, None] * K0[0][None, :] / (K0[0] @ K0[0])
    q = q.astype(np.float32)
    idx = np.arange(64, dtype=np.int32)
    out, lse = oracle_mod.attn(q, codes, scales, idx, sk, sv, sks, svs, 128, SM)
    _, V = fp4_matrix(codes, scales)
    Vs = e4m3_value(sv) * svs[:, None].astype(np.float64)
    mean = np.vstack([V, Vs]).mean(axis=0)
    np.testing.assert_allclose(out, np.broadcast_to(mean, out.shape), rtol=0, atol=2e-5)
    np.testing.assert_allclose(lse, np.log(192.0), atol=2e-5)


def test_dominant_key_returns_its_value(oracle_mod):
    q, codes, scales, sk, sv, sks, svs = make_case(oracle_mod, 5, 64, H=1)
    K, V = fp4_matrix(codes, scales)
    q = (K[17] * 50.0).astype(np.float32)[None, :]  # logit of entry 17 dominates
    idx = np.arange(64, dtype=np.int32)
    out, _ = oracle_mod.attn(q, codes, scales, idx, sk, sv, sks, svs, 0, SM)
    np.testing.assert_allclose(out[0], V[17], rtol=0, atol=1e-5)


def test_no_keys_gives_zero_and_minus_inf(oracle_mod):
    q, codes, scales, sk, sv, sks, svs = make_case(oracle_mod, 6, 8, H=2)
    idx = np.full(8, -1, np.int32)
    out, lse = oracle_mod.attn(q, codes, scales, idx, sk, sv, sks, svs, 0, SM)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_chunk_batch_is_per_query_attention_with_causal_window(oracle_mod):
    g = np.random.default_rng(7)
    n, Q, H = 200, 6, 16
    k = g.standard_normal((1, n, 128)).astype(np.float32)
    codes, scales = oracle_mod.quant_fp4(k[0], k[0])
    codes, scales = codes[None], scales[None]
    q = g.standard_normal((1, Q, H, 128)).astype(np.float32)
    idx = np.sort(g.choice(n, (1, Q, 32)), axis=-1).astype(np.int32)
    sk, sks = oracle_mod.quant_fp8_rows(g.standard_normal((1, Q, 128)).astype(np.float32))
    sv, svs = oracle_mod.quant_fp8_rows(g.standard_normal((1, Q, 128)).astype(np.float32))
    out, lse = oracle_mod.attn_chunk_batch(q, codes, scales, idx, sk, sv, sks, svs, SM)
    for i in range(Q):
        o1, l1 = oracle_mod.attn(q[0, i], codes[0], scales[0], idx[0, i], sk[0], sv[0], sks[0],
                                 svs[0], i + 1, SM)
        np.testing.assert_array_equal(out[0, i], o1)
        np.testing.assert_array_equal(lse[0, i], l1)


def test_chunk_window_slides_past_128_tokens(oracle_mod):
    """In a chunk longer than the window, token i attends to the chunk tokens
    [i - 127, i] (the last 128 up to itself): checked against a dense numpy
    attention over the independently dequantised selected entries and exactly
    those window rows."""
    g = np.random.default_rng(8)
    n, Q, H = 300, 300, 16
    k = g.standard_normal((1, n, 128)).astype(np.float32)
    codes, scales = oracle_mod.quant_fp4(k[0], k[0][::-1].copy())
    q = g.standard_normal((1, Q, H, 128)).astype(np.float32)
    idx = np.sort(g.choice(n, (1, Q, 16)), axis=-1).astype(np.int32)
    sk, sks = oracle_mod.quant_fp8_rows(g.standard_normal((1, Q, 128)).astype(np.float32))
    sv, svs = oracle_mod.quant_fp8_rows(g.standard_normal((1, Q, 128)).astype(np.float32))
    out, lse = oracle_mod.attn_chunk_batch(q, codes[None], scales[None], idx, sk, sv, sks, svs, SM)
    K, V = fp4_matrix(codes, scales)
    WK = e4m3_value(sk[0]) * sks[0][:, None].astype(np.float64)
    WV = e4m3_value(sv[0]) * svs[0][:, None].astype(np.float64)
    for i in (0, 5, 127, 128, 129, 200, 299):
        lo = max(0, i - 127)
        kk = np.concatenate([K[idx[0, i]], WK[lo:i + 1]])
        vv = np.concatenate([V[idx[0, i]], WV[lo:i + 1]])
        o, l = dense_attention(q[0, i], kk, vv, SM)
        np.testing.assert_allclose(out[0, i], o, rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(lse[0, i], l, rtol=1e-6, atol=1e-6)


def test_decode_batch_equals_single(oracle_mod):
    g = np.random.default_rng(9)
    B, H, cap, topk = 3, 16, 96, 40
    k = g.standard_normal((B * cap, 128)).astype(np.float32)
    v = g.standard_normal((B * cap, 128)).astype(np.float32)
    codes, scales = oracle_mod.quant_fp4(k, v)
    codes, scales = codes.reshape(B, cap, 128), scales.reshape(B, cap, 16)
    q = g.standard_normal((B, H, 128)).astype(np.float32)
    idx = np.stack([np.sort(g.choice(cap, topk, replace=False)) for _ in range(B)]).astype(np.int32)
    idx[1, 30:] = -1  # a row padded with -1
    sk, sks = oracle_mod.quant_fp8_rows(g.standard_normal((B, 128, 128)).astype(np.float32))
    sv, svs = oracle_mod.quant_fp8_rows(g.standard_normal((B, 128, 128)).astype(np.float32))
    swa_len = np.array([128, 0, 57], np.int32)
    out, lse = oracle_mod.attn_decode_batch(q, codes, scales, idx, sk, sv, sks, svs, swa_len, SM)
    for b in range(B):
        o1, l1 = oracle_mod.attn(q[b], codes[b], scales[b], idx[b], sk[b], sv[b], sks[b], svs[b],
                                 swa_len[b], SM)
        np.testing.assert_array_equal(out[b], o1)
        np.testing.assert_array_equal(lse[b], l1)
