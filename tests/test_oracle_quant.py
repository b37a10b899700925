"""Pins of the oracle's write path: FP4 records, pair averaging, RoPE, FP8 rows.

References: the pages' 4.5 bits per value (golden/page_constants.json), torch's
E4M3 cast, numpy float32 arithmetic (IEEE), numpy fp64 trigonometry, and
hand-derived special cases.
"""
import json
import os

import numpy as np
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e4m3_value(code):
    return torch.tensor(np.asarray(code, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e4m3_rne(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def unpack_nibbles(codes):
    codes = np.asarray(codes, np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


def fp4_dequant(codes64, scales8):
    """Independent decode of one 128-channel half-record: table x torch E4M3."""
    nib = unpack_nibbles(codes64)
    mag = E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    return mag * np.repeat(e4m3_value(scales8), 16)


def test_four_and_a_half_bits_per_value(oracle_mod):
    gold = json.load(open(os.path.join(GOLD, "page_constants.json")))
    k = np.random.default_rng(0).standard_normal((3, 128)).astype(np.float32)
    codes, scales = oracle_mod.quant_fp4(k, k)
    bits_k = (codes.shape[1] // 2 + scales.shape[1] // 2) * 8 / 128  # K half of a record
    assert bits_k == gold["bits_per_fp4_value"]["value"] == 4 + 8 / 16
    assert gold["fp4_scale_group_channels"]["value"] == 128 // (scales.shape[1] // 2)


def test_fp4_scale_is_rne_of_amax_over_6(oracle_mod):
    g = np.random.default_rng(1)
    x = (g.standard_normal((200, 128)) * np.exp2(g.integers(-12, 10, (200, 1)))).astype(np.float32)
    for row in x:
        _, scales = oracle_mod.fp4_quant_vec(row)
        amax = np.abs(row.reshape(8, 16)).max(axis=1)
        s32 = (amax / np.float32(6.0)).astype(np.float32)
        ref = np.where(s32 >= 464, 0x7E, e4m3_rne(np.minimum(s32, 463)))
        np.testing.assert_array_equal(scales, ref)


def test_fp4_reconstruction_within_half_grid_step(oracle_mod):
    g = np.random.default_rng(2)
    x = (g.standard_normal((300, 128)) * np.exp2(g.integers(-8, 8, (300, 1)))).astype(np.float32)
    for row in x:
        codes, scales = oracle_mod.fp4_quant_vec(row)
        deq = fp4_dequant(codes, scales)
        sd = np.repeat(e4m3_value(scales), 16)
        zero = sd == 0  # amax/6 rounded to a zero scale: |x| <= 6 * 2^-10, codes are zeros
        assert np.all(deq[zero] == 0) and np.all(np.abs(row[zero]) <= 6 * 2.0 ** -10)
        row, deq, sd = row[~zero], deq[~zero], sd[~zero]
        t = np.abs(row.astype(np.float64)) / sd
        half_step = np.where(t <= 2, 0.25, np.where(t <= 4, 0.5, 1.0))
        clip = np.maximum(t - 6.0, 0.0)  # saturation above 6 * scale
        err = np.abs(deq - row.astype(np.float64)) / sd
        assert np.all(err <= half_step + clip + 1e-6), err.max()
        assert np.all(np.sign(deq) * np.sign(row) >= 0)


def test_fp4_exact_group_and_nibble_order(oracle_mod):
    # amax/6 = 0.25 is an E4M3 value, so every x/scale below is on the grid
    x = np.zeros(128, np.float32)
    x[:8] = [1.5, -0.75, 0.375, 0.125, 0.0, -1.0, 0.5, 0.25]
    x[16] = -3.0  # second group, amax/6 = 0.5
    codes, scales = oracle_mod.fp4_quant_vec(x)
    assert e4m3_value(scales[0]) == 0.25 and e4m3_value(scales[1]) == 0.5
    # t = x/0.25: 6, -3, 1.5, 0.5, 0, -4, 2, 1 -> codes 7, 13, 3, 1, 0, 14, 4, 2
    assert list(unpack_nibbles(codes)[:8]) == [7, 13, 3, 1, 0, 14, 4, 2]
    assert codes[0] == 7 | (13 << 4)  # channel 0 in the low nibble
    assert unpack_nibbles(codes)[16] == 7 | 8
    # all-zero groups: scale 0 and signed zero codes
    assert all(scales[2:] == 0)
    assert all(unpack_nibbles(codes)[32:] == 0)
    y = np.zeros(128, np.float32)
    y[40] = -0.0
    codes, scales = oracle_mod.fp4_quant_vec(y)
    assert unpack_nibbles(codes)[40] == 8 and scales[2] == 0


def test_fp4_saturation_of_scale_and_values(oracle_mod):
    x = np.zeros(128, np.float32)
    x[0], x[1] = 1e5, -1e5  # amax/6 > 448: scale saturates at 448, codes at 6
    codes, scales = oracle_mod.fp4_quant_vec(x)
    assert scales[0] == 0x7E
    assert list(unpack_nibbles(codes)[:2]) == [7, 15]


def test_pair_average_is_float32_mean(oracle_mod):
    g = np.random.default_rng(3)
    a = g.standard_normal(1000).astype(np.float32)
    b = g.standard_normal(1000).astype(np.float32)
    a[:3] = [2.0 ** 24, 1.0, 3.0e38]
    b[:3] = [1.0, 2.0 ** -149, 3.0e38]
    got = oracle_mod.average_pair(a, b)
    with np.errstate(over="ignore"):
        ref = (a + b) * np.float32(0.5)  # numpy float32: IEEE add then multiply
    np.testing.assert_array_equal(got, ref)
    assert got[0] == 2.0 ** 23  # 2^24 + 1 rounds to 2^24 (tie to even)


def test_quant_fp4_ratio2_equals_quant_of_average(oracle_mod):
    g = np.random.default_rng(4)
    k = g.standard_normal((8, 128)).astype(np.float32)
    v = g.standard_normal((8, 128)).astype(np.float32)
    codes, scales = oracle_mod.quant_fp4(k, v, ratio=2)
    for e in range(4):
        ka = (k[2 * e] + k[2 * e + 1]) * np.float32(0.5)
        c, s = oracle_mod.fp4_quant_vec(ka)
        np.testing.assert_array_equal(codes[e, :64], c)
        np.testing.assert_array_equal(scales[e, :8], s)


def test_rope_table_against_numpy(oracle_mod):
    pos = np.array([0, 1, 7, 1000, 131071, 1048575], np.int64)
    cs = oracle_mod.rope_table(pos)
    j = np.arange(32)
    theta = 10000.0 ** (-j / 32.0)
    ang = pos[:, None].astype(np.float64) * theta[None, :]
    np.testing.assert_array_equal(cs[..., 0], np.cos(ang).astype(np.float32))
    np.testing.assert_array_equal(cs[..., 1], np.sin(ang).astype(np.float32))
    assert cs[0, :, 0].tolist() == [1.0] * 32 and cs[0, :, 1].tolist() == [0.0] * 32


def test_rope_apply_is_a_rotation_of_interleaved_pairs(oracle_mod):
    g = np.random.default_rng(5)
    x = g.standard_normal(128).astype(np.float32)
    cs = oracle_mod.rope_table(np.array([12345]))[0]
    y = oracle_mod.rope_apply(x, cs)
    np.testing.assert_array_equal(y[64:], x[64:])  # only channels 0..63 rotate
    z = (x[0:64:2] + 1j * x[1:64:2]).astype(np.complex128) * (cs[:, 0] + 1j * cs[:, 1])
    np.testing.assert_allclose(y[0:64:2], z.real, rtol=0, atol=4e-7 * np.abs(x[:64]).max())
    np.testing.assert_allclose(y[1:64:2], z.imag, rtol=0, atol=4e-7 * np.abs(x[:64]).max())
    y0 = oracle_mod.rope_apply(x, oracle_mod.rope_table(np.array([0]))[0])
    np.testing.assert_array_equal(y0, x)  # angle 0: identity


def test_rope_quantised_after_rotation(oracle_mod):
    g = np.random.default_rng(6)
    k = g.standard_normal((4, 128)).astype(np.float32)
    cs = oracle_mod.rope_table(np.arange(100, 104))
    codes, scales = oracle_mod.quant_fp4(k, k, ratio=1, rope_cs=cs)
    for e in range(4):
        c, s = oracle_mod.fp4_quant_vec(oracle_mod.rope_apply(k[e], cs[e]))
        np.testing.assert_array_equal(codes[e, :64], c)
        c2, _ = oracle_mod.fp4_quant_vec(k[e])
        np.testing.assert_array_equal(codes[e, 64:], c2)  # V is not rotated


def test_fp8_rows_against_torch(oracle_mod):
    g = np.random.default_rng(8)
    x = (g.standard_normal((64, 128)) * np.exp2(g.integers(-20, 20, (64, 1)))).astype(np.float32)
    x[3] = 0.0
    x[4, 5] = -0.0
    codes, sigma = oracle_mod.quant_fp8_rows(x)
    amax = np.abs(x).max(axis=1)
    np.testing.assert_array_equal(sigma, (amax / np.float32(448.0)).astype(np.float32))
    for r in range(64):
        if sigma[r] == 0:
            assert np.all(codes[r] == np.where(np.signbit(x[r]), 0x80, 0))
            continue
        t = (x[r] / sigma[r]).astype(np.float32)
        ref = e4m3_rne(np.clip(t, -463, 463))
        np.testing.assert_array_equal(codes[r], ref)
        assert np.abs(e4m3_value(codes[r])).max() == 448.0  # the amax element hits 448


# ---- indexer-key projection (write path) ---------------------------------
def _proj_case(x_vals, w_vals):
    W = np.zeros((64, 128), np.float32)
    x = np.zeros((1, 128), np.float32)
    W[0, :len(w_vals)] = w_vals
    x[0, :len(x_vals)] = x_vals
    return x, W


def test_projection_accumulates_channels_in_ascending_order(oracle_mod):
    """[2^24, 0, 1, 1]: adding the 1s one at a time to 2^24 rounds each away
    (half an ulp, ties to even), so the ascending chain gives 2^24, while a
    pairwise tree or the reverse order gives 2^24 + 2."""
    x, W = _proj_case([2.0 ** 24, 0.0, 1.0, 1.0], [1.0] * 4)
    assert oracle_mod.project_idx(x, W)[0, 0] == np.float32(2.0 ** 24)
    x, W = _proj_case([1.0, 1.0, 0.0, 2.0 ** 24], [1.0] * 4)
    assert oracle_mod.project_idx(x, W)[0, 0] == np.float32(2.0 ** 24 + 2)


def test_projection_steps_are_fused_multiply_adds(oracle_mod):
    """(1 + 2^-12)^2 - 1 = 2^-11 + 2^-24 exactly when the product is not
    rounded before the add; a rounded product would give 2^-11."""
    a = 1.0 + 2.0 ** -12
    x, W = _proj_case([-1.0, a], [1.0, a])
    assert oracle_mod.project_idx(x, W)[0, 0] == np.float32(2.0 ** -11 + 2.0 ** -24)


def test_projection_against_fp64_within_summation_bound(oracle_mod):
    """Every output within gamma_128 * sum_c |W x| of the fp64 product (the
    bound of a 128-term recursive sum with one rounding per step); a
    transposed or dropped operand misses by orders of magnitude."""
    g = np.random.default_rng(11)
    W = (g.standard_normal((64, 128)) / np.sqrt(128)).astype(np.float32)
    x = (g.standard_normal((50, 128)) * np.exp2(g.integers(-6, 6, (50, 1)))).astype(np.float32)
    got = oracle_mod.project_idx(x, W).astype(np.float64)
    exact = x.astype(np.float64) @ W.astype(np.float64).T
    mag = np.abs(x.astype(np.float64)) @ np.abs(W.astype(np.float64)).T
    u = 2.0 ** -24
    gamma = 128 * u / (1 - 128 * u)
    assert np.all(np.abs(got - exact) <= gamma * mag)
    assert np.abs(got - exact).max() > 0  # rounding does happen: fp32, not fp64


def test_projection_small_integers_exact(oracle_mod):
    """Small-integer operands: every partial sum is an integer below 2^24, so
    the chain equals the integer matrix product exactly."""
    g = np.random.default_rng(12)
    W = g.integers(-8, 9, (64, 128)).astype(np.float32)
    x = g.integers(-8, 9, (7, 128)).astype(np.float32)
    exact = x.astype(np.int64) @ W.astype(np.int64).T
    np.testing.assert_array_equal(oracle_mod.project_idx(x, W), exact.astype(np.float32))


def test_entry_k_is_what_the_fp4_write_quantises(oracle_mod):
    """The projected input is the entry's K after the pair mean / RoPE: FP4 of
    entry_k with ratio 1 and no RoPE reproduces the records of the full write."""
    g = np.random.default_rng(13)
    k = g.standard_normal((20, 128)).astype(np.float32)
    v = g.standard_normal((20, 128)).astype(np.float32)
    for ratio, cs in ((2, None), (1, oracle_mod.rope_table(np.arange(300, 320)))):
        xk = oracle_mod.entry_k(k, ratio, cs)
        xv = oracle_mod.entry_k(v, ratio, None)
        assert xk.shape == (20 // ratio, 128)
        direct = oracle_mod.quant_fp4(k, v, ratio, cs)
        again = oracle_mod.quant_fp4(xk, xv, 1, None)
        np.testing.assert_array_equal(direct[0], again[0])
        np.testing.assert_array_equal(direct[1], again[1])
    rot = oracle_mod.entry_k(k[:1], 1, oracle_mod.rope_table(np.array([0])))
    np.testing.assert_array_equal(rot, k[:1])  # position 0: cos 1, sin 0
