"""Edge cases of the sparse attention against the oracle (GPU).

The method's softmax over selected FP4 records and FP8 window tokens
("DeepSeek V4.1 Flash: architecture study notes", sections 1, 2 and 4) at the
extremes of its number formats and of the softmax itself:
  - peaked logits (queries scaled by 8 and 32) and a planted dominant key in
    the selected set, in the window, and in the last tile a wave processes,
    so that the running maximum has to move late;
  - FP4 records whose E4M3 group scales are saturated (byte 0x7E, values up
    to 6 * 448 = 2688) or subnormal (bytes 0x01..0x07);
  - window rows whose fp32 K and V scales span 2^-20 .. 2^4;
  - a single selected record and no window.
Every case runs the plain decode call, the staged pair (a gathering call that
writes the stage, then a call that reads it) and the chunk call, and compares
each (query, head) row with the oracle: max |o - o_ref| / max |o_ref| <= 2e-3,
and the log-sum-exp within 2e-3.
"""
import math

import numpy as np
import pytest
import torch

from gpu_util import dev, host, row_rel_err

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128.0)
TOL = 2e-3
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def say(msg):
    print(f"[attn-edges] {msg}", flush=True)


def e4m3_value(code):
    return torch.tensor(np.asarray(code, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def dequant_k(codes, scales):
    """K of FP4 records [n][128] codes / [n][16] scales, float64 (test side)."""
    nib = np.empty((codes.shape[0], 128), np.uint8)
    nib[:, 0::2] = codes[:, :64] & 0xF
    nib[:, 1::2] = codes[:, :64] >> 4
    val = E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    return val * np.repeat(e4m3_value(scales[:, :8]), 16, axis=1)


def records(oracle_mod, g, n, extreme=False):
    """FP4 records of N(0,1) K and V; with `extreme`, 10% of the groups get a
    saturated scale byte and 10% a subnormal one (codes unchanged)."""
    k = g.standard_normal((n, 128)).astype(np.float32)
    v = g.standard_normal((n, 128)).astype(np.float32)
    codes, scales = oracle_mod.quant_fp4(k, v)
    if extreme:
        u = g.random(scales.shape)
        scales = np.where(u < 0.1, np.uint8(0x7E), scales)
        sub = g.integers(1, 8, scales.shape).astype(np.uint8)
        scales = np.where((u >= 0.1) & (u < 0.2), sub, scales).astype(np.uint8)
    return codes, scales


def window(oracle_mod, g, rows, wide_sigma=False):
    """FP8 window rows [rows][128] with per-row fp32 scales; `wide_sigma`
    replaces the scales by 2^U(-20, 4), independently for K and V."""
    sk, sks = oracle_mod.quant_fp8_rows(g.standard_normal((rows, 128)).astype(np.float32))
    sv, svs = oracle_mod.quant_fp8_rows(g.standard_normal((rows, 128)).astype(np.float32))
    if wide_sigma:
        sks = np.exp2(g.uniform(-20.0, 4.0, rows)).astype(np.float32)
        svs = np.exp2(g.uniform(-20.0, 4.0, rows)).astype(np.float32)
    return sk, sv, sks, svs


CASES = {
    # name: (query scale, extreme FP4 scales, wide window sigmas, dominant key at)
    "peaked_x8": (8.0, False, False, None),
    "peaked_x32": (32.0, False, False, None),
    "dominant_global_last_tile": (1.0, False, False, "global_last"),
    "dominant_global_first_then_later": (4.0, False, False, "global_late"),
    "dominant_window": (1.0, False, False, "window"),
    "saturated_and_subnormal_scales": (1.0, True, False, None),
    "saturated_scales_peaked": (8.0, True, False, None),
    "window_sigmas_2^-20_to_2^4": (1.0, False, True, None),
    "window_sigmas_peaked": (8.0, False, True, "window"),
    "all_extremes": (32.0, True, True, "global_last"),
}


def build_decode_case(oracle_mod, name, B=3, cap=2048, H=64, topk=512, seed=0):
    qs, extreme, wide, dom = CASES[name]
    g = np.random.default_rng(9000 + seed)
    codes, scales = records(oracle_mod, g, B * cap, extreme)
    codes, scales = codes.reshape(B, cap, 128), scales.reshape(B, cap, 16)
    sk, sv, sks, svs = window(oracle_mod, g, B * 128, wide)
    sk, sv = sk.reshape(B, 128, 128), sv.reshape(B, 128, 128)
    sks, svs = sks.reshape(B, 128), svs.reshape(B, 128)
    idx = np.stack([np.sort(g.choice(cap, topk, replace=False)) for _ in range(B)]).astype(np.int32)
    q = (g.standard_normal((B, H, 128)) * qs).astype(np.float32)
    sl = np.resize(np.array([128, 77, 128], np.int32), B)
    for b in range(B):
        if dom == "global_last" or dom == "global_late":
            # global_last: slot 511 sits in the last selected tile (tile 15,
            # the last tile of the wave that takes tiles 7 and 15);
            # global_late: a weaker key in tile 0 sets the running maximum of
            # the wave that takes tiles 0, 8 and 16, and a stronger one in its
            # tile 8 (slot 261) has to move it
            late = 511 if dom == "global_last" else 261
            kd = dequant_k(codes[b, idx[b, late]][None], scales[b, idx[b, late]][None])[0]
            q[b] += (kd / max(np.abs(kd).max(), 1e-30) * 6.0 * qs).astype(np.float32)
            if dom == "global_late":
                k0 = dequant_k(codes[b, idx[b, 3]][None], scales[b, idx[b, 3]][None])[0]
                q[b, : H // 2] += (k0 / max(np.abs(k0).max(), 1e-30) * 3.0 * qs).astype(np.float32)
        elif dom == "window":
            t = int(sl[b]) - 1  # the window's last token
            kw = e4m3_value(sk[b, t]) * float(sks[b, t])
            q[b] += (kw / max(np.abs(kw).max(), 1e-30) * 6.0 * qs).astype(np.float32)
    return dict(codes=codes, scales=scales, sk=sk, sv=sv, sks=sks, svs=svs, idx=idx, q=q, sl=sl,
                B=B, cap=cap, H=H, topk=topk)


def upload_cache(gpu, c):
    cache = gpu.Cache(c["B"], c["cap"])
    cache.kv_codes.copy_(dev(c["codes"].reshape(-1, 128)))
    cache.kv_scales.copy_(dev(c["scales"].reshape(-1, 16)))
    return cache


def check(out, lse, ref_out, ref_lse, what):
    o, l = host(out), host(lse)
    bad = ~np.isfinite(o).all(axis=-1)
    assert not bad.any(), (what, "rows with non-finite values", np.argwhere(bad)[:8].tolist())
    err = row_rel_err(o, ref_out)
    say(f"{what}: max row error {err.max():.2e}")
    assert err.max() <= TOL, (what, float(err.max()))
    np.testing.assert_allclose(l, ref_lse, rtol=TOL, atol=TOL, err_msg=what)


@pytest.mark.parametrize("name", sorted(CASES))
def test_attn_decode_edges(gpu, oracle_mod, name):
    say(f"decode {name}")
    c = build_decode_case(oracle_mod, name)
    cache = upload_cache(gpu, c)
    ref_out, ref_lse = oracle_mod.attn_decode_batch(c["q"], c["codes"], c["scales"], c["idx"],
                                                    c["sk"], c["sv"], c["sks"], c["svs"], c["sl"], SM)
    out = torch.empty((c["B"], c["H"], 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((c["B"], c["H"]), dtype=torch.float32, device="cuda")
    win = (dev(c["sk"]), dev(c["sv"]), dev(c["sks"]), dev(c["svs"]), dev(c["sl"]))
    gpu.sparse_attn_decode(dev(c["q"]), cache, dev(c["idx"]), *win, out, lse)
    check(out, lse, ref_out, ref_lse, f"decode {name}")


@pytest.mark.parametrize("name", ["peaked_x32", "dominant_global_last_tile",
                                  "saturated_and_subnormal_scales", "all_extremes"])
def test_attn_reuse_stage_edges(gpu, oracle_mod, name):
    """The gathering call stages the records; a second layer with its own
    (edge-case) query and window reads them back."""
    say(f"reuse {name}")
    c = build_decode_case(oracle_mod, name, seed=1)
    c2 = build_decode_case(oracle_mod, name, seed=2)  # the second layer's query and window
    cache = upload_cache(gpu, c)
    stage = gpu.alloc_workspace(gpu.workspace_size(gpu.OP_ATTN_STAGE, c["B"], 1, c["cap"],
                                                   c["topk"], 0, c["H"]))
    for layer, src in enumerate((c, c2)):
        out = torch.empty((c["B"], c["H"], 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((c["B"], c["H"]), dtype=torch.float32, device="cuda")
        win = (dev(src["sk"]), dev(src["sv"]), dev(src["sks"]), dev(src["svs"]), dev(src["sl"]))
        if layer == 0:
            gpu.sparse_attn_decode_reuse(dev(src["q"]), cache, dev(c["idx"]), c["topk"], stage,
                                         gpu.STAGE_WRITE, *win, out, lse)
        else:
            gpu.sparse_attn_decode_reuse(dev(src["q"]), None, None, c["topk"], stage,
                                         gpu.STAGE_READ, *win, out, lse)
        ref_out, ref_lse = oracle_mod.attn_decode_batch(src["q"], c["codes"], c["scales"], c["idx"],
                                                        src["sk"], src["sv"], src["sks"],
                                                        src["svs"], src["sl"], SM)
        check(out, lse, ref_out, ref_lse, f"reuse layer {layer} {name}")


@pytest.mark.parametrize("name", ["peaked_x32", "dominant_window", "window_sigmas_2^-20_to_2^4",
                                  "all_extremes"])
def test_attn_chunk_edges(gpu, oracle_mod, name):
    qs, extreme, wide, dom = CASES[name]
    say(f"chunk {name}")
    g = np.random.default_rng(9100)
    B, Q, cap, H, topk = 1, 40, 1024, 32, 256
    codes, scales = records(oracle_mod, g, B * cap, extreme)
    codes, scales = codes.reshape(B, cap, 128), scales.reshape(B, cap, 16)
    sk, sv, sks, svs = window(oracle_mod, g, B * Q, wide)
    sk, sv = sk.reshape(B, Q, 128), sv.reshape(B, Q, 128)
    sks, svs = sks.reshape(B, Q), svs.reshape(B, Q)
    idx = np.full((B, Q, topk), -1, np.int32)
    for i in range(Q):
        n = min(topk, cap - Q + i + 1)
        idx[0, i, :n] = np.sort(g.choice(cap - Q + i + 1, n, replace=False))
    q = (g.standard_normal((B, Q, H, 128)) * qs).astype(np.float32)
    if dom == "window":
        for i in range(Q):  # each query's own chunk token dominates
            kw = e4m3_value(sk[0, i]) * float(sks[0, i])
            q[0, i] += (kw / max(np.abs(kw).max(), 1e-30) * 6.0 * qs).astype(np.float32)
    elif dom == "global_last":
        for i in range(Q):
            p = idx[0, i, topk - 1]
            kd = dequant_k(codes[0, p][None], scales[0, p][None])[0]
            q[0, i] += (kd / max(np.abs(kd).max(), 1e-30) * 6.0 * qs).astype(np.float32)
    cache = gpu.Cache(B, cap)
    cache.kv_codes.copy_(dev(codes.reshape(-1, 128)))
    cache.kv_scales.copy_(dev(scales.reshape(-1, 16)))
    ref_out, ref_lse = oracle_mod.attn_chunk_batch(q, codes, scales, idx, sk, sv, sks, svs, SM)
    out = torch.empty((B, Q, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Q, H), dtype=torch.float32, device="cuda")
    gpu.sparse_attn_chunk(dev(q), cache, dev(idx), dev(sk), dev(sv), dev(sks), dev(svs), out, lse)
    check(out, lse, ref_out, ref_lse, f"chunk {name}")


def test_attn_single_entry_no_window(gpu, oracle_mod):
    """One selected record, no window: the output is that record's V (exact in
    fp16, so to rounding of the fp32 normalisation) and the lse its logit."""
    say("single entry, swa_len 0")
    g = np.random.default_rng(9200)
    B, cap, H, topk = 2, 1024, 64, 512
    codes, scales = records(oracle_mod, g, B * cap)
    codes, scales = codes.reshape(B, cap, 128), scales.reshape(B, cap, 16)
    sk, sv, sks, svs = window(oracle_mod, g, B * 128)
    sk, sv = sk.reshape(B, 128, 128), sv.reshape(B, 128, 128)
    sks, svs = sks.reshape(B, 128), svs.reshape(B, 128)
    idx = np.full((B, topk), -1, np.int32)
    idx[0, 0] = 17
    idx[1, 300] = 1000  # the only entry sits in a middle tile
    q = (g.standard_normal((B, H, 128)) * 8.0).astype(np.float32)
    sl = np.zeros(B, np.int32)
    cache = gpu.Cache(B, cap)
    cache.kv_codes.copy_(dev(codes.reshape(-1, 128)))
    cache.kv_scales.copy_(dev(scales.reshape(-1, 16)))
    ref_out, ref_lse = oracle_mod.attn_decode_batch(q, codes, scales, idx, sk, sv, sks, svs, sl, SM)
    out = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    gpu.sparse_attn_decode(dev(q), cache, dev(idx), dev(sk), dev(sv), dev(sks), dev(svs), dev(sl),
                           out, lse)
    check(out, lse, ref_out, ref_lse, "single entry")
    np.testing.assert_array_equal(host(out), ref_out.astype(np.float32))
