"""GPU parity of whole layer stacks against the oracle, including the full-size
workloads in the launch configuration the bench times, checked on sampled
sequences / queries that the oracle computes one by one.

The caches are written by the library's own write path (csa2_quant_fp4 /
csa2_quant_fp8) from the seeded fp32 inputs; the oracle quantises the same
inputs itself, and the bytes of the sampled sequences are compared first.
"""
import math
import time

import numpy as np
import pytest
import torch

from compressed_kv_cache_decode_amd import synth
from gpu_util import dev, host, row_rel_err, untile_ik, untile_ik4

pytestmark = pytest.mark.gpu
SM = 1.0 / math.sqrt(128.0)


def say(msg):
    print(f"[gpu-case] {time.strftime('%H:%M:%S')} {msg}", flush=True)


def build_cache_on_gpu(gpu, inp, cap, rope=False):
    """Write the main KV and indexer K of every sequence with the library
    (indexer keys in the workload's format)."""
    B, n_tok = inp.k_tok.shape[:2]
    n_ent = n_tok // inp.wl.ratio
    cache = gpu.Cache(B, cap, idx_fp4=inp.wl.idx_fp4)
    for b in range(B):
        rows = cache.rows(b, np.arange(n_ent))
        cs = dev(gpu.rope_table(np.arange(n_ent))) if rope else None
        gpu.quant_fp4(dev(inp.k_tok[b]), dev(inp.v_tok[b]), cache.kv_codes, cache.kv_scales,
                      ratio=inp.wl.ratio, rope_cs=cs, dst_rows=rows)
        if inp.wl.idx_fp4:
            gpu.quant_idx_fp4(dev(inp.idx_k[b]), cache.ik_codes, cache.ik_scales4, dst_rows=rows)
        else:
            gpu.quant_fp8(dev(inp.idx_k[b]), cache.ik_codes, cache.ik_sigma,
                          layout=gpu.FP8_IDX_TILED, dst_rows=rows)
    return cache


def quantize_windows(gpu, swa_k, swa_v):
    """[L][B][128][128] fp32 -> device E4M3 codes and fp32 sigmas (library)."""
    shp = swa_k.shape
    out = []
    for x in (swa_k, swa_v):
        codes = torch.empty(int(np.prod(shp)), dtype=torch.uint8, device="cuda")
        sig = torch.empty(int(np.prod(shp[:-1])), dtype=torch.float32, device="cuda")
        gpu.quant_fp8(dev(x.reshape(-1, 128)), codes, sig)
        out += [codes.view(*shp), sig.view(*shp[:-1])]
    return out


def oracle_stack(oracle_mod, inp, b, topk, pool_blocks, plan, rope=False, new_entry_proj=None):
    """Oracle run of one sequence: bytes, per-layer indices and outputs.
    new_entry_proj: W [64][128]: the last entry's indexer key is the one the
    write path projects from its K (the others are the fixture's keys)."""
    n_ent = inp.k_tok.shape[1] // inp.wl.ratio
    cs = oracle_mod.rope_table(np.arange(n_ent)) if rope else None
    codes, scales = oracle_mod.quant_fp4(inp.k_tok[b], inp.v_tok[b], inp.wl.ratio, cs)
    fp4 = inp.wl.idx_fp4
    ikc, iks = (oracle_mod.idx4_quant_rows if fp4 else oracle_mod.quant_fp8_rows)(inp.idx_k[b])
    full = oracle_mod.index_full4 if fp4 else oracle_mod.index_full
    reindex = oracle_mod.index_reindex4 if fp4 else oracle_mod.index_reindex
    if new_entry_proj is not None:
        assert not fp4
        r = inp.wl.ratio
        _, _, ikc[-1:], iks[-1:] = oracle_mod.write_entries_proj(
            inp.k_tok[b, -r:], inp.v_tok[b, -r:], new_entry_proj, r,
            None if cs is None else cs[-1:])
    res = {"codes": codes, "scales": scales, "ikc": ikc, "iks": iks, "topk": [], "out": [],
           "lse": []}
    cur, pool, k = None, None, 0
    for layer, mode in enumerate(plan):
        if mode == "F":
            cur, pool = full(ikc, iks, n_ent, inp.iq[k, b], inp.iw[k, b], topk, pool_blocks)
            k += 1
        elif mode == "X":
            cur = reindex(ikc, iks, n_ent, inp.iq[k, b], inp.iw[k, b], pool, topk)
            k += 1
        sk, sks = oracle_mod.quant_fp8_rows(inp.swa_k[layer, b])
        sv, svs = oracle_mod.quant_fp8_rows(inp.swa_v[layer, b])
        o, l = oracle_mod.attn(inp.q[layer, b], codes, scales, cur, sk, sv, sks, svs,
                               int(inp.swa_len[b]), SM)
        res["topk"].append(cur)
        res["out"].append(o)
        res["lse"].append(l)
    return res


def run_stack_case(gpu, oracle_mod, wl, n_ent=None, B=None, layers=None, sample=None,
                   topk=512, pool_blocks=None):
    from compressed_kv_cache_decode_amd.stack import DecodeStack
    pool_blocks = wl.pool_blocks if pool_blocks is None else pool_blocks
    say(f"{wl.name}: drawing inputs")
    inp = synth.decode_inputs(wl, n_ent=n_ent, B=B, layers=layers)
    B, n_tok = inp.k_tok.shape[:2]
    n_ent = n_tok // wl.ratio
    plan = wl.plan if layers is None else wl.plan[:layers]
    cap = (n_ent + 63) // 64 * 64
    say(f"{wl.name}: B={B} n_ent={n_ent} plan={plan} -> writing caches on the GPU")
    cache = build_cache_on_gpu(gpu, inp, cap)
    swk, sks, swv, svs = quantize_windows(gpu, inp.swa_k, inp.swa_v)
    st = DecodeStack(cache, plan, B, wl.H, topk=topk, pool_blocks=pool_blocks)
    n_vis = dev(np.full((B, 1), n_ent, np.int32))
    say(f"{wl.name}: stack step on the GPU")
    used = st.step(dev(inp.iq[:, :, None]), dev(inp.iw[:, :, None]), n_vis, dev(inp.q), swk, swv,
                   sks, svs, dev(inp.swa_len))
    torch.cuda.synchronize()
    # Reuse layers attend with exactly their source layer's buffer
    for layer, src in enumerate(st.sources):
        assert used[layer].data_ptr() == used[src].data_ptr()
    kvc, kvs = host(cache.kv_codes), host(cache.kv_scales)
    if wl.idx_fp4:
        ikc_all = untile_ik4(host(cache.ik_codes), B, cap)
        iks_all = host(cache.ik_scales4).reshape(B, cap, 4)
    else:
        ikc_all = untile_ik(host(cache.ik_codes), B, cap)
        iks_all = host(cache.ik_sigma).reshape(B, cap)
    tk_all = [host(t) for t in used]
    out_all, lse_all = host(st.out), host(st.lse)
    sample = range(B) if sample is None else sample
    for b in sample:
        say(f"{wl.name}: oracle for sequence {b}")
        ref = oracle_stack(oracle_mod, inp, b, topk, pool_blocks, plan)
        r0 = b * cap
        np.testing.assert_array_equal(kvc[r0:r0 + n_ent], ref["codes"])
        np.testing.assert_array_equal(kvs[r0:r0 + n_ent], ref["scales"])
        np.testing.assert_array_equal(ikc_all[b, :n_ent], ref["ikc"])
        np.testing.assert_array_equal(iks_all[b, :n_ent], ref["iks"])
        for layer in range(len(plan)):
            np.testing.assert_array_equal(tk_all[layer][b, 0], ref["topk"][layer],
                                          err_msg=f"layer {layer} ({plan[layer]})")
            err = row_rel_err(out_all[layer, b], ref["out"][layer])
            assert err.max() <= 2e-3, (layer, err.max())
            np.testing.assert_allclose(lse_all[layer, b], ref["lse"][layer], rtol=2e-3, atol=2e-3)
    return inp, tk_all


def test_small_decoder_stack(gpu, oracle_mod):
    wl = synth.WORKLOADS["decoder_stack_128k"]
    run_stack_case(gpu, oracle_mod, wl, n_ent=20000, B=3, layers=9, topk=128, pool_blocks=256)


def test_full_layer_1k(gpu, oracle_mod):
    run_stack_case(gpu, oracle_mod, synth.WORKLOADS["full_1k"])


def test_encoder_group_16k(gpu, oracle_mod):
    """Encoder-style group: 32768 tokens averaged 2:1, 1 Full + 5 Reuse, batch 8."""
    run_stack_case(gpu, oracle_mod, synth.WORKLOADS["encoder_group_16k"])


def test_decoder_stack_128k_full_size(gpu, oracle_mod):
    """The 128K decoder stack at full size (B=16, 20 layers); oracle on 3 sequences."""
    run_stack_case(gpu, oracle_mod, synth.WORKLOADS["decoder_stack_128k"], sample=[0, 9, 15])


def test_decoder_stack_1m_full_size(gpu, oracle_mod):
    """1M-position stack (B=4) with planted clusters, all 20 layers; oracle on
    2 sequences; the planted blocks must dominate the Full layer's pool."""
    wl = synth.WORKLOADS["decoder_stack_1m"]
    inp, tk_all = run_stack_case(gpu, oracle_mod, wl, sample=[0, 3])
    for b in range(wl.B):
        planted = set((inp.planted[b][:, None] * 8 + np.arange(8)).ravel().tolist())
        sel = [p for p in tk_all[0][b, 0].tolist() if p >= 0]
        assert sum(p in planted for p in sel) > 0.5 * len(sel)


def test_decoder_stack_128k_fp4idx_full_size(gpu, oracle_mod):
    """The 128K decoder stack with FP4 indexer keys at full size (B=16, 20
    layers); oracle on 3 sequences."""
    run_stack_case(gpu, oracle_mod, synth.WORKLOADS["decoder_stack_128k_fp4idx"],
                   sample=[0, 7, 15])


def test_decoder_stack_1m_fp4idx_full_size(gpu, oracle_mod):
    """1M positions with FP4 indexer keys (B=4, planted clusters), all 20
    layers; oracle on one sequence; the planted blocks dominate the Full
    layer's selection."""
    wl = synth.WORKLOADS["decoder_stack_1m_fp4idx"]
    inp, tk_all = run_stack_case(gpu, oracle_mod, wl, sample=[2])
    for b in range(wl.B):
        planted = set((inp.planted[b][:, None] * 8 + np.arange(8)).ravel().tolist())
        sel = [p for p in tk_all[0][b, 0].tolist() if p >= 0]
        assert sum(p in planted for p in sel) > 0.5 * len(sel)


def test_graph_replay_matches_eager(gpu, oracle_mod):
    """The stack captured in a HIP graph replays to the same bytes as eager
    launches, on every replay, with unrelated eager work in between."""
    from compressed_kv_cache_decode_amd.stack import DecodeStack
    wl = synth.WORKLOADS["decoder_stack_128k"]
    inp = synth.decode_inputs(wl, n_ent=12000, B=2, layers=6)
    cap = 12032
    cache = build_cache_on_gpu(gpu, inp, cap)
    swk, sks, swv, svs = quantize_windows(gpu, inp.swa_k, inp.swa_v)
    st = DecodeStack(cache, wl.plan[:6], 2, wl.H, topk=256, pool_blocks=512)
    args = (dev(inp.iq[:, :, None]), dev(inp.iw[:, :, None]), dev(np.full((2, 1), 12000, np.int32)),
            dev(inp.q), swk, swv, sks, svs, dev(inp.swa_len))
    say("graph: eager reference")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        st.step(*args)
    torch.cuda.synchronize()
    ref_out, ref_lse, ref_tk = host(st.out).copy(), host(st.lse).copy(), host(st.topk_bufs).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st.step(*args)
    for rep in range(4):
        st.out.zero_()
        st.topk_bufs.fill_(-9)
        if st.stage is not None:
            st.stage.fill_(0x5A)  # each replay must write the stage before the Reuse layers read it
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"graph: replay {rep}")
        np.testing.assert_array_equal(host(st.out), ref_out)
        np.testing.assert_array_equal(host(st.lse), ref_lse)
        np.testing.assert_array_equal(host(st.topk_bufs), ref_tk)
        del junk


def test_staged_stack_equals_plain_stack(gpu, oracle_mod):
    """Reuse layers reading the staged records give the same bytes as Reuse
    layers gathering through the positions again."""
    from compressed_kv_cache_decode_amd.stack import DecodeStack
    wl = synth.WORKLOADS["decoder_stack_128k"]
    inp = synth.decode_inputs(wl, n_ent=9000, B=3, layers=10)
    cap = 9024
    cache = build_cache_on_gpu(gpu, inp, cap)
    swk, sks, swv, svs = quantize_windows(gpu, inp.swa_k, inp.swa_v)
    args = (dev(inp.iq[:, :, None]), dev(inp.iw[:, :, None]), dev(np.full((3, 1), 9000, np.int32)),
            dev(inp.q), swk, swv, sks, svs, dev(inp.swa_len))
    outs = []
    for staged in (True, False):
        say(f"stack with staging={staged}")
        st = DecodeStack(cache, wl.plan[:10], 3, wl.H, topk=512, pool_blocks=1024, stage=staged)
        assert (st.stage is not None) == staged
        st.step(*args)
        torch.cuda.synchronize()
        outs.append((host(st.out).copy(), host(st.lse).copy()))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("ratio_wl", ["decoder_stack_128k", "encoder_group_16k"])
def test_decode_step_with_write_path(gpu, oracle_mod, ratio_wl):
    """One whole decode step: the write path in one launch (every sequence's
    new entry with its indexer key projected on the device, and every layer's
    new window token appended at ring slot t mod 128), then the stack; bytes,
    indices and outputs against the oracle.  Before the step the new entry's
    cache rows and the windows' ring slots hold other data."""
    from compressed_kv_cache_decode_amd.stack import DecodeStack
    wl = synth.WORKLOADS[ratio_wl]
    layers = 9 if wl.ratio == 1 else 6
    n_ent = 6001 if wl.ratio == 1 else 3001
    inp = synth.decode_inputs(wl, n_ent=n_ent, B=3, layers=layers)
    B, plan, r = 3, wl.plan[:layers], wl.ratio
    rope = wl.ratio == 1
    cap = (n_ent + 63) // 64 * 64
    say(f"write path step {ratio_wl}: B={B} n_ent={n_ent} plan={plan}")
    cache = build_cache_on_gpu(gpu, inp, cap, rope=rope)
    last = n_ent - 1
    slot = (last * r + r - 1) % 128  # ring slot of the newest token
    stale_k, stale_v = inp.swa_k.copy(), inp.swa_v.copy()
    stale_k[:, :, slot] = 7.0
    stale_v[:, :, slot] = -3.0
    swk, sks, swv, svs = quantize_windows(gpu, stale_k, stale_v)
    for b in range(B):  # stale bytes in the new entry's rows
        cache.kv_codes[b * cap + last].fill_(0x11)
        cache.ik_sigma[b * cap + last] = 123.0
    st = DecodeStack(cache, plan, B, wl.H, topk=128, pool_blocks=256 if "X" in plan else 0)
    k_new = dev(np.ascontiguousarray(inp.k_tok[:, last * r:last * r + r].reshape(-1, 128)))
    v_new = dev(np.ascontiguousarray(inp.v_tok[:, last * r:last * r + r].reshape(-1, 128)))
    rows_new = torch.arange(B, dtype=torch.int64, device="cuda") * cap + last
    L = len(plan)
    win_rows = dev(((np.arange(L)[:, None] * B + np.arange(B)[None, :]) * 128 + slot)
                   .reshape(-1).astype(np.int64))
    win_k = dev(np.ascontiguousarray(inp.swa_k[:, :, slot].reshape(-1, 128)))
    win_v = dev(np.ascontiguousarray(inp.swa_v[:, :, slot].reshape(-1, 128)))
    st.write(k_new, v_new, rows_new, dev(inp.proj), win_k, win_v, win_rows, swk, swv, sks, svs,
             ratio=r, rope_cs=dev(gpu.rope_table(np.full(B, last))) if rope else None)
    used = st.step(dev(inp.iq[:, :, None]), dev(inp.iw[:, :, None]),
                   dev(np.full((B, 1), n_ent, np.int32)), dev(inp.q), swk, swv, sks, svs,
                   dev(inp.swa_len))
    torch.cuda.synchronize()
    kvc, kvs = host(cache.kv_codes), host(cache.kv_scales)
    ikc_all = untile_ik(host(cache.ik_codes), B, cap)
    iks_all = host(cache.ik_sigma).reshape(B, cap)
    for li in range(L):
        for b in range(B):
            ck, sk_ = oracle_mod.quant_fp8_rows(inp.swa_k[li, b])
            np.testing.assert_array_equal(host(swk[li, b]), ck)
            np.testing.assert_array_equal(host(sks[li, b]), sk_)
            cv, sv_ = oracle_mod.quant_fp8_rows(inp.swa_v[li, b])
            np.testing.assert_array_equal(host(swv[li, b]), cv)
            np.testing.assert_array_equal(host(svs[li, b]), sv_)
    for b in range(B):
        say(f"write path step {ratio_wl}: oracle for sequence {b}")
        ref = oracle_stack(oracle_mod, inp, b, 128, st.pool_blocks, plan, rope=rope,
                           new_entry_proj=inp.proj)
        r0 = b * cap
        np.testing.assert_array_equal(kvc[r0:r0 + n_ent], ref["codes"])
        np.testing.assert_array_equal(kvs[r0:r0 + n_ent], ref["scales"])
        np.testing.assert_array_equal(ikc_all[b, :n_ent], ref["ikc"])
        np.testing.assert_array_equal(iks_all[b, :n_ent], ref["iks"])
        for layer in range(L):
            np.testing.assert_array_equal(host(used[layer])[b, 0], ref["topk"][layer],
                                          err_msg=f"layer {layer} ({plan[layer]})")
            err = row_rel_err(host(st.out)[layer, b], ref["out"][layer])
            assert err.max() <= 2e-3, (layer, err.max())


def prepare_group(gpu, inp, B, plan, rope):
    """Caches and windows of one layer group with the step's ring slot and new
    entry holding stale data, and the arguments of its write and its step."""
    r = inp.wl.ratio
    n_ent = inp.k_tok.shape[1] // r
    cap = (n_ent + 63) // 64 * 64
    cache = build_cache_on_gpu(gpu, inp, cap, rope=rope)
    last = n_ent - 1
    slot = (last * r + r - 1) % 128
    stale_k, stale_v = inp.swa_k.copy(), inp.swa_v.copy()
    stale_k[:, :, slot], stale_v[:, :, slot] = 5.0, -2.0
    swk, sks, swv, svs = quantize_windows(gpu, stale_k, stale_v)
    for b in range(B):
        cache.kv_codes[b * cap + last].fill_(0x22)
        cache.ik_sigma[b * cap + last] = 77.0
    L = len(plan)
    wr = dict(k_new=dev(np.ascontiguousarray(inp.k_tok[:, last * r:last * r + r].reshape(-1, 128))),
              v_new=dev(np.ascontiguousarray(inp.v_tok[:, last * r:last * r + r].reshape(-1, 128))),
              rows_new=torch.arange(B, dtype=torch.int64, device="cuda") * cap + last,
              idx_proj=dev(inp.proj),
              win_k=dev(np.ascontiguousarray(inp.swa_k[:, :, slot].reshape(-1, 128))),
              win_v=dev(np.ascontiguousarray(inp.swa_v[:, :, slot].reshape(-1, 128))),
              win_rows=dev(((np.arange(L)[:, None] * B + np.arange(B)[None, :]) * 128 + slot)
                           .reshape(-1).astype(np.int64)),
              ratio=r, rope_cs=dev(gpu.rope_table(np.full(B, last))) if rope else None)
    args = dict(iq=dev(inp.iq[:, :, None]), iw=dev(inp.iw[:, :, None]),
                n_vis=dev(np.full((B, 1), n_ent, np.int32)), q=dev(inp.q), swk=swk, swv=swv,
                sks=sks, svs=svs, swa_len=dev(inp.swa_len))
    return cache, wr, args


def test_model_step_all_40_layers(gpu, oracle_mod):
    """One decode step of the whole layer plan (2 window-only layers, three
    encoder groups F+5R over 2:1 entries, the decoder F+4X+15R) at a 4000-token
    context: every layer's indices and output against the oracle."""
    from compressed_kv_cache_decode_amd import stack as S
    B, T, topk, pool = 2, 4000, 512, 2048
    wl_e, wl_d = synth.WORKLOADS["encoder_group_16k"], synth.WORKLOADS["decoder_stack_128k"]
    groups = [(synth.decode_inputs(wl_e, n_ent=T // 2, B=B, seed=3000 + g), S.ENCODER_GROUP_PLAN,
               False) for g in range(S.ENCODER_GROUPS)]
    groups.append((synth.decode_inputs(wl_d, n_ent=T, B=B, seed=3100), S.DECODER_PLAN, True))
    say("model step: writing four caches")
    prepared = [prepare_group(gpu, inp, B, plan, rope) for inp, plan, rope in groups]
    g = np.random.default_rng(3200)
    H, W = wl_d.H, S.ENCODER_WINDOW_ONLY
    wq = g.standard_normal((W, B, H, 128), dtype=np.float32)
    wk = g.standard_normal((W, B, 128, 128), dtype=np.float32)
    wv = g.standard_normal((W, B, 128, 128), dtype=np.float32)
    slot = (T - 1) % 128
    wsk, wsks, wsv, wsvs = quantize_windows(gpu, np.zeros_like(wk), np.zeros_like(wv))
    win = dict(q=dev(wq), swk=wsk, swv=wsv, sks=wsks, svs=wsvs,
               swa_len=dev(np.full(B, 128, np.int32)),
               win_k=dev(np.ascontiguousarray(wk[:, :, slot].reshape(-1, 128))),
               win_v=dev(np.ascontiguousarray(wv[:, :, slot].reshape(-1, 128))),
               win_rows=dev(((np.arange(W)[:, None] * B + np.arange(B)[None, :]) * 128 + slot)
                            .reshape(-1).astype(np.int64)))
    # the window-only layers' other slots are written up front
    wk_stale, wv_stale = wk.copy(), wv.copy()
    wk_stale[:, :, slot], wv_stale[:, :, slot] = 1.0, 1.0
    for x, codes, sig in ((wk_stale, wsk, wsks), (wv_stale, wsv, wsvs)):
        gpu.quant_fp8(dev(x.reshape(-1, 128)), codes, sig)
    model = S.ModelStep([p[0] for p in prepared[:3]], prepared[3][0], B, H, topk=topk,
                        pool_blocks=pool)
    assert model.layers == 40
    say("model step: one step on the GPU")
    used = model.step([p[1] for p in prepared], win, [p[2] for p in prepared[:3]],
                      prepared[3][2])
    torch.cuda.synchronize()
    for i in range(W):
        for b in range(B):
            sk, sks_ = oracle_mod.quant_fp8_rows(wk[i, b])
            sv, svs_ = oracle_mod.quant_fp8_rows(wv[i, b])
            codes = np.zeros((1, 128), np.uint8)
            scales = np.zeros((1, 16), np.uint8)
            o, _ = oracle_mod.attn(wq[i, b], codes, scales, np.full(0, -1, np.int32), sk, sv,
                                   sks_, svs_, 128, SM)
            err = row_rel_err(host(model.win_out[i, b]), o)
            assert err.max() <= 2e-3, ("window-only", i, b, err.max())
    stacks = model.enc + [model.dec]
    for gi, ((inp, plan, rope), st) in enumerate(zip(groups, stacks)):
        for b in range(B):
            say(f"model step: oracle for group {gi} sequence {b}")
            ref = oracle_stack(oracle_mod, inp, b, topk, st.pool_blocks, plan, rope=rope,
                               new_entry_proj=inp.proj)
            for layer in range(len(plan)):
                np.testing.assert_array_equal(host(used[gi][layer])[b, 0], ref["topk"][layer],
                                              err_msg=f"group {gi} layer {layer}")
                err = row_rel_err(host(st.out)[layer, b], ref["out"][layer])
                assert err.max() <= 2e-3, (gi, layer, err.max())
