"""Layer-plan drivers: one decode step of a CSA2 layer stack over a shared
cache, and one bounded-replay chunk through such a stack.

"DeepSeek V4.1 Flash: architecture study notes", section 2: every CSA2 layer
is statically Full, Reindex or Reuse; the decoder is one Full layer, four
Reindex and fifteen Reuse layers over one shared global KV; every layer keeps
its own attention query and its own local window.  "DeepSeek V4.1 Flash is
live", "CSA2 attention": the decoder's groups are headed by Reindex layers.

A plan is a string over {F, X, R}: F = Full (index_full, writes the pool),
X = Reindex (index_reindex inside the latest pool), R = Reuse (no indexer
call; attends to the most recent Full/Reindex top-K).  Every layer calls the
sparse attention with its own q and window.  With staging (the default), a
Full/Reindex layer's attention also writes the records it gathered to a
stage buffer, and the Reuse layers after it read them from there instead of
gathering through the same positions again (the cache is shared by every
layer, so the records are the same).  This module only sequences library
calls; buffers are allocated once, up front.

"DeepSeek V4.1 Flash: architecture study notes", section 5: a decoder whose
window state is gone replays the last 128 tokens; ChunkStack runs those
tokens through every layer of the plan, each replayed token with its own
Full/Reindex selection (and, for the Reindex layers, its own pool from the
Full layer) and its in-chunk causal window.
"""
import torch

from . import (DEFAULT_POOL_BLOCKS, DEFAULT_TOPK, HEAD_DIM, OP_ATTN_CHUNK, OP_ATTN_DECODE,
               OP_ATTN_STAGE, OP_INDEX_FULL, OP_INDEX_REINDEX, STAGE_READ, STAGE_WRITE,
               alloc_workspace, index_full, index_reindex, sparse_attn_chunk, sparse_attn_decode,
               sparse_attn_decode_reuse, workspace_size, write_entries)


def check_plan(plan, pool_blocks):
    if not plan or plan[0] != "F":
        raise ValueError("a plan starts with a Full layer")
    if any(m not in "FXR" for m in plan):
        raise ValueError("plan letters are F (Full), X (Reindex), R (Reuse)")
    if "X" in plan and pool_blocks <= 0:
        raise ValueError("Reindex layers need a pool (pool_blocks > 0)")


def reuse_sources(plan):
    """For each layer, the index of the layer whose top-K it attends with."""
    src, last = [], None
    for i, m in enumerate(plan):
        if m in "FX":
            last = i
        src.append(last)
    return src


class DecodeStack:
    """Buffers and workspaces for one stack of `plan` over `cache`, batch B, H heads."""

    def __init__(self, cache, plan, B, H, topk=DEFAULT_TOPK, pool_blocks=DEFAULT_POOL_BLOCKS,
                 stage=True):
        check_plan(plan, pool_blocks)
        self.cache, self.plan, self.B, self.H = cache, plan, B, H
        self.topk, self.pool_blocks = topk, pool_blocks
        dev = cache.kv_codes.device
        n_idx = sum(1 for m in plan if m in "FX")
        self.topk_bufs = torch.empty((n_idx, B, 1, topk), dtype=torch.int32, device=dev)
        self.pool = torch.empty((B, 1, max(pool_blocks, 1)), dtype=torch.int32, device=dev)
        self.ws_full = alloc_workspace(
            workspace_size(OP_INDEX_FULL, B, 1, cache.cap, topk, pool_blocks, 0), dev)
        self.ws_reindex = (alloc_workspace(
            workspace_size(OP_INDEX_REINDEX, B, 1, cache.cap, topk, pool_blocks, 0), dev)
            if "X" in plan else None)
        n_attn = workspace_size(OP_ATTN_DECODE, B, 1, cache.cap, topk, 0, H)
        self.ws_attn = alloc_workspace(n_attn, dev) if n_attn else None
        self.out = torch.empty((len(plan), B, H, HEAD_DIM), dtype=torch.float32, device=dev)
        self.lse = torch.empty((len(plan), B, H), dtype=torch.float32, device=dev)
        self.sources = reuse_sources(plan)
        self.stage = (alloc_workspace(workspace_size(OP_ATTN_STAGE, B, 1, cache.cap, topk, 0, H),
                                      dev) if stage and topk > 0 else None)

    def write(self, k_new, v_new, rows_new, idx_proj, win_k, win_v, win_rows, swa_k, swa_v,
              swa_ks, swa_vs, ratio=1, rope_cs=None, stream=None):
        """Write path of one decode step, in one launch: the new entry of every
        sequence (FP4 record and its indexer key, projected on the device from
        the entry's K by idx_proj [64][128], at rows_new [B] of the shared
        cache) and every layer's new window token (FP8 K and V rows win_k,
        win_v [L*B][128] f32 at rows win_rows [L*B] of the stacked windows
        [L][B][128][128]: slot t mod 128 of a 128-token ring for token t).
        k_new, v_new: [B*ratio][128] f32 (the tokens of each new entry)."""
        L = len(self.plan)
        write_entries(k_new, v_new, self.cache.kv_codes, self.cache.kv_scales, ratio=ratio,
                      rope_cs=rope_cs, dst_rows=rows_new, idx_proj=idx_proj,
                      ik_codes=self.cache.ik_codes, ik_sigma=self.cache.ik_sigma,
                      ik_scales4=self.cache.ik_scales4,
                      fp8_jobs=[dict(x=win_k, codes=swa_k.view(L * self.B * 128, HEAD_DIM),
                                     sigma=swa_ks.view(-1), dst_rows=win_rows),
                                dict(x=win_v, codes=swa_v.view(L * self.B * 128, HEAD_DIM),
                                     sigma=swa_vs.view(-1), dst_rows=win_rows)],
                      stream=stream)

    def step(self, iq, iw, n_vis, q, swa_k, swa_v, swa_ks, swa_vs, swa_len, stream=None,
             scan_timer=None, attn_timer=None, index_events=None):
        """One decode step.

        iq [n_idx][B][1][4][64], iw [n_idx][B][1][4]: one indexer query per
        Full/Reindex layer; n_vis [B][1] int32; q [L][B][H][128];
        swa_k/v [L][B][128][128] u8, swa_ks/vs [L][B][128] f32, swa_len [B].
        scan_timer: optional KernelTimer bracketing the Full layer's scan;
        attn_timer: optional KernelTimer bracketing every layer's attention kernel;
        index_events: optional list; each Full / Reindex call is appended to it
        as (mode, start, end) timing events recorded on the current stream.
        Returns the list of top-K buffers each layer attended with."""
        used, cur, k = [], None, 0
        for layer, mode in enumerate(self.plan):
            if index_events is not None and mode in "FX":
                ev = (mode, torch.cuda.Event(enable_timing=True),
                      torch.cuda.Event(enable_timing=True))
                ev[1].record()
            if mode == "F":
                index_full(self.cache, iq[k], iw[k], n_vis, self.topk_bufs[k],
                           self.pool if self.pool_blocks else None, topk=self.topk,
                           pool_blocks=self.pool_blocks, ws=self.ws_full, stream=stream,
                           scan_timer=scan_timer)
                cur, k = self.topk_bufs[k], k + 1
            elif mode == "X":
                index_reindex(self.cache, iq[k], iw[k], n_vis, self.pool, self.topk_bufs[k],
                              topk=self.topk, ws=self.ws_reindex, stream=stream)
                cur, k = self.topk_bufs[k], k + 1
            if index_events is not None and mode in "FX":
                ev[2].record()
                index_events.append(ev)
            if self.stage is None:
                sparse_attn_decode(q[layer], self.cache, cur.view(self.B, self.topk),
                                   swa_k[layer], swa_v[layer], swa_ks[layer], swa_vs[layer],
                                   swa_len, self.out[layer], self.lse[layer], ws=self.ws_attn,
                                   stream=stream, timer=attn_timer)
            else:
                sparse_attn_decode_reuse(
                    q[layer], self.cache, cur.view(self.B, self.topk), self.topk, self.stage,
                    STAGE_READ if mode == "R" else STAGE_WRITE, swa_k[layer], swa_v[layer],
                    swa_ks[layer], swa_vs[layer], swa_len, self.out[layer], self.lse[layer],
                    ws=self.ws_attn, stream=stream, timer=attn_timer)
            used.append(cur)
        return used


class ChunkStack:
    """Buffers and workspaces for a Q-token replay chunk through `plan` over
    `cache` (B sequences, H heads): per layer and chunk token, the indices it
    attends with, its output and lse."""

    def __init__(self, cache, plan, B, Q, H, topk=DEFAULT_TOPK, pool_blocks=DEFAULT_POOL_BLOCKS):
        check_plan(plan, pool_blocks)
        self.cache, self.plan, self.B, self.Q, self.H = cache, plan, B, Q, H
        self.topk, self.pool_blocks = topk, pool_blocks
        dev = cache.kv_codes.device
        n_idx = sum(1 for m in plan if m in "FX")
        self.topk_bufs = torch.empty((n_idx, B, Q, topk), dtype=torch.int32, device=dev)
        self.pool = torch.empty((B, Q, max(pool_blocks, 1)), dtype=torch.int32, device=dev)
        self.ws_full = alloc_workspace(
            workspace_size(OP_INDEX_FULL, B, Q, cache.cap, topk, pool_blocks, 0), dev)
        self.ws_reindex = (alloc_workspace(
            workspace_size(OP_INDEX_REINDEX, B, Q, cache.cap, topk, pool_blocks, 0), dev)
            if "X" in plan else None)
        n_attn = workspace_size(OP_ATTN_CHUNK, B, Q, cache.cap, topk, 0, H)
        self.ws_attn = alloc_workspace(n_attn, dev) if n_attn else None
        self.out = torch.empty((len(plan), B, Q, H, HEAD_DIM), dtype=torch.float32, device=dev)
        self.lse = torch.empty((len(plan), B, Q, H), dtype=torch.float32, device=dev)
        self.sources = reuse_sources(plan)

    def step(self, iq, iw, n_vis, q, swa_k, swa_v, swa_ks, swa_vs, stream=None, scan_timer=None):
        """One replay chunk through the stack.

        iq [n_idx][B][Q][4][64], iw [n_idx][B][Q][4]: per Full/Reindex layer and
        chunk token; n_vis [B][Q] int32 (token i sees entries [0, n_vis)); q
        [L][B][Q][H][128]; swa_k/v [L][B][Q][128] u8, swa_ks/vs [L][B][Q] f32:
        each layer's window over the chunk's tokens.  Returns the top-K buffer
        each layer attended with."""
        used, cur, k = [], None, 0
        for layer, mode in enumerate(self.plan):
            if mode == "F":
                index_full(self.cache, iq[k], iw[k], n_vis, self.topk_bufs[k],
                           self.pool if self.pool_blocks else None, topk=self.topk,
                           pool_blocks=self.pool_blocks, ws=self.ws_full, stream=stream,
                           scan_timer=scan_timer)
                cur, k = self.topk_bufs[k], k + 1
            elif mode == "X":
                index_reindex(self.cache, iq[k], iw[k], n_vis, self.pool, self.topk_bufs[k],
                              topk=self.topk, ws=self.ws_reindex, stream=stream)
                cur, k = self.topk_bufs[k], k + 1
            sparse_attn_chunk(q[layer], self.cache, cur, swa_k[layer], swa_v[layer],
                              swa_ks[layer], swa_vs[layer], self.out[layer], self.lse[layer],
                              ws=self.ws_attn, stream=stream)
            used.append(cur)
        return used



# The model's layer plan ("DeepSeek V4.1 Flash: architecture study notes",
# section 2, the layer table; section 3, sequence compression): encoder layers
# 1-2 attend to their window only; encoder layers 3-20 are three groups of one
# Full and five Reuse layers, each group over its own global KV of 2:1
# compressed entries; decoder layers 21-40 are one Full, four Reindex and
# fifteen Reuse layers over one shared global KV of uncompressed entries.
ENCODER_WINDOW_ONLY = 2
ENCODER_GROUP_PLAN = "FRRRRR"
ENCODER_GROUPS = 3
ENCODER_RATIO = 2
DECODER_PLAN = "FRRRXRRRXRRRXRRRXRRR"


class ModelStep:
    """One decode step of the whole 40-layer plan for B sequences: the write
    path of the new token into every global KV and every layer's window, then
    the encoder's window-only layers, its three groups and the decoder stack.

    enc_caches: three Cache objects (2:1 compressed entries), dec_cache: one
    Cache (one entry per token).  Every layer has its own window, stacked per
    group as [L][B][128][128] (window-only layers: [2][B][128][128])."""

    def __init__(self, enc_caches, dec_cache, B, H, topk=DEFAULT_TOPK,
                 pool_blocks=DEFAULT_POOL_BLOCKS):
        if len(enc_caches) != ENCODER_GROUPS:
            raise ValueError(f"{ENCODER_GROUPS} encoder caches expected")
        self.B, self.H, self.topk = B, H, topk
        self.enc = [DecodeStack(c, ENCODER_GROUP_PLAN, B, H, topk=topk, pool_blocks=0)
                    for c in enc_caches]
        self.dec = DecodeStack(dec_cache, DECODER_PLAN, B, H, topk=topk, pool_blocks=pool_blocks)
        dev = dec_cache.kv_codes.device
        W = ENCODER_WINDOW_ONLY
        self.win_out = torch.empty((W, B, H, HEAD_DIM), dtype=torch.float32, device=dev)
        self.win_lse = torch.empty((W, B, H), dtype=torch.float32, device=dev)
        self.no_idx = torch.empty((B, 0), dtype=torch.int32, device=dev)
        n_attn = workspace_size(OP_ATTN_DECODE, B, 1, dec_cache.cap, 0, 0, H)
        self.ws_win = alloc_workspace(n_attn, dev) if n_attn else None

    @property
    def layers(self):
        return ENCODER_WINDOW_ONLY + ENCODER_GROUPS * len(ENCODER_GROUP_PLAN) + len(DECODER_PLAN)

    def step(self, new, win, enc_args, dec_args, stream=None):
        """new: per global KV (three encoder groups, then the decoder) a dict
        with the arguments of DecodeStack.write (k_new, v_new, rows_new,
        idx_proj, win_k, win_v, win_rows, ratio, rope_cs); for an encoder
        group whose pair the token does not complete, k_new / v_new have no
        rows (only the window tokens are written);
        win: the window-only layers' dict: q [2][B][H][128], swk / swv
        [2][B][128][128] u8, sks / svs [2][B][128] f32, swa_len [B], the new
        window rows win_k / win_v [2*B][128] f32 with their rows win_rows;
        enc_args / dec_args: per group a dict iq, iw, n_vis, q, swk, swv, sks,
        svs, swa_len with the meaning of DecodeStack.step's arguments.
        Returns, per group, the top-K buffers its layers attended with."""
        write_entries(None, None, self.dec.cache.kv_codes, self.dec.cache.kv_scales,
                      fp8_jobs=[dict(x=win["win_k"], codes=win["swk"].view(-1, HEAD_DIM),
                                     sigma=win["sks"].view(-1), dst_rows=win["win_rows"]),
                                dict(x=win["win_v"], codes=win["swv"].view(-1, HEAD_DIM),
                                     sigma=win["svs"].view(-1), dst_rows=win["win_rows"])],
                      stream=stream)
        for i in range(ENCODER_WINDOW_ONLY):
            sparse_attn_decode(win["q"][i], self.dec.cache, self.no_idx, win["swk"][i],
                               win["swv"][i], win["sks"][i], win["svs"][i], win["swa_len"],
                               self.win_out[i], self.win_lse[i], ws=self.ws_win, stream=stream)
        used = []
        for st, wr, a in zip(self.enc + [self.dec], new, enc_args + [dec_args]):
            st.write(**wr, swa_k=a["swk"], swa_v=a["swv"], swa_ks=a["sks"], swa_vs=a["svs"],
                     stream=stream)
            used.append(st.step(a["iq"], a["iw"], a["n_vis"], a["q"], a["swk"], a["swv"],
                                a["sks"], a["svs"], a["swa_len"], stream=stream))
        return used
