"""Seeded synthetic inputs shaped like the CSA2 decode workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no quantisation, scoring, selection or attention).  The
same arrays are handed to the HIP library and, in tests, to the CPU oracle.

Workloads (positions are global-KV entries of one sequence):
  full_1k            one Full layer, 1 decode query, 1024 entries, 16 heads
  encoder_group_16k  1 Full + 5 Reuse, 32768 tokens averaged 2:1 into 16384
                     entries, batch 8, 64 heads, no pool
  decoder_stack_128k 1 Full + 4 Reindex + 15 Reuse over 131072 entries,
                     pool of 2048 blocks x 8, batch 16, 64 heads
  decoder_stack_1m   the same stack over 1048576 entries, batch 4, keys with
                     planted high-score clusters
  replay_chunk_128k  128 causal queries over 131072 entries (bounded replay)
  replay_stack_128k  the same 128 replayed queries through the whole decoder
                     stack (1 Full + 4 Reindex + 15 Reuse), per-query pools

Every array is float32 N(0,1) unless stated; the indexer head weights are
U(0,1); the indexer key of an entry is a fixed seeded 128->64 projection of
that entry's main K (fp64 product, rounded to fp32 once).
"""
from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128
IDX_HEADS = 4
IDX_DIM = 64
WINDOW = 128
TOPK = 512
POOL_BLOCKS = 2048
BLOCK = 8

# Decoder plan: one Full layer, four Reindex-headed groups, the rest Reuse.
DECODER_PLAN = "FRRRXRRRXRRRXRRRXRRR"
ENCODER_PLAN = "FRRRRR"


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int            # independent sequences
    n_ent: int        # visible global entries per sequence
    ratio: int        # tokens per entry (2 = pairs averaged)
    H: int            # attention query heads
    plan: str         # layer modes: F = Full, X = Reindex, R = Reuse
    pool_blocks: int  # 0 = no block pool
    Q: int = 1        # queries per sequence (128 for the replay chunk)
    planted: bool = False
    topk: int = TOPK
    extra: dict = field(default_factory=dict)
    idx_fp4: bool = False  # indexer keys in the FP4 format (36 B) instead of FP8 (68 B)

    @property
    def n_tok(self):
        return self.n_ent * self.ratio


WORKLOADS = {
    "full_1k": Workload("full_1k", 1000, B=1, n_ent=1024, ratio=1, H=16, plan="F",
                        pool_blocks=0),
    "encoder_group_16k": Workload("encoder_group_16k", 1001, B=8, n_ent=16384, ratio=2, H=64,
                                  plan=ENCODER_PLAN, pool_blocks=0),
    "decoder_stack_128k": Workload("decoder_stack_128k", 1002, B=16, n_ent=131072, ratio=1,
                                   H=64, plan=DECODER_PLAN, pool_blocks=POOL_BLOCKS),
    "decoder_stack_1m": Workload("decoder_stack_1m", 1003, B=4, n_ent=1048576, ratio=1, H=64,
                                 plan=DECODER_PLAN, pool_blocks=POOL_BLOCKS, planted=True),
    "decoder_stack_128k_fp4idx": Workload("decoder_stack_128k_fp4idx", 1002, B=16,
                                          n_ent=131072, ratio=1, H=64, plan=DECODER_PLAN,
                                          pool_blocks=POOL_BLOCKS, idx_fp4=True),
    "decoder_stack_1m_fp4idx": Workload("decoder_stack_1m_fp4idx", 1003, B=4, n_ent=1048576,
                                        ratio=1, H=64, plan=DECODER_PLAN,
                                        pool_blocks=POOL_BLOCKS, planted=True, idx_fp4=True),
    "replay_chunk_128k": Workload("replay_chunk_128k", 1004, B=1, n_ent=131072, ratio=1, H=64,
                                  plan="F", pool_blocks=0, Q=128),
    "replay_chunk_128k_fp4idx": Workload("replay_chunk_128k_fp4idx", 1004, B=1, n_ent=131072,
                                         ratio=1, H=64, plan="F", pool_blocks=0, Q=128,
                                         idx_fp4=True),
    "replay_stack_128k": Workload("replay_stack_128k", 1005, B=1, n_ent=131072, ratio=1, H=64,
                                  plan=DECODER_PLAN, pool_blocks=POOL_BLOCKS, Q=128),
}


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def normal(g, shape):
    return g.standard_normal(shape, dtype=np.float32)


def idx_projection(g):
    """Fixed 128 -> 64 projection, entries N(0, 1/128)."""
    return (g.standard_normal((IDX_DIM, HEAD_DIM)) / np.sqrt(HEAD_DIM)).astype(np.float64)


def project_idx_k(k_entries, proj):
    """Indexer key per entry: proj @ k in fp64, rounded once to fp32.

    k_entries [..., 128] fp32 (or fp64 for pair means built in fp64)."""
    shp = k_entries.shape[:-1]
    flat = np.asarray(k_entries, np.float64).reshape(-1, HEAD_DIM)
    return (flat @ proj.T).astype(np.float32).reshape(*shp, IDX_DIM)


def pair_mean_fp64(x):
    """fp64 mean of disjoint token pairs, used only to derive the indexer-key
    fixture for 2:1 averaged entries (the write path's own averaging is fp32)."""
    x = np.asarray(x, np.float64)
    return 0.5 * (x[..., 0::2, :] + x[..., 1::2, :])


def indexer_query(g, B, Q):
    iq = normal(g, (B, Q, IDX_HEADS, IDX_DIM))
    iw = g.random((B, Q, IDX_HEADS), dtype=np.float32)
    return iq, iw


def plant_clusters(g, idx_k, iq_full, frac=0.01, shift=3.0):
    """Add shift * sum_h unit(q_h) to every position of a random `frac` of the
    8-position blocks of each sequence (in place on fp32 idx_k [B][N][64]).

    iq_full [B][4][64] is the Full layer's indexer query of each sequence.
    Returns the planted block ids per sequence."""
    B, N, _ = idx_k.shape
    n_blocks = N // BLOCK
    n_plant = max(1, int(round(frac * n_blocks)))
    planted = []
    for b in range(B):
        qh = iq_full[b].astype(np.float64)
        qh = qh / np.linalg.norm(qh, axis=-1, keepdims=True)
        direction = (shift * qh.sum(axis=0)).astype(np.float32)
        blocks = np.sort(g.choice(n_blocks, size=n_plant, replace=False))
        pos = (blocks[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
        idx_k[b, pos, :] += direction[None, :]
        planted.append(blocks)
    return planted


@dataclass
class DecodeInputs:
    """Host arrays for one decode stack step (all float32 unless noted)."""
    wl: Workload
    k_tok: np.ndarray      # [B][n_tok][128]
    v_tok: np.ndarray      # [B][n_tok][128]
    idx_k: np.ndarray      # [B][n_ent][64]
    iq: np.ndarray         # [L_idx][B][4][64]  one per Full/Reindex layer
    iw: np.ndarray         # [L_idx][B][4]
    q: np.ndarray          # [L][B][H][128]     one per layer
    swa_k: np.ndarray      # [L][B][128][128]
    swa_v: np.ndarray      # [L][B][128][128]
    swa_len: np.ndarray    # [B] int32
    planted: list = None
    proj: np.ndarray = None  # [64][128] the indexer-key projection, rounded to fp32


def decode_inputs(wl, n_ent=None, B=None, layers=None, seed=None):
    """Draw the inputs of one decode stack step.

    n_ent / B / layers override the workload's sizes (smaller parity cases);
    the draw order is fixed: K, V, projection, indexer queries, planted
    clusters, attention queries, SWA K, SWA V."""
    n_ent = wl.n_ent if n_ent is None else n_ent
    B = wl.B if B is None else B
    plan = wl.plan if layers is None else wl.plan[:layers]
    g = rng(wl.seed if seed is None else seed)
    n_tok = n_ent * wl.ratio
    k_tok = normal(g, (B, n_tok, HEAD_DIM))
    v_tok = normal(g, (B, n_tok, HEAD_DIM))
    proj = idx_projection(g)
    if wl.ratio == 2:
        idx_k = project_idx_k(pair_mean_fp64(k_tok), proj)
    else:
        idx_k = project_idx_k(k_tok, proj)
    n_idx = sum(1 for m in plan if m in "FX")
    iq, iw = indexer_query(g, n_idx, B)
    iq = iq.reshape(n_idx, B, IDX_HEADS, IDX_DIM)
    iw = iw.reshape(n_idx, B, IDX_HEADS)
    planted = None
    if wl.planted:
        planted = plant_clusters(g, idx_k, iq[0])
    L = len(plan)
    q = normal(g, (L, B, wl.H, HEAD_DIM))
    swa_k = normal(g, (L, B, WINDOW, HEAD_DIM))
    swa_v = normal(g, (L, B, WINDOW, HEAD_DIM))
    swa_len = np.full(B, WINDOW, np.int32)
    return DecodeInputs(wl, k_tok, v_tok, idx_k, iq, iw, q, swa_k, swa_v, swa_len, planted,
                        proj.astype(np.float32))


@dataclass
class ChunkInputs:
    """Host arrays for one bounded-replay chunk (the last Q positions)."""
    wl: Workload
    k_tok: np.ndarray      # [B][N][128] all entries' raw K (last Q are the chunk's)
    v_tok: np.ndarray      # [B][N][128]
    idx_k: np.ndarray      # [B][N][64]
    iq: np.ndarray         # [B][Q][4][64]
    iw: np.ndarray         # [B][Q][4]
    q: np.ndarray          # [B][Q][H][128]
    swa_k: np.ndarray      # [B][Q][128]   the chunk's own SWA tokens
    swa_v: np.ndarray      # [B][Q][128]
    positions: np.ndarray  # [Q] int64 absolute positions of the chunk tokens
    proj: np.ndarray = None  # [64][128] the indexer-key projection, rounded to fp32


def chunk_inputs(wl, n_ent=None, Q=None, H=None, seed=None):
    n_ent = wl.n_ent if n_ent is None else n_ent
    Q = wl.Q if Q is None else Q
    H = wl.H if H is None else H
    B = wl.B
    g = rng(wl.seed if seed is None else seed)
    k_tok = normal(g, (B, n_ent, HEAD_DIM))
    v_tok = normal(g, (B, n_ent, HEAD_DIM))
    proj = idx_projection(g)
    idx_k = project_idx_k(k_tok, proj)
    iq, iw = indexer_query(g, B, Q)
    q = normal(g, (B, Q, H, HEAD_DIM))
    swa_k = normal(g, (B, Q, HEAD_DIM))
    swa_v = normal(g, (B, Q, HEAD_DIM))
    positions = np.arange(n_ent - Q, n_ent, dtype=np.int64)
    return ChunkInputs(wl, k_tok, v_tok, idx_k, iq, iw, q, swa_k, swa_v, positions,
                       proj.astype(np.float32))


@dataclass
class ChunkStackInputs:
    """Host arrays for a bounded-replay chunk through a layer stack: the last
    Q entries of each sequence are the chunk's; each Full/Reindex layer has
    its own indexer query per chunk token, each layer its own attention
    queries and its own window K / V over the chunk's tokens."""
    wl: Workload
    plan: str
    k_tok: np.ndarray      # [B][N][128]
    v_tok: np.ndarray      # [B][N][128]
    idx_k: np.ndarray      # [B][N][64]
    iq: np.ndarray         # [L_idx][B][Q][4][64]
    iw: np.ndarray         # [L_idx][B][Q][4]
    q: np.ndarray          # [L][B][Q][H][128]
    swa_k: np.ndarray      # [L][B][Q][128]
    swa_v: np.ndarray      # [L][B][Q][128]
    positions: np.ndarray  # [Q] int64
    proj: np.ndarray = None  # [64][128] the indexer-key projection, rounded to fp32


def chunk_stack_inputs(wl, n_ent=None, Q=None, H=None, B=None, layers=None, seed=None):
    """Draw order: K, V, projection, indexer queries, attention queries, SWA K, SWA V."""
    n_ent = wl.n_ent if n_ent is None else n_ent
    Q = wl.Q if Q is None else Q
    H = wl.H if H is None else H
    B = wl.B if B is None else B
    plan = wl.plan if layers is None else wl.plan[:layers]
    g = rng(wl.seed if seed is None else seed)
    k_tok = normal(g, (B, n_ent, HEAD_DIM))
    v_tok = normal(g, (B, n_ent, HEAD_DIM))
    proj = idx_projection(g)
    idx_k = project_idx_k(k_tok, proj)
    n_idx = sum(1 for m in plan if m in "FX")
    iq = normal(g, (n_idx, B, Q, IDX_HEADS, IDX_DIM))
    iw = g.random((n_idx, B, Q, IDX_HEADS), dtype=np.float32)
    L = len(plan)
    q = normal(g, (L, B, Q, H, HEAD_DIM))
    swa_k = normal(g, (L, B, Q, HEAD_DIM))
    swa_v = normal(g, (L, B, Q, HEAD_DIM))
    positions = np.arange(n_ent - Q, n_ent, dtype=np.int64)
    return ChunkStackInputs(wl, plan, k_tok, v_tok, idx_k, iq, iw, q, swa_k, swa_v, positions,
                            proj.astype(np.float32))


def device_generator(seed):
    """Seeded torch generator on the GPU, for workloads too large to draw on
    the host (their results are checked through sampled properties only)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def device_normal(gen, shape):
    """N(0, 1) fp32 tensor of `shape` on the GPU from `gen`."""
    import torch
    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
