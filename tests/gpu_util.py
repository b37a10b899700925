"""Helpers shared by the GPU parity tests: layout conversion between the
library's device layouts and the oracle's plain row layouts, uploads, and the
attention error metric.  No arithmetic of the method lives here."""
import numpy as np
import torch

IDX_DIM = 64


def tile_ik(codes):
    """Oracle row layout [B][cap][64] -> library tile layout (flat uint8).

    Position p of row r = b*cap + p: tile r // 64, lane r % 64; channel group g
    (16 bytes) at ((tile*4 + g)*64 + lane)*16."""
    B, cap, d = codes.shape
    assert d == IDX_DIM and cap % 64 == 0
    t = codes.reshape(B * cap // 64, 64, 4, 16)          # [tile][lane][g][16]
    return np.ascontiguousarray(t.transpose(0, 2, 1, 3)).reshape(-1)


def untile_ik(flat, B, cap):
    t = np.asarray(flat).reshape(B * cap // 64, 4, 64, 16)  # [tile][g][lane][16]
    return np.ascontiguousarray(t.transpose(0, 2, 1, 3)).reshape(B, cap, IDX_DIM)


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def row_rel_err(out, ref):
    """Per (query, head) row: max_c |o - o_ref| / max_c |o_ref|."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(out - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return num / np.maximum(den, 1e-30)


def tile_ik4(codes):
    """Oracle FP4 indexer codes [B][cap][32] -> library two-plane tile layout
    (flat uint8): plane h of tile t, lane i at ((t*2 + h)*64 + i)*16."""
    B, cap, d = codes.shape
    assert d == IDX_DIM // 2 and cap % 64 == 0
    t = codes.reshape(B * cap // 64, 64, 2, 16)          # [tile][lane][h][16]
    return np.ascontiguousarray(t.transpose(0, 2, 1, 3)).reshape(-1)


def untile_ik4(flat, B, cap):
    t = np.asarray(flat).reshape(B * cap // 64, 2, 64, 16)  # [tile][h][lane][16]
    return np.ascontiguousarray(t.transpose(0, 2, 1, 3)).reshape(B, cap, IDX_DIM // 2)
