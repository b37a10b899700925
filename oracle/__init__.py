"""ctypes wrapper around the CPU oracle (test infrastructure only).

Only tests/, the smoke check and the bench's CPU-baseline leg import this
package.  It shares no code with the HIP library; arrays go in and out as
numpy arrays in the oracle's own plain layouts:
  main KV   codes [n][128] uint8 (K 64 B | V 64 B, low nibble = even channel),
            scales [n][16] uint8 (K 8 E4M3 | V 8 E4M3), one per 16 channels;
  indexer K codes [n][64] uint8 E4M3, sigma [n] fp32;
  SWA       codes [n][128] uint8 E4M3, sigma [n] fp32.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
c_i64, c_int, c_f, c_d = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        sig = {
            "csa2o_e4m3_decode": (c_d, [ctypes.c_uint8]),
            "csa2o_e4m3_encode": (ctypes.c_uint8, [c_f]),
            "csa2o_e2m1_decode": (c_d, [ctypes.c_uint8]),
            "csa2o_e2m1_encode": (ctypes.c_uint8, [c_f]),
            "csa2o_average_pair": (None, [f32p, f32p, c_int, f32p]),
            "csa2o_rope_table": (None, [i64p, c_i64, c_d, f32p]),
            "csa2o_rope_apply": (None, [f32p, f32p]),
            "csa2o_fp4_quant_vec": (None, [f32p, u8p, u8p]),
            "csa2o_quant_fp4": (c_int, [f32p, f32p, c_i64, c_int, ctypes.c_void_p, u8p, u8p]),
            "csa2o_entry_k": (c_int, [f32p, c_i64, c_int, ctypes.c_void_p, f32p]),
            "csa2o_project_idx": (None, [f32p, f32p, f32p]),
            "csa2o_project_idx_rows": (None, [f32p, c_i64, f32p, f32p]),
            "csa2o_fp8_quant_row": (None, [f32p, c_int, u8p, f32p]),
            "csa2o_quant_fp8_rows": (None, [f32p, c_i64, c_int, u8p, f32p]),
            "csa2o_quant_iq": (None, [f32p, f32p, u8p, f32p]),
            "csa2o_score": (c_f, [u8p, f32p, u8p, c_f]),
            "csa2o_index_full": (c_int, [u8p, f32p, c_i64, f32p, f32p, c_int, c_int, i32p,
                                         ctypes.c_void_p, ctypes.c_void_p]),
            "csa2o_index_reindex": (c_int, [u8p, f32p, c_i64, f32p, f32p, i32p, c_int, c_int,
                                            i32p]),
            "csa2o_index_full_batch": (c_int, [u8p, f32p, c_i64, c_int, c_int, f32p, f32p, i32p,
                                               c_int, c_int, i32p, ctypes.c_void_p]),
            "csa2o_index_reindex_batch": (c_int, [u8p, f32p, c_i64, c_int, c_int, f32p, f32p,
                                                  i32p, i32p, c_int, c_int, i32p]),
            "csa2o_attn": (None, [f32p, c_int, u8p, u8p, i32p, c_int, u8p, u8p, f32p, f32p,
                                  c_int, c_f, f32p, f32p]),
            "csa2o_attn_decode_batch": (None, [f32p, c_int, c_int, u8p, u8p, c_i64, i32p, c_int,
                                               u8p, u8p, f32p, f32p, i32p, c_f, f32p, f32p]),
            "csa2o_attn_chunk_batch": (None, [f32p, c_int, c_int, c_int, u8p, u8p, c_i64, i32p,
                                              c_int, u8p, u8p, f32p, f32p, c_f, f32p, f32p]),
            "csa2o_fp4_quant_groups": (None, [f32p, c_int, u8p, u8p]),
            "csa2o_idx4_quant_rows": (None, [f32p, c_i64, u8p, u8p]),
            "csa2o_score4": (c_f, [u8p, f32p, u8p, u8p]),
            "csa2o_index_full4": (c_int, [u8p, u8p, c_i64, f32p, f32p, c_int, c_int, i32p,
                                          ctypes.c_void_p, ctypes.c_void_p]),
            "csa2o_index_reindex4": (c_int, [u8p, u8p, c_i64, f32p, f32p, i32p, c_int, c_int,
                                             i32p]),
            "csa2o_index_full4_batch": (c_int, [u8p, u8p, c_i64, c_int, c_int, f32p, f32p, i32p,
                                                c_int, c_int, i32p, ctypes.c_void_p]),
            "csa2o_index_reindex4_batch": (c_int, [u8p, u8p, c_i64, c_int, c_int, f32p, f32p,
                                                   i32p, i32p, c_int, c_int, i32p]),
            "csa2o_num_threads": (c_int, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---- formats -------------------------------------------------------------
def e4m3_decode(code):
    return lib().csa2o_e4m3_decode(int(code))


def e4m3_encode(x):
    return int(lib().csa2o_e4m3_encode(float(x)))


def e2m1_decode(code):
    return lib().csa2o_e2m1_decode(int(code))


def e2m1_encode(t):
    return int(lib().csa2o_e2m1_encode(float(t)))


def num_threads():
    return int(lib().csa2o_num_threads())


# ---- write path ----------------------------------------------------------
def average_pair(a, b):
    a, b = _c(a, np.float32), _c(b, np.float32)
    out = np.empty_like(a)
    lib().csa2o_average_pair(a, b, a.size, out)
    return out


def rope_table(pos, base=10000.0):
    pos = _c(pos, np.int64)
    cs = np.empty((pos.size, 32, 2), np.float32)
    lib().csa2o_rope_table(pos, pos.size, float(base), cs)
    return cs


def rope_apply(x, cs_row):
    x = _c(x, np.float32).copy()
    lib().csa2o_rope_apply(x, _c(cs_row, np.float32))
    return x


def fp4_quant_vec(x):
    x = _c(x, np.float32)
    codes = np.zeros(64, np.uint8)
    scales = np.zeros(8, np.uint8)
    lib().csa2o_fp4_quant_vec(x, codes, scales)
    return codes, scales


def quant_fp4(k, v, ratio=1, rope_cs=None):
    """k, v [n_tok][128] fp32 -> (codes [n_ent][128] u8, scales [n_ent][16] u8)."""
    k, v = _c(k, np.float32), _c(v, np.float32)
    n_tok = k.shape[0]
    n_ent = n_tok // ratio
    codes = np.zeros((n_ent, 128), np.uint8)
    scales = np.zeros((n_ent, 16), np.uint8)
    cs = None if rope_cs is None else _c(rope_cs, np.float32)
    rc = lib().csa2o_quant_fp4(k, v, n_tok, ratio,
                               None if cs is None else cs.ctypes.data, codes, scales)
    if rc != 0:
        raise ValueError("oracle quant_fp4 rejected its arguments")
    return codes, scales


def quant_fp8_rows(x):
    """x [..., dim] fp32 -> (codes [..., dim] u8, sigma [...] fp32)."""
    x = _c(x, np.float32)
    dim = x.shape[-1]
    n = x.size // dim
    codes = np.empty(x.shape, np.uint8)
    sigma = np.empty(x.shape[:-1], np.float32)
    lib().csa2o_quant_fp8_rows(x, n, dim, codes, sigma)
    return codes, sigma


def entry_k(k, ratio=1, rope_cs=None):
    """k [n_tok][128] fp32 -> the entries' fp32 K as the write path quantises
    them (pair mean for ratio 2, RoPE when rope_cs is given) [n_ent][128]."""
    k = _c(k, np.float32)
    out = np.empty((k.shape[0] // ratio, 128), np.float32)
    cs = None if rope_cs is None else _c(rope_cs, np.float32)
    rc = lib().csa2o_entry_k(k, k.shape[0], ratio, None if cs is None else cs.ctypes.data, out)
    if rc != 0:
        raise ValueError("oracle entry_k rejected its arguments")
    return out


def project_idx(x, W):
    """x [n][128] fp32, W [64][128] fp32 -> indexer keys [n][64] fp32."""
    x, W = _c(x, np.float32), _c(W, np.float32)
    keys = np.empty((x.shape[0], 64), np.float32)
    lib().csa2o_project_idx_rows(x, x.shape[0], W, keys)
    return keys


def write_entries_proj(k, v, W, ratio=1, rope_cs=None):
    """The write path with the indexer key projected from each entry's K:
    (codes, scales, indexer codes [n_ent][64], indexer sigma [n_ent])."""
    codes, scales = quant_fp4(k, v, ratio, rope_cs)
    ikc, iks = quant_fp8_rows(project_idx(entry_k(k, ratio, rope_cs), W))
    return codes, scales, ikc, iks


# ---- indexer ------------------------------------------------------------
def quant_iq(iq, iw):
    qc = np.empty((4, 64), np.uint8)
    wq = np.empty(4, np.float32)
    lib().csa2o_quant_iq(_c(iq, np.float32), _c(iw, np.float32), qc, wq)
    return qc, wq


def score(qc, wq, kc, sigma):
    return lib().csa2o_score(_c(qc, np.uint8), _c(wq, np.float32), _c(kc, np.uint8),
                             float(sigma))


def index_full(ikc, iks, n_vis, iq, iw, topk, pool_blocks, want_scores=False):
    ikc, iks = _c(ikc, np.uint8), _c(iks, np.float32)
    topk_idx = np.empty(topk, np.int32)
    pool = np.empty(max(pool_blocks, 1), np.int32)
    sc = np.empty(max(int(n_vis), 1), np.float32)
    rc = lib().csa2o_index_full(ikc, iks, int(n_vis), _c(iq, np.float32), _c(iw, np.float32),
                                topk, pool_blocks, topk_idx, pool.ctypes.data,
                                sc.ctypes.data if want_scores else None)
    if rc != 0:
        raise ValueError("oracle index_full rejected its arguments")
    out = [topk_idx, pool[:pool_blocks]]
    if want_scores:
        out.append(sc[:int(n_vis)])
    return tuple(out)


def index_reindex(ikc, iks, n_vis, iq, iw, pool_idx, topk):
    pool_idx = _c(pool_idx, np.int32)
    topk_idx = np.empty(topk, np.int32)
    rc = lib().csa2o_index_reindex(_c(ikc, np.uint8), _c(iks, np.float32), int(n_vis),
                                   _c(iq, np.float32), _c(iw, np.float32), pool_idx,
                                   pool_idx.size, topk, topk_idx)
    if rc != 0:
        raise ValueError("oracle index_reindex rejected its arguments")
    return topk_idx


def index_full_batch(ikc, iks, iq, iw, n_vis, topk, pool_blocks):
    """ikc [B][cap][64], iks [B][cap], iq [B][Q][4][64], iw [B][Q][4], n_vis [B][Q]."""
    ikc, iks = _c(ikc, np.uint8), _c(iks, np.float32)
    B, cap = iks.shape
    Q = iq.shape[1]
    topk_idx = np.empty((B, Q, topk), np.int32)
    pool = np.empty((B, Q, max(pool_blocks, 1)), np.int32)
    rc = lib().csa2o_index_full_batch(ikc, iks, cap, B, Q, _c(iq, np.float32),
                                      _c(iw, np.float32), _c(n_vis, np.int32), topk, pool_blocks,
                                      topk_idx, pool.ctypes.data)
    if rc != 0:
        raise ValueError("oracle index_full_batch rejected its arguments")
    return topk_idx, pool[:, :, :pool_blocks]


def index_reindex_batch(ikc, iks, iq, iw, n_vis, pool_idx, topk):
    ikc, iks = _c(ikc, np.uint8), _c(iks, np.float32)
    B, cap = iks.shape
    Q = iq.shape[1]
    pool_idx = _c(pool_idx, np.int32)
    topk_idx = np.empty((B, Q, topk), np.int32)
    rc = lib().csa2o_index_reindex_batch(ikc, iks, cap, B, Q, _c(iq, np.float32),
                                         _c(iw, np.float32), _c(n_vis, np.int32), pool_idx,
                                         pool_idx.shape[-1], topk, topk_idx)
    if rc != 0:
        raise ValueError("oracle index_reindex_batch rejected its arguments")
    return topk_idx


# ---- FP4 indexer key -----------------------------------------------------
# layout: codes [n][32] uint8 (low nibble = even channel), scales [n][4] uint8
# (E4M3, one per 16 channels)
def idx4_quant_rows(x):
    """x [..., 64] fp32 -> (codes [..., 32] u8, scales [..., 4] u8)."""
    x = _c(x, np.float32)
    n = x.size // 64
    codes = np.zeros(x.shape[:-1] + (32,), np.uint8)
    scales = np.zeros(x.shape[:-1] + (4,), np.uint8)
    lib().csa2o_idx4_quant_rows(x, n, codes, scales)
    return codes, scales


def score4(qc, wq, kc4, ks4):
    return lib().csa2o_score4(_c(qc, np.uint8), _c(wq, np.float32), _c(kc4, np.uint8),
                              _c(ks4, np.uint8))


def index_full4(kc4, ks4, n_vis, iq, iw, topk, pool_blocks, want_scores=False):
    kc4, ks4 = _c(kc4, np.uint8), _c(ks4, np.uint8)
    topk_idx = np.empty(topk, np.int32)
    pool = np.empty(max(pool_blocks, 1), np.int32)
    sc = np.empty(max(int(n_vis), 1), np.float32)
    rc = lib().csa2o_index_full4(kc4, ks4, int(n_vis), _c(iq, np.float32), _c(iw, np.float32),
                                 topk, pool_blocks, topk_idx, pool.ctypes.data,
                                 sc.ctypes.data if want_scores else None)
    if rc != 0:
        raise ValueError("oracle index_full4 rejected its arguments")
    out = [topk_idx, pool[:pool_blocks]]
    if want_scores:
        out.append(sc[:int(n_vis)])
    return tuple(out)


def index_reindex4(kc4, ks4, n_vis, iq, iw, pool_idx, topk):
    pool_idx = _c(pool_idx, np.int32)
    topk_idx = np.empty(topk, np.int32)
    rc = lib().csa2o_index_reindex4(_c(kc4, np.uint8), _c(ks4, np.uint8), int(n_vis),
                                    _c(iq, np.float32), _c(iw, np.float32), pool_idx,
                                    pool_idx.size, topk, topk_idx)
    if rc != 0:
        raise ValueError("oracle index_reindex4 rejected its arguments")
    return topk_idx


def index_full4_batch(kc4, ks4, iq, iw, n_vis, topk, pool_blocks):
    """kc4 [B][cap][32], ks4 [B][cap][4], iq [B][Q][4][64], iw [B][Q][4], n_vis [B][Q]."""
    kc4, ks4 = _c(kc4, np.uint8), _c(ks4, np.uint8)
    B, cap = ks4.shape[:2]
    Q = iq.shape[1]
    topk_idx = np.empty((B, Q, topk), np.int32)
    pool = np.empty((B, Q, max(pool_blocks, 1)), np.int32)
    rc = lib().csa2o_index_full4_batch(kc4, ks4, cap, B, Q, _c(iq, np.float32),
                                       _c(iw, np.float32), _c(n_vis, np.int32), topk,
                                       pool_blocks, topk_idx, pool.ctypes.data)
    if rc != 0:
        raise ValueError("oracle index_full4_batch rejected its arguments")
    return topk_idx, pool[:, :, :pool_blocks]


def index_reindex4_batch(kc4, ks4, iq, iw, n_vis, pool_idx, topk):
    kc4, ks4 = _c(kc4, np.uint8), _c(ks4, np.uint8)
    B, cap = ks4.shape[:2]
    Q = iq.shape[1]
    pool_idx = _c(pool_idx, np.int32)
    topk_idx = np.empty((B, Q, topk), np.int32)
    rc = lib().csa2o_index_reindex4_batch(kc4, ks4, cap, B, Q, _c(iq, np.float32),
                                          _c(iw, np.float32), _c(n_vis, np.int32), pool_idx,
                                          pool_idx.shape[-1], topk, topk_idx)
    if rc != 0:
        raise ValueError("oracle index_reindex4_batch rejected its arguments")
    return topk_idx


# ---- attention ------------------------------------------------------------
def attn(q, codes, scales, idx, swa_k, swa_v, swa_ks, swa_vs, swa_len, sm_scale):
    q = _c(q, np.float32)
    H = q.shape[0]
    idx = _c(idx, np.int32)
    out = np.empty((H, 128), np.float32)
    lse = np.empty(H, np.float32)
    lib().csa2o_attn(q, H, _c(codes, np.uint8), _c(scales, np.uint8), idx, idx.size,
                     _c(swa_k, np.uint8), _c(swa_v, np.uint8), _c(swa_ks, np.float32),
                     _c(swa_vs, np.float32), int(swa_len), float(sm_scale), out, lse)
    return out, lse


def attn_decode_batch(q, codes, scales, idx, swa_k, swa_v, swa_ks, swa_vs, swa_len, sm_scale):
    """q [B][H][128]; codes [B][cap][128]; scales [B][cap][16]; idx [B][topk];
    swa_k/v [B][128][128]; swa_ks/vs [B][128]; swa_len [B]."""
    q = _c(q, np.float32)
    B, H = q.shape[:2]
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    cap = codes.shape[1]
    idx = _c(idx, np.int32)
    out = np.empty((B, H, 128), np.float32)
    lse = np.empty((B, H), np.float32)
    lib().csa2o_attn_decode_batch(q, B, H, codes, scales, cap, idx, idx.shape[-1],
                                  _c(swa_k, np.uint8), _c(swa_v, np.uint8),
                                  _c(swa_ks, np.float32), _c(swa_vs, np.float32),
                                  _c(swa_len, np.int32), float(sm_scale), out, lse)
    return out, lse


def attn_chunk_batch(q, codes, scales, idx, swa_k, swa_v, swa_ks, swa_vs, sm_scale):
    """q [B][Q][H][128]; idx [B][Q][topk]; chunk SWA [B][Q][128], [B][Q]."""
    q = _c(q, np.float32)
    B, Q, H = q.shape[:3]
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    cap = codes.shape[1]
    idx = _c(idx, np.int32)
    out = np.empty((B, Q, H, 128), np.float32)
    lse = np.empty((B, Q, H), np.float32)
    lib().csa2o_attn_chunk_batch(q, B, Q, H, codes, scales, cap, idx, idx.shape[-1],
                                 _c(swa_k, np.uint8), _c(swa_v, np.uint8),
                                 _c(swa_ks, np.float32), _c(swa_vs, np.float32),
                                 float(sm_scale), out, lse)
    return out, lse
