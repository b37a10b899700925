"""Python binding of libcsa2 (CSA2 decode hot path, HIP for MI355X / gfx950).

Argument marshalling only: torch tensors on the GPU are checked for dtype,
shape and contiguity, and their device pointers plus torch's current HIP
stream are passed to the C ABI declared in include/csa2.h.  Every step of the
path runs in the library's kernels; there is no fallback.  If libcsa2.so is
missing or cannot be loaded, importing the binding's entry points raises.

torch is imported before the library is loaded so that both use the one HIP
runtime torch has already mapped (they share the soname libamdhip64.so.7).
"""
import ctypes
import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

HEAD_DIM = 128
KV_CODE_BYTES = 128
KV_SCALE_BYTES = 16
IDX_HEADS = 4
IDX_DIM = 64
IDX_TILE = 64
BLOCK = 8
WINDOW = 128
DEFAULT_TOPK = 512
DEFAULT_POOL_BLOCKS = 2048

FP8_ROWS = 0
FP8_IDX_TILED = 1
OP_INDEX_FULL = 1
OP_INDEX_REINDEX = 2
OP_ATTN_DECODE = 3
OP_ATTN_CHUNK = 4
OP_ATTN_STAGE = 5
STAGE_WRITE = 1
STAGE_READ = 2

STATUS = {0: "ok", -1: "CSA2_E_ARG", -2: "CSA2_E_UNSUPPORTED", -3: "CSA2_E_WORKSPACE",
          -4: "CSA2_E_HIP"}

EXPORTS = ("csa2_quant_fp4", "csa2_quant_fp8", "csa2_write_entries", "csa2_write_entries_proj",
           "csa2_index_full",
           "csa2_index_full_timed",
           "csa2_index_reindex",
           "csa2_sparse_attn_decode", "csa2_sparse_attn_decode_timed",
           "csa2_sparse_attn_decode_reuse", "csa2_sparse_attn_chunk",
           "csa2_workspace_size",
           "csa2_status_str", "csa2_abi_version", "csa2_codec_probe",
           "csa2_quant_idx_fp4", "csa2_write_entries_proj_fp4", "csa2_index_full_fp4",
           "csa2_index_full_fp4_timed", "csa2_index_reindex_fp4", "csa2_rope_table",
           "csa2_index_full_noalloc", "csa2_stream_probe", "csa2_gather_probe")

_lib = None

_vp, _i64, _int, _f, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
MAX_FP8_JOBS = 3


class _Fp8Job(ctypes.Structure):
    """csa2_fp8_job of include/csa2.h."""
    _fields_ = [("x", ctypes.c_void_p), ("n_rows", ctypes.c_int64), ("dim", ctypes.c_int),
                ("layout", ctypes.c_int), ("dst_rows", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("sigma", ctypes.c_void_p)]


_SIGS = {
    "csa2_quant_fp4": (_int, [_vp, _vp, _i64, _int, _vp, _vp, _vp, _vp, _vp]),
    "csa2_write_entries": (_int, [_vp, _vp, _i64, _int, _vp, _vp, _vp, _vp,
                                  ctypes.POINTER(_Fp8Job), _int, _vp]),
    "csa2_write_entries_proj": (_int, [_vp, _vp, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       ctypes.POINTER(_Fp8Job), _int, _vp]),
    "csa2_quant_fp8": (_int, [_vp, _i64, _int, _int, _vp, _vp, _vp, _vp]),
    "csa2_index_full": (_int, [_vp, _vp, _i64, _int, _int, _vp, _vp, _vp, _int, _int, _vp, _vp,
                               _vp, _sz, _vp]),
    "csa2_index_full_timed": (_int, [_vp, _vp, _i64, _int, _int, _vp, _vp, _vp, _int, _int, _vp,
                                     _vp, _vp, _sz, _vp, _vp, _vp]),
    "csa2_index_reindex": (_int, [_vp, _vp, _i64, _int, _int, _vp, _vp, _vp, _vp, _int, _int,
                                  _vp, _vp, _sz, _vp]),
    "csa2_sparse_attn_decode": (_int, [_vp, _int, _int, _vp, _vp, _i64, _vp, _int, _vp, _vp, _vp,
                                       _vp, _vp, _f, _vp, _vp, _vp, _sz, _vp]),
    "csa2_sparse_attn_decode_timed": (_int, [_vp, _int, _int, _vp, _vp, _i64, _vp, _int, _vp, _vp,
                                             _vp, _vp, _vp, _f, _vp, _vp, _vp, _sz, _vp, _vp,
                                             _vp]),
    "csa2_sparse_attn_decode_reuse": (_int, [_vp, _int, _int, _vp, _vp, _i64, _vp, _int, _vp, _sz,
                                             _int, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp,
                                             _sz, _vp, _vp, _vp]),
    "csa2_sparse_attn_chunk": (_int, [_vp, _int, _int, _int, _vp, _vp, _i64, _vp, _int, _vp, _vp,
                                      _vp, _vp, _f, _vp, _vp, _vp, _sz, _vp]),
    "csa2_workspace_size": (_sz, [_int, _int, _int, _i64, _int, _int, _int]),
    "csa2_status_str": (ctypes.c_char_p, [_int]),
    "csa2_abi_version": (_int, []),
    "csa2_rope_table": (_int, [_vp, _i64, ctypes.c_double, _vp]),
    "csa2_stream_probe": (_int, [_int, _vp, _vp, _sz, _vp, _int, _vp]),
    "csa2_gather_probe": (_int, [_vp, _vp, _vp, _int, _int, _i64, _vp, _vp, _vp, _vp, _vp, _int,
                                 _vp, _vp, _vp, _vp]),
    "csa2_index_full_noalloc": (_int, [_vp, _vp, _i64, _int, _int, _vp, _vp, _vp, _int, _int, _vp,
                                       _vp, _vp]),
    "csa2_codec_probe": (_int, [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp]),
    "csa2_quant_idx_fp4": (_int, [_vp, _i64, _vp, _vp, _vp, _vp]),
    "csa2_write_entries_proj_fp4": (_int, [_vp, _vp, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp,
                                           _vp, ctypes.POINTER(_Fp8Job), _int, _vp]),
    "csa2_index_full_fp4": (_int, [_vp, _vp, _i64, _int, _int, _vp, _vp, _vp, _int, _int, _vp,
                                   _vp, _vp, _sz, _vp]),
    "csa2_index_full_fp4_timed": (_int, [_vp, _vp, _i64, _int, _int, _vp, _vp, _vp, _int, _int,
                                         _vp, _vp, _vp, _sz, _vp, _vp, _vp]),
    "csa2_index_reindex_fp4": (_int, [_vp, _vp, _i64, _int, _int, _vp, _vp, _vp, _vp, _int, _int,
                                      _vp, _vp, _sz, _vp]),
}


class Csa2Error(RuntimeError):
    pass


def lib():
    """Load libcsa2.so (built in-tree by build.py); raise if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Csa2Error(f"{LIB_PATH} is missing: build it with "
                            "`python compressed_kv_cache_decode_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc, what):
    if rc != 0:
        msg = lib().csa2_status_str(rc).decode()
        raise Csa2Error(f"{what}: {STATUS.get(rc, rc)} ({msg})")


def _ptr(t, dtype, name, numel=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()}")
    return t.data_ptr()


def _check_batch(cache, B, what):
    """The kernels address cache rows b*cap + position for b < B: a query batch
    larger than the cache's would read past its arrays."""
    if B < 0 or B > cache.B:
        raise ValueError(f"{what}: a batch of {B} sequences does not fit the cache's {cache.B}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def workspace_size(op, B, Q, cap, topk, pool_blocks, H):
    n = lib().csa2_workspace_size(op, B, Q, cap, topk, pool_blocks, H)
    if n == ctypes.c_size_t(-1).value:
        raise Csa2Error("workspace_size: invalid sizes")
    return n


def alloc_workspace(nbytes, device=None):
    """A caller-owned byte buffer for the workspace argument."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8,
                       device=device or torch.cuda.current_device())


# ---------------------------------------------------------------------------
# caches
# ---------------------------------------------------------------------------
class Cache:
    """Device arrays of one shared global KV (B sequences x cap entries).

    kv_codes [B*cap][128] u8, kv_scales [B*cap][16] u8: FP4 main KV;
    indexer K, FP8 (default): ik_codes [B*cap*64] u8 (tile layout), ik_sigma
    [B*cap] f32; FP4 (idx_fp4=True): ik_codes [B*cap*32] u8 (two-plane tile
    layout), ik_scales4 [B*cap][4] u8 E4M3 (ik_sigma is None)."""

    def __init__(self, B, cap, device=None, idx_fp4=False):
        if cap % IDX_TILE:
            raise ValueError("cap must be a multiple of 64")
        dev = device or torch.cuda.current_device()
        self.B, self.cap, self.idx_fp4 = B, cap, idx_fp4
        n = B * cap
        self.kv_codes = torch.zeros((n, KV_CODE_BYTES), dtype=torch.uint8, device=dev)
        self.kv_scales = torch.zeros((n, KV_SCALE_BYTES), dtype=torch.uint8, device=dev)
        if idx_fp4:
            self.ik_codes = torch.zeros(n * IDX_DIM // 2, dtype=torch.uint8, device=dev)
            self.ik_scales4 = torch.zeros((n, 4), dtype=torch.uint8, device=dev)
            self.ik_sigma = None
        else:
            self.ik_codes = torch.zeros(n * IDX_DIM, dtype=torch.uint8, device=dev)
            self.ik_sigma = torch.zeros(n, dtype=torch.float32, device=dev)
            self.ik_scales4 = None

    @property
    def ik_aux(self):
        """The indexer key's per-row array: fp32 sigma (FP8) or scale bytes (FP4)."""
        return self.ik_scales4 if self.idx_fp4 else self.ik_sigma

    def rows(self, b, positions):
        """int64 device tensor of row numbers b*cap + positions."""
        pos = torch.as_tensor(positions, dtype=torch.int64)
        return (pos + b * self.cap).to(self.kv_codes.device)

    @property
    def nbytes(self):
        return sum(t.numel() * t.element_size()
                   for t in (self.kv_codes, self.kv_scales, self.ik_codes, self.ik_aux))


def rope_table(positions, base=10000.0):
    """The write path's rotation table for these positions: [n][32][2] float32
    (cos, sin), computed by the library's host function csa2_rope_table."""
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64).reshape(-1))
    cs = np.empty((pos.size, 32, 2), np.float32)
    rc = lib().csa2_rope_table(pos.ctypes.data, pos.size, float(base), cs.ctypes.data)
    _check(rc, "csa2_rope_table")
    return cs


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def quant_fp4(k_tok, v_tok, kv_codes, kv_scales, ratio=1, rope_cs=None, dst_rows=None,
              stream=None):
    if k_tok is None and v_tok is None:  # FP8 jobs only
        k_tok = v_tok = torch.empty((0, HEAD_DIM), dtype=torch.float32, device=kv_codes.device)
    n_tok = k_tok.shape[0] if k_tok.dim() > 1 else 0
    if k_tok.shape != v_tok.shape or (k_tok.dim() != 2 or k_tok.shape[1] != HEAD_DIM):
        raise ValueError("k_tok, v_tok must be [n_tok][128]")
    n_ent = n_tok // ratio
    rc = lib().csa2_quant_fp4(
        _ptr(k_tok, torch.float32, "k_tok"), _ptr(v_tok, torch.float32, "v_tok"), n_tok, ratio,
        _ptr(rope_cs, torch.float32, "rope_cs", n_ent * 64),
        _ptr(dst_rows, torch.int64, "dst_rows", n_ent),
        _ptr(kv_codes, torch.uint8, "kv_codes"), _ptr(kv_scales, torch.uint8, "kv_scales"),
        _stream(stream))
    _check(rc, "csa2_quant_fp4")


def quant_fp8(x, codes, sigma, layout=FP8_ROWS, dst_rows=None, stream=None):
    if x.dim() != 2:
        raise ValueError("x must be [n_rows][dim]")
    n, dim = x.shape
    rc = lib().csa2_quant_fp8(_ptr(x, torch.float32, "x"), n, dim, layout,
                              _ptr(dst_rows, torch.int64, "dst_rows", n),
                              _ptr(codes, torch.uint8, "codes"),
                              _ptr(sigma, torch.float32, "sigma"), _stream(stream))
    _check(rc, "csa2_quant_fp8")


def write_entries(k_tok, v_tok, kv_codes, kv_scales, ratio=1, rope_cs=None, dst_rows=None,
                  fp8_jobs=(), stream=None, idx_proj=None, ik_codes=None, ik_sigma=None,
                  ik_scales4=None):
    """quant_fp4(k_tok, v_tok, ...) and quant_fp8 of each job in one launch
    (k_tok = v_tok = None: the FP8 jobs only).

    fp8_jobs: up to 3 dicts with the arguments of quant_fp8: x, codes, sigma,
    and optionally layout (FP8_ROWS) and dst_rows.
    idx_proj [64][128] f32 (optional): also each entry's indexer key, projected
    on the device from its fp32 K and written in FP8 to ik_codes (tile layout)
    and ik_sigma at the entry's row (csa2_write_entries_proj), or as FP4 keys to
    ik_codes and ik_scales4 when ik_scales4 is given (csa2_write_entries_proj_fp4)."""
    if k_tok is None and v_tok is None:  # FP8 jobs only
        k_tok = v_tok = torch.empty((0, HEAD_DIM), dtype=torch.float32, device=kv_codes.device)
    n_tok = k_tok.shape[0] if k_tok.dim() > 1 else 0
    if k_tok.shape != v_tok.shape or (k_tok.dim() != 2 or k_tok.shape[1] != HEAD_DIM):
        raise ValueError("k_tok, v_tok must be [n_tok][128]")
    if len(fp8_jobs) > MAX_FP8_JOBS:
        raise ValueError(f"at most {MAX_FP8_JOBS} FP8 jobs")
    n_ent = n_tok // ratio
    jobs = (_Fp8Job * max(len(fp8_jobs), 1))()
    for i, jb in enumerate(fp8_jobs):
        x = jb["x"]
        if x.dim() != 2:
            raise ValueError("an FP8 job's x must be [n_rows][dim]")
        n, dim = x.shape
        jobs[i] = _Fp8Job(_ptr(x, torch.float32, "x"), n, dim, jb.get("layout", FP8_ROWS),
                          _ptr(jb.get("dst_rows"), torch.int64, "dst_rows", n),
                          _ptr(jb["codes"], torch.uint8, "codes"),
                          _ptr(jb["sigma"], torch.float32, "sigma"))
    head = (_ptr(k_tok, torch.float32, "k_tok"), _ptr(v_tok, torch.float32, "v_tok"), n_tok,
            ratio, _ptr(rope_cs, torch.float32, "rope_cs", n_ent * 64),
            _ptr(dst_rows, torch.int64, "dst_rows", n_ent),
            _ptr(kv_codes, torch.uint8, "kv_codes"), _ptr(kv_scales, torch.uint8, "kv_scales"))
    if idx_proj is None:
        rc = lib().csa2_write_entries(*head, jobs, len(fp8_jobs), _stream(stream))
        _check(rc, "csa2_write_entries")
        return
    if tuple(idx_proj.shape) != (IDX_DIM, HEAD_DIM):
        raise ValueError("idx_proj must be [64][128]")
    if ik_scales4 is not None:
        rc = lib().csa2_write_entries_proj_fp4(
            *head, _ptr(idx_proj, torch.float32, "idx_proj"),
            _ptr(ik_codes, torch.uint8, "ik_codes"), _ptr(ik_scales4, torch.uint8, "ik_scales4"),
            jobs, len(fp8_jobs), _stream(stream))
        _check(rc, "csa2_write_entries_proj_fp4")
        return
    rc = lib().csa2_write_entries_proj(
        *head, _ptr(idx_proj, torch.float32, "idx_proj"), _ptr(ik_codes, torch.uint8, "ik_codes"),
        _ptr(ik_sigma, torch.float32, "ik_sigma"), jobs, len(fp8_jobs), _stream(stream))
    _check(rc, "csa2_write_entries_proj")


def _ik_aux_ptr(cache):
    if cache.idx_fp4:
        return _ptr(cache.ik_scales4, torch.uint8, "ik_scales4")
    return _ptr(cache.ik_sigma, torch.float32, "ik_sigma")


def quant_idx_fp4(x, ik_codes, ik_scales4, dst_rows=None, stream=None):
    """x [n][64] f32 -> FP4 indexer keys at rows dst_rows (or 0..n-1)."""
    if x.dim() != 2 or x.shape[1] != IDX_DIM:
        raise ValueError("x must be [n][64]")
    n = x.shape[0]
    rc = lib().csa2_quant_idx_fp4(_ptr(x, torch.float32, "x"), n,
                                  _ptr(dst_rows, torch.int64, "dst_rows", n),
                                  _ptr(ik_codes, torch.uint8, "ik_codes"),
                                  _ptr(ik_scales4, torch.uint8, "ik_scales4"), _stream(stream))
    _check(rc, "csa2_quant_idx_fp4")


def index_full(cache, iq, iw, n_vis, topk_idx, pool_idx=None, topk=DEFAULT_TOPK,
               pool_blocks=0, ws=None, stream=None, scan_timer=None):
    """iq [B][Q][4][64] f32, iw [B][Q][4] f32, n_vis [B][Q] i32 ->
    topk_idx [B][Q][topk] i32, pool_idx [B][Q][pool_blocks] i32.
    scan_timer: optional KernelTimer whose events bracket the scan kernel."""
    B, Q = iq.shape[0], iq.shape[1]
    _check_batch(cache, B, "index_full")
    need = workspace_size(OP_INDEX_FULL, B, Q, cache.cap, topk, pool_blocks, 0)
    if ws is None:
        ws = alloc_workspace(need, iq.device)
    ev = scan_timer.next_pair() if scan_timer is not None else (None, None)
    fn = lib().csa2_index_full_fp4_timed if cache.idx_fp4 else lib().csa2_index_full_timed
    rc = fn(
        _ptr(cache.ik_codes, torch.uint8, "ik_codes"), _ik_aux_ptr(cache), cache.cap, B, Q, _ptr(iq, torch.float32, "iq", B * Q * 256),
        _ptr(iw, torch.float32, "iw", B * Q * 4), _ptr(n_vis, torch.int32, "n_vis", B * Q),
        topk, pool_blocks, _ptr(topk_idx, torch.int32, "topk_idx", B * Q * topk),
        _ptr(pool_idx, torch.int32, "pool_idx", B * Q * pool_blocks) if pool_blocks else None,
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream), ev[0], ev[1])
    _check(rc, "csa2_index_full")


NOALLOC_SCRATCH_BYTES = 32 << 20


def index_full_noalloc(cache, iq, iw, n_vis, topk_idx, pool_idx=None, topk=DEFAULT_TOPK,
                       pool_blocks=0, stream=None):
    """index_full without a workspace (FP8 indexer keys): the library's own
    fixed scratch of NOALLOC_SCRATCH_BYTES per GPU; calls that overlap on one
    GPU race."""
    B, Q = iq.shape[0], iq.shape[1]
    _check_batch(cache, B, "index_full_noalloc")
    if cache.idx_fp4:
        raise ValueError("index_full_noalloc takes FP8 indexer keys")
    rc = lib().csa2_index_full_noalloc(
        _ptr(cache.ik_codes, torch.uint8, "ik_codes"), _ik_aux_ptr(cache), cache.cap, B, Q,
        _ptr(iq, torch.float32, "iq", B * Q * 256), _ptr(iw, torch.float32, "iw", B * Q * 4),
        _ptr(n_vis, torch.int32, "n_vis", B * Q), topk, pool_blocks,
        _ptr(topk_idx, torch.int32, "topk_idx", B * Q * topk),
        _ptr(pool_idx, torch.int32, "pool_idx", B * Q * pool_blocks) if pool_blocks else None,
        _stream(stream))
    _check(rc, "csa2_index_full_noalloc")


def index_reindex(cache, iq, iw, n_vis, pool_idx, topk_idx, topk=DEFAULT_TOPK, ws=None,
                  stream=None):
    B, Q = iq.shape[0], iq.shape[1]
    _check_batch(cache, B, "index_reindex")
    pool_blocks = pool_idx.shape[-1]
    need = workspace_size(OP_INDEX_REINDEX, B, Q, cache.cap, topk, pool_blocks, 0)
    if ws is None:
        ws = alloc_workspace(need, iq.device)
    fn = lib().csa2_index_reindex_fp4 if cache.idx_fp4 else lib().csa2_index_reindex
    rc = fn(
        _ptr(cache.ik_codes, torch.uint8, "ik_codes"), _ik_aux_ptr(cache), cache.cap, B, Q, _ptr(iq, torch.float32, "iq", B * Q * 256),
        _ptr(iw, torch.float32, "iw", B * Q * 4), _ptr(n_vis, torch.int32, "n_vis", B * Q),
        _ptr(pool_idx, torch.int32, "pool_idx", B * Q * pool_blocks), pool_blocks, topk,
        _ptr(topk_idx, torch.int32, "topk_idx", B * Q * topk),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream))
    _check(rc, "csa2_index_reindex")


def sparse_attn_decode(q, cache, topk_idx, swa_k, swa_v, swa_ks, swa_vs, swa_len, out, lse,
                       sm_scale=None, ws=None, stream=None, timer=None):
    """q [B][H][128] f32; topk_idx [B][topk]; swa_k/v [B][128][128] u8; swa_ks/vs [B][128];
    swa_len [B] i32 -> out [B][H][128], lse [B][H].
    timer: optional KernelTimer; its next event pair brackets the kernel's dispatch."""
    B, H = q.shape[0], q.shape[1]
    _check_batch(cache, B, "sparse_attn_decode")
    topk = topk_idx.shape[-1]
    sm = 1.0 / math.sqrt(HEAD_DIM) if sm_scale is None else sm_scale
    need = workspace_size(OP_ATTN_DECODE, B, 1, cache.cap, topk, 0, H)
    if ws is None and need:
        ws = alloc_workspace(need, q.device)
    ev = timer.next_pair() if timer is not None else (None, None)
    rc = lib().csa2_sparse_attn_decode_timed(
        _ptr(q, torch.float32, "q", B * H * HEAD_DIM), B, H,
        _ptr(cache.kv_codes, torch.uint8, "kv_codes"), _ptr(cache.kv_scales, torch.uint8, "kv_scales"),
        cache.cap, _ptr(topk_idx, torch.int32, "topk_idx", B * topk), topk,
        _ptr(swa_k, torch.uint8, "swa_k", B * WINDOW * HEAD_DIM),
        _ptr(swa_v, torch.uint8, "swa_v", B * WINDOW * HEAD_DIM),
        _ptr(swa_ks, torch.float32, "swa_ks", B * WINDOW),
        _ptr(swa_vs, torch.float32, "swa_vs", B * WINDOW),
        _ptr(swa_len, torch.int32, "swa_len", B), sm,
        _ptr(out, torch.float32, "out", B * H * HEAD_DIM), _ptr(lse, torch.float32, "lse", B * H),
        _ptr(ws, torch.uint8, "ws") if ws is not None else None,
        ws.numel() if ws is not None else 0, _stream(stream), ev[0], ev[1])
    _check(rc, "csa2_sparse_attn_decode")


def sparse_attn_decode_reuse(q, cache, topk_idx, topk, stage, stage_mode, swa_k, swa_v, swa_ks,
                             swa_vs, swa_len, out, lse, sm_scale=None, ws=None, stream=None,
                             timer=None):
    """sparse_attn_decode for layers sharing one selection.  stage_mode
    STAGE_WRITE: gather through topk_idx [B][topk] (cache required) and write
    the staged records to `stage` (u8, workspace_size(OP_ATTN_STAGE, ...)
    bytes); STAGE_READ: take the records from `stage` (cache and topk_idx may
    be None)."""
    B, H = q.shape[0], q.shape[1]
    if cache is not None:
        _check_batch(cache, B, "sparse_attn_decode_reuse")
    sm = 1.0 / math.sqrt(HEAD_DIM) if sm_scale is None else sm_scale
    cap = cache.cap if cache is not None else 1
    need = workspace_size(OP_ATTN_DECODE, B, 1, cap, topk, 0, H)
    if ws is None and need:
        ws = alloc_workspace(need, q.device)
    if stage_mode == STAGE_WRITE:
        if cache is None or topk_idx is None:
            raise ValueError("STAGE_WRITE gathers through the cache: cache and topk_idx needed")
        if topk_idx.shape[-1] != topk:
            raise ValueError("topk_idx must be [B][topk]")
    ev = timer.next_pair() if timer is not None else (None, None)
    rc = lib().csa2_sparse_attn_decode_reuse(
        _ptr(q, torch.float32, "q", B * H * HEAD_DIM), B, H,
        _ptr(cache.kv_codes, torch.uint8, "kv_codes") if cache is not None else None,
        _ptr(cache.kv_scales, torch.uint8, "kv_scales") if cache is not None else None, cap,
        _ptr(topk_idx, torch.int32, "topk_idx", B * topk) if topk_idx is not None else None, topk,
        _ptr(stage, torch.uint8, "stage") if stage is not None else None,
        stage.numel() if stage is not None else 0, stage_mode,
        _ptr(swa_k, torch.uint8, "swa_k", B * WINDOW * HEAD_DIM),
        _ptr(swa_v, torch.uint8, "swa_v", B * WINDOW * HEAD_DIM),
        _ptr(swa_ks, torch.float32, "swa_ks", B * WINDOW),
        _ptr(swa_vs, torch.float32, "swa_vs", B * WINDOW),
        _ptr(swa_len, torch.int32, "swa_len", B), sm,
        _ptr(out, torch.float32, "out", B * H * HEAD_DIM), _ptr(lse, torch.float32, "lse", B * H),
        _ptr(ws, torch.uint8, "ws") if ws is not None else None,
        ws.numel() if ws is not None else 0, _stream(stream), ev[0], ev[1])
    _check(rc, "csa2_sparse_attn_decode_reuse")


def sparse_attn_chunk(q, cache, topk_idx, swa_k, swa_v, swa_ks, swa_vs, out, lse, sm_scale=None,
                      ws=None, stream=None):
    """q [B][Q][H][128]; topk_idx [B][Q][topk]; chunk window swa_k/v [B][Q][128], swa_ks/vs [B][Q]."""
    B, Q, H = q.shape[0], q.shape[1], q.shape[2]
    _check_batch(cache, B, "sparse_attn_chunk")
    topk = topk_idx.shape[-1]
    sm = 1.0 / math.sqrt(HEAD_DIM) if sm_scale is None else sm_scale
    need = workspace_size(OP_ATTN_CHUNK, B, Q, cache.cap, topk, 0, H)
    if ws is None and need:
        ws = alloc_workspace(need, q.device)
    rc = lib().csa2_sparse_attn_chunk(
        _ptr(q, torch.float32, "q", B * Q * H * HEAD_DIM), B, Q, H,
        _ptr(cache.kv_codes, torch.uint8, "kv_codes"), _ptr(cache.kv_scales, torch.uint8, "kv_scales"),
        cache.cap, _ptr(topk_idx, torch.int32, "topk_idx", B * Q * topk), topk,
        _ptr(swa_k, torch.uint8, "swa_k", B * Q * HEAD_DIM),
        _ptr(swa_v, torch.uint8, "swa_v", B * Q * HEAD_DIM),
        _ptr(swa_ks, torch.float32, "swa_ks", B * Q), _ptr(swa_vs, torch.float32, "swa_vs", B * Q),
        sm, _ptr(out, torch.float32, "out", B * Q * H * HEAD_DIM),
        _ptr(lse, torch.float32, "lse", B * Q * H),
        _ptr(ws, torch.uint8, "ws") if ws is not None else None,
        ws.numel() if ws is not None else 0, _stream(stream))
    _check(rc, "csa2_sparse_attn_chunk")


def codec_probe(x, stream=None):
    """Run the device codecs: returns (E4M3 decode [256] via the scan's fp32
    converter, E4M3 decode [256] via the attention's fp16 converter, FP4 code x
    scale products [256][16], E4M3 encode of x, E2M1 encode of x)."""
    dev = x.device
    e4 = torch.empty(256, dtype=torch.float32, device=dev)
    e4h = torch.empty(256, dtype=torch.float32, device=dev)
    fp4 = torch.empty((256, 16), dtype=torch.float32, device=dev)
    enc4 = torch.empty(x.numel(), dtype=torch.uint8, device=dev)
    enc2 = torch.empty(x.numel(), dtype=torch.uint8, device=dev)
    rc = lib().csa2_codec_probe(_ptr(e4, torch.float32, "e4m3_dec"),
                                _ptr(e4h, torch.float32, "e4m3_dec16"),
                                _ptr(fp4, torch.float32, "fp4_dec16"),
                                _ptr(x, torch.float32, "x"), x.numel(),
                                _ptr(enc4, torch.uint8, "e4m3_enc"), _ptr(enc2, torch.uint8, "e2m1_enc"),
                                _stream(stream))
    _check(rc, "csa2_codec_probe")
    return e4, e4h, fp4, enc4, enc2


def stream_probe(mode, src, dst=None, sink=None, n_blocks=2048, stream=None):
    """Diagnostics: mode 0 streams src (u8, a multiple of 16 bytes) with
    16-byte loads (grid-stride), mode 2 with one load per thread, mode 3 in
    16 KB chunks (one per workgroup, four loads per thread), mode 1 copies it
    to dst (csa2_stream_probe)."""
    if sink is None and mode != 1:
        sink = torch.empty(n_blocks, dtype=torch.int32, device=src.device)
    rc = lib().csa2_stream_probe(mode, _ptr(src, torch.uint8, "src"),
                                 _ptr(dst, torch.uint8, "dst", src.numel()) if dst is not None else None,
                                 src.numel(), _ptr(sink, torch.int32, "sink", n_blocks) if sink is not None else None,
                                 n_blocks, _stream(stream))
    _check(rc, "csa2_stream_probe")


def gather_probe(q, cache, topk_idx, swa_k, swa_v, swa_ks, swa_vs, out, stream=None, timer=None):
    """Diagnostics: reads what sparse_attn_decode reads for a full window
    (q [B][H][128], the selected records, the 128 window rows) and writes out
    [B][H][128] with no arithmetic: each word i of a query's row is word
    i mod 4 of the XOR of every 16-byte unit read for it (csa2_gather_probe).
    timer: optional KernelTimer; its next event pair brackets the dispatch."""
    B, H = q.shape[0], q.shape[1]
    _check_batch(cache, B, "gather_probe")
    topk = topk_idx.shape[-1]
    ev = timer.next_pair() if timer is not None else (None, None)
    rc = lib().csa2_gather_probe(
        _ptr(cache.kv_codes, torch.uint8, "kv_codes"), _ptr(cache.kv_scales, torch.uint8, "kv_scales"),
        _ptr(topk_idx, torch.int32, "topk_idx", B * topk), B, topk, cache.cap,
        _ptr(swa_k, torch.uint8, "swa_k", B * WINDOW * HEAD_DIM),
        _ptr(swa_v, torch.uint8, "swa_v", B * WINDOW * HEAD_DIM),
        _ptr(swa_ks, torch.float32, "swa_ks", B * WINDOW),
        _ptr(swa_vs, torch.float32, "swa_vs", B * WINDOW),
        _ptr(q, torch.float32, "q", B * H * HEAD_DIM), H,
        _ptr(out, torch.float32, "out", B * H * HEAD_DIM), _stream(stream), ev[0], ev[1])
    _check(rc, "csa2_gather_probe")


# ---------------------------------------------------------------------------
# HIP events for kernel timing (plumbing for the bench)
# ---------------------------------------------------------------------------
_hip = None


def _hiprt():
    """The HIP runtime torch has loaded (same soname as the one libcsa2 uses)."""
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so.7", mode=ctypes.RTLD_GLOBAL)
        h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        _hip = h
    return _hip


class KernelTimer:
    """A ring of (start, stop) HIP event pairs; elapsed_ms() averages them."""

    def __init__(self, n):
        h = _hiprt()
        self.events = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            if h.hipEventCreate(ctypes.byref(e)) != 0:
                raise Csa2Error("hipEventCreate failed")
            self.events.append(e)
        self.n, self.used = n, 0

    def next_pair(self):
        i = self.used % self.n
        self.used += 1
        return self.events[2 * i], self.events[2 * i + 1]

    def durations_ms(self):
        h = _hiprt()
        out = []
        for i in range(min(self.used, self.n)):
            a, b = self.events[2 * i], self.events[2 * i + 1]
            h.hipEventSynchronize(b)
            ms = ctypes.c_float()
            if h.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
                raise Csa2Error("hipEventElapsedTime failed")
            out.append(ms.value)
        return out

    def reset(self):
        self.used = 0

    def close(self):
        h = _hiprt()
        for e in self.events:
            h.hipEventDestroy(e)
        self.events = []
