"""The C ABI on a machine without a GPU: the library loads, exports every
function include/csa2.h declares, and rejects bad scalar arguments with the
documented status codes before touching the HIP runtime."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import torch  # noqa: F401  (same HIP runtime as the binding)
    import compressed_kv_cache_decode_amd as csa2
    return csa2.lib()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    import compressed_kv_cache_decode_amd as csa2
    assert set(csa2.EXPORTS) == set(names)


def test_version_and_status_strings(lib):
    assert lib.csa2_abi_version() == 4
    for st in (0, -1, -2, -3, -4):
        assert lib.csa2_status_str(st)
    assert lib.csa2_status_str(12345) == b"unknown status"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def test_quant_validation(lib):
    q = lib.csa2_quant_fp4
    assert q(FAKE, FAKE, 8, 3, None, None, FAKE, FAKE, None) == -2   # ratio
    assert q(FAKE, FAKE, 8, 2, FAKE, None, FAKE, FAKE, None) == -2   # RoPE with ratio 2
    assert q(FAKE, FAKE, 7, 2, None, None, FAKE, FAKE, None) == -1   # odd token count
    assert q(None, FAKE, 8, 1, None, None, FAKE, FAKE, None) == -1   # null
    assert q(FAKE, FAKE, -1, 1, None, None, FAKE, FAKE, None) == -1
    assert q(None, None, 0, 1, None, None, None, None, None) == 0    # nothing to do
    f8 = lib.csa2_quant_fp8
    assert f8(FAKE, 4, 96, 0, None, FAKE, FAKE, None) == -2          # dim
    assert f8(FAKE, 4, 128, 1, None, FAKE, FAKE, None) == -2         # tiled needs dim 64
    assert f8(FAKE, 4, 64, 7, None, FAKE, FAKE, None) == -1          # layout
    assert f8(FAKE, 4, 64, 0, None, None, FAKE, None) == -1


def test_write_entries_validation(lib):
    import compressed_kv_cache_decode_amd as csa2
    w = lib.csa2_write_entries
    J = csa2._Fp8Job

    def jobs(*js):
        arr = (J * max(len(js), 1))()
        for i, j in enumerate(js):
            arr[i] = j
        return arr

    ok = J(FAKE, 4, 64, 1, None, FAKE, FAKE)
    # the FP4 part is checked as csa2_quant_fp4 checks it
    assert w(FAKE, FAKE, 8, 3, None, None, FAKE, FAKE, jobs(), 0, None) == -2
    assert w(None, FAKE, 8, 1, None, None, FAKE, FAKE, jobs(), 0, None) == -1
    # job count and table
    assert w(FAKE, FAKE, 8, 1, None, None, FAKE, FAKE, jobs(ok), 4, None) == -1
    assert w(FAKE, FAKE, 8, 1, None, None, FAKE, FAKE, jobs(ok), -1, None) == -1
    assert w(FAKE, FAKE, 8, 1, None, None, FAKE, FAKE, None, 1, None) == -1
    # each job is checked as csa2_quant_fp8 checks it
    assert w(FAKE, FAKE, 8, 1, None, None, FAKE, FAKE, jobs(ok, J(FAKE, 4, 96, 0, None, FAKE, FAKE)), 2, None) == -2
    assert w(FAKE, FAKE, 8, 1, None, None, FAKE, FAKE, jobs(J(FAKE, 4, 128, 1, None, FAKE, FAKE)), 1, None) == -2
    assert w(FAKE, FAKE, 8, 1, None, None, FAKE, FAKE, jobs(J(FAKE, 4, 64, 0, None, None, FAKE)), 1, None) == -1
    assert w(FAKE, FAKE, 8, 1, None, None, FAKE, FAKE, jobs(J(FAKE, -2, 64, 0, None, FAKE, FAKE)), 1, None) == -1
    # nothing to write: no launch
    assert w(None, None, 0, 1, None, None, None, None, jobs(J(None, 0, 64, 0, None, None, None)), 1, None) == 0


def test_index_validation(lib):
    f = lib.csa2_index_full
    ok = dict(cap=1024, B=2, Q=1, topk=512, pool=2048)

    def call(cap=1024, B=2, Q=1, topk=512, pool=2048, ws=FAKE, ws_bytes=1 << 40, ptr=FAKE):
        return f(ptr, FAKE, cap, B, Q, FAKE, FAKE, FAKE, topk, pool, FAKE, FAKE, ws, ws_bytes, None)

    assert call(ptr=None) == -1
    assert call(cap=1000) == -1          # not a multiple of 64
    assert call(cap=0) == -1
    assert call(B=0) == -1
    assert call(topk=0) == -1
    assert call(topk=4096) == -2
    assert call(pool=8192) == -2
    assert call(pool=256) == -2          # pool < topk blocks
    assert call(ws=None) == -3
    assert call(ws_bytes=10) == -3
    r = lib.csa2_index_reindex
    assert r(FAKE, FAKE, 1024, 1, 1, FAKE, FAKE, FAKE, None, 16, 8, FAKE, FAKE, 1 << 40, None) == -1
    assert r(FAKE, FAKE, 1024, 1, 1, FAKE, FAKE, FAKE, FAKE, 0, 8, FAKE, FAKE, 1 << 40, None) == -1
    assert r(FAKE, FAKE, 1024, 1, 1, FAKE, FAKE, FAKE, FAKE, 16, 8, FAKE, FAKE, 0, None) == -3
    del ok


def test_attention_validation(lib):
    a = lib.csa2_sparse_attn_decode

    def call(B=4, H=64, topk=512, sm=0.088, swa_len=FAKE, q=FAKE, ws=FAKE, wsb=1 << 40):
        return a(q, B, H, FAKE, FAKE, 4096, FAKE, topk, FAKE, FAKE, FAKE, FAKE, swa_len,
                 ctypes.c_float(sm), FAKE, FAKE, ws, wsb, None)

    assert call(q=None) == -1
    assert call(H=24) == -2
    assert call(H=256) == -2
    assert call(topk=-1) == -1
    assert call(topk=4096) == -2
    assert call(sm=float("nan")) == -1
    assert call(swa_len=None) == -1
    r = lib.csa2_sparse_attn_decode_reuse

    def reuse(mode=2, stage=FAKE, stage_bytes=1 << 40, topk=512, ws=FAKE):
        return r(FAKE, 4, 64, None, None, 0, None, topk, stage, stage_bytes, mode, FAKE, FAKE,
                 FAKE, FAKE, FAKE, ctypes.c_float(0.088), FAKE, FAKE, ws, 1 << 40, None, None, None)

    assert reuse(mode=0) == -1 and reuse(mode=3) == -1
    assert reuse(stage=None) == -1                    # records must come from somewhere
    assert reuse(stage_bytes=4 * 16 * 4672 - 1) == -3  # B * ceil(topk / 32) tiles of 4672 B
    assert reuse(mode=1) == -1                        # a writing call gathers: cache needed
    c = lib.csa2_sparse_attn_chunk
    assert c(FAKE, 1, 128, 40, FAKE, FAKE, 4096, FAKE, 512, FAKE, FAKE, FAKE, FAKE,
             ctypes.c_float(0.088), FAKE, FAKE, FAKE, 1 << 40, None) == -2


def test_workspace_sizes(lib):
    ws = lib.csa2_workspace_size
    big = ctypes.c_size_t(-1).value
    n_full = ws(1, 16, 1, 131072, 512, 2048, 0)
    # keys (4 B/position) + block keys (0.5 B/position) dominate
    assert 16 * 131072 * 4.5 <= n_full < 16 * 131072 * 4.5 + (1 << 20)
    assert ws(1, 16, 1, 131072, 512, 0, 0) == n_full         # internal pool lives in LDS
    assert ws(2, 16, 1, 131072, 512, 2048, 0) >= 16 * 2048 * 8 * 4
    # Reindex: the pool keys (4 B per pool position) and a 16-byte summary
    # per 64 of them (the selection's lower bound), each 256-byte aligned
    al = lambda n: (n + 255) // 256 * 256
    assert ws(2, 16, 1, 131072, 512, 2048, 0) == al(16 * 2048 * 8 * 4) + al(16 * 256 * 16)
    assert ws(2, 3, 1, 4096, 100, 61, 0) == al(3 * 61 * 8 * 4) + al(3 * 8 * 16)
    assert ws(1, 16, 1, 1000, 512, 2048, 0) == big
    assert ws(99, 1, 1, 64, 1, 1, 16) == big
    assert ws(5, 16, 1, 131072, 512, 0, 64) == 16 * 16 * 4672  # staged records
    assert ws(5, 2, 1, 131072, 100, 0, 64) == 2 * 4 * 4672
    assert ws(5, 2, 1, 131072, 0, 0, 64) == 0
    assert ws(3, 16, 1, 131072, 512, 0, 64) == 0              # attention needs no workspace
    assert ws(4, 1, 128, 131072, 512, 0, 64) == 0


def test_projected_write_and_fp4_key_validation(lib):
    import compressed_kv_cache_decode_amd as csa2
    J = csa2._Fp8Job
    none = (J * 1)()
    for w in (lib.csa2_write_entries_proj, lib.csa2_write_entries_proj_fp4):
        # the FP4 part as csa2_quant_fp4, then the projection arrays
        assert w(FAKE, FAKE, 8, 3, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, none, 0, None) == -2
        assert w(FAKE, FAKE, 8, 1, None, None, FAKE, FAKE, None, FAKE, FAKE, none, 0, None) == -1
        assert w(FAKE, FAKE, 8, 1, None, None, FAKE, FAKE, FAKE, None, FAKE, none, 0, None) == -1
        assert w(FAKE, FAKE, 8, 1, None, None, FAKE, FAKE, FAKE, FAKE, None, none, 0, None) == -1
        assert w(FAKE, FAKE, 8, 1, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, none, 4, None) == -1
        bad = (J * 1)(J(FAKE, 4, 96, 0, None, FAKE, FAKE))
        assert w(FAKE, FAKE, 8, 1, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, bad, 1, None) == -2
        # no entries and no rows: nothing to launch, the projection is not needed
        assert w(None, None, 0, 1, None, None, None, None, None, None, None, none, 0, None) == 0
    q4 = lib.csa2_quant_idx_fp4
    assert q4(FAKE, -1, None, FAKE, FAKE, None) == -1
    assert q4(None, 4, None, FAKE, FAKE, None) == -1
    assert q4(FAKE, 4, None, FAKE, None, None) == -1
    assert q4(None, 0, None, None, None, None) == 0

    f = lib.csa2_index_full_fp4

    def call(cap=1024, B=2, Q=1, topk=512, pool=2048, ws=FAKE, ws_bytes=1 << 40, ptr=FAKE):
        return f(ptr, FAKE, cap, B, Q, FAKE, FAKE, FAKE, topk, pool, FAKE, FAKE, ws, ws_bytes, None)

    assert call(ptr=None) == -1
    assert call(cap=1000) == -1
    assert call(topk=0) == -1
    assert call(topk=4096) == -2
    assert call(pool=256) == -2
    assert call(ws=None) == -3
    assert call(ws_bytes=10) == -3
    r = lib.csa2_index_reindex_fp4
    assert r(FAKE, FAKE, 1024, 1, 1, FAKE, FAKE, FAKE, None, 16, 8, FAKE, FAKE, 1 << 40, None) == -1
    assert r(FAKE, None, 1024, 1, 1, FAKE, FAKE, FAKE, FAKE, 16, 8, FAKE, FAKE, 1 << 40, None) == -1
    assert r(FAKE, FAKE, 1024, 1, 1, FAKE, FAKE, FAKE, FAKE, 16, 8, FAKE, FAKE, 0, None) == -3


def test_reindex_query_count_limit(lib):
    r = lib.csa2_index_reindex
    assert r(FAKE, FAKE, 1024, 2, 40000, FAKE, FAKE, FAKE, FAKE, 16, 8, FAKE, FAKE, 1 << 40, None) == -2


def test_rope_table_host_export(lib, oracle_mod):
    """The library's rotation table equals the oracle's independent one bit for
    bit, at small and large positions, and rejects bad arguments."""
    import numpy as np
    import compressed_kv_cache_decode_amd as csa2
    pos = np.concatenate([np.arange(0, 300), np.arange(131000, 131100), [1 << 20, (1 << 24) - 1]])
    np.testing.assert_array_equal(csa2.rope_table(pos), oracle_mod.rope_table(pos))
    assert csa2.rope_table(np.zeros(0, np.int64)).shape == (0, 32, 2)
    out = (ctypes.c_float * 64)()
    p = (ctypes.c_int64 * 1)(5)
    assert lib.csa2_rope_table(p, -1, 10000.0, out) == -1
    assert lib.csa2_rope_table(p, 1, 1.0, out) == -1
    assert lib.csa2_rope_table(None, 1, 10000.0, out) == -1
    assert lib.csa2_rope_table(p, 1, 10000.0, out) == 0


def test_batch_larger_than_the_cache_is_rejected_before_any_launch():
    """The binding refuses a query batch larger than the cache's: the kernels
    would address rows past the cache arrays.  Checked on the host first, so
    no GPU is needed here."""
    import types
    import torch
    import compressed_kv_cache_decode_amd as csa2
    cache = types.SimpleNamespace(B=2, cap=64, idx_fp4=False)
    iq = torch.zeros((3, 1, 4, 64))
    with pytest.raises(ValueError, match="does not fit"):
        csa2.index_full(cache, iq, None, None, None)
    with pytest.raises(ValueError, match="does not fit"):
        csa2.index_reindex(cache, iq, None, None, torch.zeros((3, 1, 8)), None)
    q = torch.zeros((3, 16, 128))
    with pytest.raises(ValueError, match="does not fit"):
        csa2.sparse_attn_decode(q, cache, None, None, None, None, None, None, None, None)
    with pytest.raises(ValueError, match="does not fit"):
        csa2.sparse_attn_decode_reuse(q, cache, None, 512, None, csa2.STAGE_READ, None, None,
                                      None, None, None, None, None)
    with pytest.raises(ValueError, match="does not fit"):
        csa2.sparse_attn_chunk(torch.zeros((3, 4, 16, 128)), cache, None, None, None, None, None,
                               None, None)


def test_noalloc_index_full_rejects_before_touching_the_gpu(lib):
    """csa2_index_full_noalloc refuses sizes whose workspace exceeds its fixed
    scratch, and bad scalars, with the documented codes and no HIP call."""
    f = lib.csa2_index_full_noalloc
    big = 1 << 24  # 16 sequences x 16M positions need far more than 32 MiB
    assert f(FAKE, FAKE, big, 16, 1, FAKE, FAKE, FAKE, 512, 2048, FAKE, FAKE, None) == -3
    assert f(None, FAKE, 1024, 1, 1, FAKE, FAKE, FAKE, 512, 0, FAKE, None, None) == -1
    assert f(FAKE, FAKE, 1000, 1, 1, FAKE, FAKE, FAKE, 512, 0, FAKE, None, None) == -1  # cap % 64
    assert f(FAKE, FAKE, 1024, 1, 1, FAKE, FAKE, FAKE, 4096, 0, FAKE, None, None) == -2  # topk
    import compressed_kv_cache_decode_amd as csa2
    need = csa2.workspace_size(csa2.OP_INDEX_FULL, 16, 1, 131072, 512, 2048, 0)
    assert need <= csa2.NOALLOC_SCRATCH_BYTES


def test_probes_reject_bad_arguments_before_touching_the_gpu(lib):
    """The measurement probes (stream and gather) validate their scalars and
    pointers on the host."""
    s = lib.csa2_stream_probe
    assert s(4, FAKE, FAKE, 64, FAKE, 16, None) == -1          # mode
    assert s(-1, FAKE, FAKE, 64, FAKE, 16, None) == -1         # mode
    assert s(0, FAKE, None, 63, FAKE, 16, None) == -1          # not a multiple of 16
    assert s(0, FAKE, None, 64, None, 16, None) == -1          # read without a sink
    assert s(1, FAKE, None, 64, None, 16, None) == -1          # copy without dst
    assert s(0, FAKE, None, 64, FAKE, 0, None) == -1           # no workgroups
    assert s(0, FAKE, None, 0, FAKE, 16, None) == 0            # nothing to do
    g = lib.csa2_gather_probe
    args = [FAKE, FAKE, FAKE, 4, 512, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, None, None, None]
    for i, v in ((4, 4096), (4, -1), (5, 0), (11, 0), (0, None), (12, None),
                 (6, ctypes.c_void_p(0x1008))):  # topk, cap, H, null and misaligned pointers
        a = list(args)
        a[i] = v
        assert g(*a) == -1, (i, v)
    a = list(args)
    a[3] = 0
    assert g(*a) == 0  # no queries
