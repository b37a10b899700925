"""The measurement probes on the GPU: the copy probe copies, and the gather
probe reads exactly the bytes the gathering decode attention reads (each
output word is the XOR of every 16-byte unit read for the query, computed
here on the host from the same arrays)."""
import numpy as np
import pytest
import torch

from gpu_util import dev, host

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[probe] {msg}", flush=True)


def xor_units(*arrays):
    acc = np.zeros(4, np.uint32)
    for a in arrays:
        u = np.ascontiguousarray(a).view(np.uint32).reshape(-1, 4)
        acc ^= np.bitwise_xor.reduce(u, axis=0) if len(u) else 0
    return acc


def test_stream_copy_probe_copies(gpu):
    say("stream copy 3 MiB")
    src = torch.randint(0, 256, (3 << 20,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    gpu.stream_probe(1, src, dst, n_blocks=300)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("mode", [0, 2, 3])
def test_stream_read_probes_cover_a_ragged_buffer(gpu, mode):
    """The read probes run over a buffer that is not a whole number of their
    chunks (the last workgroup partly past it) and leave the sink untouched:
    only a data-dependent test on an all-ones buffer could write it (mode 0
    writes its per-workgroup XOR, zero for an even number of equal words)."""
    say(f"stream read mode {mode}, 3 MiB + 48 bytes")
    src = torch.ones((3 << 20) + 48, dtype=torch.uint8, device="cuda")
    sink = torch.full((300,), 7, dtype=torch.int32, device="cuda")
    gpu.stream_probe(mode, src, sink=sink, n_blocks=300)
    torch.cuda.synchronize()
    if mode == 0:
        assert torch.all(sink == 0)
    else:
        assert torch.all(sink == 7)


@pytest.mark.parametrize("B,cap,H,topk", [(3, 1024, 16, 512), (2, 4096, 64, 700), (1, 256, 128, 5)])
def test_gather_probe_reads_the_attention_bytes(gpu, B, cap, H, topk):
    say(f"gather B={B} cap={cap} H={H} topk={topk}")
    g = np.random.default_rng(50 + B)
    codes = g.integers(0, 256, (B, cap, 128), dtype=np.uint8)
    scales = g.integers(0, 256, (B, cap, 16), dtype=np.uint8)
    idx = np.stack([g.choice(cap, topk, replace=topk > cap) for _ in range(B)]).astype(np.int32)
    idx[0, :3] = [-1, cap, cap + 7]  # skipped: padding and positions past the cache
    swk = g.integers(0, 256, (B, 128, 128), dtype=np.uint8)
    swv = g.integers(0, 256, (B, 128, 128), dtype=np.uint8)
    sks = g.standard_normal((B, 128)).astype(np.float32)
    svs = g.standard_normal((B, 128)).astype(np.float32)
    q = g.standard_normal((B, H, 128)).astype(np.float32)
    cache = gpu.Cache(B, cap)
    cache.kv_codes.copy_(dev(codes.reshape(-1, 128)))
    cache.kv_scales.copy_(dev(scales.reshape(-1, 16)))
    out = torch.zeros((B, H, 128), dtype=torch.float32, device="cuda")
    gpu.gather_probe(dev(q), cache, dev(idx), dev(swk), dev(swv), dev(sks), dev(svs), out)
    got = host(out).view(np.uint32).reshape(B, -1)
    for b in range(B):
        sel = idx[b][(idx[b] >= 0) & (idx[b] < cap)]
        acc = xor_units(codes[b][sel], scales[b][sel], swk[b], swv[b], sks[b], svs[b], q[b])
        np.testing.assert_array_equal(got[b], np.tile(acc, H * 32), err_msg=f"query {b}")
