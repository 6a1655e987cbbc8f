"""grad_global_norm_noalloc: the allocation-free norm entry point, called
through the C ABI, against grad_global_norm with a caller workspace (same
kernels, so the same bits) and the oracle, on two calls in a row, the second
with a smaller input; and its size limit."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as o
from bf16_numerics_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def bfo():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from bf16_numerics_amd import binding
    torch.cuda.set_device(0)
    return binding


def _noalloc(bfo, T, G, res, max_norm=1.0):
    lib = bfo.library()
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    return lib.grad_global_norm_noalloc(T.handle, ctypes.c_void_p(G.data_ptr()), ctypes.c_float(max_norm),
                                        ctypes.c_void_p(res.data_ptr()), stream)


def _grads(n, std, step):
    G = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    W.fill_grads(torch, W.Workload("g", [("g", (n,))], grad_std=std), G, 0, step)
    return G


@pytest.mark.parametrize("sizes", [(40_000_003, 3_000_011), (300_000_000, 65_537)])
def test_noalloc_norm_equals_workspace_norm_twice(bfo, sizes):
    # The second call is smaller: the array keeps the first call's partials
    # beyond the second's, which nothing may read.  The 300M-element shard
    # (36,622 tiles) takes the intermediate reduction pass as well.
    for k, n in enumerate(sizes):
        T = bfo.Table([(0, n // 2, 1), (n // 2, n - n // 2, 0)])
        G = _grads(n, 1e-3 * (k + 1), k + 1)
        ws = bfo.new_norm_workspace(T)
        want = bfo.new_norm_result(DEV)
        bfo.grad_global_norm(T, G, want, 1.0, workspace=ws)
        got = bfo.new_norm_result(DEV)
        assert _noalloc(bfo, T, G, got) == bfo.OK
        torch.cuda.synchronize()
        assert got.cpu().numpy().tobytes() == want.cpu().numpy().tobytes(), (n, k)
        sumsq, norm, scale = bfo.read_norm_result(got)
        ref = o.grad_norm(W.bf16_bits_numpy(torch, G), 1.0)
        assert abs(sumsq - ref[0]) <= 1e-5 * ref[0] and abs(norm - ref[1]) <= 1e-5 * ref[1]
        assert abs(scale - ref[2]) <= 1e-5 * ref[2]
        T.close()


def test_noalloc_norm_small_and_per_tensor(bfo):
    # One-workgroup path (no partials) and a per-tensor table (planned loads).
    w = W.tiny()
    T = bfo.Table(w.entries())
    G = torch.empty(w.n, dtype=torch.bfloat16, device=DEV)
    W.fill_grads(torch, w, G, 0, 1)
    a, b = bfo.new_norm_result(DEV), bfo.new_norm_result(DEV)
    bfo.grad_global_norm(T, G, a, 1.0)
    assert _noalloc(bfo, T, G, b) == bfo.OK
    torch.cuda.synchronize()
    assert a.cpu().numpy().tobytes() == b.cpu().numpy().tobytes()
    w = W.gpt2_124m()
    T = bfo.Table(w.entries(), 4, 3, layout=bfo.LAYOUT_PER_TENSOR)
    G = torch.empty(w.n, dtype=torch.bfloat16, device=DEV)
    W.fill_grads(torch, w, G, 0, 2)
    bfo.grad_global_norm(T, G, a, 1.0, workspace=bfo.new_norm_workspace(T))
    assert _noalloc(bfo, T, G, b) == bfo.OK
    torch.cuda.synchronize()
    assert a.cpu().numpy().tobytes() == b.cpu().numpy().tobytes()


def test_noalloc_norm_refuses_shards_beyond_its_array(bfo):
    # 8,587,837,440 elements fill the 8 MiB array exactly; one more tile does
    # not fit.  The size is refused before any work is queued, so the small
    # buffer passed as grads is never read.
    limit = 1_048_320 * 8192
    G = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    res = bfo.new_norm_result(DEV)
    T = bfo.Table([(0, limit + 8192, 0)])
    assert bfo.norm_workspace_bytes(T) > 8 << 20
    assert _noalloc(bfo, T, G, res) == bfo.ERANGE
    T.close()
    T = bfo.Table([(0, limit, 0)])
    assert bfo.norm_workspace_bytes(T) == 8 << 20
    T.close()
    T = bfo.Table([(0, 16, 0)])
    assert _noalloc(bfo, T, G, res, max_norm=0.0) == bfo.EINVAL
    assert _noalloc(bfo, T, G, res, max_norm=float("nan")) == bfo.EINVAL
    torch.cuda.synchronize()
