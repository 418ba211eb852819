"""The allocation-free GEMM entry point (qwg_gemm_q4k_noalloc) against the
allocating one (qwg_gemm_q4k): the same kernels and plans, so the outputs must
be bit-identical, and both within the oracle's bound. Two calls in a row per
case, the second on a smaller input, so the shared scratch array is reused with
a different plan."""
import numpy as np
import pytest
import torch

import oracle
import quantized_weight_decode_gemv_amd as qwg
from quantized_weight_decode_gemv_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-6


def _case(n_out, n_in, batch, seed):
    w = synth.q4k_weights(n_out, n_in, 190, seed)
    x = synth.activations(n_in, 190, seed, batch=batch)
    return w, x


def _check(w, x, n_in, n_out, batch):
    wd = torch.from_numpy(w).to(DEV)
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    y_ref = qwg.gemm_q4k(wd, xd)
    y = torch.full((batch, n_out), float("nan"), device=DEV)
    qwg.gemm_q4k_noalloc(wd, xd, out=y)
    torch.cuda.synchronize()
    a, b = y.cpu().numpy(), y_ref.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{batch}x{n_out}x{n_in}"
    yr, sr = oracle.gemm_q4k(w, x, n_in, n_out)
    assert (np.abs(a.astype(np.float64) - yr) <= TOL * sr).all(), f"{batch}x{n_out}x{n_in}"


@pytest.fixture(scope="module", autouse=True)
def _ready():
    oracle.build(force=False)
    qwg.lib()


@pytest.mark.parametrize("first,second", [
    # (n_out, n_in, batch): split plans on the batch-1 engines and on the
    # matrix cores (batch >= 2), then a smaller input
    ((2048, 5632, 1), (200, 5632, 1)),
    ((2048, 5632, 1), (256, 2048, 1)),
    ((2048, 2048, 8), (130, 768, 3)),
    ((5632, 2048, 1), (7, 256, 1)),
    ((32000, 2048, 1), (64, 512, 2)),
])
def test_noalloc_matches_gemm_q4k_two_calls(first, second):
    for k, (n_out, n_in, batch) in enumerate((first, second)):
        w, x = _case(n_out, n_in, batch, 10 * k + batch)
        _check(w, x, n_in, n_out, batch)


def test_noalloc_under_graph_capture_on_a_fresh_stream():
    # A stream with no split workspace: the allocating entry point would refuse
    # to allocate under capture; the allocation-free one records its kernels.
    n_out, n_in = 2048, 2048
    w, x = _case(n_out, n_in, 1, 50)
    wd = torch.from_numpy(w).to(DEV)
    xd = torch.from_numpy(x).to(DEV)
    y = torch.full((1, n_out), float("nan"), device=DEV)
    side = torch.cuda.Stream()
    qwg.workspace_release(side)
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        qwg.gemm_q4k_noalloc(wd, xd, out=y)
    ref = qwg.gemm_q4k(wd, xd)
    for _ in range(3):
        y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref)
