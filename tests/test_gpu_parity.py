"""GPU parity: the HIP kernels, called through the C ABI (ctypes binding), against
the CPU oracle on the same seeded inputs.

Bars: dequantization is bit-exact; a GEMV/GEMM output passes when
|y_gpu - y_oracle| <= 2e-6 * sum_k |w_k x_k| for every row (the oracle sums in
fp64); integer-valued and one-hot cases must match exactly.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import quantized_weight_decode_gemv_amd as qwg
from golden_io import floats, hexbytes, ints, load
from quantized_weight_decode_gemv_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-6


@pytest.fixture(scope="module", autouse=True)
def _ready():
    oracle.build(force=False)
    qwg.lib()


def dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_bound(y_gpu, y_ref, s_ref, what=""):
    y_gpu = np.asarray(y_gpu, np.float64).reshape(y_ref.shape)
    err = np.abs(y_gpu - y_ref)
    bad = err > TOL * s_ref
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(s_ref, 1e-300)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} rows outside the bound; worst at {i}: "
                             f"gpu {y_gpu[i]!r} oracle {y_ref[i]!r} sum|wx| {s_ref[i]!r}")


def assert_bits(a, b, what=""):
    a = np.ascontiguousarray(a, np.float32).view(np.uint32)
    b = np.ascontiguousarray(b, np.float32).view(np.uint32)
    diff = np.nonzero(a != b)[0]
    assert diff.size == 0, f"{what}: {diff.size} mismatching words, first at {diff[:5]}"


_STREAMS = {}


def stream_case(key, make):
    """Host weights and inputs of a whole per-token stream and the oracle's full
    result (y, s) for every GEMV of it, computed once per module: make() returns
    (problems, weights, inputs, oracle_fn) with oracle_fn(p, w, x) -> (y, s)."""
    if key not in _STREAMS:
        probs, ws, xs, fn = make()
        refs = [fn(p, w, x) for p, w, x in zip(probs, ws, xs)]
        _STREAMS[key] = (probs, ws, xs, refs)
    return _STREAMS[key]


def q4k_c5():
    return stream_case("q4k_c5", lambda: (
        synth.config(5), [synth.weights(p) for p in synth.config(5)],
        [synth.inputs(p) for p in synth.config(5)],
        lambda p, w, x: oracle.gemv_q4k(w, x, p.n_in, p.n_out)))


def nan_outputs(probs):
    return [torch.full((p.n_out,), float("nan"), device=DEV) for p in probs]


def assert_stream(probs, refs, Y, what):
    """Every row of every GEMV of a stream within the bound (NaN rows, left
    unwritten, fail it)."""
    for p, (yr, sr), y in zip(probs, refs, Y):
        assert_bound(host(y), yr, sr, f"{what} {p.name}")


# ---------------------------------------------------------------- dequant

def test_dequant_q4k_hand_blocks():
    for name in ("q4k_block_A.txt", "q4k_block_C.txt"):
        g = load(name)
        blk = np.array(hexbytes(g["head"]) + [int(g["quant_fill"], 16)] * 128, np.uint8)
        w = host(qwg.dequant_q4k(dev(blk)))
        assert_bits(w, np.repeat(np.array(floats(g["subblock_values"]), np.float32), 32), name)
    g = load("q4k_nibble_order.txt")
    blk = np.array(hexbytes(g["head"]) + list(range(128)), np.uint8)
    assert_bits(host(qwg.dequant_q4k(dev(blk))), np.array(ints(g["weights"]), np.float32))


@pytest.mark.parametrize("n_out,n_in", [(1, 256), (3, 512), (2048, 2048), (256, 2048),
                                        (5632, 2048), (2048, 5632)])
def test_dequant_q4k_matches_oracle(n_out, n_in):
    w = synth.q4k_weights(n_out, n_in, 91, n_out + n_in)
    got = host(qwg.dequant_q4k(dev(w)))
    assert_bits(got, oracle.dequant_q4k(w, n_out * n_in), f"{n_out}x{n_in}")


# Past one grid's worth of blocks: the dequant launchers cap the grid at 65,536
# four-wavefront workgroups (262,144 blocks), and wavefronts walk further
# blocks in a grid-stride loop. The C3 LM head (256,000 blocks) is just below
# the cap; 266,241 blocks take a second, partial trip; 786,433 a third.
@pytest.mark.parametrize("nblocks", [256000, 262144 + 4097, 3 * 262144 + 1])
def test_dequant_q4k_grid_stride(nblocks):
    w = synth.q4k_weights(nblocks, 256, 93, nblocks % 1000)
    got = qwg.dequant_q4k(dev(w))
    ref = oracle.dequant_q4k(w, nblocks * 256)
    bad = int((host(got).view(np.uint32) != ref.view(np.uint32)).sum())
    assert bad == 0, f"{bad} mismatching weights"


@pytest.mark.parametrize("fmt", ["iq3", "iq3_xxs", "iq3s", "iq4xs"])
def test_dequant_codebooks_grid_stride(fmt):
    nblocks = 262144 + 4097
    if fmt == "iq3":
        w, tab = synth.iq3_weights(nblocks, 256, 94, 0), synth.iq3_grid()
        got, ref = qwg.dequant_iq3(dev(w), dev(tab)), oracle.dequant_iq3(w, tab, nblocks * 256)
    elif fmt == "iq3_xxs":
        w, tab = synth.iq3_xxs_weights(nblocks, 256, 94, 1), synth.iq3_xxs_grid()
        got, ref = qwg.dequant_iq3_xxs(dev(w), dev(tab)), oracle.dequant_iq3_xxs(w, tab, nblocks * 256)
    else:
        c = CB[fmt]
        w, tab = c["weights"](nblocks, 256, 94, 2), c["table"]()
        got, ref = c["dequant"](dev(w), dev(tab)), c["o_dequant"](w, tab, nblocks * 256)
    bad = int((host(got).reshape(-1).view(np.uint32) != ref.reshape(-1).view(np.uint32)).sum())
    assert bad == 0, f"{fmt}: {bad} mismatching weights"


def test_dequant_q4k_special_scales():
    # subnormal, negative, zero and large fp16 d / dmin
    rng = np.random.default_rng(11)
    blocks = synth.q4k_weights(64, 256, 92, 0).copy()
    specials = [0x0001, 0x03FF, 0x0400, 0x8001, 0xBC00, 0x0000, 0x8000, 0x7BFF, 0xFBFF, 0x3C00]
    for r in range(64):
        d, dm = specials[r % len(specials)], specials[(3 * r + 1) % len(specials)]
        blocks[r, 0], blocks[r, 1] = d & 0xFF, d >> 8
        blocks[r, 2], blocks[r, 3] = dm & 0xFF, dm >> 8
    got = host(qwg.dequant_q4k(dev(blocks)))
    ref = oracle.dequant_q4k(blocks, 64 * 256)
    # signed zeros may differ only where both sides are zero (x - x with negative d)
    both0 = (got == 0) & (ref == 0)
    got = np.where(both0, 0.0, got).astype(np.float32)
    ref = np.where(both0, 0.0, ref).astype(np.float32)
    assert_bits(got, ref, "special scales")
    del rng


def _grid_from(spec):
    grid = np.full((256, 4), 2.0, np.float32)
    for item in spec.split():
        k, _, vals = item.partition(":")
        grid[int(k)] = [float(v) for v in vals.split(",")]
    return grid


def test_dequant_iq3_hand_blocks():
    for name in ("iq3_block_B.txt", "iq3_block_D.txt"):
        g = load(name)
        idx = np.zeros(64, int) if g["idx"] == "zeros" else np.arange(64) % 4
        blk = oracle.iq3_block(idx, [int(t, 16) for t in g["words"].split()], int(g["d_bits"], 16))
        grid = _grid_from(g["grid_rows"])
        got = host(qwg.dequant_iq3(dev(blk), dev(grid)))
        assert_bits(got, oracle.dequant_iq3(blk, grid, 256), name)


@pytest.mark.parametrize("n_out,n_in", [(1, 256), (3, 768), (5632, 2048), (2048, 5632)])
def test_dequant_iq3_matches_oracle(n_out, n_in):
    grid = synth.iq3_grid()
    w = synth.iq3_weights(n_out, n_in, 93, n_out + n_in)
    got = host(qwg.dequant_iq3(dev(w), dev(grid)))
    assert_bits(got, oracle.dequant_iq3(w, grid, n_out * n_in), f"{n_out}x{n_in}")


# ---------------------------------------------------------------- Q4_K GEMV

def _gemv_q4k_case(n_out, n_in, cfg=94, tensor=0):
    w = synth.q4k_weights(n_out, n_in, cfg, tensor)
    x = synth.activations(n_in, cfg, tensor)
    return w, x


@pytest.mark.parametrize("p", synth.config(1) + synth.config(2) + synth.config(3)[:1],
                         ids=lambda p: f"c{p.cfg}-{p.name}")
def test_gemv_q4k_configs(p):
    w, x = synth.weights(p), synth.inputs(p)
    y = host(qwg.gemv_q4k(dev(w), dev(x)))
    yr, sr = oracle.gemv_q4k(w, x, p.n_in, p.n_out)
    assert_bound(y, yr, sr, p.name)


@pytest.mark.parametrize("n_out,n_in", [(1, 256), (2, 256), (63, 512), (64, 768), (65, 1024),
                                        (127, 1280), (200, 5632), (1000, 2048), (4097, 256),
                                        (131072 + 5, 256), (3, 65536)])
def test_gemv_q4k_ragged(n_out, n_in):
    w, x = _gemv_q4k_case(n_out, n_in, 95, n_out)
    y = host(qwg.gemv_q4k(dev(w), dev(x)))
    yr, sr = oracle.gemv_q4k(w, x, n_in, n_out)
    assert_bound(y, yr, sr, f"{n_out}x{n_in} splits={qwg.plan_splits(0, n_in, n_out)}")


@pytest.mark.parametrize("waves", [4, 8, 16])
@pytest.mark.parametrize("n_out,n_in,splits", [(70, 256, 1), (70, 2048, 1), (70, 2048, 3),
                                               (130, 5632, 1), (130, 5632, 5), (130, 5632, 22),
                                               (1, 1024, 4), (300, 1280, 2)])
def test_gemv_q4k_every_plan(waves, n_out, n_in, splits):
    w, x = _gemv_q4k_case(n_out, n_in, 107, n_out + splits)
    wd, xd = dev(w), dev(x)
    yr, sr = oracle.gemv_q4k(w, x, n_in, n_out)
    y = host(qwg.gemm_q4k(wd, xd.reshape(1, -1), waves=waves, splits=splits))
    assert_bound(y[0], yr, sr, f"waves={waves} splits={splits}")
    X = synth.activations(n_in, 107, 500 + n_out, batch=3)
    Yr, Sr = oracle.gemm_q4k(w, X, n_in, n_out)
    Y = host(qwg.gemm_q4k(wd, dev(X), waves=waves, splits=splits))
    assert_bound(Y, Yr, Sr, f"batch 3 waves={waves} splits={splits}")


def test_gemm_q4k_ex_rejects_bad_plans():
    w, x = _gemv_q4k_case(64, 512, 108, 0)
    for waves, splits in [(2, 1), (32, 1), (4, 3), (16, -1)]:
        with pytest.raises(qwg.QwgError) as e:
            qwg.gemm_q4k(dev(w), dev(x).reshape(1, -1), waves=waves, splits=splits)
        assert e.value.status == 2


def test_gemv_q4k_covers_split_and_unsplit_plans():
    # vector engine: many tiles (no split), a long row (split); short-call
    # kernel: up to one workgroup per compute unit, at most 8 splits; rows of
    # at most 8 super-blocks on those matrices: the row-group kernel (no split)
    assert qwg.plan_splits(0, 256, 131072 + 5) == 1
    assert qwg.plan_splits(0, 65536, 3) > 8
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for n_in, n_out in [(2048, 2048), (5632, 2048), (5632, 200), (2048, 5632), (256, 64),
                        (3072, 640)]:
        tiles, nb = -(-n_out // 64), n_in // 256
        want = 1 if nb <= 8 else min(cus // tiles, nb, 8)
        assert qwg.plan_splits(0, n_in, n_out) == want, (n_in, n_out)


@pytest.mark.parametrize("n_out,n_in", [(1, 256), (7, 512), (9, 2048), (63, 1792), (65, 768),
                                        (1000, 2048), (2047, 1280), (8192, 2048)])
def test_gemv_q4k_row_groups(n_out, n_in):
    # Row-group kernel (batch 1, at most 8 super-blocks per row, a matrix the
    # split short-call plan covers: at least two workgroups per tile fit the
    # compute units): eight whole rows per workgroup, lanes over (row,
    # super-block); ragged last groups, rows past n_out untouched, both layouts
    # with the same bits, repeat calls with the same bits.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert -(-n_out // 64) <= cus // 2
    assert qwg.plan_splits(0, n_in, n_out) == 1
    w, x = _gemv_q4k_case(n_out, n_in, 111, n_in // 256)
    wd, xd = dev(w), dev(x)
    yr, sr = oracle.gemv_q4k(w, x, n_in, n_out)
    buf = torch.full((n_out + 16,), float("nan"), device="cuda")
    qwg.gemv_q4k(wd, xd, out=buf[:n_out])
    y = host(buf)
    assert np.isnan(y[n_out:]).all()
    assert_bound(y[:n_out], yr, sr, f"{n_out}x{n_in}")
    wt = qwg.pack_q4k_tiles(wd, n_in)
    t = host(qwg.gemv_q4k_tiled(wt, xd, n_out))
    assert_bits(t, y[:n_out], "tile layout")
    for _ in range(2):
        assert_bits(host(qwg.gemv_q4k(wd, xd)), y[:n_out], "repeat")


@pytest.mark.parametrize("n_out,n_in", [(64, 3584), (64, 3840), (200, 5632), (2048, 5632),
                                        (100, 28672), (1, 7168), (130, 3328)])
def test_gemv_q4k_short_calls_split_and_repeat(n_out, n_in):
    # Short-call kernel: rows split into tagged words that the last split adds
    # up (up to 8 splits of 1..4 columns), on row-major and tile-layout
    # weights; repeated calls, with another shape in between on the same
    # stream, advance the tiles' epochs and give the same bits. (100 x 28672
    # has more columns per split than the kernel holds: the vector engine.)
    w, x = _gemv_q4k_case(n_out, n_in, 109, n_in // 256)
    wd, xd = dev(w), dev(x)
    wt = qwg.pack_q4k_tiles(wd, n_in)
    yr, sr = oracle.gemv_q4k(w, x, n_in, n_out)
    y1 = host(qwg.gemv_q4k(wd, xd)).copy()
    assert_bound(y1, yr, sr, f"{n_out}x{n_in} splits={qwg.plan_splits(0, n_in, n_out)}")
    t1 = host(qwg.gemv_q4k_tiled(wt, xd, n_out)).copy()
    assert_bound(t1, yr, sr, "tile layout")
    if n_in <= 8192:   # one kernel for both layouts: the same bits
        assert_bits(t1, y1, "tile layout")
    wo, xo = _gemv_q4k_case(300, 7168, 110, 0)
    other = qwg.gemv_q4k(dev(wo), dev(xo))
    for _ in range(3):
        assert_bits(host(qwg.gemv_q4k(wd, xd)), y1, "repeat")
        assert_bits(host(qwg.gemv_q4k_tiled(wt, xd, n_out)), t1, "repeat, tile layout")
    yo, so = oracle.gemv_q4k(wo, xo, 7168, 300)
    assert_bound(host(other), yo, so, "other shape")


def _integer_q4k(n_out, n_in, seed):
    # d = dmin = 1, every 6-bit scale/min in 0..7: bytes 4..11 masked to 0x07,
    # bytes 12..15 (low nibbles of scales 4..7 and mins 4..7) to 0x77.
    w = synth.q4k_weights(n_out, n_in, 96, seed).reshape(-1, 144).copy()
    w[:, 0:4] = [0x00, 0x3C, 0x00, 0x3C]
    w[:, 4:12] &= 0x07
    w[:, 12:16] &= 0x77
    return w.reshape(n_out, -1)


@pytest.mark.parametrize("n_out,n_in", [(64, 2048), (300, 5632), (7, 256)])
def test_gemv_q4k_integer_exact(n_out, n_in):
    w = _integer_q4k(n_out, n_in, n_out)
    x = np.random.default_rng(n_in).integers(-8, 9, n_in).astype(np.float32)
    y = host(qwg.gemv_q4k(dev(w), dev(x)))
    yr, _ = oracle.gemv_q4k(w, x, n_in, n_out)
    assert np.array_equal(y.astype(np.float64), yr)


def test_gemv_q4k_one_hot_is_exact_column():
    n_out, n_in = 130, 1024
    w, _ = _gemv_q4k_case(n_out, n_in, 97, 1)
    deq = oracle.dequant_q4k(w, n_out * n_in).reshape(n_out, n_in)
    wd = dev(w)
    for k in (0, 31, 32, 63, 64, 100, 255, 256, 511, 700, 1023):
        x = np.zeros(n_in, np.float32)
        x[k] = 1.0
        y = host(qwg.gemv_q4k(wd, dev(x)))
        assert_bits(y + 0.0, deq[:, k] + 0.0, f"k={k}")


def test_gemv_q4k_deterministic_and_stream_aware():
    n_out, n_in = 2048, 2048
    w, x = _gemv_q4k_case(n_out, n_in, 98, 2)
    wd, xd = dev(w), dev(x)
    y1 = host(qwg.gemv_q4k(wd, xd))
    y2 = host(qwg.gemv_q4k(wd, xd))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y3 = qwg.gemv_q4k(wd, xd)
    s.synchronize()
    assert_bits(y1, y2)
    assert_bits(y1, host(y3))


def test_gemv_q4k_c5_stream_all_rows():
    # The full per-token stream (22 layers x 7 projections + LM head) at its real
    # shapes, 155 qwg_gemv_q4k calls back to back on row-major weights; every
    # row of every output (NaN-filled first) against the oracle.
    probs, ws, xs, refs = q4k_c5()
    Y = nan_outputs(probs)
    for p, w, x, y in zip(probs, ws, xs, Y):
        qwg.gemv_q4k(dev(w), dev(x), out=y)
    assert_stream(probs, refs, Y, "single call")


def test_first_split_call_under_capture_returns_a_status():
    # A stream without a split workspace, being captured: the call must not
    # allocate (it cannot, under capture) and reports QWG_ERR_CAPTURE. After
    # qwg_workspace_reserve the same capture records the kernels, and replays
    # reproduce the eager result.
    n_out, n_in = 2048, 5632
    assert qwg.plan_splits(0, n_in, n_out) > 1
    w, x = _gemv_q4k_case(n_out, n_in, 97, 3)
    wd, xd = dev(w), dev(x)
    y = torch.full((n_out,), float("nan"), device=DEV)
    side = torch.cuda.Stream()
    qwg.workspace_release(side)
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(qwg.QwgError) as e:
        with torch.cuda.graph(graph, stream=side):
            qwg.gemv_q4k(wd, xd, out=y)
    assert e.value.status == 7
    torch.cuda.synchronize()
    qwg.workspace_reserve(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        qwg.gemv_q4k(wd, xd, out=y)
    ref = host(qwg.gemv_q4k(wd, xd)).copy()
    for _ in range(3):
        y.fill_(float("nan"))
        graph.replay()
        assert_bits(host(y), ref, "replay after reserve")
        # eager calls on the same stream between replays advance the split epochs
        with torch.cuda.stream(side):
            assert_bits(host(qwg.gemv_q4k(wd, xd)), ref, "eager between replays")
    yr, sr = oracle.gemv_q4k(w, x, n_in, n_out)
    assert_bound(ref, yr, sr, "eager")


def test_gemv_q4k_misaligned_input_is_an_error():
    w, x = _gemv_q4k_case(4, 256, 99, 0)
    xd = dev(np.concatenate([[0.0], x]).astype(np.float32))[1:]
    with pytest.raises(qwg.QwgError) as e:
        qwg.gemv_q4k(dev(w), xd)
    assert e.value.status == 3


def test_group_c2_layer_and_repeat_runs():
    # One TinyLlama layer's seven projections as one grouped launch, run twice
    # (the plan is reusable; the second run sees a changed x in place).
    probs = synth.config(2)
    ws = [synth.weights(p) for p in probs]
    xs = [synth.inputs(p) for p in probs]
    W = [dev(w) for w in ws]
    X = [dev(x) for x in xs]
    Y = [torch.full((p.n_out,), float("nan"), device=DEV) for p in probs]
    g = qwg.Q4kGroup(zip(W, X, Y))
    assert g.workgroups == sum((p.n_out + 63) // 64 for p in probs)
    g.run()
    for p, w, x, y in zip(probs, ws, xs, Y):
        yr, sr = oracle.gemv_q4k(w, x, p.n_in, p.n_out)
        assert_bound(host(y), yr, sr, "group " + p.name)
    X[0].mul_(-0.5)
    g.run()
    yr, sr = oracle.gemv_q4k(ws[0], -0.5 * xs[0], probs[0].n_in, probs[0].n_out)
    assert_bound(host(Y[0]), yr, sr, "group rerun")
    g.close()


def test_group_and_single_calls_are_within_bound_and_deterministic():
    # Large members run through the persistent stream engine in both entry
    # points (different workgroup shapes, so different summation orders): both
    # must meet the bound, and each must be bitwise reproducible.
    shapes = [(16384 + 7, 256), (32000, 2048)]
    ws = [synth.q4k_weights(o, i, 105, k) for k, (o, i) in enumerate(shapes)]
    xs = [synth.activations(i, 105, k) for k, (o, i) in enumerate(shapes)]
    W, X = [dev(w) for w in ws], [dev(x) for x in xs]
    Y = [torch.empty(o, device=DEV) for o, _ in shapes]
    g = qwg.Q4kGroup(zip(W, X, Y))
    g.run()
    first = [host(y).copy() for y in Y]
    g.run()
    for (o, i), w, x, wd, xd, y, y0 in zip(shapes, ws, xs, W, X, Y, first):
        assert qwg.plan_splits(0, i, o) == 1
        yr, sr = oracle.gemv_q4k(w, x, i, o)
        assert_bound(y0, yr, sr, f"group {o}x{i}")
        assert_bits(host(y), y0, f"group rerun {o}x{i}")
        ys = host(qwg.gemv_q4k(wd, xd))
        assert_bound(ys, yr, sr, f"single {o}x{i}")
        assert_bits(host(qwg.gemv_q4k(wd, xd)), ys, f"single rerun {o}x{i}")


def test_group_ragged_members():
    shapes = [(1, 256), (65, 512), (200, 5632), (3, 65536), (4097, 768), (64, 2048)]
    ws = [synth.q4k_weights(o, i, 106, k) for k, (o, i) in enumerate(shapes)]
    xs = [synth.activations(i, 106, k) for k, (o, i) in enumerate(shapes)]
    Y = [torch.empty(o, device=DEV) for o, _ in shapes]
    g = qwg.Q4kGroup(zip([dev(w) for w in ws], [dev(x) for x in xs], Y))
    g.run()
    for (o, i), w, x, y in zip(shapes, ws, xs, Y):
        yr, sr = oracle.gemv_q4k(w, x, i, o)
        assert_bound(host(y), yr, sr, f"group member {o}x{i}")


def test_group_c5_stream_all_rows():
    # The 155 GEMVs as one grouped launch on row-major weights: every row, after
    # the first run and again after two more runs into NaN-filled outputs.
    probs, ws, xs, refs = q4k_c5()
    Y = nan_outputs(probs)
    g = qwg.Q4kGroup(zip([dev(w) for w in ws], [dev(x) for x in xs], Y))
    g.run()
    assert_stream(probs, refs, Y, "group")
    for y in Y:
        y.fill_(float("nan"))
    for _ in range(2):
        g.run()
    assert_stream(probs, refs, Y, "group rerun")
    g.close()


# ---------------------------------------------------------------- GEMM

@pytest.mark.parametrize("batch", range(1, 9))
def test_gemm_q4k_batches(batch):
    n_out, n_in = 333, 1536
    w, _ = _gemv_q4k_case(n_out, n_in, 100, batch)
    X = synth.activations(n_in, 100, 50 + batch, batch=batch)
    Y = host(qwg.gemm_q4k(dev(w), dev(X)))
    Yr, Sr = oracle.gemm_q4k(w, X, n_in, n_out)
    assert_bound(Y, Yr, Sr, f"batch {batch}")
    if batch == 1:
        assert_bits(Y[0], host(qwg.gemv_q4k(dev(w), dev(X[0]))))


def test_gemm_q4k_lm_head_b8():
    p = synth.config(3)[1]
    w, X = synth.weights(p), synth.inputs(p)
    Y = host(qwg.gemm_q4k(dev(w), dev(X)))
    Yr, Sr = oracle.gemm_q4k(w, X, p.n_in, p.n_out)
    assert_bound(Y, Yr, Sr, "lm_head b8")


def test_gemm_q4k_integer_exact():
    n_out, n_in = 100, 2048
    w = _integer_q4k(n_out, n_in, 7)
    X = np.random.default_rng(3).integers(-8, 9, (8, n_in)).astype(np.float32)
    Y = host(qwg.gemm_q4k(dev(w), dev(X)))
    Yr, _ = oracle.gemm_q4k(w, X, n_in, n_out)
    assert np.array_equal(Y.astype(np.float64), Yr)


# ---------------------------------------------------------------- batched GEMM on matrix cores

@pytest.mark.parametrize("batch", [2, 3, 5, 8])
@pytest.mark.parametrize("n_out,n_in", [(333, 1536), (64, 256), (130, 5632), (1, 512)])
def test_gemm_q4k_mfma_every_split(batch, n_out, n_in):
    w, _ = _gemv_q4k_case(n_out, n_in, 101, batch)
    X = synth.activations(n_in, 101, 60 + batch, batch=batch)
    Yr, Sr = oracle.gemm_q4k(w, X, n_in, n_out)
    wd, xd = dev(w), dev(X)
    nb = n_in // 256
    for splits in sorted({1, 2, nb} & set(range(1, nb + 1))):
        for cols in (1, 2):   # super-block columns per stage (waves=1: one, waves=2: two)
            Y = host(qwg.gemm_q4k(wd, xd, waves=cols, splits=splits))
            assert_bound(Y, Yr, Sr, f"mfma batch {batch} splits {splits} cols {cols}")
            assert_bits(host(qwg.gemm_q4k(wd, xd, waves=cols, splits=splits)), Y, "mfma rerun")
    # the vector-ALU engine on the same problem, same bound
    assert_bound(host(qwg.gemm_q4k(wd, xd, waves=4, splits=1)), Yr, Sr, "valu engine")


def test_gemm_q4k_mfma_wide_range_activations():
    # magnitudes from 1e-30 to 1e30 in one row: every bf16 part of the split matters
    n_out, n_in, batch = 200, 2048, 8
    w, _ = _gemv_q4k_case(n_out, n_in, 102, 0)
    g = np.random.default_rng(21)
    X = (g.standard_normal((batch, n_in)) * 10.0 ** g.integers(-30, 31, (batch, n_in))).astype(np.float32)
    Y = host(qwg.gemm_q4k(dev(w), dev(X)))
    Yr, Sr = oracle.gemm_q4k(w, X, n_in, n_out)
    assert_bound(Y, Yr, Sr, "wide range")


@pytest.mark.parametrize("batch", [2, 4, 7])
def test_gemm_q4k_mfma_integer_exact(batch):
    n_out, n_in = 190, 5632
    w = _integer_q4k(n_out, n_in, 8 + batch)
    X = np.random.default_rng(batch).integers(-8, 9, (batch, n_in)).astype(np.float32)
    Yr, _ = oracle.gemm_q4k(w, X, n_in, n_out)
    for splits in (1, 3):   # ranges of 22 and of 7, 7, 8 super-blocks
        for cols in (1, 2):
            Y = host(qwg.gemm_q4k(dev(w), dev(X), waves=cols, splits=splits))
            assert np.array_equal(Y.astype(np.float64), Yr), f"splits {splits} cols {cols}"


def test_gemm_q4k_mfma_one_hot_columns():
    # x = e_k in batch row b picks column k of the dequantized matrix exactly
    n_out, n_in = 96, 1024
    w, _ = _gemv_q4k_case(n_out, n_in, 103, 1)
    deq = oracle.dequant_q4k(w, n_out * n_in).reshape(n_out, n_in)
    cols = [0, 31, 32, 255, 256, 700, 1023, 513]
    X = np.zeros((8, n_in), np.float32)
    for b, k in enumerate(cols):
        X[b, k] = 1.0
    for waves, splits in [(0, 0), (1, 1), (2, 1), (2, 3)]:
        Y = host(qwg.gemm_q4k(dev(w), dev(X), waves=waves, splits=splits))
        for b, k in enumerate(cols):
            assert np.array_equal(Y[b], deq[:, k]), f"column {k} waves {waves} splits {splits}"


@pytest.mark.parametrize("batch", [2, 3, 5, 8])
@pytest.mark.parametrize("n_out,n_in", [(333, 1536), (64, 256), (130, 5632), (1, 512), (700, 2048)])
def test_gemm_q4k_mstream_every_split(batch, n_out, n_in):
    # the persistent matrix-core stream (waves=3): whole rows and split ranges
    # (two, three: 7/7/8-style uneven ranges, and one super-block each)
    w, _ = _gemv_q4k_case(n_out, n_in, 109, batch)
    X = synth.activations(n_in, 109, 70 + batch, batch=batch)
    Yr, Sr = oracle.gemm_q4k(w, X, n_in, n_out)
    wd, xd = dev(w), dev(X)
    nb = n_in // 256
    for splits in sorted({1, 2, 3, nb} & set(range(1, nb + 1))):
        out = torch.full((batch, n_out), float("nan"), device=DEV)
        Y = host(qwg.gemm_q4k(wd, xd, out=out, waves=3, splits=splits)).copy()
        assert_bound(Y, Yr, Sr, f"mstream batch {batch} splits {splits}")
        assert_bits(host(qwg.gemm_q4k(wd, xd, waves=3, splits=splits)), Y, "mstream rerun")
    # whole rows: the same sums in the same order as the per-tile pipeline
    assert_bits(host(qwg.gemm_q4k(wd, xd, waves=3, splits=1)),
                host(qwg.gemm_q4k(wd, xd, waves=1, splits=1)), "mstream vs per-tile pipeline")


@pytest.mark.parametrize("batch", [2, 6, 8])
def test_gemm_q4k_mstream_integer_exact(batch):
    n_out, n_in = 190, 5632
    w = _integer_q4k(n_out, n_in, 40 + batch)
    X = np.random.default_rng(40 + batch).integers(-8, 9, (batch, n_in)).astype(np.float32)
    Yr, _ = oracle.gemm_q4k(w, X, n_in, n_out)
    for splits in (1, 3, 22):
        Y = host(qwg.gemm_q4k(dev(w), dev(X), waves=3, splits=splits))
        assert np.array_equal(Y.astype(np.float64), Yr), f"splits {splits}"


def test_gemm_q4k_batch2_many_tiles_runs_on_the_vector_alus():
    # batch 2 with >= 256 tiles takes the vector-ALU engine (8 wavefronts per tile)
    p = synth.config(3)[1]
    w = synth.weights(p)
    X = synth.activations(p.n_in, 3, 2, batch=2)
    wd, xd = dev(w), dev(X)
    Y = host(qwg.gemm_q4k(wd, xd)).copy()
    Yr, Sr = oracle.gemm_q4k(w, X, p.n_in, p.n_out)
    assert_bound(Y, Yr, Sr, "lm_head b2")
    assert_bits(host(qwg.gemm_q4k(wd, xd, waves=8)), Y, "the vector-ALU engine's result")


def test_gemm_q4k_lm_head_b8_tiled_all_rows():
    p = synth.config(3)[1]
    w, X = synth.weights(p), synth.inputs(p)
    out = torch.full((8, p.n_out), float("nan"), device=DEV)
    qwg.gemm_q4k_tiled(qwg.pack_q4k_tiles(dev(w), p.n_in), dev(X), p.n_out, out=out)
    Yr, Sr = oracle.gemm_q4k(w, X, p.n_in, p.n_out)
    assert_bound(host(out), Yr, Sr, "lm_head b8 tiled")


# ---------------------------------------------------------------- batched groups (matrix cores)

def test_batched_group_c5_stream_all_rows():
    # the per-token stream's 155 products for 8 sequences, tile layout, as the
    # batched bench runs them (XCD-ordered work list); every row of every member
    probs = synth.config(5)
    ws = [synth.weights(p) for p in probs]
    Xs = [synth.activations(p.n_in, 5, k, batch=8) for k, p in enumerate(probs)]
    WT = [qwg.pack_q4k_tiles(dev(w), p.n_in) for p, w in zip(probs, ws)]
    Y = [torch.full((8, p.n_out), float("nan"), device=DEV) for p in probs]
    g = qwg.Q4kBatchedGroup(zip(WT, [dev(x) for x in Xs], Y), tiled=True)
    g.run()
    for p, w, x, y in zip(probs, ws, Xs, Y):
        Yr, Sr = oracle.gemm_q4k(w, x, p.n_in, p.n_out)
        assert_bound(host(y), Yr, Sr, f"batched stream {p.name}")
    g.close()


BATCHED_SHAPES = [(333, 1536), (64, 256), (130, 5632), (1, 512), (2000, 2048), (65, 768)]


@pytest.mark.parametrize("batch", [2, 3, 5, 8])
def test_batched_group_within_bound_and_equal_to_gemm(batch):
    ws = [synth.q4k_weights(o, i, 105, k) for k, (o, i) in enumerate(BATCHED_SHAPES)]
    Xs = [synth.activations(i, 105, 10 * batch + k, batch=batch) for k, (o, i) in enumerate(BATCHED_SHAPES)]
    W = [dev(w) for w in ws]
    X = [dev(x) for x in Xs]
    Y = [torch.full((batch, o), float("nan"), device=DEV) for o, _ in BATCHED_SHAPES]
    g = qwg.Q4kBatchedGroup(zip(W, X, Y))
    assert g.workgroups == sum((o + 63) // 64 for o, _ in BATCHED_SHAPES)
    g.run()
    cols = 1   # the group's columns per stage; a single launch with the same shape matches it
    for k, ((o, i), w, x, y) in enumerate(zip(BATCHED_SHAPES, ws, Xs, Y)):
        Yr, Sr = oracle.gemm_q4k(w, x, i, o)
        got = host(y)
        assert_bound(got, Yr, Sr, f"member {k} batch {batch}")
        single = host(qwg.gemm_q4k(W[k], X[k], waves=cols, splits=1))
        assert_bits(got, single, f"member {k}: group vs single launch")
    # a second run, after new activations, recomputes every member
    X[0].copy_(dev(synth.activations(BATCHED_SHAPES[0][1], 106, 1, batch=batch)))
    g.run()
    Yr, Sr = oracle.gemm_q4k(ws[0], host(X[0]), BATCHED_SHAPES[0][1], BATCHED_SHAPES[0][0])
    assert_bound(host(Y[0]), Yr, Sr, "rerun")
    g.close()


@pytest.mark.parametrize("batch", [1, 2, 4, 5, 8])
@pytest.mark.parametrize("n_out,n_in", [(333, 1536), (64, 256), (130, 5632), (1, 512), (2000, 2048)])
def test_gemm_q4k_tiled_equals_row_major(batch, n_out, n_in):
    # the same decomposition on both layouts: only where a stage is copied from differs
    w = synth.q4k_weights(n_out, n_in, 107, batch)
    X = dev(synth.activations(n_in, 107, 20 + batch, batch=batch))
    wd = dev(w)
    wt = qwg.pack_q4k_tiles(wd, n_in)
    got = host(qwg.gemm_q4k_tiled(wt, X, n_out))
    if batch == 1:
        assert_bits(got[0], host(qwg.gemv_q4k_tiled(wt, X[0], n_out)), "batch 1 = tiled GEMV")
    else:
        assert_bits(got, host(qwg.gemm_q4k(wd, X)), f"tiled vs row-major, batch {batch}")
    Yr, Sr = oracle.gemm_q4k(w, host(X), n_in, n_out)
    assert_bound(got, Yr, Sr, f"tiled gemm batch {batch}")


@pytest.mark.parametrize("batch", [3, 8])
def test_batched_group_tiled_equals_row_major(batch):
    ws = [dev(synth.q4k_weights(o, i, 108, k)) for k, (o, i) in enumerate(BATCHED_SHAPES)]
    X = [dev(synth.activations(i, 108, k, batch=batch)) for k, (o, i) in enumerate(BATCHED_SHAPES)]
    Y = [torch.empty(batch, o, device=DEV) for o, _ in BATCHED_SHAPES]
    Yt = [torch.empty(batch, o, device=DEV) for o, _ in BATCHED_SHAPES]
    WT = [qwg.pack_q4k_tiles(w, i) for w, (_, i) in zip(ws, BATCHED_SHAPES)]
    g = qwg.Q4kBatchedGroup(zip(ws, X, Y))
    gt = qwg.Q4kBatchedGroup(zip(WT, X, Yt), tiled=True)
    g.run()
    gt.run()
    for k, (a, b) in enumerate(zip(Y, Yt)):
        assert_bits(host(b), host(a), f"member {k}")
    g.close()
    gt.close()


@pytest.mark.parametrize("batch", [2, 7])
def test_batched_group_integer_exact(batch):
    shapes = [(190, 5632), (64, 2048), (3, 256)]
    ws = [_integer_q4k(o, i, 30 + k) for k, (o, i) in enumerate(shapes)]
    g_ = np.random.default_rng(batch)
    Xs = [g_.integers(-8, 9, (batch, i)).astype(np.float32) for _, i in shapes]
    Y = [torch.empty(batch, o, device=DEV) for o, _ in shapes]
    g = qwg.Q4kBatchedGroup(zip([dev(w) for w in ws], [dev(x) for x in Xs], Y))
    g.run()
    for (o, i), w, x, y in zip(shapes, ws, Xs, Y):
        Yr, _ = oracle.gemm_q4k(w, x, i, o)
        assert np.array_equal(host(y).astype(np.float64), Yr)
    g.close()


def test_batched_group_rejects_mixed_batches():
    w = dev(synth.q4k_weights(64, 256, 105, 0))
    a = (w, torch.zeros(2, 256, device=DEV), torch.zeros(2, 64, device=DEV))
    b = (w, torch.zeros(3, 256, device=DEV), torch.zeros(3, 64, device=DEV))
    with pytest.raises(ValueError):
        qwg.Q4kBatchedGroup([a, b])
    with pytest.raises(ValueError):
        qwg.Q4kBatchedGroup([(w, torch.zeros(1, 256, device=DEV), torch.zeros(1, 64, device=DEV))])


# ---------------------------------------------------------------- IQ3 GEMV

@pytest.mark.parametrize("p", synth.config(4), ids=lambda p: p.name)
def test_gemv_iq3_configs(p):
    grid = synth.iq3_grid()
    w, x = synth.weights(p), synth.inputs(p)
    y = host(qwg.gemv_iq3(dev(w), dev(x), dev(grid)))
    yr, sr = oracle.gemv_iq3(w, grid, x, p.n_in, p.n_out)
    assert_bound(y, yr, sr, p.name)


@pytest.mark.parametrize("n_out,n_in", [(1, 256), (3, 256), (65, 768), (100, 1280), (129, 5632),
                                        (2000, 768), (131072 + 3, 256)])
def test_gemv_iq3_ragged(n_out, n_in):
    grid = synth.iq3_grid()
    w = synth.iq3_weights(n_out, n_in, 101, n_out)
    x = synth.activations(n_in, 101, n_out)
    y = host(qwg.gemv_iq3(dev(w), dev(x), dev(grid)))
    yr, sr = oracle.gemv_iq3(w, grid, x, n_in, n_out)
    assert_bound(y, yr, sr, f"{n_out}x{n_in}")


def test_gemv_iq3_two_byte_aligned_base():
    # rows of 98-byte blocks at a base address that is 2 mod 4
    n_out, n_in = 70, 768
    grid = synth.iq3_grid()
    w = synth.iq3_weights(n_out, n_in, 102, 0)
    buf = torch.zeros(w.size + 16, dtype=torch.uint8, device=DEV)
    buf[2:2 + w.size] = dev(w.reshape(-1))
    wd = buf[2:2 + w.size]
    assert wd.data_ptr() % 4 == 2
    x = synth.activations(n_in, 102, 0)
    y = host(qwg.gemv_iq3(wd, dev(x), dev(grid)))
    yr, sr = oracle.gemv_iq3(w, grid, x, n_in, n_out)
    assert_bound(y, yr, sr, "2 mod 4 base")
    got = host(qwg.dequant_iq3(wd, dev(grid)))
    assert_bits(got, oracle.dequant_iq3(w, grid, n_out * n_in), "dequant 2 mod 4 base")


def test_gemv_iq3_integer_exact():
    # d = 4 and code in 0..3 make every sub-block scale an odd integer (1, 3, 5, 7)
    n_out, n_in = 150, 2048
    grid = synth.iq3_grid()
    w = synth.iq3_weights(n_out, n_in, 103, 0).reshape(-1, 98).copy()
    w[:, 96], w[:, 97] = 0x00, 0x44
    words = w[:, 64:96].copy().view("<u4") & np.uint32(0x3FFFFFFF)
    w[:, 64:96] = words.view(np.uint8)
    w = w.reshape(n_out, -1)
    x = np.random.default_rng(9).integers(-8, 9, n_in).astype(np.float32)
    y = host(qwg.gemv_iq3(dev(w), dev(x), dev(grid)))
    yr, _ = oracle.gemv_iq3(w, grid, x, n_in, n_out)
    assert np.array_equal(y.astype(np.float64), yr)


def test_gemv_iq3_one_hot_is_exact_column():
    n_out, n_in = 66, 512
    grid = synth.iq3_grid()
    w = synth.iq3_weights(n_out, n_in, 104, 0)
    deq = oracle.dequant_iq3(w, grid, n_out * n_in).reshape(n_out, n_in)
    wd, gd = dev(w), dev(grid)
    for k in (0, 3, 4, 7, 8, 31, 32, 100, 255, 256, 511):
        x = np.zeros(n_in, np.float32)
        x[k] = 1.0
        y = host(qwg.gemv_iq3(wd, dev(x), gd))
        assert_bits(y + 0.0, deq[:, k] + 0.0, f"k={k}")


@pytest.mark.parametrize("waves", [4, 8, 16])
@pytest.mark.parametrize("n_out,n_in,splits", [(70, 256, 1), (70, 2048, 1), (70, 2048, 3),
                                               (130, 5632, 1), (130, 5632, 5), (130, 5632, 22),
                                               (1, 1024, 4), (300, 1280, 2), (2000, 768, 1)])
def test_gemv_iq3_every_plan(waves, n_out, n_in, splits):
    grid = synth.iq3_grid()
    w = synth.iq3_weights(n_out, n_in, 110, n_out + splits)
    x = synth.activations(n_in, 110, n_out + splits)
    y = host(qwg.gemv_iq3(dev(w), dev(x), dev(grid), waves=waves, splits=splits))
    yr, sr = oracle.gemv_iq3(w, grid, x, n_in, n_out)
    assert_bound(y, yr, sr, f"waves={waves} splits={splits}")


def test_gemv_iq3_ex_rejects_bad_plans():
    grid = synth.iq3_grid()
    w = synth.iq3_weights(64, 512, 111, 0)
    x = synth.activations(512, 111, 0)
    for waves, splits in [(2, 1), (32, 1), (4, 3), (16, -1)]:
        with pytest.raises(qwg.QwgError) as e:
            qwg.gemv_iq3(dev(w), dev(x), dev(grid), waves=waves, splits=splits)
        assert e.value.status == 2


def _guarded_iq3(w: np.ndarray, offset: int, fill: int = 0xFF):
    """w placed at `offset` bytes past a 256-byte boundary inside a larger
    buffer whose other bytes are `fill` (0xFF: NaN as an fp16 scale), so that
    any use of a byte outside w shows in the result."""
    buf = torch.full((w.size + offset + 64,), fill, dtype=torch.uint8, device=DEV)
    buf[offset:offset + w.size] = dev(w.reshape(-1))
    wd = buf[offset:offset + w.size]
    assert wd.data_ptr() % 256 == offset
    return wd


@pytest.mark.parametrize("offset", [0, 2, 4, 6, 8, 10, 12, 14, 18, 30])
@pytest.mark.parametrize("n_out,n_in", [(1, 256), (3, 512), (65, 768), (64, 5632), (129, 2048)])
def test_gemv_iq3_buffer_edges(offset, n_out, n_in):
    # The first and last 16-byte granules of w reach outside it unless w starts
    # and ends on a granule boundary; those bytes must never reach the result,
    # and y must be written only inside its own range.
    grid = synth.iq3_grid()
    w = synth.iq3_weights(n_out, n_in, 112, offset)
    x = synth.activations(n_in, 112, offset)
    wd, xd, gd = _guarded_iq3(w, offset), dev(x), dev(grid)
    yr, sr = oracle.gemv_iq3(w, grid, x, n_in, n_out)
    ybuf = torch.full((n_out + 130,), -7.0, device=DEV)
    for waves, splits in [(0, 0), (4, 1), (16, 1), (8, n_in // 256)]:
        y = ybuf[64:64 + n_out]
        qwg.gemv_iq3(wd, xd, gd, out=y, waves=waves, splits=splits)
        yb = host(ybuf)
        assert_bound(yb[64:64 + n_out], yr, sr, f"offset={offset} waves={waves} splits={splits}")
        assert (yb[:64] == -7.0).all() and (yb[64 + n_out:] == -7.0).all(), "write outside y"


@pytest.mark.parametrize("waves", [4, 8, 16])
def test_gemv_iq3_integer_exact_every_shape(waves):
    # d = 4 and code in 0..3: every partial sum is an exact integer, so every
    # decomposition must give the oracle's value exactly
    n_out, n_in = 130, 5632
    grid = synth.iq3_grid()
    w = synth.iq3_weights(n_out, n_in, 113, 0).reshape(-1, 98).copy()
    w[:, 96], w[:, 97] = 0x00, 0x44
    words = w[:, 64:96].copy().view("<u4") & np.uint32(0x3FFFFFFF)
    w[:, 64:96] = words.view(np.uint8)
    w = w.reshape(n_out, -1)
    x = np.random.default_rng(10).integers(-8, 9, n_in).astype(np.float32)
    yr, _ = oracle.gemv_iq3(w, grid, x, n_in, n_out)
    for splits in (1, 2, 7, 22):
        y = host(qwg.gemv_iq3(dev(w), dev(x), dev(grid), waves=waves, splits=splits))
        assert np.array_equal(y.astype(np.float64), yr), f"splits={splits}"


def test_gemv_iq3_deterministic():
    p = synth.config(4)[1]
    grid = dev(synth.iq3_grid())
    w, x = dev(synth.weights(p)), dev(synth.inputs(p))
    y0 = host(qwg.gemv_iq3(w, x, grid)).copy()
    for _ in range(3):
        assert_bits(host(qwg.gemv_iq3(w, x, grid)), y0, "rerun")


# ---------------------------------------------------------------- IQ3 groups

def test_iq3_group_layer_and_repeat_runs():
    probs = synth.config(7)
    grid = synth.iq3_grid()
    ws = [synth.weights(p) for p in probs]
    xs = [synth.inputs(p) for p in probs]
    W, X = [dev(w) for w in ws], [dev(x) for x in xs]
    Y = [torch.full((p.n_out,), float("nan"), device=DEV) for p in probs]
    g = qwg.Iq3Group(zip(W, X, Y), dev(grid))
    assert g.workgroups == sum((p.n_out + 63) // 64 for p in probs)
    g.run()
    first = [host(y).copy() for y in Y]
    for p, w, x, y in zip(probs, ws, xs, first):
        yr, sr = oracle.gemv_iq3(w, grid, x, p.n_in, p.n_out)
        assert_bound(y, yr, sr, "iq3 group " + p.name)
    g.run()
    for p, y, y0 in zip(probs, Y, first):
        assert_bits(host(y), y0, "iq3 group rerun " + p.name)
    X[4].mul_(-0.5)
    g.run()
    yr, sr = oracle.gemv_iq3(ws[4], grid, -0.5 * xs[4], probs[4].n_in, probs[4].n_out)
    assert_bound(host(Y[4]), yr, sr, "iq3 group rerun with new x")
    g.close()


def test_iq3_group_ragged_members_at_odd_offsets():
    shapes = [(1, 256), (65, 512), (200, 5632), (3, 65536), (4097, 768), (64, 2048)]
    grid = synth.iq3_grid()
    ws = [synth.iq3_weights(o, i, 114, k) for k, (o, i) in enumerate(shapes)]
    xs = [synth.activations(i, 114, k) for k, (o, i) in enumerate(shapes)]
    W = [_guarded_iq3(w, 2 * k + 2) for k, w in enumerate(ws)]
    Y = [torch.empty(o, device=DEV) for o, _ in shapes]
    g = qwg.Iq3Group(zip(W, [dev(x) for x in xs], Y), dev(grid))
    g.run()
    for (o, i), w, x, y in zip(shapes, ws, xs, Y):
        yr, sr = oracle.gemv_iq3(w, grid, x, i, o)
        assert_bound(host(y), yr, sr, f"iq3 group member {o}x{i}")


def iq3_c6():
    grid = synth.iq3_grid()
    return grid, stream_case("iq3_c6", lambda: (
        synth.config(6), [synth.weights(p) for p in synth.config(6)],
        [synth.inputs(p) for p in synth.config(6)],
        lambda p, w, x: oracle.gemv_iq3(w, grid, x, p.n_in, p.n_out)))


def test_iq3_group_stream_all_rows():
    grid, (probs, ws, xs, refs) = iq3_c6()
    Y = nan_outputs(probs)
    g = qwg.Iq3Group(zip([dev(w) for w in ws], [dev(x) for x in xs], Y), dev(grid))
    g.run()
    assert_stream(probs, refs, Y, "iq3 group")
    for y in Y:
        y.fill_(float("nan"))
    for _ in range(2):
        g.run()
    assert_stream(probs, refs, Y, "iq3 group rerun")
    g.close()


# ---------------------------------------------------------------- Q4_K tile layout

def _tile_layout(w: np.ndarray, n_in: int) -> np.ndarray:
    """The tile layout written out: block (r, b) at ((r//64)*nb + b)*9216 + (r%64)*144,
    rows past n_out as zero blocks."""
    n_out, nb = w.shape[0], n_in // 256
    tiles = (n_out + 63) // 64
    blocks = np.zeros((tiles * 64, nb, 144), np.uint8)
    blocks[:n_out] = w.reshape(n_out, nb, 144)
    return blocks.reshape(tiles, 64, nb, 144).transpose(0, 2, 1, 3).reshape(-1)


@pytest.mark.parametrize("n_out,n_in", [(1, 256), (64, 512), (65, 768), (300, 2048), (2048, 5632)])
def test_pack_q4k_tiles_is_the_layout(n_out, n_in):
    w = synth.q4k_weights(n_out, n_in, 120, n_out)
    got = host(qwg.pack_q4k_tiles(dev(w), n_in))
    assert np.array_equal(got, _tile_layout(w, n_in))


@pytest.mark.parametrize("n_out,n_in", [(1, 256), (3, 512), (65, 768), (130, 5632), (2048, 2048),
                                        (32000, 2048), (4097, 1280)])
def test_gemv_q4k_tiled(n_out, n_in):
    w, x = _gemv_q4k_case(n_out, n_in, 121, n_out)
    wt = qwg.pack_q4k_tiles(dev(w), n_in)
    xd = dev(x)
    yr, sr = oracle.gemv_q4k(w, x, n_in, n_out)
    y = host(qwg.gemv_q4k_tiled(wt, xd, n_out))
    assert_bound(y, yr, sr, f"tiled {n_out}x{n_in}")
    assert_bits(host(qwg.gemv_q4k_tiled(wt, xd, n_out)), y, "tiled rerun")


def test_q4k_tiled_group_layer_and_integer_exact():
    probs = synth.config(2)
    ws = [synth.weights(p) for p in probs]
    xs = [synth.inputs(p) for p in probs]
    W = [qwg.pack_q4k_tiles(dev(w), p.n_in) for p, w in zip(probs, ws)]
    Y = [torch.full((p.n_out,), float("nan"), device=DEV) for p in probs]
    g = qwg.Q4kGroup(zip(W, [dev(x) for x in xs], Y), tiled=True)
    g.run()
    for p, w, x, y in zip(probs, ws, xs, Y):
        yr, sr = oracle.gemv_q4k(w, x, p.n_in, p.n_out)
        assert_bound(host(y), yr, sr, "tiled group " + p.name)
    g.close()
    # integer-valued weights and activations: every order of summation is exact
    n_out, n_in = 129, 5632
    w = _integer_q4k(n_out, n_in, 122)
    x = np.random.default_rng(12).integers(-8, 9, n_in).astype(np.float32)
    yr, _ = oracle.gemv_q4k(w, x, n_in, n_out)
    y = torch.empty(n_out, device=DEV)
    g = qwg.Q4kGroup([(qwg.pack_q4k_tiles(dev(w), n_in), dev(x), y)], tiled=True)
    g.run()
    assert np.array_equal(host(y).astype(np.float64), yr)


def test_q4k_tiled_group_stream_all_rows():
    # The launch bench.py times for the independent-input stream: 155 members on
    # tile-layout weights, the weighted static schedule with its hole table.
    # Every row of every member (426,240 rows) against the full oracle, from
    # NaN-filled outputs, on the first run and on a later one; runs are
    # bitwise reproducible.
    probs, ws, xs, refs = q4k_c5()
    Y = nan_outputs(probs)
    W = [qwg.pack_q4k_tiles(dev(w), p.n_in) for p, w in zip(probs, ws)]
    g = qwg.Q4kGroup(zip(W, [dev(x) for x in xs], Y), tiled=True)
    assert g.workgroups == sum((p.n_out + 63) // 64 for p in probs)
    g.run()
    assert_stream(probs, refs, Y, "tiled group")
    first = [host(y).copy() for y in Y]
    for y in Y:
        y.fill_(float("nan"))
    for _ in range(3):
        g.run()
    for p, y, y0 in zip(probs, Y, first):
        assert_bits(host(y), y0, "tiled group rerun " + p.name)
    g.close()


@pytest.mark.parametrize("tiled", [False, True])
def test_q4k_group_many_items_repeat_runs(tiled):
    # Many more items than resident workgroups, one-stage items (n_in = 256)
    # mixed with 22-block ones, ragged row counts. Each run uses new
    # activations and NaN-filled outputs, so a skipped or repeated item shows
    # up as stale or NaN rows.
    shapes = [(64 * 8000 + 5, 256), (64 * 300, 5632), (64 * 700 - 3, 2048)]
    ws = [synth.q4k_weights(n_out, n_in, 123, i) for i, (n_out, n_in) in enumerate(shapes)]
    W = [qwg.pack_q4k_tiles(dev(w), n_in) if tiled else dev(w) for w, (_, n_in) in zip(ws, shapes)]
    X = [torch.empty(n_in, device=DEV) for _, n_in in shapes]
    Y = [torch.empty(n_out, device=DEV) for n_out, _ in shapes]
    g = qwg.Q4kGroup(zip(W, X, Y), tiled=tiled)
    assert g.workgroups > 4 * 2048
    for run in range(4):
        xs = [synth.activations(n_in, 123, 10 * run + i) for i, (_, n_in) in enumerate(shapes)]
        for xd, x in zip(X, xs):
            xd.copy_(torch.from_numpy(x))
        for y in Y:
            y.fill_(float("nan"))
        g.run()
        for (n_out, n_in), w, x, y in zip(shapes, ws, xs, Y):
            yh = host(y)
            assert not np.isnan(yh).any(), f"run {run}: rows left unwritten"
            yr, sr = oracle.gemv_q4k(w, x, n_in, n_out)
            assert_bound(yh, yr, sr, f"run {run} {n_out}x{n_in}")
    g.close()


# ---------------------------------------------------------------- IQ3 tile layout

def _sign_bytes(words: np.ndarray) -> np.ndarray:
    """Each 32-bit sign/scale word -> its four groups of eight signs as bytes:
    the seven stored bits, then the eighth that makes the count of set bits
    even (the container's sign rule)."""
    out = np.zeros(words.shape, np.uint32)
    for k in range(4):
        g = (words >> np.uint32(7 * k)) & np.uint32(0x7F)
        odd = np.zeros_like(g)
        for bit in range(7):
            odd ^= (g >> np.uint32(bit)) & np.uint32(1)
        out |= (g | (odd << np.uint32(7))) << np.uint32(8 * k)
    return out


def _iq3_tile_layout(w: np.ndarray, n_in: int) -> np.ndarray:
    """The IQ3 tile layout written out: per (tile, block column), index bytes
    [G][row][16], sign bytes [G][row][8] (words 2G, 2G+1 as eight signs per
    byte), scales [G][row] (word 2G's in the low nibble, 2G+1's in the high
    one), d [row][2]; rows past n_out as zero blocks."""
    n_out, nb = w.shape[0], n_in // 256
    tiles = (n_out + 63) // 64
    blk = np.zeros((tiles * 64, nb, 98), np.uint8)
    blk[:n_out] = w.reshape(n_out, nb, 98)
    blk = blk.reshape(tiles, 64, nb, 98).transpose(0, 2, 1, 3)       # [t][b][row][98]
    idx = blk[..., :64].reshape(tiles, nb, 64, 4, 16).transpose(0, 1, 3, 2, 4)
    words = np.ascontiguousarray(blk[..., 64:96]).view("<u4")       # [t][b][row][8]
    signs = _sign_bytes(words).view(np.uint8).reshape(tiles, nb, 64, 4, 8).transpose(0, 1, 3, 2, 4)
    code = (words >> np.uint32(28)).astype(np.uint8)
    scales = (code[..., 0::2] | (code[..., 1::2] << 4)).transpose(0, 1, 3, 2)   # [t][b][G][row]
    d = blk[..., 96:98]
    return np.concatenate([idx.reshape(tiles, nb, -1), signs.reshape(tiles, nb, -1),
                           scales.reshape(tiles, nb, -1), d.reshape(tiles, nb, -1)],
                          axis=2).reshape(-1)


@pytest.mark.parametrize("n_out,n_in", [(1, 256), (64, 512), (65, 768), (300, 2048), (2048, 5632)])
def test_pack_iq3_tiles_is_the_layout(n_out, n_in):
    w = synth.iq3_weights(n_out, n_in, 130, n_out)
    got = host(qwg.pack_iq3_tiles(dev(w), n_in))
    assert np.array_equal(got, _iq3_tile_layout(w, n_in))


@pytest.mark.parametrize("n_out,n_in", [(1, 256), (3, 512), (65, 768), (130, 5632), (2048, 2048),
                                        (32000, 2048), (4097, 1280)])
def test_gemv_iq3_tiled(n_out, n_in):
    grid = synth.iq3_grid()
    w = synth.iq3_weights(n_out, n_in, 131, n_out)
    x = synth.activations(n_in, 131, n_out)
    wt = qwg.pack_iq3_tiles(dev(w), n_in)
    gd, xd = dev(grid), dev(x)
    yr, sr = oracle.gemv_iq3(w, grid, x, n_in, n_out)
    y = host(qwg.gemv_iq3_tiled(wt, xd, gd, n_out))
    assert_bound(y, yr, sr, f"iq3 tiled {n_out}x{n_in}")
    assert_bits(host(qwg.gemv_iq3_tiled(wt, xd, gd, n_out)), y, "iq3 tiled rerun")


@pytest.mark.parametrize("n_out,n_in", [(2048, 2048), (5632, 2048), (2048, 5632), (256, 2048),
                                        (130, 3328), (1, 7168), (64, 3840)])
def test_gemv_iq3_short_calls_layouts_and_repeat(n_out, n_in):
    # The short-call IQ3 kernels (row groups for rows of at most 8 blocks, else
    # split rows through tagged words) on row-major, llama.cpp-order and
    # tile-layout weights: the same kernel, so the same
    # bits for the container and its tile layout, the llama.cpp order with the
    # doubled grid exactly twice that; repeated calls give the same bits.
    grid = synth.iq3_grid()
    w = synth.iq3_weights(n_out, n_in, 133, n_in // 256)
    x = synth.activations(n_in, 133, n_out)
    wd, xd, gd = dev(w), dev(x), dev(grid)
    yr, sr = oracle.gemv_iq3(w, grid, x, n_in, n_out)
    y = host(qwg.gemv_iq3(wd, xd, gd)).copy()
    assert_bound(y, yr, sr, f"iq3 {n_out}x{n_in} splits={qwg.plan_splits(1, n_in, n_out)}")
    t = host(qwg.gemv_iq3_tiled(qwg.pack_iq3_tiles(wd, n_in), xd, gd, n_out))
    assert_bits(t, y, "tile layout")
    wx = dev(synth.iq3_xxs_weights(n_out, n_in, 133, n_in // 256))
    gx = dev(synth.iq3_xxs_grid())
    assert_bits(host(qwg.gemv_iq3_xxs(wx, xd, gx)), 2 * y, "llama.cpp order, doubled grid")
    for _ in range(2):
        assert_bits(host(qwg.gemv_iq3(wd, xd, gd)), y, "repeat")


@pytest.mark.parametrize("offset", [0, 2, 6, 14])
@pytest.mark.parametrize("n_out,n_in", [(1, 256), (7, 512), (9, 2048), (63, 1792), (65, 768),
                                        (1000, 2048), (5632, 2048), (3, 2304), (130, 4096),
                                        (2048, 5632), (17, 6144)])
def test_gemv_iq3_row_groups(offset, n_out, n_in):
    # Row-group IQ3 kernel (batch 1, at most 24 blocks per row: one, two or
    # three block sets per workgroup, a matrix the
    # split short-call plan covers): eight whole rows per workgroup; row-major
    # weights at 2-byte offsets from a 16-byte boundary (the contiguous granule
    # run of each group, clamped at the buffer's ends), ragged last groups,
    # rows past n_out untouched; the tile layout and the llama.cpp order with
    # the same (doubled) bits; repeat calls with the same bits.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert -(-n_out // 64) <= cus // 2
    assert qwg.plan_splits(1, n_in, n_out) == 1
    grid = synth.iq3_grid()
    w = synth.iq3_weights(n_out, n_in, 135, offset)
    x = synth.activations(n_in, 135, n_out)
    wd, xd, gd = _guarded_iq3(w, offset), dev(x), dev(grid)
    yr, sr = oracle.gemv_iq3(w, grid, x, n_in, n_out)
    ybuf = torch.full((n_out + 128,), float("nan"), device=DEV)
    qwg.gemv_iq3(wd, xd, gd, out=ybuf[64:64 + n_out])
    yb = host(ybuf)
    assert np.isnan(yb[:64]).all() and np.isnan(yb[64 + n_out:]).all(), "write outside y"
    y = yb[64:64 + n_out]
    assert_bound(y, yr, sr, f"iq3 rows {n_out}x{n_in} offset {offset}")
    t = host(qwg.gemv_iq3_tiled(qwg.pack_iq3_tiles(dev(w), n_in), xd, gd, n_out))
    assert_bits(t, y, "tile layout")
    wx = synth.iq3_xxs_weights(n_out, n_in, 135, offset)
    gx = dev(synth.iq3_xxs_grid())
    assert_bits(host(qwg.gemv_iq3_xxs(_guarded_iq3(wx, offset), xd, gx)), 2 * y,
                "llama.cpp order, doubled grid")
    assert_bits(host(qwg.gemv_iq3(wd, xd, gd)), y, "repeat")


@pytest.mark.parametrize("waves", [0, 16])
def test_gemv_iq3_inexact_grid_gives_nan_rows(waves):
    # A grid value that fp16 cannot hold: every engine stores NaN in every row.
    grid = synth.iq3_grid().copy()
    grid[17, 2] = 0.1
    n_out, n_in = 300, 2048
    w = synth.iq3_weights(n_out, n_in, 134, 0)
    x = synth.activations(n_in, 134, 0)
    y = host(qwg.gemv_iq3(dev(w), dev(x), dev(grid), waves=waves, splits=1 if waves else 0))
    assert np.isnan(y).all()


def test_iq3_tiled_integer_exact_and_group_layer():
    grid = synth.iq3_grid()
    gd = dev(grid)
    # integer case (as test_gemv_iq3_integer_exact): exact in every summation order
    n_out, n_in = 150, 2048
    w = synth.iq3_weights(n_out, n_in, 103, 0).reshape(-1, 98).copy()
    w[:, 96], w[:, 97] = 0x00, 0x44
    words = w[:, 64:96].copy().view("<u4") & np.uint32(0x3FFFFFFF)
    w[:, 64:96] = words.view(np.uint8)
    w = w.reshape(n_out, -1)
    x = np.random.default_rng(9).integers(-8, 9, n_in).astype(np.float32)
    yr, _ = oracle.gemv_iq3(w, grid, x, n_in, n_out)
    y = host(qwg.gemv_iq3_tiled(qwg.pack_iq3_tiles(dev(w), n_in), dev(x), gd, n_out))
    assert np.array_equal(y.astype(np.float64), yr)
    # one layer's seven projections as a tiled group, three runs
    probs = synth.config(7)
    ws = [synth.weights(p) for p in probs]
    xs = [synth.inputs(p) for p in probs]
    W = [qwg.pack_iq3_tiles(dev(w), p.n_in) for p, w in zip(probs, ws)]
    Y = [torch.full((p.n_out,), float("nan"), device=DEV) for p in probs]
    g = qwg.Iq3Group(zip(W, [dev(x) for x in xs], Y), gd, tiled=True)
    for _ in range(3):
        g.run()
    for p, w, x, y in zip(probs, ws, xs, Y):
        yr, sr = oracle.gemv_iq3(w, grid, x, p.n_in, p.n_out)
        assert_bound(host(y), yr, sr, "iq3 tiled group " + p.name)
    g.close()


def test_iq3_tiled_group_stream_all_rows():
    grid, (probs, ws, xs, refs) = iq3_c6()
    Y = nan_outputs(probs)
    W = [qwg.pack_iq3_tiles(dev(w), p.n_in) for p, w in zip(probs, ws)]
    g = qwg.Iq3Group(zip(W, [dev(x) for x in xs], Y), dev(grid), tiled=True)
    g.run()
    assert_stream(probs, refs, Y, "iq3 tiled stream")
    for y in Y:
        y.fill_(float("nan"))
    g.run()
    assert_stream(probs, refs, Y, "iq3 tiled stream rerun")
    g.close()


# ---------------------------------------------------------------- IQ3_XXS, llama.cpp byte order
# synth.iq3_xxs_weights(n_out, n_in, cfg, t) holds the bytes of
# synth.iq3_weights(n_out, n_in, cfg, t) in llama.cpp's order, and
# synth.iq3_xxs_grid() is the container grid doubled (llama.cpp's convention).

@pytest.mark.parametrize("n_out,n_in", [(1, 256), (3, 768), (5632, 2048), (2048, 5632)])
def test_dequant_iq3_xxs_matches_oracle(n_out, n_in):
    grid = synth.iq3_xxs_grid()
    w = synth.iq3_xxs_weights(n_out, n_in, 140, n_out + n_in)
    got = host(qwg.dequant_iq3_xxs(dev(w), dev(grid)))
    assert_bits(got, oracle.dequant_iq3_xxs(w, grid, n_out * n_in), f"{n_out}x{n_in}")


def test_dequant_iq3_xxs_two_byte_aligned_base():
    n_out, n_in = 5, 768
    grid = synth.iq3_xxs_grid()
    w = synth.iq3_xxs_weights(n_out, n_in, 141, 0)
    wd = _guarded_iq3(w, 6)
    got = host(qwg.dequant_iq3_xxs(wd, dev(grid)))
    assert_bits(got, oracle.dequant_iq3_xxs(w, grid, n_out * n_in), "2 mod 4 base")


@pytest.mark.parametrize("p", synth.config(4), ids=lambda p: p.name)
def test_gemv_iq3_xxs_configs(p):
    grid = synth.iq3_xxs_grid()
    w = synth.iq3_xxs_weights(p.n_out, p.n_in, p.cfg, p.tensor)
    x = synth.inputs(p)
    y = host(qwg.gemv_iq3_xxs(dev(w), dev(x), dev(grid)))
    yr, sr = oracle.gemv_iq3_xxs(w, grid, x, p.n_in, p.n_out)
    assert_bound(y, yr, sr, p.name)


@pytest.mark.parametrize("n_out,n_in", [(1, 256), (3, 256), (65, 768), (100, 1280), (129, 5632),
                                        (2000, 768), (32000, 2048)])
def test_gemv_iq3_xxs_ragged(n_out, n_in):
    grid = synth.iq3_xxs_grid()
    w = synth.iq3_xxs_weights(n_out, n_in, 142, n_out)
    x = synth.activations(n_in, 142, n_out)
    y = torch.full((n_out,), float("nan"), device=DEV)
    qwg.gemv_iq3_xxs(dev(w), dev(x), dev(grid), out=y)
    yr, sr = oracle.gemv_iq3_xxs(w, grid, x, n_in, n_out)
    assert_bound(host(y), yr, sr, f"{n_out}x{n_in}")


@pytest.mark.parametrize("offset", [0, 2, 4, 6, 8, 10, 12, 14, 18, 30])
@pytest.mark.parametrize("n_out,n_in", [(1, 256), (3, 512), (65, 768), (64, 5632), (129, 2048)])
def test_gemv_iq3_xxs_buffer_edges(offset, n_out, n_in):
    # as test_gemv_iq3_buffer_edges: bytes outside w (0xFF) must never reach y
    grid = synth.iq3_xxs_grid()
    w = synth.iq3_xxs_weights(n_out, n_in, 143, offset)
    x = synth.activations(n_in, 143, offset)
    wd = _guarded_iq3(w, offset)
    yr, sr = oracle.gemv_iq3_xxs(w, grid, x, n_in, n_out)
    ybuf = torch.full((n_out + 130,), -7.0, device=DEV)
    qwg.gemv_iq3_xxs(wd, dev(x), dev(grid), out=ybuf[64:64 + n_out])
    yb = host(ybuf)
    assert_bound(yb[64:64 + n_out], yr, sr, f"offset={offset}")
    assert (yb[:64] == -7.0).all() and (yb[64 + n_out:] == -7.0).all(), "write outside y"


def test_gemv_iq3_xxs_integer_exact():
    # d = 4 and s in 0..3 make every sub-block scale an odd integer with the
    # doubled grid's integer entries: every partial sum is an exact integer
    n_out, n_in = 150, 5632
    grid = synth.iq3_xxs_grid()
    w = synth.iq3_xxs_weights(n_out, n_in, 144, 0).reshape(-1, 98).copy()
    w[:, 0], w[:, 1] = 0x00, 0x44
    words = w[:, 66:98].copy().view("<u4") & np.uint32(0x3FFFFFFF)
    w[:, 66:98] = words.view(np.uint8)
    w = w.reshape(n_out, -1)
    x = np.random.default_rng(11).integers(-8, 9, n_in).astype(np.float32)
    yr, _ = oracle.gemv_iq3_xxs(w, grid, x, n_in, n_out)
    y = host(qwg.gemv_iq3_xxs(dev(w), dev(x), dev(grid)))
    assert np.array_equal(y.astype(np.float64), yr)


@pytest.mark.parametrize("n_out,n_in", [(65, 768), (5632, 2048), (2048, 5632)])
def test_gemv_iq3_xxs_is_the_container_gemv(n_out, n_in):
    # the same fields in the two byte orders with the same grid: identical sums
    grid = dev(synth.iq3_xxs_grid())
    x = dev(synth.activations(n_in, 145, n_out))
    y5 = host(qwg.gemv_iq3(dev(synth.iq3_weights(n_out, n_in, 145, n_out)), x, grid)).copy()
    yx = host(qwg.gemv_iq3_xxs(dev(synth.iq3_xxs_weights(n_out, n_in, 145, n_out)), x, grid))
    assert_bits(yx, y5, f"{n_out}x{n_in}")


@pytest.mark.parametrize("n_out,n_in", [(1, 256), (65, 768), (300, 2048), (2048, 5632)])
def test_pack_iq3_xxs_tiles_is_the_iq3_tile_layout(n_out, n_in):
    wx = synth.iq3_xxs_weights(n_out, n_in, 146, n_out)
    w5 = synth.iq3_weights(n_out, n_in, 146, n_out)
    got = host(qwg.pack_iq3_xxs_tiles(dev(wx), n_in))
    assert np.array_equal(got, _iq3_tile_layout(w5, n_in))
    grid = synth.iq3_xxs_grid()
    x = synth.activations(n_in, 146, n_out)
    y = host(qwg.gemv_iq3_tiled(dev(got), dev(x), dev(grid), n_out))
    yr, sr = oracle.gemv_iq3_xxs(wx, grid, x, n_in, n_out)
    assert_bound(y, yr, sr, f"xxs tiled {n_out}x{n_in}")


# ---------------------------------------------------------------- split sums in stream launches
# A grouped launch (or a tiled single GEMV) with fewer 64-row tiles than
# resident workgroups splits each member's super-block range across
# workgroups; the partial sums meet in the member's own workspace.

def _integer_iq3(n_out, n_in, seed):
    # d = 4 and code in 0..3: every sub-block scale is an odd integer
    w = synth.iq3_weights(n_out, n_in, 150, seed).reshape(-1, 98).copy()
    w[:, 96], w[:, 97] = 0x00, 0x44
    words = w[:, 64:96].copy().view("<u4") & np.uint32(0x3FFFFFFF)
    w[:, 64:96] = words.view(np.uint8)
    return w.reshape(n_out, -1)


@pytest.mark.parametrize("fmt,tiled", [("q4k", False), ("q4k", True), ("iq3", False), ("iq3", True)])
def test_split_group_integer_exact_repeat_runs(fmt, tiled):
    # Integer data: every summation order gives the oracle's value exactly.
    # Members with one super-block per row are never split, so split and
    # whole-row members share the launch. Each run has new activations and
    # NaN-filled outputs: a tile counter that did not return to zero, or a
    # partial sum from the previous run, shows up as a wrong or NaN row.
    shapes = [(2048, 5632), (256, 2048), (65, 256), (1, 768), (130, 1280), (2048, 2048)]
    grid = synth.iq3_grid()
    if fmt == "q4k":
        ws = [_integer_q4k(o, i, 151 + k) for k, (o, i) in enumerate(shapes)]
        pack = qwg.pack_q4k_tiles
    else:
        ws = [_integer_iq3(o, i, 151 + k) for k, (o, i) in enumerate(shapes)]
        pack = qwg.pack_iq3_tiles
    W = [pack(dev(w), i) if tiled else dev(w) for w, (_, i) in zip(ws, shapes)]
    X = [torch.empty(i, device=DEV) for _, i in shapes]
    Y = [torch.empty(o, device=DEV) for o, _ in shapes]
    members = list(zip(W, X, Y))
    g = qwg.Q4kGroup(members, tiled=tiled) if fmt == "q4k" else \
        qwg.Iq3Group(members, dev(grid), tiled=tiled)
    assert g.workgroups == sum((o + 63) // 64 for o, _ in shapes)
    rng = np.random.default_rng(152)
    for run in range(4):
        xs = [rng.integers(-8, 9, i).astype(np.float32) for _, i in shapes]
        for xd, x in zip(X, xs):
            xd.copy_(torch.from_numpy(x))
        for y in Y:
            y.fill_(float("nan"))
        g.run()
        for (o, i), w, x, y in zip(shapes, ws, xs, Y):
            if fmt == "q4k":
                yr, _ = oracle.gemv_q4k(w, x, i, o)
            else:
                yr, _ = oracle.gemv_iq3(w, grid, x, i, o)
            assert np.array_equal(host(y).astype(np.float64), yr), f"run {run} {o}x{i}"
    g.close()


@pytest.mark.parametrize("n_out,n_in", [(7, 256), (64, 2048), (130, 5632), (2048, 5632),
                                        (300, 65536), (5632, 2048)])
def test_gemv_q4k_tiled_split_integer_exact(n_out, n_in):
    w = _integer_q4k(n_out, n_in, 153)
    wt = qwg.pack_q4k_tiles(dev(w), n_in)
    rng = np.random.default_rng(n_out + n_in)
    for _ in range(2):
        x = rng.integers(-8, 9, n_in).astype(np.float32)
        yr, _ = oracle.gemv_q4k(w, x, n_in, n_out)
        y = host(qwg.gemv_q4k_tiled(wt, dev(x), n_out))
        assert np.array_equal(y.astype(np.float64), yr)


def test_layered_decode_groups_within_bound():
    # The dependent per-layer launches of a decoder (q|k|v, o, gate|up, down),
    # each a small split group, on tile-layout weights.
    probs = synth.config(2)
    ws = [synth.weights(p) for p in probs]
    xs = [synth.inputs(p) for p in probs]
    W = [qwg.pack_q4k_tiles(dev(w), p.n_in) for p, w in zip(probs, ws)]
    X = [dev(x) for x in xs]
    Y = [torch.full((p.n_out,), float("nan"), device=DEV) for p in probs]
    names = [p.name.split(".")[-1] for p in probs]
    parts = [[0, 1, 2], [3], [4, 5], [6]] if names[:4] == ["q", "k", "v", "o"] else \
        [[i] for i in range(len(probs))]
    groups = [qwg.Q4kGroup([(W[i], X[i], Y[i]) for i in part], tiled=True) for part in parts]
    for _ in range(3):
        for g in groups:
            g.run()
    for p, w, x, y in zip(probs, ws, xs, Y):
        yr, sr = oracle.gemv_q4k(w, x, p.n_in, p.n_out)
        assert_bound(host(y), yr, sr, "layered " + p.name)
    for g in groups:
        g.close()


def test_graph_replays_match_eager():
    # A decoder layer's launches (split groups on tile-layout weights, per-call
    # GEMVs on the per-stream split workspace, a batched GEMM, an IQ3 GEMV)
    # captured once in a HIP graph after one eager call on the capture stream.
    # Three replays, each after an eager run on another stream, must reproduce
    # the eager outputs bit for bit.
    probs = synth.config(2)
    W = [qwg.pack_q4k_tiles(dev(synth.weights(p)), p.n_in) for p in probs]
    X = [dev(synth.inputs(p)) for p in probs]
    Y = [torch.empty(p.n_out, device=DEV) for p in probs]
    names = [p.name.split(".")[-1] for p in probs]
    parts = [[0, 1, 2], [3], [4, 5], [6]] if names[:4] == ["q", "k", "v", "o"] else \
        [[i] for i in range(len(probs))]
    groups = [qwg.Q4kGroup([(W[i], X[i], Y[i]) for i in part], tiled=True) for part in parts]
    wr, xr = dev(synth.weights(probs[0])), X[0]
    yr = torch.empty(probs[0].n_out, device=DEV)
    wg = dev(synth.q4k_weights(512, 2048, 104, 1))
    xg = dev(synth.activations(2048, 104, 2, batch=4))
    yg = torch.empty(4, 512, device=DEV)
    grid = dev(synth.iq3_grid())
    w3 = dev(synth.iq3_weights(300, 5632, 104, 3))
    x3 = dev(synth.activations(5632, 104, 4))
    y3 = torch.empty(300, device=DEV)
    xb = [dev(synth.activations(p.n_in, 104, 10 + i, batch=3)) for i, p in enumerate(probs[:3])]
    yb = [torch.empty(3, p.n_out, device=DEV) for p in probs[:3]]
    batched = qwg.Q4kBatchedGroup(zip(W[:3], xb, yb), tiled=True)
    outs = Y + [yr, yg, y3] + yb

    def step(s):
        for g in groups + [batched]:
            g.run(s)
        with torch.cuda.stream(s):
            qwg.gemv_q4k(wr, xr, out=yr)
            qwg.gemm_q4k(wg, xg, out=yg)
            qwg.gemv_iq3(w3, x3, grid, out=y3)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    step(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(side)
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    for r in range(3):
        step(main)
        torch.cuda.synchronize()
        ref = [o.clone() for o in outs]
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, outs)):
            assert torch.equal(a, b), f"replay {r}, output {i}"
    for g in groups + [batched]:
        g.close()


# ---------------------------------------------------------------- layer chain

def layer_phases(probs):
    """The per-token stream's problems grouped into the phases of a decoder's
    dependency chain (picoLM's model_forward: per layer q|k|v, o, gate|up,
    down; then the LM head), as lists of indices."""
    phases, i = [], 0
    while i < len(probs):
        name = probs[i].name.split(".")[-1]
        n = 3 if name == "q" else 2 if name == "gate" else 1
        phases.append(list(range(i, i + n)))
        i += n
    return phases


def c5_decode_step_chain(tagged=True):
    """The chain the bench times: the per-token stream's 155 products in the 89
    phases of a decode step, each product reading the output of the product
    that stands in for its input (synth.chain_sources; layer 0 reads the step's
    input x0), weights that keep the chained norms in range
    (synth.q4k_chain_weights), outputs NaN-filled. Returns the chain, the host
    weights, x0, the sources and the outputs."""
    probs = synth.config(5)
    ws = _C5_CHAIN_W.setdefault("w", [synth.q4k_chain_weights(p.n_out, p.n_in, p.cfg, p.tensor)
                                      for p in probs])
    x0 = synth.activations(2048, 5, 0)
    src = synth.chain_sources(probs)
    X0 = dev(x0)
    Y = nan_outputs(probs)
    X = [X0 if j < 0 else Y[j] for j in src]
    W = [qwg.pack_q4k_tiles(dev(w), p.n_in) for p, w in zip(probs, ws)]
    phases = layer_phases(probs)
    assert len(phases) == 89
    env = os.environ.pop("QWG_CHAIN_TAGGED", None)
    if not tagged:
        os.environ["QWG_CHAIN_TAGGED"] = "0"
    try:
        ch = qwg.Q4kChain([[(W[i], X[i], Y[i]) for i in ph] for ph in phases])
    finally:
        os.environ.pop("QWG_CHAIN_TAGGED", None)
        if env is not None:
            os.environ["QWG_CHAIN_TAGGED"] = env
    assert ch.tagged == tagged
    return ch, probs, ws, x0, src, Y, (W, X0)


_C5_CHAIN_W = {}


def test_chain_c5_decode_step_all_rows_and_repeat_runs():
    # The headline launch: every row of every product against the oracle applied
    # to that product's actual input (the step input or its producer's output);
    # later runs bitwise equal; the same chain with a flag barrier per phase
    # gives the same bits.
    ch, probs, ws, x0, src, Y, keep = c5_decode_step_chain()
    assert ch.launch_phases >= 89
    ch.run()
    ch.status()
    out = [host(y).copy() for y in Y]
    for k, (p, w) in enumerate(zip(probs, ws)):
        xin = x0 if src[k] < 0 else out[src[k]]
        assert not np.isnan(xin).any(), f"{p.name}: input left unwritten"
        yr, sr = oracle.gemv_q4k(w, xin, p.n_in, p.n_out)
        assert_bound(out[k], yr, sr, "chain " + p.name)
    assert 1.0 < np.linalg.norm(out[-2]) < 1e4   # the chained norms stay in range
    for y in Y:
        y.fill_(float("nan"))
    for _ in range(3):
        ch.run()
    ch.status()
    for p, y, y0 in zip(probs, Y, out):
        assert_bits(host(y), y0, "chain rerun " + p.name)
    ch.close()
    cb, _, _, _, _, Yb, keep_b = c5_decode_step_chain(tagged=False)
    cb.run()
    cb.status()
    for p, y, y0 in zip(probs, Yb, out):
        assert_bits(host(y), y0, "flag-barrier chain " + p.name)
    cb.close()


def test_chain_c5_independent_inputs_all_rows():
    # The same 89 phases with an independent input per product (done-word waits
    # only, no tagged rows): every row against the oracle, reruns bitwise equal.
    probs, ws, xs, refs = q4k_c5()
    W = [qwg.pack_q4k_tiles(dev(w), p.n_in) for p, w in zip(probs, ws)]
    X = [dev(x) for x in xs]
    Y = nan_outputs(probs)
    phases = layer_phases(probs)
    ch = qwg.Q4kChain([[(W[i], X[i], Y[i]) for i in ph] for ph in phases])
    assert ch.tagged
    ch.run()
    ch.status()
    assert_stream(probs, refs, Y, "chain")
    first = [host(y).copy() for y in Y]
    for y in Y:
        y.fill_(float("nan"))
    for _ in range(2):
        ch.run()
    ch.status()
    for p, y, y0 in zip(probs, Y, first):
        assert_bits(host(y), y0, "chain rerun " + p.name)
    ch.close()


def test_chain_overwriting_an_earlier_input_uses_flag_barriers():
    # Phase 1 writes the buffer phase 0 read: a tagged launch could let a fast
    # workgroup overwrite it early, so the chain falls back to flag barriers.
    n = 2048
    wa, wb = _small_q4k(n, n, 301), _small_q4k(n, n, 302)
    x0 = synth.activations(n, 203, 0)
    xd, ya = dev(x0), torch.full((n,), float("nan"), device=DEV)
    ch = qwg.Q4kChain([[(qwg.pack_q4k_tiles(dev(wa), n), xd, ya)],
                       [(qwg.pack_q4k_tiles(dev(wb), n), ya, xd)]])
    assert not ch.tagged
    ch.run()
    ch.status()
    yah = host(ya).copy()
    yr, sr = oracle.gemv_q4k(wa, x0, n, n)
    assert_bound(yah, yr, sr, "phase 0")
    yr, sr = oracle.gemv_q4k(wb, yah, n, n)
    assert_bound(host(xd), yr, sr, "phase 1 (written over phase 0's input)")
    ch.close()


def test_chain_input_inside_a_larger_output():
    # A consumer reads 2048 rows at an offset inside a 5632-row output (tagged
    # rows read at that offset), another the output's head; a third phase
    # reads both consumers' outputs through one more producer.
    wp = _small_q4k(5632, 2048, 303)
    wc1, wc2 = _small_q4k(2048, 2048, 304), _small_q4k(256, 2048, 305)
    wl = _small_q4k(1000, 2048, 306)
    x0 = synth.activations(2048, 204, 0)
    xd = dev(x0)
    yp = torch.full((5632,), float("nan"), device=DEV)
    y1 = torch.full((2048,), float("nan"), device=DEV)
    y2 = torch.full((256,), float("nan"), device=DEV)
    yl = torch.full((1000,), float("nan"), device=DEV)
    pk = lambda w, k: qwg.pack_q4k_tiles(dev(w), k)   # noqa: E731
    ch = qwg.Q4kChain([[(pk(wp, 2048), xd, yp)],
                       [(pk(wc1, 2048), yp[1024:3072], y1), (pk(wc2, 2048), yp[:2048], y2)],
                       [(pk(wl, 2048), y1, yl)]])
    assert ch.tagged
    for _ in range(2):
        ch.run()
    ch.status()
    yph = host(yp).copy()
    for w, xin, y, n_out in ((wp, x0, yp, 5632), (wc1, yph[1024:3072], y1, 2048),
                             (wc2, yph[:2048], y2, 256), (wl, host(y1).copy(), yl, 1000)):
        yr, sr = oracle.gemv_q4k(w, np.ascontiguousarray(xin), 2048, n_out)
        assert_bound(host(y), yr, sr, f"member with {n_out} rows")
    ch.close()


def _small_q4k(n_out, n_in, seed, d=2e-5):
    """Q4_K weights with d and dmin near `d` (fp16), so that products chained
    over many phases stay far inside the fp32 range."""
    w = synth.q4k_weights(n_out, n_in, 201, seed).reshape(-1, 144).copy()
    rng = np.random.default_rng(seed)
    w[:, 0:2] = (rng.uniform(0.5, 1.5, len(w)) * d).astype(np.float16).view(np.uint8).reshape(-1, 2)
    w[:, 2:4] = (rng.uniform(0.5, 1.5, len(w)) * d).astype(np.float16).view(np.uint8).reshape(-1, 2)
    return w.reshape(n_out, -1)


def test_chain_wired_phases_read_the_previous_outputs():
    # Each phase reads what the phase before it wrote: q|k|v read x (then the
    # previous down's y), o reads y_q, gate|up read y_o, down reads y_gate, and
    # an LM-head-shaped last phase reads the last y_down. Outputs start as NaN
    # and the input changes every run, so a phase that read its input before
    # the producer finished (or a stale copy of an earlier run) fails the bound
    # against the oracle applied to the producer's final output.
    layers = 4
    shapes = {"q": (2048, 2048), "k": (256, 2048), "v": (256, 2048), "o": (2048, 2048),
              "gate": (5632, 2048), "up": (5632, 2048), "down": (2048, 5632)}
    x0 = torch.empty(2048, device=DEV)
    members, phases = [], []
    src = x0
    for l in range(layers):
        mk = {}
        for k, name in enumerate(shapes):
            n_out, n_in = shapes[name]
            w = _small_q4k(n_out, n_in, 10 * l + k)
            mk[name] = [w, qwg.pack_q4k_tiles(dev(w), n_in), None,
                        torch.empty(n_out, device=DEV)]
        for name in ("q", "k", "v"):
            mk[name][2] = src
        mk["o"][2] = mk["q"][3]
        mk["gate"][2] = mk["o"][3]
        mk["up"][2] = mk["o"][3]
        mk["down"][2] = mk["gate"][3]
        src = mk["down"][3]
        for group in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
            phases.append([len(members) + i for i in range(len(group))])
            members += [mk[name] for name in group]
    wh = _small_q4k(32000, 2048, 99)
    members.append([wh, qwg.pack_q4k_tiles(dev(wh), 2048), src, torch.empty(32000, device=DEV)])
    phases.append([len(members) - 1])
    ch = qwg.Q4kChain([[tuple(members[i][1:]) for i in ph] for ph in phases])
    assert ch.tagged
    for run in range(3):
        x0.copy_(torch.from_numpy(synth.activations(2048, 201, run)))
        for m in members:
            m[3].fill_(float("nan"))
        ch.run()
        ch.status()
        for i, (w, _, x, y) in enumerate(members):
            xh = host(x).copy()
            assert not np.isnan(xh).any(), f"run {run} member {i}: input left unwritten"
            yr, sr = oracle.gemv_q4k(w, xh, x.numel(), y.numel())
            assert_bound(host(y), yr, sr, f"run {run} wired member {i}")
    ch.close()


def test_chain_ragged_members_and_one_phase():
    # Ragged row counts, one-block rows, 256-block rows (256 units per tile),
    # several members in a phase, and a chain of a single phase.
    shapes = [[(1, 256), (65, 512)], [(300, 65536)], [(4097, 768), (64, 2048), (129, 5632)]]
    members, refs = [], []
    for pi, ph in enumerate(shapes):
        row = []
        for k, (n_out, n_in) in enumerate(ph):
            w = synth.q4k_weights(n_out, n_in, 202, 10 * pi + k)
            x = synth.activations(n_in, 202, 10 * pi + k)
            y = torch.full((n_out,), float("nan"), device=DEV)
            row.append((qwg.pack_q4k_tiles(dev(w), n_in), dev(x), y))
            refs.append((w, x, y, n_in, n_out))
        members.append(row)
    for chain_phases in (members, [members[2]]):
        ch = qwg.Q4kChain(chain_phases)
        for _ in range(2):
            ch.run()
        ch.status()
        for w, x, y, n_in, n_out in refs if chain_phases is members else refs[3:]:
            yr, sr = oracle.gemv_q4k(w, x, n_in, n_out)
            assert_bound(host(y), yr, sr, f"chain {n_out}x{n_in}")
        ch.close()


# ---------------------------------------------------------------- IQ3_S and IQ4_XS

CB_FMT = {"iq3s": qwg.QWG_FMT_IQ3_S, "iq4xs": qwg.QWG_FMT_IQ4_XS}
CB = {
    "iq3s": dict(weights=synth.iq3s_weights, table=synth.iq3s_grid, nbytes=110,
                 dequant=qwg.dequant_iq3s, pack=qwg.pack_iq3s_tiles, gemv=qwg.gemv_iq3s_tiled,
                 rows=qwg.gemv_iq3s,
                 group=qwg.Iq3sGroup, o_dequant=oracle.dequant_iq3s, o_gemv=oracle.gemv_iq3s,
                 o_rows=oracle.gemv_iq3s_rows),
    "iq4xs": dict(weights=synth.iq4xs_weights, table=synth.iq4nl_table, nbytes=136,
                  dequant=qwg.dequant_iq4xs, pack=qwg.pack_iq4xs_tiles, gemv=qwg.gemv_iq4xs_tiled,
                  rows=qwg.gemv_iq4xs,
                  group=qwg.Iq4xsGroup, o_dequant=oracle.dequant_iq4xs, o_gemv=oracle.gemv_iq4xs,
                  o_rows=oracle.gemv_iq4xs_rows),
}


def _cb_tile_layout(fmt: str, w: np.ndarray, n_in: int) -> np.ndarray:
    """The tile layouts written out from their description in include/qwg.h."""
    nbytes = CB[fmt]["nbytes"]
    n_out, nb = w.shape[0], n_in // 256
    tiles = (n_out + 63) // 64
    blk = np.zeros((tiles * 64, nb, nbytes), np.uint8)
    blk[:n_out] = w.reshape(n_out, nb, nbytes)
    blk = blk.reshape(tiles, 64, nb, nbytes).transpose(0, 2, 1, 3)       # [t][b][row][bytes]

    def per_g(a, b, width):    # bytes a..b of each block as [G][row][width]
        return blk[..., a:b].reshape(tiles, nb, 64, 4, width).transpose(0, 1, 3, 2, 4).reshape(tiles, nb, -1)

    def per_row(a, b):
        return blk[..., a:b].reshape(tiles, nb, -1)

    if fmt == "iq3s":
        parts = [per_g(2, 66, 16), per_g(74, 106, 8), per_g(66, 74, 2), per_row(106, 110),
                 per_row(0, 2)]
    else:
        parts = [per_g(8, 136, 32), per_row(0, 8)]
    return np.concatenate(parts, axis=2).reshape(-1)


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
@pytest.mark.parametrize("n_out,n_in", [(1, 256), (3, 768), (5632, 2048), (2048, 5632)])
def test_dequant_codebook_matches_oracle(fmt, n_out, n_in):
    c = CB[fmt]
    tab = c["table"]()
    w = c["weights"](n_out, n_in, 160, n_out + n_in)
    got = host(c["dequant"](dev(w), dev(tab)))
    assert_bits(got, c["o_dequant"](w, tab, n_out * n_in), f"{fmt} {n_out}x{n_in}")


def test_dequant_iq3s_two_byte_aligned_base():
    tab = synth.iq3s_grid()
    w = synth.iq3s_weights(3, 512, 161, 0)
    wd = _guarded_iq3(w, 2)
    assert wd.data_ptr() % 4 == 2
    assert_bits(host(qwg.dequant_iq3s(wd, dev(tab))), oracle.dequant_iq3s(w, tab, 3 * 512), "2 mod 4")


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
@pytest.mark.parametrize("n_out,n_in", [(1, 256), (65, 768), (300, 2048), (2048, 5632)])
def test_pack_codebook_tiles_is_the_layout(fmt, n_out, n_in):
    c = CB[fmt]
    w = c["weights"](n_out, n_in, 162, n_out)
    got = host(c["pack"](dev(w), n_in))
    assert np.array_equal(got, _cb_tile_layout(fmt, w, n_in))


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
@pytest.mark.parametrize("n_out,n_in", [(1, 256), (3, 512), (65, 768), (130, 5632), (2048, 2048),
                                        (5632, 2048), (2048, 5632), (4097, 1280)])
def test_gemv_codebook_tiled(fmt, n_out, n_in):
    c = CB[fmt]
    tab = c["table"]()
    w = c["weights"](n_out, n_in, 163, n_out)
    x = synth.activations(n_in, 163, n_out)
    wt, xd, td = c["pack"](dev(w), n_in), dev(x), dev(tab)
    y = host(c["gemv"](wt, xd, td, n_out)).copy()
    yr, sr = c["o_gemv"](w, tab, x, n_in, n_out)
    assert_bound(y, yr, sr, f"{fmt} tiled {n_out}x{n_in}")
    assert_bits(host(c["gemv"](wt, xd, td, n_out)), y, f"{fmt} rerun")


def _guarded_cb(w: np.ndarray, offset: int):
    """Row-major codebook weights at `offset` (a multiple of 16) past a 256-byte
    boundary, with 0xFF bytes (an fp16 NaN scale) before and after them, so that
    a byte used from outside w shows as NaN rows."""
    buf = torch.full((w.size + offset + 160,), 0xFF, dtype=torch.uint8, device=DEV)
    buf[offset:offset + w.size] = dev(w.reshape(-1))
    wd = buf[offset:offset + w.size]
    assert wd.data_ptr() % 256 == offset
    return wd


# Row-major blocks as a file stores them. (n_out * n_in/256) odd: the buffer
# ends off a 16-byte boundary (the last row's last block is read directly);
# 130 x 5632 and 7 x 2816 rows are not multiples of 16 bytes, so every row's
# blocks start at a different offset within their granules.
@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
@pytest.mark.parametrize("n_out,n_in", [(1, 256), (3, 768), (65, 768), (7, 2816), (130, 5632),
                                        (2048, 2048), (5632, 2048), (2048, 5632), (4097, 1280)])
def test_gemv_codebook_rows(fmt, n_out, n_in):
    c = CB[fmt]
    tab = c["table"]()
    w = c["weights"](n_out, n_in, 168, n_out)
    x = synth.activations(n_in, 168, n_out)
    wd, xd, td = dev(w), dev(x), dev(tab)
    y = torch.full((n_out,), float("nan"), device=DEV)
    c["rows"](wd, xd, td, out=y)
    y = host(y).copy()
    yr, sr = c["o_gemv"](w, tab, x, n_in, n_out)
    assert_bound(y, yr, sr, f"{fmt} rows {n_out}x{n_in} splits={qwg.plan_splits(CB_FMT[fmt], n_in, n_out)}")
    assert_bits(host(c["rows"](wd, xd, td)), y, f"{fmt} rows rerun")


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
@pytest.mark.parametrize("offset", [0, 16, 48, 240])
@pytest.mark.parametrize("n_out,n_in", [(1, 256), (3, 768), (65, 1280), (129, 2048)])
def test_gemv_codebook_rows_reads_only_the_weights(fmt, offset, n_out, n_in):
    c = CB[fmt]
    tab = c["table"]()
    w = c["weights"](n_out, n_in, 169, offset + n_out)
    x = synth.activations(n_in, 169, n_out)
    y = host(c["rows"](_guarded_cb(w, offset), dev(x), dev(tab)))
    yr, sr = c["o_gemv"](w, tab, x, n_in, n_out)
    assert_bound(y, yr, sr, f"{fmt} rows at +{offset} {n_out}x{n_in}")


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
@pytest.mark.parametrize("n_out,n_in", [(1, 256), (9, 2048), (63, 1792), (1000, 2048),
                                        (5632, 2048), (3, 2304), (130, 4096), (2048, 5632),
                                        (17, 6144)])
def test_gemv_codebook_row_groups(fmt, n_out, n_in):
    # Row-group kernel for IQ3_S / IQ4_XS single GEMVs (at most 24 blocks per
    # row, a matrix the split short-call plan covers): eight whole rows per
    # workgroup; row-major weights between guard bytes, ragged last groups,
    # rows past n_out untouched; the tile layout with the same bits (the same
    # kernel and order); repeat calls with the same bits.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert -(-n_out // 64) <= cus // 2
    assert qwg.plan_splits(CB_FMT[fmt], n_in, n_out) == 1
    c = CB[fmt]
    tab = c["table"]()
    w = c["weights"](n_out, n_in, 172, n_out)
    x = synth.activations(n_in, 172, n_out)
    wd, xd, td = _guarded_cb(w, 16), dev(x), dev(tab)
    yr, sr = c["o_gemv"](w, tab, x, n_in, n_out)
    ybuf = torch.full((n_out + 128,), float("nan"), device=DEV)
    c["rows"](wd, xd, td, out=ybuf[64:64 + n_out])
    yb = host(ybuf)
    assert np.isnan(yb[:64]).all() and np.isnan(yb[64 + n_out:]).all(), "write outside y"
    y = yb[64:64 + n_out]
    assert_bound(y, yr, sr, f"{fmt} row groups {n_out}x{n_in}")
    t = host(c["gemv"](c["pack"](dev(w), n_in), xd, td, n_out))
    assert_bits(t, y, f"{fmt} tile layout")
    assert_bits(host(c["rows"](wd, xd, td)), y, f"{fmt} repeat")


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
def test_gemv_codebook_rows_misaligned_weights_rejected(fmt):
    c = CB[fmt]
    w = c["weights"](2, 256, 170, 0)
    buf = torch.zeros(w.size + 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(qwg.QwgError) as e:
        c["rows"](buf[8:8 + w.size], dev(synth.activations(256, 170, 0)), dev(c["table"]()))
    assert e.value.status == 3


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
def test_gemv_codebook_rows_lm_head_all_rows(fmt):
    c = CB[fmt]
    n_out, n_in = 32000, 2048
    tab = c["table"]()
    w = c["weights"](n_out, n_in, 171, 0)
    x = synth.activations(n_in, 171, 0)
    y = torch.full((n_out,), float("nan"), device=DEV)
    c["rows"](dev(w), dev(x), dev(tab), out=y)
    yr, sr = c["o_gemv"](w, tab, x, n_in, n_out)
    assert_bound(host(y), yr, sr, f"{fmt} rows lm head")


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
@pytest.mark.parametrize("n_out,n_in", [(150, 2048), (64, 5632), (7, 256), (33, 2816)])
def test_gemv_codebook_rows_integer_exact(fmt, n_out, n_in):
    c = CB[fmt]
    tab = c["table"]()
    w = _integer_cb(fmt, n_out, n_in, n_out + 1)
    x = np.random.default_rng(n_in + n_out + 1).integers(-8, 9, n_in).astype(np.float32)
    yr, _ = c["o_gemv"](w, tab, x, n_in, n_out)
    y = host(c["rows"](dev(w), dev(x), dev(tab)))
    assert np.array_equal(y.astype(np.float64), yr)


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
def test_codebook_rows_group_stream_all_rows(fmt):
    c = CB[fmt]
    tab = c["table"]()
    probs, ws, xs, refs = stream_case(fmt + "_c6", lambda: (
        synth.config(6), [c["weights"](p.n_out, p.n_in, 167, k) for k, p in enumerate(synth.config(6))],
        [synth.inputs(p) for p in synth.config(6)],
        lambda p, w, x: c["o_gemv"](w, tab, x, p.n_in, p.n_out)))
    Y = nan_outputs(probs)
    g = c["group"](zip([dev(w) for w in ws], [dev(x) for x in xs], Y), dev(tab), tiled=False)
    for _ in range(2):
        g.run()
    assert_stream(probs, refs, Y, f"{fmt} rows stream")
    g.close()


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
def test_codebook_rows_groups_layer_repeat_runs(fmt):
    c = CB[fmt]
    tab = c["table"]()
    probs = synth.config(2)
    ws = [c["weights"](p.n_out, p.n_in, 172, k) for k, p in enumerate(probs)]
    X = [torch.empty(p.n_in, device=DEV) for p in probs]
    Y = [torch.empty(p.n_out, device=DEV) for p in probs]
    g = c["group"](zip([dev(w) for w in ws], X, Y), dev(tab), tiled=False)
    for run in range(3):
        xs = [synth.activations(p.n_in, 172, 10 * run + k) for k, p in enumerate(probs)]
        for xd, x in zip(X, xs):
            xd.copy_(torch.from_numpy(x))
        for y in Y:
            y.fill_(float("nan"))
        g.run()
        for p, w, x, y in zip(probs, ws, xs, Y):
            yr, sr = c["o_gemv"](w, tab, x, p.n_in, p.n_out)
            assert_bound(host(y), yr, sr, f"{fmt} rows layer run {run} {p.name}")
    g.close()


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
def test_gemv_codebook_lm_head_all_rows(fmt):
    c = CB[fmt]
    n_out, n_in = 32000, 2048
    tab = c["table"]()
    w = c["weights"](n_out, n_in, 164, 0)
    x = synth.activations(n_in, 164, 0)
    y = torch.full((n_out,), float("nan"), device=DEV)
    c["gemv"](c["pack"](dev(w), n_in), dev(x), dev(tab), n_out, out=y)
    yr, sr = c["o_gemv"](w, tab, x, n_in, n_out)
    assert_bound(host(y), yr, sr, f"{fmt} lm head")


def _integer_cb(fmt, n_out, n_in, seed):
    w = CB[fmt]["weights"](n_out, n_in, 165, seed).reshape(-1, CB[fmt]["nbytes"]).copy()
    w[:, 0], w[:, 1] = 0x00, 0x3C                   # d = 1
    if fmt == "iq3s":
        w[:, 106:110] &= 0x33                       # s in 0..3: eff 1, 3, 5, 7
    else:
        w[:, 2:4] = [0xAA, 0xAA]                    # top bits 2: s = 32 + low nibble
        w[:, 4:8] &= 0x33                           # eff = s - 32 in 0..3
    return w.reshape(n_out, -1)


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
@pytest.mark.parametrize("n_out,n_in", [(150, 2048), (64, 5632), (7, 256)])
def test_gemv_codebook_integer_exact(fmt, n_out, n_in):
    c = CB[fmt]
    tab = c["table"]()
    w = _integer_cb(fmt, n_out, n_in, n_out)
    x = np.random.default_rng(n_in + n_out).integers(-8, 9, n_in).astype(np.float32)
    yr, _ = c["o_gemv"](w, tab, x, n_in, n_out)
    y = host(c["gemv"](c["pack"](dev(w), n_in), dev(x), dev(tab), n_out))
    assert np.array_equal(y.astype(np.float64), yr)


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
def test_codebook_groups_layer_stream_repeat_runs(fmt):
    c = CB[fmt]
    tab = c["table"]()
    td = dev(tab)
    # one layer's seven projections (split sums), four runs with new activations
    probs = synth.config(2)
    ws = [c["weights"](p.n_out, p.n_in, 166, k) for k, p in enumerate(probs)]
    W = [c["pack"](dev(w), p.n_in) for p, w in zip(probs, ws)]
    X = [torch.empty(p.n_in, device=DEV) for p in probs]
    Y = [torch.empty(p.n_out, device=DEV) for p in probs]
    g = c["group"](zip(W, X, Y), td)
    for run in range(3):
        xs = [synth.activations(p.n_in, 166, 10 * run + k) for k, p in enumerate(probs)]
        for xd, x in zip(X, xs):
            xd.copy_(torch.from_numpy(x))
        for y in Y:
            y.fill_(float("nan"))
        g.run()
        for p, w, x, y in zip(probs, ws, xs, Y):
            yr, sr = c["o_gemv"](w, tab, x, p.n_in, p.n_out)
            assert_bound(host(y), yr, sr, f"{fmt} layer run {run} {p.name}")
    g.close()


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
def test_codebook_group_stream_all_rows(fmt):
    c = CB[fmt]
    tab = c["table"]()
    probs, ws, xs, refs = stream_case(fmt + "_c6", lambda: (
        synth.config(6), [c["weights"](p.n_out, p.n_in, 167, k) for k, p in enumerate(synth.config(6))],
        [synth.inputs(p) for p in synth.config(6)],
        lambda p, w, x: c["o_gemv"](w, tab, x, p.n_in, p.n_out)))
    Y = nan_outputs(probs)
    W = [c["pack"](dev(w), p.n_in) for p, w in zip(probs, ws)]
    g = c["group"](zip(W, [dev(x) for x in xs], Y), dev(tab))
    for _ in range(2):
        g.run()
    assert_stream(probs, refs, Y, f"{fmt} stream")
    g.close()


# ---------------------------------------------------------------- codebooks fp16 cannot hold

@pytest.mark.parametrize("fmt", ["iq3", "iq3s", "iq4xs"])
def test_codebook_not_fp16_exact_is_reported(fmt):
    # The GEMV engines keep the codebook in fp16. A value fp16 cannot hold
    # (2 + 2^-20) makes every output row of a single call NaN, and group
    # creation return QWG_ERR_GRID; the same call with the value rounded to
    # fp16 (2.0) is within the bound.
    n_out, n_in = 130, 768
    x = synth.activations(n_in, 220, 0)
    rows = None
    if fmt == "iq3":
        tab = synth.iq3_grid().copy()
        w = synth.iq3_weights(n_out, n_in, 220, 1)
        call = lambda t: qwg.gemv_iq3(dev(w), dev(x), dev(t))   # noqa: E731
        group = lambda t: qwg.Iq3Group([(dev(w), dev(x), torch.empty(n_out, device=DEV))], dev(t))   # noqa: E731
        ref = lambda t: oracle.gemv_iq3(w, t, x, n_in, n_out)   # noqa: E731
    else:
        c = CB[fmt]
        tab = c["table"]().copy()
        w = c["weights"](n_out, n_in, 220, 2)
        wt = c["pack"](dev(w), n_in)
        call = lambda t: c["gemv"](wt, dev(x), dev(t), n_out)   # noqa: E731
        rows = lambda t: c["rows"](dev(w), dev(x), dev(t))   # noqa: E731
        group = lambda t: c["group"]([(wt, dev(x), torch.empty(n_out, device=DEV))], dev(t))   # noqa: E731
        ref = lambda t: c["o_gemv"](w, t, x, n_in, n_out)   # noqa: E731
    bad = tab.copy()
    bad.reshape(-1)[5] = np.float32(2.0 + 2.0 ** -20)
    assert float(np.float16(bad.reshape(-1)[5])) != float(bad.reshape(-1)[5])
    for f in (call, rows) if rows else (call,):
        y = host(f(bad))
        assert np.isnan(y).all(), f"{fmt}: {int((~np.isnan(y)).sum())} rows not NaN"
    with pytest.raises(qwg.QwgError) as e:
        group(bad)
    assert e.value.status == 9
    good = bad.copy()
    good.reshape(-1)[5] = np.float32(2.0)
    yr, sr = ref(good)
    for f in (call, rows) if rows else (call,):
        assert_bound(host(f(good)), yr, sr, f"{fmt} exact codebook")


# ---------------------------------------------------------------- IQ3 encoder
# Every step of the encoder is float32 in a fixed order on both sides, so the
# bytes must be identical.

def _enc_input(n_rows, n_in, seed, scale=0.02):
    return (np.random.default_rng(seed).standard_normal((n_rows, n_in)) * scale).astype(np.float32)


@pytest.mark.parametrize("n_rows,n_in", [(1, 256), (3, 2048), (64, 5632), (200, 768)])
def test_encode_iq3_bytes_match_oracle(n_rows, n_in):
    grid = synth.iq3_grid()
    x = _enc_input(n_rows, n_in, 170 + n_rows)
    got = host(qwg.encode_iq3(dev(x), dev(grid)))
    want = oracle.encode_iq3(x, grid)
    diff = np.nonzero((got != want).any(axis=1))[0]
    assert diff.size == 0, f"rows {diff[:5]} differ"


def test_encode_iq3_edge_values():
    grid = synth.iq3_grid()
    rng = np.random.default_rng(171)
    rows = [np.zeros(512, np.float32),                                  # d = 0
            (rng.standard_normal(512) * 1e-6).astype(np.float32),      # subnormal fp16 d
            (rng.standard_normal(512) * 1e5).astype(np.float32),       # large d
            (rng.standard_normal(512) * 1e7).astype(np.float32),       # d overflows to infinity
            np.where(rng.random(512) < 0.5, -1.0, 1.0).astype(np.float32),   # equal magnitudes
            -np.abs(rng.standard_normal(512)).astype(np.float32),      # all negative
            np.repeat(rng.standard_normal(64), 8).astype(np.float32)]  # ties inside groups
    x = np.stack(rows)
    got = host(qwg.encode_iq3(dev(x), dev(grid)))
    want = oracle.encode_iq3(x, grid)
    for r in range(len(rows)):
        assert np.array_equal(got[r], want[r]), f"row {r}"


def test_encode_iq3_duplicate_grid_rows_and_gemv_roundtrip():
    grid = synth.iq3_grid().copy()
    grid[200] = grid[3]
    x = _enc_input(96, 2048, 172)
    b = qwg.encode_iq3(dev(x), dev(grid))
    assert np.array_equal(host(b), oracle.encode_iq3(x, grid))
    # the encoded matrix multiplies as its decode
    v = synth.activations(2048, 172, 0)
    y = host(qwg.gemv_iq3(b, dev(v), dev(grid)))
    yr, sr = oracle.gemv_iq3(host(b), grid, v, 2048, 96)
    assert_bound(y, yr, sr, "encoded gemv")
