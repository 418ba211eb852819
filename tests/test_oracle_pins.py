"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test checks the oracle against something the pages or the mathematics fix:
hand-expanded blocks (tests/golden/), closed forms, exhaustive enumerations,
library routines for the special cases that reduce to them (numpy's binary16
conversion, numpy's fp64 matmul), and structural invariants of a matrix-vector
product. Together they are chosen so that a dropped term, a wrong sign, a wrong
bit or byte index, or a transposed operand in the oracle fails at least one.
"""
import numpy as np
import pytest

import oracle
from golden_io import floats, hexbytes, ints, load
from quantized_weight_decode_gemv_amd import synth


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


# ---------------------------------------------------------------- constants

def test_block_sizes_and_density():
    # "用 Python 重写 picoLM", dequantize_q4_K docstring: 144 bytes, 256 weights, 4.5 bpw.
    assert 2 + 2 + 12 + 128 == oracle.Q4K_BYTES == 144
    assert oracle.Q4K_BYTES * 8 / oracle.QK == 4.5
    # iq3_pack.py: 64 index bytes + 8 words + fp16 d = 98 bytes, 3.0625 bpw.
    assert 256 // 4 + (256 // 32) * 4 + 2 == oracle.IQ3_BYTES == 98
    assert oracle.IQ3_BYTES * 8 / oracle.QK == 3.0625


# ---------------------------------------------------------------- fp16

def test_f16_known_values():
    cases = {0x3C00: 1.0, 0x3800: 0.5, 0x4000: 2.0, 0xC000: -2.0, 0x7BFF: 65504.0,
             0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24, 0x0400: 2.0 ** -14,
             0x2C00: 0.0625, 0x3400: 0.25, 0x3555: 0.333251953125}
    for bits, val in cases.items():
        assert oracle.f16_to_f32(bits) == val, hex(bits)
    assert np.signbit(oracle.f16_to_f32(0x8000)) and oracle.f16_to_f32(0x8000) == 0.0
    assert oracle.f16_to_f32(0x7C00) == np.inf and oracle.f16_to_f32(0xFC00) == -np.inf
    assert np.isnan(oracle.f16_to_f32(0x7E00))


def test_f16_all_patterns_match_numpy():
    # numpy's binary16 -> binary32 widening is a library routine for the same definition.
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(b)) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ---------------------------------------------------------------- Q4_K scales

@pytest.mark.parametrize("name", ["q4k_block_A.txt", "q4k_block_C.txt"])
def test_q4k_scale_unpack_hand(name):
    g = load(name)
    head = hexbytes(g["head"])
    sc, mn = oracle.unpack_q4k_scales(np.array(head[4:16], np.uint8))
    assert list(sc) == ints(g["sc"])
    assert list(mn) == ints(g["mn"])
    assert list(oracle.pack_q4k_scales(sc, mn)) == head[4:16]


def test_q4k_scale_roundtrip_every_field_value():
    rng = np.random.default_rng(1)
    for field in range(16):
        for v in range(64):
            sc = rng.integers(0, 64, 8)
            mn = rng.integers(0, 64, 8)
            (sc if field < 8 else mn)[field % 8] = v
            p = oracle.pack_q4k_scales(sc, mn)
            sc2, mn2 = oracle.unpack_q4k_scales(p)
            assert list(sc2) == list(sc) and list(mn2) == list(mn)


def test_q4k_scale_pack_of_unpack_is_identity():
    # 96 bits <-> sixteen 6-bit fields is a bijection: every byte string is reached.
    rng = np.random.default_rng(2)
    for _ in range(2000):
        p = rng.integers(0, 256, 12).astype(np.uint8)
        sc, mn = oracle.unpack_q4k_scales(p)
        assert sc.max() < 64 and mn.max() < 64
        assert np.array_equal(oracle.pack_q4k_scales(sc, mn), p)


def test_q4k_scale_top_bits_land_in_byte_top():
    p = oracle.pack_q4k_scales([0, 0, 0, 0, 63, 0, 0, 0], [0] * 8)
    assert p[0] == 0xC0 and p[8] == 0x0F and not p[1:8].any() and not p[9:].any()
    p = oracle.pack_q4k_scales([0] * 8, [0, 0, 0, 0, 0, 0, 0, 48])
    assert p[7] == 0xC0 and p[11] == 0x00 and not p[:7].any()


# ---------------------------------------------------------------- Q4_K dequant

@pytest.mark.parametrize("name", ["q4k_block_A.txt", "q4k_block_C.txt"])
def test_q4k_hand_blocks(name):
    g = load(name)
    block = np.array(hexbytes(g["head"]) + [int(g["quant_fill"], 16)] * 128, np.uint8)
    w = oracle.dequant_q4k(block, 256)
    want = np.repeat(np.array(floats(g["subblock_values"]), np.float32), 32)
    assert np.array_equal(w.view(np.uint32), want.view(np.uint32))


def test_q4k_nibble_order():
    g = load("q4k_nibble_order.txt")
    block = np.array(hexbytes(g["head"]) + list(range(128)), np.uint8)
    w = oracle.dequant_q4k(block, 256)
    assert np.array_equal(w, np.array(ints(g["weights"]), np.float32))


def test_q4k_zero_quants_give_minus_dmin_mn():
    rng = np.random.default_rng(3)
    for _ in range(200):
        d = rng.uniform(1e-3, 2e-2, 2).astype(np.float16)
        sc = rng.integers(0, 64, 8)
        mn = rng.integers(0, 64, 8)
        mn[rng.integers(0, 8)] = 0
        blk = oracle.q4k_block(int(d[0].view(np.uint16)), int(d[1].view(np.uint16)), sc, mn,
                               np.zeros(256, int))
        w = oracle.dequant_q4k(blk, 256)
        dmin = np.float32(d[1])
        want = np.repeat(-(dmin * mn.astype(np.float32)), 32)
        want[want == 0] = 0.0  # 0 - 0 is +0 under round-to-nearest
        assert np.array_equal(w.view(np.uint32), want.astype(np.float32).view(np.uint32))


def test_q4k_single_quant_scales_linearly():
    # With dmin = 0 each weight is d*sc_j*q: moving one quant moves one weight only.
    rng = np.random.default_rng(4)
    sc = rng.integers(1, 64, 8)
    mn = np.zeros(8, int)
    for i in rng.choice(256, 24, replace=False):
        q = np.zeros(256, int)
        q[i] = 7
        w = oracle.dequant_q4k(oracle.q4k_block(0x3C00, 0, sc, mn, q), 256)
        nz = np.nonzero(w)[0]
        assert list(nz) == [i] and w[i] == 7 * sc[i // 32]


def test_q4k_fp32_equals_rounded_exact():
    # The products d*sc*q and dmin*mn are exact in fp32, so the fp32 result is the
    # fp64 (here: exact) value rounded once.
    g = synth.rng(99, 0, 0)
    blocks = synth.q4k_weights(64, 256, 99, 0)
    w = oracle.dequant_q4k(blocks, 64 * 256).reshape(64, 256)
    for r in range(64):
        b = blocks[r]
        d = float(b[0:2].view(np.float16)[0])
        dmin = float(b[2:4].view(np.float16)[0])
        sc, mn = oracle.unpack_q4k_scales(b[4:16])
        qs = b[16:]
        for i in g.choice(256, 16, replace=False):
            j, c = i // 32, i // 64
            byte = int(qs[32 * c + i % 32])
            q = byte & 15 if j % 2 == 0 else byte >> 4
            exact = d * sc[j] * q - dmin * mn[j]
            assert w[r, i] == np.float32(exact)


# ---------------------------------------------------------------- IQ3 dequant

def _grid_from(spec: str) -> np.ndarray:
    grid = np.full((256, 4), 2.0, np.float32)
    for item in spec.split():
        k, _, vals = item.partition(":")
        grid[int(k)] = [float(v) for v in vals.split(",")]
    return grid


def _iq3_from(g) -> tuple:
    idx = np.zeros(64, int) if g["idx"] == "zeros" else np.arange(64) % 4
    words = [int(t, 16) for t in g["words"].split()]
    return oracle.iq3_block(idx, words, int(g["d_bits"], 16)), _grid_from(g["grid_rows"])


def test_iq3_hand_block_B():
    g = load("iq3_block_B.txt")
    blk, grid = _iq3_from(g)
    w = oracle.dequant_iq3(blk, grid, 256)
    want = np.concatenate([floats(g["weights_sb0"]), np.tile(floats(g["weights_other"]), 56)])
    assert np.array_equal(w, want.astype(np.float32))


def test_iq3_hand_block_D():
    g = load("iq3_block_D.txt")
    blk, grid = _iq3_from(g)
    w = oracle.dequant_iq3(blk, grid, 256)
    other = floats(g["weights_other"])
    want = np.concatenate([other, floats(g["weights_sb1"])] + [other] * 6)
    assert np.array_equal(w, np.array(want, np.float32))


def test_iq3_parity_exhaustive():
    grid = np.full((256, 4), 2.0, np.float32)
    for l in range(4):
        for seven in range(128):
            words = [0] * 8
            words[3] = seven << (7 * l)
            w = oracle.dequant_iq3(oracle.iq3_block(np.zeros(64), words, 0x3C00), grid, 256)
            neg = (w[96 + 8 * l: 96 + 8 * l + 8] < 0)
            assert neg.sum() % 2 == 0
            assert list(neg[:7]) == [bool((seven >> j) & 1) for j in range(7)]
            assert (w < 0).sum() == neg.sum()
    w = oracle.dequant_iq3(oracle.iq3_block(np.zeros(64), [0x01] + [0] * 7, 0x3C00), grid, 256)
    assert list(np.nonzero(w < 0)[0]) == [0, 7]
    w = oracle.dequant_iq3(oracle.iq3_block(np.zeros(64), [0x7F] + [0] * 7, 0x3C00), grid, 256)
    assert list(np.nonzero(w < 0)[0]) == list(range(8))


def test_iq3_code_sweep():
    grid = np.zeros((256, 4), np.float32)
    grid[0] = [2, 6, 10, 14]
    mags = np.tile([2, 6, 10, 14], 8)
    for first in (0, 8):
        words = [(first + ib) << 28 for ib in range(8)]
        w = oracle.dequant_iq3(oracle.iq3_block(np.zeros(64), words, 0x3C00), grid, 256)
        for ib in range(8):
            s = first + ib
            assert np.array_equal(w[32 * ib:32 * ib + 32], ((0.5 + s) * 0.5 * mags).astype(np.float32))


def test_iq3_fp32_equals_exact():
    # d (11 significant bits) * (2*code+1) (5 bits) * magnitude (5 bits) fits in fp32.
    grid = synth.iq3_grid()
    blocks = synth.iq3_weights(16, 512, 99, 1)
    w = oracle.dequant_iq3(blocks, grid, 16 * 512).reshape(16, 2, 256)
    for r in range(16):
        for sb in range(2):
            b = blocks[r, 98 * sb: 98 * sb + 98]
            d = float(b[96:98].view(np.float16)[0])
            for ib in range(8):
                word = int(b[64 + 4 * ib: 68 + 4 * ib].view("<u4")[0])
                code = word >> 28
                for t in (0, 5, 7, 13, 23, 31):
                    l, j = t // 8, t % 8
                    seven = (word >> (7 * l)) & 0x7F
                    neg = bin(seven).count("1") % 2 if j == 7 else (seven >> j) & 1
                    m = grid[b[8 * ib + t // 4], t % 4]
                    exact = (-1 if neg else 1) * m * d * (0.5 + code) * 0.5
                    assert w[r, sb, 32 * ib + t] == exact


# ---------------------------------------------------------------- IQ3_XXS, llama.cpp byte order
# Pins from the codebook.py page: its format table (98 bytes; eff = d*(0.5+s)*0.5;
# d at bytes 0-1; s in the top four bits of the uint32s at bytes 66-97; the
# decode unit 0.25 = eff at d = 1, s = 0), the even-negatives sign rule of its
# free-code section, and the iq3_pack.py page's statement that its container is
# the same scheme with the grid stored halved.

def _xxs(idx, words, d_bits, grid):
    return oracle.dequant_iq3_xxs(oracle.iq3_xxs_block(idx, words, d_bits), grid, 256)


def test_iq3_xxs_unit_and_scale_table():
    grid = np.zeros((256, 4), np.float32)
    grid[0] = [4, 12, 20, 62]
    mags = np.tile([4, 12, 20, 62], 8).astype(np.float64)
    # d = 1, s = 0: every weight is 0.25 x its codebook value (the page's decode unit)
    w = _xxs(np.zeros(64), [0] * 8, 0x3C00, grid)
    assert np.array_equal(w, np.tile(0.25 * mags, 8).astype(np.float32))
    # s = 0..15 across two blocks: eff = (0.5 + s) * 0.5 per sub-block, d = 2
    for first in (0, 8):
        w = _xxs(np.zeros(64), [(first + ib) << 28 for ib in range(8)], 0x4000, grid)
        for ib in range(8):
            s = first + ib
            assert np.array_equal(w[32 * ib:32 * ib + 32],
                                  (2.0 * (0.5 + s) * 0.5 * mags).astype(np.float32))


def test_iq3_xxs_field_positions():
    grid = np.arange(1024, dtype=np.float32).reshape(256, 4) % 61 + 1
    idx = np.zeros(64, int)
    idx[8 * 5 + 3] = 200        # sub-block 5, weights 12..15
    b = oracle.iq3_xxs_block(idx, [0] * 8, 0x3C00)
    assert b[2 + 8 * 5 + 3] == 200 and b[0] == 0x00 and b[1] == 0x3C
    w = oracle.dequant_iq3_xxs(b, grid, 256)
    assert np.array_equal(w[32 * 5 + 12:32 * 5 + 16], 0.25 * grid[200])
    assert np.array_equal(np.delete(w, np.arange(172, 176)),
                          np.delete(np.tile(0.25 * np.tile(grid[0], 8), 8), np.arange(172, 176)))
    # s of sub-block 6 lives in the top nibble of byte 66 + 4*6 + 3
    b = oracle.iq3_xxs_block(np.zeros(64), [0] * 8, 0x3C00)
    b[66 + 4 * 6 + 3] = 0x30
    w = oracle.dequant_iq3_xxs(b, grid, 256)
    assert np.array_equal(w[192:224], (3.5 * 0.5 * np.tile(grid[0], 8)).astype(np.float32))
    assert np.array_equal(w[:192], np.tile(0.25 * grid[0], 48))
    # d is the fp16 at bytes 0-1: 0x4400 = 4.0
    b[0], b[1] = 0x00, 0x44
    assert np.array_equal(oracle.dequant_iq3_xxs(b, grid, 256), 4.0 * w)


def test_iq3_xxs_signs_even_negatives_exhaustive():
    grid = np.full((256, 4), 4.0, np.float32)
    for l in range(4):
        for seven in range(128):
            words = [0] * 8
            words[2] = seven << (7 * l)
            w = _xxs(np.zeros(64), words, 0x3C00, grid)
            neg = w[64 + 8 * l: 64 + 8 * l + 8] < 0
            assert neg.sum() % 2 == 0
            assert list(neg[:7]) == [bool((seven >> j) & 1) for j in range(7)]
            assert (w < 0).sum() == neg.sum()


def test_iq3_xxs_is_the_iq3_container_with_a_doubled_grid():
    # Same random fields in both orders; the llama.cpp convention's grid is the
    # container's grid doubled, so every weight doubles exactly.
    n_out, n_in = 6, 768
    fmt5 = synth.iq3_weights(n_out, n_in, 91, 3)
    xxs = synth.iq3_xxs_weights(n_out, n_in, 91, 3)
    a = fmt5.reshape(-1, 98)
    b = xxs.reshape(-1, 98)
    assert np.array_equal(b[:, 0:2], a[:, 96:98]) and np.array_equal(b[:, 2:66], a[:, 0:64])
    assert np.array_equal(b[:, 66:98], a[:, 64:96])
    w5 = oracle.dequant_iq3(fmt5, synth.iq3_grid(), n_out * n_in)
    wx = oracle.dequant_iq3_xxs(xxs, synth.iq3_xxs_grid(), n_out * n_in)
    assert np.array_equal(wx, 2 * w5)
    # and with the same grid passed to both, the weights agree exactly
    assert np.array_equal(oracle.dequant_iq3_xxs(xxs, synth.iq3_grid(), n_out * n_in), w5)


def test_iq3_xxs_fp32_equals_exact():
    grid = synth.iq3_xxs_grid()
    blocks = synth.iq3_xxs_weights(8, 512, 99, 2)
    w = oracle.dequant_iq3_xxs(blocks, grid, 8 * 512).reshape(8, 2, 256)
    for r in range(8):
        for sb in range(2):
            b = blocks[r, 98 * sb: 98 * sb + 98]
            d = float(b[0:2].view(np.float16)[0])
            for ib in range(8):
                word = int(b[66 + 4 * ib: 70 + 4 * ib].view("<u4")[0])
                s = word >> 28
                for t in (0, 6, 7, 14, 25, 31):
                    l, j = t // 8, t % 8
                    seven = (word >> (7 * l)) & 0x7F
                    neg = bin(seven).count("1") % 2 if j == 7 else (seven >> j) & 1
                    v = (-1 if neg else 1) * grid[b[2 + 8 * ib + t // 4], t % 4]
                    assert w[r, sb, 32 * ib + t] == v * d * (0.5 + s) * 0.5


def test_gemv_iq3_xxs_matches_numpy_matmul():
    n_out, n_in = 11, 1024
    grid = synth.iq3_xxs_grid()
    w = synth.iq3_xxs_weights(n_out, n_in, 90, 9)
    x = synth.activations(n_in, 90, 9)
    deq = oracle.dequant_iq3_xxs(w, grid, n_out * n_in).reshape(n_out, n_in).astype(np.float64)
    y, s = oracle.gemv_iq3_xxs(w, grid, x, n_in, n_out)
    sref = np.abs(deq) @ np.abs(x.astype(np.float64))
    assert np.allclose(y, deq @ x.astype(np.float64), rtol=0, atol=1e-12 * sref.max())
    assert np.allclose(s, sref, rtol=1e-13)
    rows = np.array([10, 0, 4])
    yr, sr = oracle.gemv_iq3_xxs_rows(w, grid, x, n_in, rows)
    assert np.array_equal(yr, y[rows]) and np.array_equal(sr, s[rows])


# ---------------------------------------------------------------- IQ3_S and IQ4_XS
# Pins from the codebook.py page: its format table (110 and 136 bytes; eff =
# d*(1+2s) and d*(s-32); the Format rows' neutral sub-scale and decode unit:
# IQ3_S s = 0 gives eff = d, IQ4_XS s = 33 gives eff = d), get_s's field
# positions (written here by the test-side builders, which follow set_s and the
# IQ3_S branch of encode), and exactness.

def test_iq3s_iq4xs_block_sizes():
    assert oracle.IQ3S_BYTES == 2 + 64 + 8 + 32 + 4 == 110
    assert oracle.IQ4XS_BYTES == 2 + 2 + 4 + 128 == 136
    assert oracle.IQ3S_BYTES * 8 / 256 == 3.4375 and oracle.IQ4XS_BYTES * 8 / 256 == 4.25


def _iq3s_grid_seq():
    return (np.arange(2048, dtype=np.float32).reshape(512, 4) % 15) + 1


def test_iq3s_unit_scale_sweep_and_signs():
    grid = _iq3s_grid_seq()
    idx = (np.arange(64) * 37) % 512
    want = grid[idx].reshape(256).astype(np.float64)
    # d = 1, s = 0: eff = 1, every weight is its grid value (the page's unit 1.0)
    w = oracle.dequant_iq3s(oracle.iq3s_block(idx, np.zeros(256, bool), [0] * 8, 0x3C00), grid, 256)
    assert np.array_equal(w, want.astype(np.float32))
    # s = 0..15 over two blocks: eff = 1 + 2s per sub-block (d = 0.5)
    for first in (0, 8):
        s = [first + ib for ib in range(8)]
        w = oracle.dequant_iq3s(oracle.iq3s_block(idx, np.zeros(256, bool), s, 0x3800), grid, 256)
        for ib in range(8):
            assert np.array_equal(w[32 * ib:32 * ib + 32],
                                  (0.5 * (1 + 2 * s[ib]) * want[32 * ib:32 * ib + 32]).astype(np.float32))
    # every sign bit negates exactly its own weight
    rng = np.random.default_rng(5)
    neg = rng.random(256) < 0.5
    w = oracle.dequant_iq3s(oracle.iq3s_block(idx, neg, [0] * 8, 0x3C00), grid, 256)
    assert np.array_equal(w, np.where(neg, -want, want).astype(np.float32))


def test_iq3s_ninth_index_bit():
    grid = _iq3s_grid_seq()
    for k in (0, 7, 8, 31, 63):
        idx = np.zeros(64, int)
        idx[k] = 256 + 5
        b = oracle.iq3s_block(idx, np.zeros(256, bool), [0] * 8, 0x3C00)
        assert b[66 + k // 8] == 1 << (k % 8) and b[2 + k] == 5
        w = oracle.dequant_iq3s(b, grid, 256)
        assert np.array_equal(w[4 * k:4 * k + 4], grid[261])
        assert np.array_equal(np.delete(w, np.arange(4 * k, 4 * k + 4)),
                              np.tile(grid[0], 63))


def test_iq3s_random_fields_roundtrip_exact():
    grid = synth.iq3s_grid()
    rng = np.random.default_rng(6)
    for _ in range(20):
        idx = rng.integers(0, 512, 64)
        neg = rng.random(256) < 0.5
        s = rng.integers(0, 16, 8)
        d_bits = int(rng.integers(0x0400, 0x5000))
        d = float(np.array([d_bits], np.uint16).view(np.float16)[0])
        w = oracle.dequant_iq3s(oracle.iq3s_block(idx, neg, s, d_bits), grid, 256)
        for t in range(256):
            v = (-1 if neg[t] else 1) * grid[idx[t // 4], t % 4]
            assert w[t] == v * d * (1 + 2 * s[t // 32])


def test_iq4xs_unit_and_scale_sweep():
    table = synth.iq4nl_table()
    q = (np.arange(256) * 7) % 16
    want = table[q].astype(np.float64)
    # d = 1, s = 33: eff = 1, every weight is its table value (neutral s, unit 1.0)
    w = oracle.dequant_iq4xs(oracle.iq4xs_block(q, [33] * 8, 0x3C00), table, 256)
    assert np.array_equal(w, want.astype(np.float32))
    # s = 0..63 in every sub-block position: eff = s - 32 (d = 2)
    for s0 in range(0, 64, 8):
        s = [(s0 + 5 * ib) % 64 for ib in range(8)]
        w = oracle.dequant_iq4xs(oracle.iq4xs_block(q, s, 0x4000), table, 256)
        for ib in range(8):
            assert np.array_equal(w[32 * ib:32 * ib + 32],
                                  (2.0 * (s[ib] - 32) * want[32 * ib:32 * ib + 32]).astype(np.float32))


def test_iq4xs_scale_and_nibble_positions():
    table = np.arange(16, dtype=np.float32) - 8.0
    # the top two bits of sub-block ib's scale at bits 2ib of bytes 2-3, the low
    # four in nibble ib of bytes 4-7
    for ib in range(8):
        s = [32] * 8
        s[ib] = 32 + 16      # only bit 4 set beyond 32's bit 5
        b = oracle.iq4xs_block(np.full(256, 9), s, 0x3C00)
        hi = int(b[2]) | (int(b[3]) << 8)
        assert (hi >> (2 * ib)) & 3 == 3 and b[4 + ib // 2] >> (4 * (ib % 2)) & 15 == 0
        w = oracle.dequant_iq4xs(b, table, 256)
        assert np.array_equal(w[32 * ib:32 * ib + 32], np.full(32, 16.0, np.float32))
        assert np.array_equal(np.delete(w, np.arange(32 * ib, 32 * ib + 32)), np.zeros(224, np.float32))
    # byte 8 + 16ib + j: weight j in the low nibble, weight j + 16 in the high one
    q = np.zeros(256, int)
    q[32 * 3 + 5] = 1
    q[32 * 3 + 16 + 5] = 2
    b = oracle.iq4xs_block(q, [33] * 8, 0x3C00)
    assert b[8 + 16 * 3 + 5] == 0x21
    w = oracle.dequant_iq4xs(b, table, 256)
    assert w[32 * 3 + 5] == -7.0 and w[32 * 3 + 21] == -6.0
    assert (np.delete(w, [101, 117]) == -8.0).all()


def test_iq4xs_fp32_equals_exact():
    table = synth.iq4nl_table()
    blocks = synth.iq4xs_weights(4, 512, 99, 3)
    w = oracle.dequant_iq4xs(blocks, table, 4 * 512).reshape(4, 2, 256)
    for r in range(4):
        for sb in range(2):
            b = blocks[r, 136 * sb: 136 * sb + 136]
            d = float(b[0:2].view(np.float16)[0])
            hi = int(b[2]) | (int(b[3]) << 8)
            for ib in range(8):
                s = ((b[4 + ib // 2] >> (4 * (ib % 2))) & 15) | (((hi >> (2 * ib)) & 3) << 4)
                for j in (0, 5, 15, 16, 30, 31):
                    byte = b[8 + 16 * ib + j % 16]
                    q = byte & 15 if j < 16 else byte >> 4
                    assert w[r, sb, 32 * ib + j] == table[q] * d * (int(s) - 32)


@pytest.mark.parametrize("fmt", ["iq3s", "iq4xs"])
def test_gemv_codebook_formats_match_numpy_matmul(fmt):
    n_out, n_in = 9, 768
    if fmt == "iq3s":
        tab, w = synth.iq3s_grid(), synth.iq3s_weights(n_out, n_in, 90, 10)
        deq = oracle.dequant_iq3s(w, tab, n_out * n_in)
        y, s = oracle.gemv_iq3s(w, tab, synth.activations(n_in, 90, 10), n_in, n_out)
        yr, sr = oracle.gemv_iq3s_rows(w, tab, synth.activations(n_in, 90, 10), n_in, [8, 0, 3])
    else:
        tab, w = synth.iq4nl_table(), synth.iq4xs_weights(n_out, n_in, 90, 11)
        deq = oracle.dequant_iq4xs(w, tab, n_out * n_in)
        y, s = oracle.gemv_iq4xs(w, tab, synth.activations(n_in, 90, 10), n_in, n_out)
        yr, sr = oracle.gemv_iq4xs_rows(w, tab, synth.activations(n_in, 90, 10), n_in, [8, 0, 3])
    x = synth.activations(n_in, 90, 10).astype(np.float64)
    deq = deq.reshape(n_out, n_in).astype(np.float64)
    sref = np.abs(deq) @ np.abs(x)
    assert np.allclose(y, deq @ x, rtol=0, atol=1e-12 * sref.max())
    assert np.allclose(s, sref, rtol=1e-13)
    assert np.array_equal(yr, y[[8, 0, 3]]) and np.array_equal(sr, s[[8, 0, 3]])


# ---------------------------------------------------------------- IQ3 encoder
# Pins of the iq3_pack.py page's encode(): fp16 rounding against numpy's, the
# stored d against numpy's float32 RMS formula, the parity-fix rule, the
# sub-block search against an fp64 brute force (where no near-tie decides),
# and closed-form special cases.

def test_f32_to_f16_matches_numpy():
    rng = np.random.default_rng(40)
    specials = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e30, -1e30,
                2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -24, 2.0 ** -26, 6.1e-5, 1e-12,
                np.inf, -np.inf, 0.000123, 1024.5, 2049.0, 2051.0, 3.0 * 2.0 ** -25]
    vals = np.concatenate([np.array(specials, np.float32),
                           rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-9, 6, 20000),
                           rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32)])
    vals = vals[~np.isnan(vals)]
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16(v) for v in vals], np.uint16)
    assert np.array_equal(got, want)


def _encode_case(n_rows, n_in, seed, scale=0.02):
    x = (np.random.default_rng(seed).standard_normal((n_rows, n_in)) * scale).astype(np.float32)
    grid = synth.iq3_grid()
    return x, grid, oracle.encode_iq3(x, grid)


def test_encode_d_is_the_rms_anchor():
    x, grid, b = _encode_case(3, 768, 41)
    blocks = b.reshape(-1, 98)
    xs = x.reshape(-1, 256)
    mag = np.abs(xs)
    d = np.sqrt((mag * mag).mean(-1, keepdims=True)) / 20.0 + 1e-12
    assert d.dtype == np.float32
    want = d.astype(np.float16).view(np.uint16)[:, 0]
    got = blocks[:, 96:98].copy().view(np.uint16)[:, 0]
    assert np.array_equal(got, want)


def test_encode_parity_fix():
    x, grid, b = _encode_case(4, 512, 42)
    # decode with an all-ones grid: the output's signs are the stored signs
    ones = np.ones((256, 4), np.float32)
    w = oracle.dequant_iq3(b, ones, x.size).reshape(-1, 8)
    xs = x.reshape(-1, 8)
    for g in range(xs.shape[0]):
        want = xs[g] < 0
        if want.sum() % 2:
            want = want.copy()
            am = int(np.argmin(np.abs(xs[g])))
            want[am] = not want[am]
        got = w[g] < 0
        assert np.array_equal(got, want), g
        assert got.sum() % 2 == 0


def test_encode_search_matches_fp64_brute_force():
    x, grid, b = _encode_case(2, 1024, 43)
    g64 = grid.astype(np.float64)
    blocks = b.reshape(-1, 98)
    xs = np.abs(x.reshape(-1, 256)).astype(np.float64)
    checked = 0
    for k in range(blocks.shape[0]):
        d = float(blocks[k, 96:98].copy().view(np.float16)[0])
        for ib in range(8):
            m = xs[k, 32 * ib:32 * ib + 32].reshape(8, 4)
            errs, idxs = [], []
            for code in range(16):
                db = d * (0.5 + code) * 0.5
                dist = ((g64[None, :, :] * db - m[:, None, :]) ** 2).sum(-1)   # [8 groups, 256]
                idx = dist.argmin(-1)
                idxs.append(idx)
                errs.append(dist[np.arange(8), idx].sum())
            errs = np.array(errs)
            best = int(errs.argmin())
            second = np.partition(errs, 1)[1]
            if second - errs[best] < 1e-4 * errs[best]:
                continue          # a near-tie: fp32 may pick either
            word = int(blocks[k, 64 + 4 * ib:68 + 4 * ib].view("<u4")[0])
            assert word >> 28 == best, (k, ib)
            # the chosen rows: nearest per group unless that group is itself near-tied
            db = d * (0.5 + best) * 0.5
            dist = ((g64[None, :, :] * db - m[:, None, :]) ** 2).sum(-1)
            srt = np.sort(dist, -1)
            for g in range(8):
                if srt[g, 1] - srt[g, 0] > 1e-5 * max(srt[g, 0], 1e-30):
                    assert blocks[k, 8 * ib + g] == idxs[best][g], (k, ib, g)
            checked += 1
    assert checked >= 24


def test_encode_zero_and_exact_grid_cases():
    grid = synth.iq3_grid()
    g2 = (grid.astype(np.float32) ** 2).sum(-1)
    b = oracle.encode_iq3(np.zeros((1, 256), np.float32), grid)[0]
    # d = fp16(1e-12) = 0, every code reconstructs zero: code 0, the first row of least norm
    assert b[96] == 0 and b[97] == 0
    assert (b[:64] == int(np.argmin(g2))).all()
    assert all(int(b[64 + 4 * ib:68 + 4 * ib].view("<u4")[0]) == 0 for ib in range(8))
    # every group an exact grid row: the encoder returns those rows and reconstructs the
    # magnitudes exactly for the code whose db makes them fit
    rows = np.random.default_rng(44).integers(0, 256, 64)
    mag = grid[rows].reshape(256).astype(np.float32)
    d_bits = oracle.f32_to_f16(np.sqrt(np.float32((mag * mag).mean())) / np.float32(20) + np.float32(1e-12))
    d = float(np.array([d_bits], np.uint16).view(np.float16)[0])
    b = oracle.encode_iq3(mag.reshape(1, 256), grid)[0]
    w = oracle.dequant_iq3(b, grid, 256)
    assert int(b[96]) | int(b[97]) << 8 == d_bits
    err = np.abs(w - mag)
    assert (w >= 0).all() and err.max() <= 0.5 * d * 31 * 1.0 + 1e-6


def test_encode_ties_go_to_the_first_row():
    # Duplicate grid rows score identically in any arithmetic: the later copy
    # must never be chosen (the page's argmin keeps the first minimum).
    grid = synth.iq3_grid().copy()
    for a, b in ((3, 200), (17, 18), (0, 255)):
        grid[b] = grid[a]
    x = (np.random.default_rng(46).standard_normal((8, 1024)) * 0.02).astype(np.float32)
    idx = oracle.encode_iq3(x, grid).reshape(-1, 98)[:, :64]
    used = set(np.unique(idx).tolist())
    assert used.isdisjoint({200, 18, 255})
    assert {3, 17, 0} & used


def test_encode_roundtrip_error_and_threads():
    x, grid, b = _encode_case(4, 2048, 45)
    w = oracle.dequant_iq3(b, grid, x.size).reshape(x.shape)
    rel = np.sqrt(((w - x) ** 2).mean()) / np.sqrt((x ** 2).mean())
    assert rel < 0.3
    oracle.set_threads(1)
    try:
        assert np.array_equal(oracle.encode_iq3(x, grid), b)
    finally:
        oracle.set_threads(0)


# ---------------------------------------------------------------- GEMV / GEMM

def _q4k_case(n_out, n_in, seed):
    w = synth.q4k_weights(n_out, n_in, 90, seed)
    x = synth.activations(n_in, 90, seed)
    return w, x


def test_gemv_one_hot_is_a_column():
    n_out, n_in = 5, 512
    w, _ = _q4k_case(n_out, n_in, 1)
    deq = oracle.dequant_q4k(w, n_out * n_in).reshape(n_out, n_in)
    for k in (0, 1, 31, 32, 255, 256, 300, 511):
        x = np.zeros(n_in, np.float32)
        x[k] = 1.0
        y, s = oracle.gemv_q4k(w, x, n_in, n_out)
        assert np.array_equal(y, deq[:, k].astype(np.float64))
        assert np.array_equal(s, np.abs(deq[:, k]).astype(np.float64))


def test_gemv_matches_numpy_matmul():
    n_out, n_in = 37, 1024
    w, x = _q4k_case(n_out, n_in, 2)
    deq = oracle.dequant_q4k(w, n_out * n_in).reshape(n_out, n_in).astype(np.float64)
    y, s = oracle.gemv_q4k(w, x, n_in, n_out)
    ref = deq @ x.astype(np.float64)
    sref = np.abs(deq) @ np.abs(x.astype(np.float64))
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * sref.max())
    assert np.allclose(s, sref, rtol=1e-13)


def test_gemv_structure():
    n_out, n_in = 9, 768
    w, x = _q4k_case(n_out, n_in, 3)
    y, s = oracle.gemv_q4k(w, x, n_in, n_out)
    y2, s2 = oracle.gemv_q4k(w, 2 * x, n_in, n_out)
    assert np.array_equal(y2, 2 * y) and np.array_equal(s2, 2 * s)
    perm = np.random.default_rng(0).permutation(n_out)
    yp, _ = oracle.gemv_q4k(np.ascontiguousarray(w[perm]), x, n_in, n_out)
    assert np.array_equal(yp, y[perm])
    assert (np.abs(y) <= s).all()


def test_gemv_integer_case_exact():
    # d = dmin = 1, sc and mn in 0..7, integer x: every term and partial sum is an
    # integer far below 2^53, so the result is the exact integer sum.
    rng = np.random.default_rng(5)
    n_out, n_in = 3, 512
    rows = []
    ws = []
    for r in range(n_out):
        row = []
        for b in range(n_in // 256):
            sc = rng.integers(0, 8, 8)
            mn = rng.integers(0, 8, 8)
            q = rng.integers(0, 16, 256)
            row.append(oracle.q4k_block(0x3C00, 0x3C00, sc, mn, q))
            ws.append([int(sc[i // 32]) * int(q[i]) - int(mn[i // 32]) for i in range(256)])
        rows.append(np.concatenate(row))
    w = np.stack(rows)
    wint = np.array(ws, dtype=np.int64).reshape(n_out, n_in)
    x = rng.integers(-8, 9, n_in).astype(np.float32)
    y, s = oracle.gemv_q4k(w, x, n_in, n_out)
    exact = wint @ x.astype(np.int64)
    assert np.array_equal(y, exact.astype(np.float64))
    assert np.array_equal(s, (np.abs(wint) @ np.abs(x.astype(np.int64))).astype(np.float64))


def test_gemm_rows_are_gemvs():
    n_out, n_in = 11, 512
    w, _ = _q4k_case(n_out, n_in, 4)
    X = synth.activations(n_in, 90, 5, batch=8)
    Y, S = oracle.gemm_q4k(w, X, n_in, n_out)
    for b in range(8):
        y, s = oracle.gemv_q4k(w, X[b], n_in, n_out)
        assert np.array_equal(Y[b], y) and np.array_equal(S[b], s)
    Y1, _ = oracle.gemm_q4k(w, X[:1], n_in, n_out)
    assert np.array_equal(Y1[0], Y[0])


def test_rows_variant_matches_full():
    n_out, n_in = 20, 512
    w, x = _q4k_case(n_out, n_in, 6)
    y, s = oracle.gemv_q4k(w, x, n_in, n_out)
    rows = np.array([19, 0, 7, 7, 3])
    yr, sr = oracle.gemv_q4k_rows(w, x, n_in, rows)
    assert np.array_equal(yr, y[rows]) and np.array_equal(sr, s[rows])
    grid = synth.iq3_grid()
    wi = synth.iq3_weights(n_out, n_in, 90, 7)
    yi, si = oracle.gemv_iq3(wi, grid, x, n_in, n_out)
    yir, sir = oracle.gemv_iq3_rows(wi, grid, x, n_in, rows)
    assert np.array_equal(yir, yi[rows]) and np.array_equal(sir, si[rows])


def test_gemv_iq3_matches_numpy_matmul():
    n_out, n_in = 13, 768
    grid = synth.iq3_grid()
    w = synth.iq3_weights(n_out, n_in, 90, 8)
    x = synth.activations(n_in, 90, 8)
    deq = oracle.dequant_iq3(w, grid, n_out * n_in).reshape(n_out, n_in).astype(np.float64)
    y, s = oracle.gemv_iq3(w, grid, x, n_in, n_out)
    sref = np.abs(deq) @ np.abs(x.astype(np.float64))
    assert np.allclose(y, deq @ x.astype(np.float64), rtol=0, atol=1e-12 * sref.max())
    assert np.allclose(s, sref, rtol=1e-13)


def test_thread_count_does_not_change_results():
    n_out, n_in = 64, 1024
    w, x = _q4k_case(n_out, n_in, 9)
    old = oracle.get_threads()
    try:
        oracle.set_threads(1)
        y1, _ = oracle.gemv_q4k(w, x, n_in, n_out)
        oracle.set_threads(4)
        y4, _ = oracle.gemv_q4k(w, x, n_in, n_out)
    finally:
        oracle.set_threads(old)
    assert np.array_equal(y1, y4)


def test_size_errors():
    with pytest.raises(ValueError):
        oracle.dequant_q4k(np.zeros(144, np.uint8), 255)
    L = oracle.lib()
    buf = np.zeros(1024, np.float64)
    assert L.orc_gemv_q4k(buf.ctypes.data, buf.ctypes.data, 300, 1, buf.ctypes.data, None) == 2
    assert L.orc_gemm_q4k(buf.ctypes.data, buf.ctypes.data, 256, 1, 9, buf.ctypes.data, None) == 2
    assert L.orc_gemv_q4k(None, buf.ctypes.data, 256, 1, buf.ctypes.data, None) == 1
