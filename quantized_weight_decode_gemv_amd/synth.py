"""Seeded synthetic inputs for the quantized GEMV workloads.

This module only draws random bytes and vectors in the shapes of the formats; it
holds none of the codec arithmetic (no unpacking, no dequantization, no dot
products), so both the HIP path's tests and the CPU oracle can take their inputs
from it without sharing any of the method.

Recipe (every tensor gets its own generator ``default_rng([2026, cfg, tensor,
role])``, role 0 = weight fields, 1 = activations, 2 = IQ3 grid):

* Q4_K blocks (144 B): d and dmin are fp16 draws from U[1e-3, 2e-2] rounded to
  nearest fp16; bytes 4..143 are uniform random bytes. The 12 scale bytes encode
  sixteen 6-bit fields through a bijection and the 128 quant bytes hold 256
  nibbles, so uniform bytes are the same as uniform 6-bit scales/mins and uniform
  4-bit quants.
* IQ3 blocks (98 B): 64 uniform index bytes, 8 uniform uint32 words (every 7-bit
  sign pattern is valid and the 4-bit code is uniform), fp16 d as above.
* IQ3 grid: 256 distinct 4-tuples over the eight magnitudes
  {2, 6, 10, 14, 18, 22, 26, 31} (the published grid is absent; this is a
  stand-in with the same value range), fp32 [256, 4].
* IQ3_XXS blocks in llama.cpp's byte order: the same draws as the IQ3 blocks of
  the same (cfg, tensor), placed as d (bytes 0-1), indices (2-65), words
  (66-97); their grid is the IQ3 grid doubled (integer entries 4..62, the
  convention of llama.cpp's own table).
* IQ3_S blocks (110 B): fp16 d as above, bytes 2..109 uniform (every index,
  sign pattern and 4-bit sub-scale is valid). Grid: 512 distinct 4-tuples over
  the eight odd magnitudes 1..15 (the published table is absent).
* IQ4_XS blocks (136 B): fp16 d as above, bytes 2..135 uniform (uniform 6-bit
  sub-scales and 4-bit codes). Table: 16 distinct integers in [-127, 127],
  ascending (the published table is absent).
* Q4_K blocks of a chained stream (a product's output is the next one's
  input, ``q4k_chain_weights``): as above, but d and dmin are fp16 draws of
  random sign and magnitude U[0.5, 1.5] / (336.7 sqrt(n_out)): zero-mean
  weights whose products keep the norm of their input, so that 89 chained
  products stay inside the fp32 range (a decoder's norms do this in the model).
* Activations: fp32 standard normal.

The published TinyLlama-1.1B Q4_K_M weights and real IQ3 tensors are absent; the
kernels do data-independent work, so these stand in for them at the same shapes.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

QK = 256
Q4K_BYTES = 144
IQ3_BYTES = 98
IQ3_LEVELS = (2, 6, 10, 14, 18, 22, 26, 31)
IQ3S_BYTES = 110
IQ4XS_BYTES = 136
IQ3S_LEVELS = (1, 3, 5, 7, 9, 11, 13, 15)

ROLE_W, ROLE_X, ROLE_GRID = 0, 1, 2


def rng(cfg: int, tensor: int, role: int) -> np.random.Generator:
    return np.random.default_rng([2026, cfg, tensor, role])


def _fp16_uniform(g: np.random.Generator, n: int) -> np.ndarray:
    return g.uniform(1e-3, 2e-2, n).astype(np.float16)


def q4k_weights(n_out: int, n_in: int, cfg: int, tensor: int) -> np.ndarray:
    """uint8 [n_out, n_in/256*144]."""
    if n_in % QK:
        raise ValueError("n_in must be a multiple of 256")
    nb = n_out * (n_in // QK)
    g = rng(cfg, tensor, ROLE_W)
    d = _fp16_uniform(g, nb)
    dmin = _fp16_uniform(g, nb)
    blocks = np.empty((nb, Q4K_BYTES), np.uint8)
    blocks[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    blocks[:, 2:4] = dmin.view(np.uint8).reshape(nb, 2)
    blocks[:, 4:] = g.integers(0, 256, (nb, Q4K_BYTES - 4), dtype=np.uint8)
    return blocks.reshape(n_out, -1)


# Mean square of a Q4_K weight per unit of d^2 when d and dmin have the same
# magnitude distribution (U[0.5, 1.5] x scale, independent random signs) and the
# 6-bit scales/mins and 4-bit quants are uniform: E[a^2] (E[sc^2] E[q^2] +
# E[mn^2]) = (13/12) * 1333.5 * 78.5 = 113,370 (sqrt 336.7).
CHAIN_W_RMS_PER_SCALE = 336.7


def q4k_chain_weights(n_out: int, n_in: int, cfg: int, tensor: int) -> np.ndarray:
    """Q4_K blocks for a product whose output is the next product's input: as
    q4k_weights, but d and dmin are fp16 draws of random sign and magnitude
    U[0.5, 1.5] / (336.7 sqrt(n_out)), so that the weights have zero mean and
    a product's output has about the norm of its input (a chain of many such
    products stays inside the fp32 range, as a decoder's normalized layers
    do). uint8 [n_out, n_in/256*144]."""
    if n_in % QK:
        raise ValueError("n_in must be a multiple of 256")
    nb = n_out * (n_in // QK)
    g = rng(cfg, tensor, ROLE_W)
    scale = 1.0 / (CHAIN_W_RMS_PER_SCALE * np.sqrt(n_out))
    d = (g.choice([-1.0, 1.0], nb) * g.uniform(0.5, 1.5, nb) * scale).astype(np.float16)
    dmin = (g.choice([-1.0, 1.0], nb) * g.uniform(0.5, 1.5, nb) * scale).astype(np.float16)
    blocks = np.empty((nb, Q4K_BYTES), np.uint8)
    blocks[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    blocks[:, 2:4] = dmin.view(np.uint8).reshape(nb, 2)
    blocks[:, 4:] = g.integers(0, 256, (nb, Q4K_BYTES - 4), dtype=np.uint8)
    return blocks.reshape(n_out, -1)


def iq3_weights(n_out: int, n_in: int, cfg: int, tensor: int) -> np.ndarray:
    """uint8 [n_out, n_in/256*98]."""
    if n_in % QK:
        raise ValueError("n_in must be a multiple of 256")
    nb = n_out * (n_in // QK)
    g = rng(cfg, tensor, ROLE_W)
    d = _fp16_uniform(g, nb)
    blocks = np.empty((nb, IQ3_BYTES), np.uint8)
    blocks[:, 0:64] = g.integers(0, 256, (nb, 64), dtype=np.uint8)
    words = g.integers(0, 2 ** 32, (nb, 8), dtype=np.uint32).astype("<u4")
    blocks[:, 64:96] = words.view(np.uint8).reshape(nb, 32)
    blocks[:, 96:98] = d.view(np.uint8).reshape(nb, 2)
    return blocks.reshape(n_out, -1)


def iq3_xxs_weights(n_out: int, n_in: int, cfg: int, tensor: int) -> np.ndarray:
    """uint8 [n_out, n_in/256*98], llama.cpp byte order; the bytes of
    iq3_weights(n_out, n_in, cfg, tensor), block by block, in that order."""
    src = iq3_weights(n_out, n_in, cfg, tensor).reshape(-1, IQ3_BYTES)
    blocks = np.empty_like(src)
    blocks[:, 0:2] = src[:, 96:98]
    blocks[:, 2:66] = src[:, 0:64]
    blocks[:, 66:98] = src[:, 64:96]
    return blocks.reshape(n_out, -1)


def iq3_xxs_grid(cfg: int = 4, tensor: int = 0) -> np.ndarray:
    """fp32 [256, 4]: iq3_grid doubled (entries in {4, 12, ..., 62})."""
    return iq3_grid(cfg, tensor) * np.float32(2)


def _d_then_uniform(n_out: int, n_in: int, cfg: int, tensor: int, nbytes: int) -> np.ndarray:
    if n_in % QK:
        raise ValueError("n_in must be a multiple of 256")
    nb = n_out * (n_in // QK)
    g = rng(cfg, tensor, ROLE_W)
    d = _fp16_uniform(g, nb)
    blocks = np.empty((nb, nbytes), np.uint8)
    blocks[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    blocks[:, 2:] = g.integers(0, 256, (nb, nbytes - 2), dtype=np.uint8)
    return blocks.reshape(n_out, -1)


def iq3s_weights(n_out: int, n_in: int, cfg: int, tensor: int) -> np.ndarray:
    """uint8 [n_out, n_in/256*110] IQ3_S blocks."""
    return _d_then_uniform(n_out, n_in, cfg, tensor, IQ3S_BYTES)


def iq4xs_weights(n_out: int, n_in: int, cfg: int, tensor: int) -> np.ndarray:
    """uint8 [n_out, n_in/256*136] IQ4_XS blocks."""
    return _d_then_uniform(n_out, n_in, cfg, tensor, IQ4XS_BYTES)


def iq3s_grid(cfg: int = 4, tensor: int = 0) -> np.ndarray:
    """fp32 [512, 4]: 512 distinct base-8 4-digit tuples mapped onto IQ3S_LEVELS."""
    g = rng(cfg, tensor, ROLE_GRID)
    pick = g.choice(4096, 512, replace=False)
    digits = np.stack([(pick >> (3 * i)) & 7 for i in range(4)], axis=1)
    return np.asarray(IQ3S_LEVELS, np.float32)[digits]


def iq4nl_table(cfg: int = 4, tensor: int = 0) -> np.ndarray:
    """fp32 [16]: 16 distinct integers in [-127, 127], ascending."""
    g = rng(cfg, tensor, ROLE_GRID)
    return np.sort(g.choice(255, 16, replace=False) - 127).astype(np.float32)


def iq3_grid(cfg: int = 4, tensor: int = 0) -> np.ndarray:
    """fp32 [256, 4]: 256 distinct base-8 4-digit tuples mapped onto IQ3_LEVELS."""
    g = rng(cfg, tensor, ROLE_GRID)
    pick = g.choice(4096, 256, replace=False)
    digits = np.stack([(pick >> (3 * i)) & 7 for i in range(4)], axis=1)
    return np.asarray(IQ3_LEVELS, np.float32)[digits]


def activations(n: int, cfg: int, tensor: int, batch: int | None = None) -> np.ndarray:
    """fp32 [n] (or [batch, n]) standard normal."""
    g = rng(cfg, tensor, ROLE_X)
    shape = (n,) if batch is None else (batch, n)
    return g.standard_normal(shape).astype(np.float32)


# ---------------------------------------------------------------- workload table

@dataclass(frozen=True)
class Problem:
    name: str
    fmt: str        # "q4k" or "iq3"
    n_out: int
    n_in: int
    batch: int      # 1 for GEMV
    cfg: int
    tensor: int

    @property
    def row_bytes(self) -> int:
        return (self.n_in // QK) * (Q4K_BYTES if self.fmt == "q4k" else IQ3_BYTES)

    @property
    def weight_bytes(self) -> int:
        return self.n_out * self.row_bytes

    @property
    def algorithmic_bytes(self) -> int:
        """Weights read once, activations read once, outputs written once (fp32)."""
        return self.weight_bytes + 4 * self.batch * (self.n_in + self.n_out)


DIM, KV, FF, VOCAB, LAYERS = 2048, 256, 5632, 32000, 22
PROJ = (("q", DIM, DIM), ("k", KV, DIM), ("v", KV, DIM), ("o", DIM, DIM),
        ("gate", FF, DIM), ("up", FF, DIM), ("down", DIM, FF))


def config(cfg: int) -> list[Problem]:
    """The five workloads: 1 = Q4_K 2048x2048; 2 = one TinyLlama-1.1B layer's
    seven projections; 3 = LM head 2048->32000 as GEMV and as B=8 GEMM; 4 = IQ3
    5632x2048 and 2048x5632; 5 = the full per-token stream (22 layers x 7
    projections + LM head). Two more at the same shapes in IQ3: 6 = the
    per-token stream, 7 = one layer's seven projections."""
    if cfg == 1:
        return [Problem("q4k_2048x2048", "q4k", DIM, DIM, 1, 1, 0)]
    if cfg == 2:
        return [Problem(n, "q4k", o, i, 1, 2, t) for t, (n, o, i) in enumerate(PROJ)]
    if cfg == 3:
        return [Problem("lm_head", "q4k", VOCAB, DIM, 1, 3, 0),
                Problem("lm_head_b8", "q4k", VOCAB, DIM, 8, 3, 1)]
    if cfg == 4:
        return [Problem("iq3_5632x2048", "iq3", FF, DIM, 1, 4, 0),
                Problem("iq3_2048x5632", "iq3", DIM, FF, 1, 4, 1)]
    if cfg == 5:
        out = []
        for layer in range(LAYERS):
            for p, (n, o, i) in enumerate(PROJ):
                out.append(Problem(f"L{layer}.{n}", "q4k", o, i, 1, 5, 7 * layer + p))
        out.append(Problem("lm_head", "q4k", VOCAB, DIM, 1, 5, 7 * LAYERS))
        return out
    if cfg == 6:
        out = []
        for layer in range(LAYERS):
            for p, (n, o, i) in enumerate(PROJ):
                out.append(Problem(f"L{layer}.{n}", "iq3", o, i, 1, 6, 7 * layer + p))
        out.append(Problem("lm_head", "iq3", VOCAB, DIM, 1, 6, 7 * LAYERS))
        return out
    if cfg == 7:
        return [Problem(n, "iq3", o, i, 1, 7, t) for t, (n, o, i) in enumerate(PROJ)]
    raise ValueError(cfg)


def chain_sources(probs: list[Problem]) -> list[int]:
    """For a per-token stream (config 5 or 6 order: per layer q, k, v, o, gate,
    up, down, then the LM head), the index of the product whose output stands
    in for each product's input in a decode step, or -1 for the step's own
    input (one vector): q, k and v read the previous layer's down (layer 0:
    the step's input), o reads q (standing in for
    the attention output), gate and up read o (the normalized residual), down
    reads gate (the SwiGLU activation), the LM head reads the last down. The
    operations between the products are not part of this workload."""
    src, last_down, mine = [], -1, {}
    for i, p in enumerate(probs):
        name = p.name.split(".")[-1]
        if name in ("q", "k", "v"):
            if name == "q":
                mine = {"q": i}
            src.append(last_down)
        elif name == "o":
            src.append(mine["q"])
            mine["o"] = i
        elif name in ("gate", "up"):
            src.append(mine["o"])
            if name == "gate":
                mine["gate"] = i
        elif name == "down":
            src.append(mine["gate"])
            last_down = i
        else:
            src.append(last_down)
    return src


def weights(p: Problem) -> np.ndarray:
    # B=8 LM head reuses the LM-head weights of its config (tensor 0).
    tensor = 0 if (p.cfg == 3 and p.batch > 1) else p.tensor
    if p.fmt == "q4k":
        return q4k_weights(p.n_out, p.n_in, p.cfg, tensor)
    return iq3_weights(p.n_out, p.n_in, p.cfg, tensor)


def inputs(p: Problem) -> np.ndarray:
    return activations(p.n_in, p.cfg, p.tensor, None if p.batch == 1 else p.batch)
