"""Seeded synthetic inputs shared by the tests and the benchmark.

This module draws random block fields and lays them out as packed GGUF bytes
(Q8_0: 34 B per 32 weights, Q4_K: 144 B, Q5_K: 176 B and Q6_K: 210 B per 256
weights, Q5_0: 22 B per 32 weights). It holds none of the
method's arithmetic: nothing here dequantises or multiplies. Both the oracle
and the GPU library receive the very same bytes.

Recipe (numpy PCG64, ``default_rng([seed, matrix_id])``; per matrix the draw
order is scales, then quants, then the activation vector):

* Q8_0 (SmolLM-135M / Qwen2.5-0.5B lm_head shapes): per block the scale is
  ``fp16(max|N(0, 0.02)| over 32 draws / 127)``; the maximum of 32 half-normal
  draws is sampled directly by inverting its CDF,
  ``t = 0.02 * sqrt(2) * erfinv(u ** (1/32))``, which has the same
  distribution as drawing the 32 normals. The 32 quants are independent and
  uniform over the integers -127..127.
* Q4_K (Qwen2.5-0.5B and Llama-3-8B shapes): per super-block
  ``d = fp16(U[0.5, 1.5) * 1.2e-4)`` and ``dmin = fp16(U[0.5, 1.5) * 9.2e-4)``
  (a sub-block range of about 2 * 0.058 mapped onto 15 * 63 steps, and 0.058
  onto 63 steps); the other 140 bytes are uniform random, i.e. every 6-bit
  scale / min code is uniform on 0..63 and every 4-bit code on 0..15.
* Q5_0: per block ``d = fp16(max|N(0, 0.02)| over 32 draws / 16)`` (drawn
  as for Q8_0), then 20 uniform random bytes (every 5-bit code uniform on
  0..31).
* Q5_K: per super-block ``d = fp16(U[0.5, 1.5) * 5.9e-5)`` (2 * 0.058 onto
  31 * 63 steps) and ``dmin = fp16(U[0.5, 1.5) * 9.2e-4)``, then 172 uniform
  random bytes (scale / min codes, high bits and nibbles).
* Q6_K: per super-block 208 uniform random bytes (nibbles, high bit pairs
  and sixteen int8 scales uniform on -128..127), then
  ``d = fp16(U[0.5, 1.5) * 1.4e-5)`` (0.058 onto 32 * 127 steps; like the
  scales of real Q6_K tensors this lies in fp16's subnormal range).
* Activations: ``standard_normal`` in float64, rounded to float32.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erfinv

FMT_Q8_0 = 8
FMT_Q4_K = 12
FMT_Q5_0 = 6
FMT_Q5_K = 13
FMT_Q6_K = 14

_QK = {FMT_Q8_0: 32, FMT_Q4_K: 256, FMT_Q5_0: 32, FMT_Q5_K: 256, FMT_Q6_K: 256}
_BLOCK_BYTES = {FMT_Q8_0: 34, FMT_Q4_K: 144, FMT_Q5_0: 22, FMT_Q5_K: 176,
                FMT_Q6_K: 210}


def blocks_per_row(fmt: int, cols: int) -> int:
    return -(-cols // _QK[fmt])


def packed_row_bytes(fmt: int, cols: int) -> int:
    return blocks_per_row(fmt, cols) * _BLOCK_BYTES[fmt]


def rng_for(seed: int, matrix_id: int) -> np.random.Generator:
    return np.random.default_rng([seed, matrix_id])


def _fp16_bits(values: np.ndarray) -> np.ndarray:
    return np.asarray(values, dtype=np.float64).astype(np.float16).view(np.uint16)


def q8_0_weights(rows: int, cols: int, rng: np.random.Generator) -> np.ndarray:
    """Packed Q8_0 bytes for a rows x cols matrix (flat uint8 array)."""
    nb = blocks_per_row(FMT_Q8_0, cols)
    nblk = rows * nb
    u = rng.random(nblk)
    amax = 0.02 * np.sqrt(2.0) * erfinv(u ** (1.0 / 32.0))
    d16 = _fp16_bits(amax / 127.0)
    q = rng.integers(-127, 128, size=(nblk, 32), dtype=np.int16).astype(np.int8)
    blk = np.empty((nblk, 34), np.uint8)
    blk[:, 0] = (d16 & 0xFF).astype(np.uint8)
    blk[:, 1] = (d16 >> 8).astype(np.uint8)
    blk[:, 2:] = q.view(np.uint8)
    return blk.reshape(-1)


def q4_k_weights(rows: int, cols: int, rng: np.random.Generator,
                 chunk_blocks: int = 1 << 22) -> np.ndarray:
    """Packed Q4_K bytes for a rows x cols matrix (flat uint8 array)."""
    nb = blocks_per_row(FMT_Q4_K, cols)
    nblk = rows * nb
    d16 = _fp16_bits(rng.uniform(0.5, 1.5, nblk) * 1.2e-4)
    dmin16 = _fp16_bits(rng.uniform(0.5, 1.5, nblk) * 9.2e-4)
    out = np.empty((nblk, 144), np.uint8)
    out[:, 0] = (d16 & 0xFF).astype(np.uint8)
    out[:, 1] = (d16 >> 8).astype(np.uint8)
    out[:, 2] = (dmin16 & 0xFF).astype(np.uint8)
    out[:, 3] = (dmin16 >> 8).astype(np.uint8)
    for b0 in range(0, nblk, chunk_blocks):
        b1 = min(nblk, b0 + chunk_blocks)
        out[b0:b1, 4:] = rng.integers(0, 256, size=(b1 - b0, 140), dtype=np.uint8)
    return out.reshape(-1)


def _random_fill(out: np.ndarray, c0: int, c1: int, rng: np.random.Generator,
                 chunk_blocks: int = 1 << 22) -> None:
    """Uniform random bytes into columns c0..c1-1 of a [blocks, bytes] array,
    drawn in chunks of blocks so that no huge temporary is made."""
    nblk = out.shape[0]
    for b0 in range(0, nblk, chunk_blocks):
        b1 = min(nblk, b0 + chunk_blocks)
        out[b0:b1, c0:c1] = rng.integers(0, 256, size=(b1 - b0, c1 - c0), dtype=np.uint8)


def _put_f16(out: np.ndarray, col: int, bits: np.ndarray) -> None:
    out[:, col] = (bits & 0xFF).astype(np.uint8)
    out[:, col + 1] = (bits >> 8).astype(np.uint8)


def q5_0_weights(rows: int, cols: int, rng: np.random.Generator) -> np.ndarray:
    """Packed Q5_0 bytes for a rows x cols matrix (flat uint8 array)."""
    nblk = rows * blocks_per_row(FMT_Q5_0, cols)
    u = rng.random(nblk)
    amax = 0.02 * np.sqrt(2.0) * erfinv(u ** (1.0 / 32.0))
    out = np.empty((nblk, 22), np.uint8)
    _put_f16(out, 0, _fp16_bits(amax / 16.0))
    _random_fill(out, 2, 22, rng)
    return out.reshape(-1)


def q5_k_weights(rows: int, cols: int, rng: np.random.Generator) -> np.ndarray:
    """Packed Q5_K bytes for a rows x cols matrix (flat uint8 array)."""
    nblk = rows * blocks_per_row(FMT_Q5_K, cols)
    d16 = _fp16_bits(rng.uniform(0.5, 1.5, nblk) * 5.9e-5)
    dmin16 = _fp16_bits(rng.uniform(0.5, 1.5, nblk) * 9.2e-4)
    out = np.empty((nblk, 176), np.uint8)
    _put_f16(out, 0, d16)
    _put_f16(out, 2, dmin16)
    _random_fill(out, 4, 176, rng)
    return out.reshape(-1)


def q6_k_weights(rows: int, cols: int, rng: np.random.Generator) -> np.ndarray:
    """Packed Q6_K bytes for a rows x cols matrix (flat uint8 array)."""
    nblk = rows * blocks_per_row(FMT_Q6_K, cols)
    out = np.empty((nblk, 210), np.uint8)
    _random_fill(out, 0, 208, rng)
    _put_f16(out, 208, _fp16_bits(rng.uniform(0.5, 1.5, nblk) * 1.4e-5))
    return out.reshape(-1)


def weights(fmt: int, rows: int, cols: int, rng: np.random.Generator) -> np.ndarray:
    if fmt == FMT_Q8_0:
        return q8_0_weights(rows, cols, rng)
    if fmt == FMT_Q4_K:
        return q4_k_weights(rows, cols, rng)
    if fmt == FMT_Q5_0:
        return q5_0_weights(rows, cols, rng)
    if fmt == FMT_Q5_K:
        return q5_k_weights(rows, cols, rng)
    if fmt == FMT_Q6_K:
        return q6_k_weights(rows, cols, rng)
    raise ValueError(f"unknown format {fmt}")


def activations(shape, rng: np.random.Generator) -> np.ndarray:
    return rng.standard_normal(shape).astype(np.float32)


def matrix_and_x(fmt: int, rows: int, cols: int, seed: int, matrix_id: int,
                 M: int | None = None):
    """(W bytes, x) for one matrix; x is [cols] or [M, cols]."""
    rng = rng_for(seed, matrix_id)
    W = weights(fmt, rows, cols, rng)
    x = activations(cols if M is None else (M, cols), rng)
    return W, x


# --------------------------------------------------------------- workloads
# Shapes are (rows = output features, cols = input features).

SMOLLM_FFN_UP = (FMT_Q8_0, 1536, 576)
QWEN05_DECODE = [(FMT_Q4_K, 896, 896), (FMT_Q4_K, 128, 896),
                 (FMT_Q4_K, 4864, 896), (FMT_Q4_K, 896, 4864)]
QWEN05_LM_HEAD = (FMT_Q8_0, 151936, 896)
LLAMA3_8B_LAYER = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096),
                   ("o", 4096, 4096), ("gate", 14336, 4096), ("up", 14336, 4096),
                   ("down", 4096, 14336)]
LLAMA3_8B_LAYERS = 32
PREFILL_M = (16, 64, 512)

# Shapes of the other formats that Q4_K_M / Q5_K_M files mix in: the
# Llama-3-8B lm_head and some ffn_down tensors are Q6_K, Qwen2.5-0.5B's
# 896-wide tensors (not a multiple of 256 columns) use Q5_0, and Q5_K_M
# files store the Llama-3-8B projections as Q5_K. Seed 5, matrix_id = index.
MIXED_FORMATS = [
    ("llama3_8b_lm_head_q6_k", FMT_Q6_K, 128256, 4096),
    ("llama3_8b_down_q6_k", FMT_Q6_K, 4096, 14336),
    ("llama3_8b_q_q5_k", FMT_Q5_K, 4096, 4096),
    ("llama3_8b_gate_q5_k", FMT_Q5_K, 14336, 4096),
    ("llama3_8b_down_q5_k", FMT_Q5_K, 4096, 14336),
    ("qwen05b_896x896_q5_0", FMT_Q5_0, 896, 896),
    ("qwen05b_128x896_q5_0", FMT_Q5_0, 128, 896),
    ("qwen05b_4864x896_q5_0", FMT_Q5_0, 4864, 896),
]

WORKLOADS = {
    "smollm135m_ffn_up_q8_0": dict(seed=0, shapes=[SMOLLM_FFN_UP]),
    "qwen05b_decode_q4_k": dict(seed=1, shapes=QWEN05_DECODE),
    "qwen05b_lm_head_q8_0": dict(seed=2, shapes=[QWEN05_LM_HEAD]),
    "llama3_8b_decode_step_q4_k": dict(seed=3),
    "llama3_8b_prefill_q4_k": dict(seed=4),
    "mixed_formats": dict(seed=5, shapes=[(f, r, c) for _, f, r, c in MIXED_FORMATS]),
}


def mixed_format_weight_and_x(i: int):
    """(name, fmt, rows, cols, W bytes, x) of MIXED_FORMATS[i]."""
    name, fmt, rows, cols = MIXED_FORMATS[i]
    W, x = matrix_and_x(fmt, rows, cols, 5, i)
    return name, fmt, rows, cols, W, x


def llama3_8b_matrix(layer: int, proj: int):
    """(name, rows, cols, seed, matrix_id) of one Llama-3-8B-shaped matrix."""
    name, rows, cols = LLAMA3_8B_LAYER[proj]
    return name, rows, cols, 3, 7 * layer + proj


def llama3_8b_weight_and_x(layer: int, proj: int):
    name, rows, cols, seed, mid = llama3_8b_matrix(layer, proj)
    return matrix_and_x(FMT_Q4_K, rows, cols, seed, mid)


def prefill_inputs(which: str, M: int):
    """Layer-0 gate (4096 -> 14336) or down (14336 -> 4096) Q4_K weights of
    the Llama-3-8B-shaped stack, and X [M, cols] ~ N(0,1) with seed 4."""
    proj = {"gate": 4, "down": 6}[which]
    name, rows, cols, seed, mid = llama3_8b_matrix(0, proj)
    W = weights(FMT_Q4_K, rows, cols, rng_for(seed, mid))
    X = activations((M, cols), rng_for(4, 1000 * proj + M))
    return W, X, rows, cols
