"""Seeded synthetic inputs for the block-quantized MUL_MAT workloads.

This module only draws random numbers and lays them out in GGUF block order
(binary16 scale first, then the code bytes). It performs none of the
method's arithmetic: nothing here decodes a scale, applies a zero point or
multiplies anything. Both the HIP path's tests/benchmark and the CPU oracle
are fed from here, and from nowhere else.

Workload shapes follow the Llama-7B projections a ggml model creates
([Bind] = "llama.cpp 源码分析：GGUF 权重与计算图的绑定", section 3.2: attn_q/k/v/o
are {n_embd, n_embd}, ffn_gate/ffn_up are {n_embd, n_ff}, ffn_down is
{n_ff, n_embd}, with ne0 = k the contiguous dimension and ne1 = rows).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TYPE_Q4_0 = 2
TYPE_Q4_1 = 3
TYPE_Q5_0 = 6
TYPE_Q5_1 = 7
TYPE_Q8_0 = 8
TYPE_Q4_K = 12
QK = 32
QK_K = 256
BLOCK_BYTES = {TYPE_Q4_0: 18, TYPE_Q4_1: 20, TYPE_Q5_0: 22, TYPE_Q5_1: 24, TYPE_Q8_0: 34, TYPE_Q4_K: 144}
BLOCK_WEIGHTS = {TYPE_Q4_0: QK, TYPE_Q4_1: QK, TYPE_Q5_0: QK, TYPE_Q5_1: QK, TYPE_Q8_0: QK, TYPE_Q4_K: QK_K}
TYPE_NAMES = {TYPE_Q4_0: "q4_0", TYPE_Q4_1: "q4_1", TYPE_Q5_0: "q5_0", TYPE_Q5_1: "q5_1", TYPE_Q8_0: "q8_0",
              TYPE_Q4_K: "q4_k"}

N_EMBD = 4096
N_FF = 11008
N_LAYER = 32
N_VOCAB = 32000

# (name, rows, k) of one Llama-7B-shaped layer, in the order the layer uses them.
LAYER_TENSORS = (
    ("attn_q", N_EMBD, N_EMBD),
    ("attn_k", N_EMBD, N_EMBD),
    ("attn_v", N_EMBD, N_EMBD),
    ("attn_output", N_EMBD, N_EMBD),
    ("ffn_gate", N_FF, N_EMBD),
    ("ffn_up", N_FF, N_EMBD),
    ("ffn_down", N_EMBD, N_FF),
)

WHAT_WEIGHTS = 0
WHAT_ACTIVATIONS = 1


def rng_for(config: int, layer: int, tensor: int, what: int) -> np.random.Generator:
    """Independent PCG64 stream per (workload, layer, tensor, weights/activations)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config, layer, tensor, what])))


def dense_row_bytes(qtype: int, k: int) -> int:
    return (k // BLOCK_WEIGHTS[qtype]) * BLOCK_BYTES[qtype]


def assemble_rows(d_bits: np.ndarray, code_bytes: np.ndarray, nb1: int,
                  pad_bytes: np.ndarray | None = None) -> np.ndarray:
    """Place per-block scale bits (uint16 [rows, nblk]) and code bytes
    (uint8 [rows, nblk, payload]) into rows of stride nb1 bytes; the bytes
    after the blocks are filled from pad_bytes (zeros if None)."""
    d_bits = np.ascontiguousarray(d_bits, dtype=np.uint16)
    rows, nblk = d_bits.shape
    payload = code_bytes.shape[2]
    bpb = 2 + payload
    dense = nblk * bpb
    if nb1 < dense:
        raise ValueError("nb1 smaller than the dense row")
    W = np.empty((rows, nb1), dtype=np.uint8)
    blk = W[:, :dense].reshape(rows, nblk, bpb)
    blk[:, :, 0:2] = d_bits.view(np.uint8).reshape(rows, nblk, 2)  # little-endian
    blk[:, :, 2:] = code_bytes
    if nb1 > dense:
        W[:, dense:] = 0 if pad_bytes is None else pad_bytes
    return W


def make_weights(qtype: int, rows: int, k: int, nb1: int | None, rng: np.random.Generator,
                 d_lo: float = 0.001, d_hi: float = 0.05) -> np.ndarray:
    """Random quantised rows: d = fp16(U[d_lo, d_hi]) (round to nearest even);
    Q4_0 code bytes uniform 0..255 (both nibbles uniform 0..15); Q4_1 the
    same code bytes after a minimum m = fp16(-U[6, 9] * |d draw|) (blocks spanning
    about [-7.5 d, 7.5 d], as a min/max quantiser makes them); Q5_0 four
    random bytes of fifth bits then the code bytes; Q5_1 a minimum
    fp16(-U[12, 18] * |d draw|), then the same as Q5_0; Q8_0 codes uniform
    integers in [-127, 127]; Q4_K (256-weight super-blocks) d and dmin =
    fp16(U[d_lo, d_hi] / 25), then 12 uniform random scale bytes (so every
    6-bit sub-block scale and minimum value occurs) and 128 uniform random
    code bytes; padding bytes uniform 0..255."""
    if qtype == TYPE_Q4_K:
        if k % QK_K:
            raise ValueError("k must be a multiple of 256")
        nsb = k // QK_K
        dense = dense_row_bytes(qtype, k)
        nb1 = dense if nb1 is None else nb1
        dd = rng.uniform(d_lo / 25, d_hi / 25, size=(rows, nsb, 2)).astype(np.float16).view(np.uint8)
        W = np.empty((rows, nb1), dtype=np.uint8)
        blk = W[:, :dense].reshape(rows, nsb, 144)
        blk[:, :, 0:4] = dd.reshape(rows, nsb, 4)  # d then dmin, little-endian
        blk[:, :, 4:] = rng.integers(0, 256, size=(rows, nsb, 140), dtype=np.uint8)
        if nb1 > dense:
            W[:, dense:] = rng.integers(0, 256, size=(rows, nb1 - dense), dtype=np.uint8)
        return W
    if k % QK:
        raise ValueError("k must be a multiple of 32")
    nblk = k // QK
    dense = dense_row_bytes(qtype, k)
    nb1 = dense if nb1 is None else nb1
    d_draw = rng.uniform(d_lo, d_hi, size=(rows, nblk))
    d_bits = d_draw.astype(np.float16).view(np.uint16)
    if qtype == TYPE_Q4_0:
        codes = rng.integers(0, 256, size=(rows, nblk, 16), dtype=np.uint8)
    elif qtype == TYPE_Q4_1:
        m_bits = (-rng.uniform(6.0, 9.0, size=(rows, nblk)) * np.abs(d_draw)).astype(np.float16).view(np.uint16)
        codes = np.empty((rows, nblk, 18), dtype=np.uint8)
        codes[:, :, 0:2] = m_bits.view(np.uint8).reshape(rows, nblk, 2)  # little-endian
        codes[:, :, 2:] = rng.integers(0, 256, size=(rows, nblk, 16), dtype=np.uint8)
    elif qtype in (TYPE_Q5_0, TYPE_Q5_1):
        lead = 2 if qtype == TYPE_Q5_1 else 0
        codes = np.empty((rows, nblk, lead + 20), dtype=np.uint8)
        if lead:
            m_bits = (-rng.uniform(12.0, 18.0, size=(rows, nblk)) * np.abs(d_draw)).astype(np.float16).view(np.uint16)
            codes[:, :, 0:2] = m_bits.view(np.uint8).reshape(rows, nblk, 2)
        codes[:, :, lead:] = rng.integers(0, 256, size=(rows, nblk, 20), dtype=np.uint8)
    elif qtype == TYPE_Q8_0:
        codes = rng.integers(-127, 128, size=(rows, nblk, 32), dtype=np.int8).view(np.uint8)
    else:
        raise ValueError(f"unsupported type {qtype}")
    pad = rng.integers(0, 256, size=(rows, nb1 - dense), dtype=np.uint8) if nb1 > dense else None
    return assemble_rows(d_bits, codes, nb1, pad)


def make_activations(n_tokens: int, k: int, rng: np.random.Generator, dtype=np.float32) -> np.ndarray:
    """X [n_tokens][k] ~ N(0, 1); fp16 activations are the fp32 draws rounded
    to nearest binary16."""
    x = rng.standard_normal((n_tokens, k), dtype=np.float32)
    return x.astype(dtype) if dtype != np.float32 else x


@dataclass(frozen=True)
class Case:
    """One MUL_MAT workload: a quantised W and n_tokens activations."""
    name: str
    config: int
    qtype: int
    rows: int
    k: int
    nb1: int
    n_tokens: int
    x_dtype: type = np.float32
    layer: int = 0
    tensor: int = 0

    def weights(self) -> np.ndarray:
        return make_weights(self.qtype, self.rows, self.k, self.nb1,
                            rng_for(self.config, self.layer, self.tensor, WHAT_WEIGHTS))

    def activations(self) -> np.ndarray:
        return make_activations(self.n_tokens, self.k,
                                rng_for(self.config, self.layer, self.tensor, WHAT_ACTIVATIONS),
                                self.x_dtype)

    def w_bytes(self) -> int:
        """Algorithmic weight bytes (blocks only, padding excluded)."""
        return self.rows * dense_row_bytes(self.qtype, self.k)


def config_cases() -> dict[int, list[Case]]:
    """The five configured workloads, keyed 1..5."""
    q4, q8 = TYPE_Q4_0, TYPE_Q8_0
    c = {}
    c[1] = [Case("q4_0 256x512 n1", 1, q4, 256, 512, dense_row_bytes(q4, 512), 1)]
    c2 = []
    for t, qt in enumerate((q4, q8)):
        for j, (nm, rows, k) in enumerate((("attn_q", 4096, 4096), ("ffn_up", 11008, 4096),
                                            ("ffn_down", 4096, 11008))):
            c2.append(Case(f"{TYPE_NAMES[qt]} {nm} {rows}x{k} n1", 2, qt, rows, k,
                           dense_row_bytes(qt, k), 1, tensor=3 * t + j))
    c[2] = c2
    # one output-projection matrix, four activation batch sizes
    c[3] = [Case(f"q4_0 output 32000x4096 nb1=2560 n{n}", 3, q4, N_VOCAB, N_EMBD, 2560, n)
            for n in (1, 2, 4, 8)]
    c[4] = [Case(f"q4_0 {nm} {rows}x{k} prefill n512 x16", 4, q4, rows, k, dense_row_bytes(q4, k), 512,
                 np.float16, tensor=j)
            for j, (nm, rows, k) in enumerate((("attn_q", 4096, 4096), ("ffn_up", 11008, 4096)))]
    c[5] = stack_cases(1) + stack_cases(2048)
    return c


def stack_cases(n_tokens: int, layers: int = N_LAYER) -> list[Case]:
    """The 32-layer Llama-7B-shaped Q4_0 stack as independent MUL_MATs; decode
    (n_tokens <= 8) takes fp32 activations, prefill takes fp16 activations."""
    xdt = np.float32 if n_tokens <= 8 else np.float16
    out = []
    for layer in range(layers):
        for j, (nm, rows, k) in enumerate(LAYER_TENSORS):
            out.append(Case(f"blk.{layer}.{nm} {rows}x{k} n{n_tokens}", 5, TYPE_Q4_0, rows, k,
                            dense_row_bytes(TYPE_Q4_0, k), n_tokens, xdt, layer, j))
    return out
