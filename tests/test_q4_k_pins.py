"""Pins of the oracle's Q4_K reading (CPU only).

The pages describe k-quants only in outline: 256-weight super-blocks whose
scales and minimums are stored in two levels ("llama.cpp 源码完全拆解(一)：整体架构
与模块全景", section "权重装载：GGUF、mmap 与 4 bit 块"; the byte count of a Q4_K
tensor is ne[0] / 256 blocks in "llama.cpp 源码完全拆解(二)：ggml 计算图与内存分配器").
The bit layout is a reading (the GGUF layout). These tests tie the oracle to
a super-block worked out by hand from that reading, to every 6-bit scale and
minimum at every position, to every code at every position, to exact
rational arithmetic, and they plant plausible mistakes that must be caught.
Parity of the reading against GGUF files written elsewhere is not pinned
(no such file exists here).
"""
from fractions import Fraction

import numpy as np
import pytest

from conftest import read_golden
import oracle.qmm_oracle as O

QK4 = O.TYPE_Q4_K


def _golden_block():
    g = read_golden("q4_k_block.txt")
    head = np.array([int(v, 16) for v in g["header"]], np.uint8)
    chunk = np.array([int(v, 16) for v in g["chunk"]], np.uint8)
    raw = np.concatenate([head] + [chunk] * 4).reshape(1, 144)
    return g, raw


def test_golden_super_block_fields_and_values():
    g, raw = _golden_block()
    d, dmin, sc, m, q = O.q4_k_fields(raw, 1, 256, 144)
    assert d[0, 0] == 0.5 and dmin[0, 0] == 0.25
    assert sc[0, 0].tolist() == [int(v) for v in g["scales"]]
    assert m[0, 0].tolist() == [int(v) for v in g["mins"]]
    w = O.dequantize(raw, QK4, 1, 256, 144)[0]
    at = [int(v) for v in g["at"]]
    assert w[at].tolist() == [float(v) for v in g["values"]]
    # every element from the hand-derived scales, minimums and code rule
    scs = [int(v) for v in g["scales"]]
    ms = [int(v) for v in g["mins"]]
    for i in range(256):
        c, r = divmod(i, 64)
        j = 2 * c + (r >= 32)
        l = r % 32
        qv = l % 16 if r < 32 else 15 - l % 16
        assert w[i] == np.float32(0.5 * scs[j] * qv - 0.25 * ms[j]), i


def test_every_scale_and_min_at_every_position():
    # each sub-block position j, each 6-bit value v, the others set to a
    # distinct background, packed and read back; the golden block above pins
    # where the bits live, this pins that no value or position is mangled
    for j in range(8):
        for v in range(64):
            sc = np.array([[[(7 * i + 3) % 64 for i in range(8)]]])
            m = np.array([[[(11 * i + 5) % 64 for i in range(8)]]])
            sc[0, 0, j] = v
            m[0, 0, 7 - j] = 63 - v
            raw = O.q4_k_pack(np.array([[0x3C00]]), np.array([[0x3C00]]), sc, m, np.zeros((1, 1, 256), np.int64))
            _, _, sc2, m2, _ = O.q4_k_fields(raw, 1, 256, 144)
            assert np.array_equal(sc2, sc) and np.array_equal(m2, m), (j, v)


def test_every_code_at_every_position():
    # one code of 15 at element i, zeros elsewhere; d = 1, dmin = 1, sc_j = j + 1,
    # m_j = 2 j: element i is (j + 1) * 15 - 2 j, every other element of
    # sub-block j' is -2 j'
    sc = np.arange(1, 9).reshape(1, 1, 8)
    m = (2 * np.arange(8)).reshape(1, 1, 8)
    for i in range(256):
        q = np.zeros((1, 1, 256), np.int64)
        q[0, 0, i] = 15
        raw = O.q4_k_pack(np.array([[0x3C00]]), np.array([[0x3C00]]), sc, m, q)
        w = O.dequantize(raw, QK4, 1, 256, 144)[0]
        want = np.array([-2.0 * (e // 32) for e in range(256)], np.float32)
        want[i] = (i // 32 + 1) * 15 - 2 * (i // 32)
        assert np.array_equal(w, want), i


def test_code_byte_layout_by_hand():
    # code byte 0 holds element 0 (low nibble) and element 32 (high nibble);
    # code byte 32 holds elements 64 and 96; byte 127 (chunk 3, l = 31) elements 223 and 255
    raw = O.q4_k_pack(np.array([[0x3C00]]), np.array([[0x0000]]), np.ones((1, 1, 8), np.int64),
                      np.zeros((1, 1, 8), np.int64), np.zeros((1, 1, 256), np.int64))
    raw[0, 16 + 0] = 0x21     # element 0 <- 1, element 32 <- 2
    raw[0, 16 + 32] = 0x43    # element 64 <- 3, element 96 <- 4
    raw[0, 16 + 127] = 0x65   # element 223 <- 5, element 255 <- 6
    w = O.dequantize(raw, QK4, 1, 256, 144)[0]
    got = {i: float(w[i]) for i in np.flatnonzero(w)}
    assert got == {0: 1.0, 32: 2.0, 64: 3.0, 96: 4.0, 223: 5.0, 255: 6.0}


def test_single_rounding_to_fp32():
    # d * sc * q - dmin * m with d = 1 + 2^-10 (0x3C01), sc = 63, q = 15 and
    # dmin = 2^-24 (0x0001), m = 1: exact value 945 + 945 * 2^-10 - 2^-24,
    # which needs more than 24 significant bits; fp32 rounds it once
    sc = np.full((1, 1, 8), 63)
    m = np.ones((1, 1, 8), np.int64)
    q = np.full((1, 1, 256), 15)
    raw = O.q4_k_pack(np.array([[0x3C01]]), np.array([[0x0001]]), sc, m, q)
    w = O.dequantize(raw, QK4, 1, 256, 144)[0, 0]
    exact = Fraction(945) + Fraction(945, 1024) - Fraction(1, 2**24)
    # the two float32 neighbours of the exact value, and the nearer one
    lo = np.float32(float(exact))
    cands = [np.nextafter(lo, np.float32(-np.inf)), lo, np.nextafter(lo, np.float32(np.inf))]
    best = min(cands, key=lambda c: abs(Fraction(float(c)) - exact))
    assert w == best
    assert Fraction(float(w)) != exact


@pytest.mark.parametrize("k", [256, 512])
def test_matmul_brute_force_fraction(k):
    rng = np.random.default_rng(17 + k)
    rows, nsb, n = 3, k // 256, 2
    d = rng.uniform(0.01, 0.1, (rows, nsb)).astype(np.float16).view(np.uint16)
    dmin = rng.uniform(0.01, 0.1, (rows, nsb)).astype(np.float16).view(np.uint16)
    sc, m = rng.integers(0, 64, (rows, nsb, 8)), rng.integers(0, 64, (rows, nsb, 8))
    q = rng.integers(0, 16, (rows, nsb, 256))
    W = O.q4_k_pack(d, dmin, sc, m, q)
    X = rng.standard_normal((n, k)).astype(np.float32)
    y, s = O.matmul(W, QK4, rows, k, W.shape[1], X)
    dh, dmh = d.view(np.float16), dmin.view(np.float16)
    for t in range(n):
        for r in range(rows):
            acc = Fraction(0)
            for i in range(k):
                b, e = divmod(i, 256)
                j = e // 32
                wv = Fraction(float(dh[r, b])) * int(sc[r, b, j]) * int(q[r, b, e]) - \
                    Fraction(float(dmh[r, b])) * int(m[r, b, j])
                acc += Fraction(float(np.float32(float(wv)))) * Fraction(float(X[t, i]))
            assert abs(Fraction(y[t, r]) - acc) <= Fraction(k) * Fraction(1, 2**52) * Fraction(s[t, r]) + \
                Fraction(1, 2**60)


def test_round_trip_codes():
    rng = np.random.default_rng(5)
    rows, nsb = 4, 2
    d = rng.uniform(0.01, 0.1, (rows, nsb)).astype(np.float16)
    dmin = rng.uniform(0.01, 0.1, (rows, nsb)).astype(np.float16)
    sc, m = rng.integers(1, 64, (rows, nsb, 8)), rng.integers(0, 64, (rows, nsb, 8))
    q = rng.integers(0, 16, (rows, nsb, 256))
    W = O.q4_k_pack(d.view(np.uint16), dmin.view(np.uint16), sc, m, q)
    w = O.dequantize(W, QK4, rows, 512, W.shape[1]).reshape(rows, nsb, 256)
    q2 = O.q4_k_quantize_codes(w, d.astype(np.float64), dmin.astype(np.float64), sc, m)
    assert np.array_equal(q2, q)


def test_sizes():
    # 144 bytes per 256 weights: 4.5 bits per weight, the same as Q4_0
    assert O.row_bytes(QK4, 256) == 144
    assert O.row_bytes(QK4, 4096) == 2304 and O.row_bytes(QK4, 11008) == 43 * 144
    for bad in (32, 255, 300, 0):
        with pytest.raises(ValueError):
            O.row_bytes(QK4, bad)


# ------------------------------------------------------------ planted mistakes
def _golden_passes():
    try:
        g, raw = _golden_block()
        w = O.dequantize(raw, QK4, 1, 256, 144)[0]
        return w[[int(v) for v in g["at"]]].tolist() == [float(v) for v in g["values"]]
    except Exception:
        return False


def test_planted_mistakes_are_caught(monkeypatch):
    assert _golden_passes()
    orig_unpack = O.q4_k_unpack_scales
    orig_fields = O.q4_k_fields

    def swapped_sc_m(s):
        sc, m = orig_unpack(s)
        return m, sc

    def high_bits_from_wrong_byte(s):
        s = np.asarray(s, np.int64)
        sc, m = orig_unpack(s)
        for j in range(4, 8):
            sc[..., j] = (s[..., j + 4] & 15) | ((s[..., j] >> 6) << 4)
            m[..., j] = (s[..., j + 4] >> 4) | ((s[..., j - 4] >> 6) << 4)
        return sc, m

    def low_nibbles_swapped(s):
        s = np.asarray(s, np.int64)
        sc, m = orig_unpack(s)
        for j in range(4, 8):
            sc[..., j] = (s[..., j + 4] >> 4) | ((s[..., j - 4] >> 6) << 4)
            m[..., j] = (s[..., j + 4] & 15) | ((s[..., j] >> 6) << 4)
        return sc, m

    for bad in (swapped_sc_m, high_bits_from_wrong_byte, low_nibbles_swapped):
        monkeypatch.setattr(O, "q4_k_unpack_scales", bad)
        assert not _golden_passes(), bad.__name__
    monkeypatch.setattr(O, "q4_k_unpack_scales", orig_unpack)

    def interleaved_codes(W, n_rows, k, nb1):
        d, dmin, sc, m, q = orig_fields(W, n_rows, k, nb1)
        q = q.reshape(n_rows, -1, 4, 2, 32).transpose(0, 1, 2, 4, 3).reshape(n_rows, -1, 256)
        return d, dmin, sc, m, q

    def plus_min(W, n_rows, k, nb1):
        d, dmin, sc, m, q = orig_fields(W, n_rows, k, nb1)
        return d, -dmin, sc, m, q

    def d_dmin_swapped(W, n_rows, k, nb1):
        d, dmin, sc, m, q = orig_fields(W, n_rows, k, nb1)
        return dmin, d, sc, m, q

    for bad in (interleaved_codes, plus_min, d_dmin_swapped):
        monkeypatch.setattr(O, "q4_k_fields", bad)
        assert not _golden_passes(), bad.__name__
    monkeypatch.setattr(O, "q4_k_fields", orig_fields)
    assert _golden_passes()
