"""Pins for the CPU oracle: facts that do not come from the oracle's own code.

Each test checks the oracle against something fixed independently of it:
sizes printed on the GSQ model card, packed words derived by hand, numpy's bit
packer, PyTorch's bf16 rounding, exact rational arithmetic and closed forms.
Together they are chosen so that a plausible slip in the oracle (a wrong bit
order, a dropped or extra bit, the wrong code offset or sign, the wrong scale
index, a transposed operand, a dropped term) fails at least one of them.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def packbits_twin(codes: np.ndarray) -> np.ndarray:
    """Exact-width LSB-first packing by numpy's own bit routines."""
    n, k = codes.shape
    bits = np.unpackbits(codes[..., None], axis=-1, bitorder="little")[..., :3]
    return np.packbits(bits.reshape(n, 3 * k), axis=-1, bitorder="little").view("<u4")


def bf16_to_fraction(b: int) -> Fraction:
    f = np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(f))


# ---------------------------------------------------------------- sizes ----

def _card_sizes():
    rows, bpp = [], []
    with open(os.path.join(GOLDEN, "card_sizes.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] == "bpp":
                bpp.append(tuple(int(v) for v in parts[1:]))
            else:
                rows.append(tuple(int(v) for v in parts))
    return rows, bpp


def test_card_sizes():
    rows, _ = _card_sizes()
    assert rows, "golden file lost its rows"
    for n, k, wcols, scols in rows:
        assert oracle.words_per_row(k) == wcols
        assert oracle.groups_per_row(k) == scols
        codes = np.full((2, k), 4, dtype=np.uint8)
        assert oracle.pack(codes).shape == (2, wcols)


def test_bits_per_weight():
    _, bpp = _card_sizes()
    for k, num, den in bpp:
        bits = 8 * (4 * oracle.words_per_row(k) + 2 * oracle.groups_per_row(k))
        assert Fraction(bits, k) == Fraction(num, den)
    # other layer widths of the 70B layer
    assert (oracle.words_per_row(28672), oracle.groups_per_row(28672)) == (2688, 224)
    assert (oracle.words_per_row(1024), oracle.groups_per_row(1024)) == (96, 8)


# ------------------------------------------------------------ pack/unpack --

def _golden_rows():
    out = []
    with open(os.path.join(GOLDEN, "pack_examples.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            left, right = line.split("|")
            name, rule = left.split()
            words = np.array([int(w, 16) for w in right.split()], dtype=np.uint32)
            if rule.startswith("fill:"):
                codes = np.full(128, int(rule[5:]), dtype=np.uint8)
            elif rule == "kmod8":
                codes = (np.arange(128) % 8).astype(np.uint8)
            elif rule.startswith("seven_at:"):
                codes = np.zeros(128, dtype=np.uint8)
                codes[[int(v) for v in rule[9:].split(",")]] = 7
            else:
                raise AssertionError(rule)
            out.append((name, codes, words))
    return out


@pytest.mark.parametrize("name,codes,words", _golden_rows(), ids=lambda v: v if isinstance(v, str) else "")
def test_pack_worked_examples(name, codes, words):
    got = oracle.pack(codes[None, :])[0]
    assert got.tolist() == words.tolist(), name
    assert oracle.unpack(words[None, :], 128)[0].tolist() == codes.tolist()


def test_all4_word_as_int32():
    # the zero-weight row's third word has its top bit set: as int32 it is negative
    w = oracle.pack(np.full((1, 128), 4, dtype=np.uint8))
    assert int(w.view(np.int32)[0, 2]) == -1840700270


@pytest.mark.parametrize("n,k", [(3, 128), (5, 384), (2, 1024), (1, 8192)])
def test_pack_matches_numpy_packbits(n, k):
    c = synth.codes_all8(11 + k, n, k)
    assert np.array_equal(oracle.pack(c), packbits_twin(c))


def test_unpack_roundtrip_all_codes():
    c = synth.codes_all8(5, 7, 896)
    w = oracle.pack(c)
    assert np.array_equal(oracle.unpack(w, 896), c)
    # unpack also inverts numpy's packing, so it is not just the inverse of our pack
    assert np.array_equal(oracle.unpack(packbits_twin(c), 896), c)


def test_pack_rejects_bad_inputs():
    with pytest.raises(ValueError):
        oracle.pack(np.full((1, 128), 8, dtype=np.uint8))
    with pytest.raises(ValueError):
        oracle.pack(np.zeros((1, 96), dtype=np.uint8))


# ------------------------------------------ 4-bit-container intermediate ---
# Reading of the GSQ model card ("Storage layout", the note on the
# pack-quantized shards): nibble k % 8 of word k / 8, least significant first,
# holds code k in its low 3 bits; the top bit is padding.

def nibbles_twin(w4: np.ndarray) -> np.ndarray:
    """Codes from 4-bit-container words with numpy shifts (independent of oracle.c)."""
    w4 = np.asarray(w4, dtype=np.uint32)
    sh = (4 * np.arange(8)).astype(np.uint32)
    return ((w4[:, :, None] >> sh) & np.uint32(7)).astype(np.uint8).reshape(w4.shape[0], -1)


def test_repack_w4c_worked_example():
    """Codes k mod 8 in nibble order are words 0x76543210; with every padding
    bit set they are 0xFEDCBA98.  Both repack to the pinned k-mod-8 stream."""
    kmod8 = [w for name, _, w in _golden_rows() if name == "kmod8"][0]
    for word in (0x76543210, 0xFEDCBA98):
        w4 = np.full((1, 16), word, dtype=np.uint32)
        assert oracle.repack_w4c(w4)[0].tolist() == kmod8.tolist(), hex(word)


def test_repack_w4c_nibble_order():
    """One code per word: code 5 in nibble 3 of word 2 of a 128-wide row is
    weight k = 19, i.e. stream bits 57 (set) and 59 (set) of word 1."""
    w4 = np.zeros((1, 16), dtype=np.uint32)
    w4[0, 2] = 5 << 12
    words = oracle.repack_w4c(w4)[0]
    expect = np.zeros(12, dtype=np.uint32)
    expect[1] = (1 << (57 - 32)) | (1 << (59 - 32))
    assert words.tolist() == expect.tolist()


@pytest.mark.parametrize("n,k", [(3, 128), (5, 384), (2, 8192)])
def test_repack_w4c_matches_twin(n, k):
    rng = np.random.default_rng(40 + k)
    w4 = rng.integers(0, 2 ** 32, size=(n, k // 8), dtype=np.uint64).astype(np.uint32)
    codes = nibbles_twin(w4)
    assert np.array_equal(oracle.repack_w4c(w4), packbits_twin(codes))
    assert np.array_equal(oracle.unpack(oracle.repack_w4c(w4), k), codes)


# --------------------------------------------------------------- dequant ---

def test_dequant_special_values():
    # scales with 8 significant bits, codes 0..7 in every group
    k = 256
    s = synth.scales(3, 4, 2, sigma=1.0, eps=0.0)
    c = np.tile(np.arange(8, dtype=np.uint8), (4, k // 8))
    w = oracle.dequant_bf16(packbits_twin(c), s, k)
    sf = synth.bf16_bits_to_f32(s).astype(np.float64)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    for n in range(4):
        for kk in range(k):
            sv = sf[n, kk // 128]
            q = int(c[n, kk]) - 4
            if q == 0:
                assert w[n, kk] == 0x0000  # +0, not -0
            elif q in (-4, -2, -1, 1, 2):
                assert wf[n, kk] == q * sv  # exact
            else:  # |q| = 3 rounds to 8 bits
                assert abs(wf[n, kk] - q * sv) <= abs(q * sv) * 2.0 ** -8


def test_dequant_matches_torch_bf16_rounding():
    k = 1024
    c = synth.codes_all8(21, 16, k)
    s = synth.scales(22, 16, k // 128, sigma=0.3, eps=1e-3)
    w = oracle.dequant_bf16(packbits_twin(c), s, k)
    sf = torch.from_numpy(synth.bf16_bits_to_f32(s)).repeat_interleave(128, dim=1)
    ref = ((torch.from_numpy(c).float() - 4.0) * sf).to(torch.bfloat16)
    ref_bits = ref.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(w, ref_bits)


# ------------------------------------------------------------------ gemm ---

@pytest.mark.parametrize("m,n,k,seed", [(1, 3, 128, 1), (3, 5, 256, 2), (4, 8, 128, 3), (2, 2, 256, 4)])
def test_gemm_exact_rationals(m, n, k, seed):
    """Brute force with exact rationals: every input is a dyadic rational."""
    c = synth.codes_all8(seed, n, k)
    s = synth.scales(seed + 50, n, k // 128, sigma=0.05, eps=1e-3)
    x = synth.activations(seed + 90, m, k)
    y, a = oracle.gemm(x, packbits_twin(c), s, k)
    for mi in range(m):
        for ni in range(n):
            exact = Fraction(0)
            exact_abs = Fraction(0)
            for kk in range(k):
                t = bf16_to_fraction(x[mi, kk]) * (int(c[ni, kk]) - 4) * bf16_to_fraction(s[ni, kk // 128])
                exact += t
                exact_abs += abs(t)
            assert abs(Fraction(y[mi, ni]) - exact) <= exact_abs * Fraction(k, 2 ** 52)
            assert abs(Fraction(a[mi, ni]) - exact_abs) <= exact_abs * Fraction(k, 2 ** 52)


def test_gemm_textbook_twin():
    """Dense fp64 dequant from the codes, then numpy matmul: Y = X W^T."""
    m, n, k = 3, 37, 640
    c = synth.codes_all8(31, n, k)
    s = synth.scales(32, n, k // 128, sigma=0.02, eps=1e-4)
    x = synth.activations(33, m, k)
    y, a = oracle.gemm(x, packbits_twin(c), s, k)
    w = (c.astype(np.float64) - 4.0) * np.repeat(synth.bf16_bits_to_f32(s).astype(np.float64), 128, axis=1)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    ref = xf @ w.T
    ref_abs = np.abs(xf) @ np.abs(w).T
    assert np.all(np.abs(y - ref) <= 1e-12 * ref_abs)
    assert np.allclose(a, ref_abs, rtol=1e-12, atol=0)


def test_gemm_row_subset_matches_full():
    m, n, k = 2, 50, 384
    c = synth.codes(41, n, k)
    s = synth.scales(42, n, k // 128)
    x = synth.activations(43, m, k)
    w = packbits_twin(c)
    y_full, a_full = oracle.gemm(x, w, s, k)
    rows = np.array([49, 0, 17, 17, 3], dtype=np.int64)
    y_sub, a_sub = oracle.gemm(x, w, s, k, rows=rows)
    assert np.array_equal(y_sub, y_full[:, rows])
    assert np.array_equal(a_sub, a_full[:, rows])


def test_gemm_zero_rows_give_exact_zero():
    k = 512
    c = np.full((4, k), 4, dtype=np.uint8)
    s = synth.scales(51, 4, k // 128)
    x = synth.activations(52, 2, k)
    y, a = oracle.gemm(x, packbits_twin(c), s, k)
    assert np.all(y == 0.0) and np.all(a == 0.0)


def test_gemm_one_hot_closed_form():
    """One nonzero weight per row against a one-hot x: y = q * s * x exactly."""
    k = 384
    n = 8
    c = np.full((n, k), 4, dtype=np.uint8)
    s = synth.scales(61, n, k // 128, sigma=0.1, eps=1e-3)
    pos = [5, 127, 128, 200, 255, 256, 300, 383]
    for i in range(n):
        c[i, pos[i]] = [0, 1, 2, 3, 5, 6, 7, 0][i]
    sf = synth.bf16_bits_to_f32(s).astype(np.float64)
    for j in range(n):
        x = np.zeros((1, k), dtype=np.uint16)
        x[0, pos[j]] = 0x3FC0  # 1.5
        y, _ = oracle.gemm(x, packbits_twin(c), s, k)
        for i in range(n):
            expect = (int(c[i, pos[j]]) - 4) * sf[i, pos[j] // 128] * 1.5
            assert y[0, i] == expect
        assert y[0, j] != 0.0


def test_gemm_ones_closed_form():
    """x = 1 and every code 5 (q = +1): y[n] = 128 * sum_g s[n][g]."""
    k = 1024
    n = 6
    c = np.full((n, k), 5, dtype=np.uint8)
    s = synth.scales(71, n, k // 128, sigma=0.01, eps=1e-4)
    x = np.full((1, k), 0x3F80, dtype=np.uint16)  # bf16 1.0
    y, _ = oracle.gemm(x, packbits_twin(c), s, k)
    sf = synth.bf16_bits_to_f32(s).astype(np.float64)
    for i in range(n):
        assert y[0, i] == pytest.approx(128.0 * sf[i].sum(), rel=1e-15)
    # and q = -1 everywhere gives the exact negative
    y2, _ = oracle.gemm(x, packbits_twin(np.full((n, k), 3, dtype=np.uint8)), s, k)
    assert np.array_equal(y2, -y)


def test_gemm_transpose_sensitivity():
    """A non-square case where W and W^T would give different shapes and values."""
    m, n, k = 2, 3, 256
    c = synth.codes_all8(81, n, k)
    s = synth.scales(82, n, k // 128, sigma=0.05, eps=1e-3)
    x = synth.activations(83, m, k)
    y, _ = oracle.gemm(x, packbits_twin(c), s, k)
    assert y.shape == (m, n)
