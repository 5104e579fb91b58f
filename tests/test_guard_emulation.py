"""CPU emulation of the fast paths' fp16 operand conversions and of the
exactness guard that covers them (no GPU).

The fused kernels multiply fp16 operands.  Activations are scaled per
exponent set (a 128-group at batch 1, an 8-group slice per token in batched
decode, a whole token on the many-token tiles) so that the set's largest
magnitude maps to [2^14, 2^15), times a slot factor 2^-p with p <= 7, and
rounded to fp16; the many-token tiles also fold the group scale into the fp16
weight as s * 2^-E with E chosen per row.  These tests emulate those
conversions in numpy (np.float16 rounds to nearest-even, subnormals included)
and check three things:

  1. the adversarial inputs of the review break |y - y_ref| <= 1e-4 a + 1e-6
     when the fast conversion is used alone -- so a guard is needed;
  2. the guard flags those outputs: its bound 4 sum_g |s_g| D_g, with D the
     summed conversion error |x - x'| of a group (fp16 subnormals kept, as
     the hardware does), exceeds 2^-21, and a row with a scale below
     2^(E-17) counts as not folding exactly; the kernels' cheap pre-test
     (every value at least 2^(e-7) converts exactly, so D is only computed
     when a smaller one exists) holds for every slot offset;
  3. the bound is a true bound on random inputs with wide magnitude spreads,
     and on the synthetic workloads' own activations it stays far inside the
     budget, so the fast path is what runs there.

The emulation is written from the conversion rule stated in the library
header, not from the kernels' source; the products themselves are checked on
the GPU against the oracle (tests/test_gpu_guard.py).
"""
import numpy as np
import pytest

import synth

RTOL, ATOL = 1e-4, 1e-6
BUDGET = 2.0 ** -21


def set_exponent(a):
    """e with max|a| * 2^-e in [2^14, 2^15) (frexp's exponent minus 15)."""
    m = float(np.max(np.abs(a))) if a.size else 0.0
    return int(np.frexp(m)[1]) - 15


def convert(x, e, p):
    """x (float64 values exactly representable in bf16) -> the value the fp16
    operand stands for: fp16(x * 2^-(e+p)) * 2^(e+p)."""
    h = np.ldexp(x, -(e + p)).astype(np.float16).astype(np.float64)
    return np.ldexp(h, e + p)


def error_mass(x, e, p):
    """D: summed conversion error |x - x'| of the values x under exponent e and
    slot offsets p."""
    return float(np.abs(x - convert(x, e, p)).sum())


def bf16(a):
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))).astype(np.float64)


def exact(x, q, s):
    """sum_g s_g sum_{k in g} q_k x_k in fp64 (exact for these magnitudes)."""
    g = q.size // 128
    return float(sum(s[i] * np.dot(q[128 * i:128 * (i + 1)], x[128 * i:128 * (i + 1)]) for i in range(g)))


def tolerance(x, q, s):
    g = q.size // 128
    a = sum(abs(s[i]) * np.abs(q[128 * i:128 * (i + 1)] * x[128 * i:128 * (i + 1)]).sum() for i in range(g))
    return RTOL * a + ATOL


def emulate_sets(x, q, s, set_len, rng):
    """Fast result with one exponent per `set_len` consecutive activations
    and random slot offsets, plus the guard's bound for that output."""
    k = x.size
    p = rng.integers(0, 8, size=k)
    xt = np.empty_like(x)
    d = np.zeros(k // 128)
    for b in range(0, k, set_len):
        e = set_exponent(x[b:b + set_len])
        xt[b:b + set_len] = convert(x[b:b + set_len], e, p[b:b + set_len])
        for g in range(b // 128, (b + set_len) // 128):
            d[g] = error_mass(x[128 * g:128 * (g + 1)], e, p[128 * g:128 * (g + 1)])
    y_fast = exact(xt, q, s)
    bound = 4.0 * float(np.dot(np.abs(s), d))
    return y_fast, bound


def adversarial_row(rng, k, big=2.0 ** 12, small=2.0 ** -22):
    """Large activations on code-4 (zero) weights, tiny ones on the rest."""
    q = rng.integers(-4, 4, size=k).astype(np.float64)
    q[q == 0] = 1.0
    x = bf16(rng.standard_normal(k) * small)
    zero_at = np.zeros(k, dtype=bool)
    zero_at[::8] = True  # every 8th weight is code 4 and meets a large activation
    q[zero_at] = 0.0
    x[zero_at] = bf16(rng.standard_normal(int(zero_at.sum())) * big)
    return x, q


@pytest.mark.parametrize("set_len,what", [(128, "batch 1: one exponent per group"),
                                          (1024, "batched decode: one exponent per 8-group slice"),
                                          (8192, "many-token tiles: one exponent per token")])
def test_adversarial_activations_need_the_guard(set_len, what):
    """Review case 2 (and its batch-1 and per-token forms), spread to 2^34:
    x ~ 2^12 on code-4 weights and ~2^-22 on the others, s = 1.  The
    conversion alone misses the tolerance; the guard's bound flags the
    output and covers the error."""
    rng = np.random.default_rng(11)
    k = 8192
    x, q = adversarial_row(rng, k)
    s = np.ones(k // 128)
    y_ref = exact(x, q, s)
    y_fast, bound = emulate_sets(x, q, s, set_len, rng)
    assert abs(y_fast - y_ref) > tolerance(x, q, s), what
    assert bound > BUDGET, what
    assert abs(y_fast - y_ref) <= bound * (1 + 1e-9), what


def fold(q, p, s_row, E):
    """The many-token tiles' weight operand: fp16(q 2^p * fp16(s 2^-E)) and the
    weight it stands for."""
    sv = np.ldexp(s_row, -E).astype(np.float16)
    b = (np.ldexp(q, p).astype(np.float16) * sv).astype(np.float64)
    return np.ldexp(b, E - p)


def row_exponent(s_row):
    return int(np.frexp(float(np.max(np.abs(s_row))))[1]) - 4  # largest -> [8, 16)


def fold_inexact(s_row):
    """The guard's test: some non-zero scale below 2^(E-17)."""
    E = row_exponent(s_row)
    nz = np.abs(s_row)[s_row != 0]
    return bool(nz.size) and float(nz.min()) < np.ldexp(1.0, E - 17)


def test_adversarial_scale_fold_needs_the_guard():
    """Review case 1: row scales {1024, 2^-18}, group 0 all code 4, x ~ N(0,1).
    The folded weight of group 1 flushes to zero, so the tile result misses
    the tolerance; the guard marks the row as not folding exactly."""
    rng = np.random.default_rng(12)
    k = 256
    s = np.array([1024.0, 2.0 ** -18])
    q = np.concatenate([np.zeros(128), rng.integers(-4, 4, size=128).astype(np.float64)])
    q[128:][q[128:] == 0] = 2.0
    x = bf16(rng.standard_normal(k))
    p = rng.integers(0, 8, size=k)
    E = row_exponent(s)
    w = np.concatenate([fold(q[:128], p[:128], s[0], E), fold(q[128:], p[128:], s[1], E)])
    y_fast = float(np.dot(w, x))
    y_ref = exact(x, q, s)
    assert y_fast == 0.0
    assert abs(y_fast - y_ref) > tolerance(x, q, s)
    assert fold_inexact(s)


def test_fold_is_exact_inside_the_window():
    """Every code and slot offset, scales down to 2^-17 * 2^E: the folded
    weight equals q * s exactly, and the guard does not flag the row."""
    rng = np.random.default_rng(13)
    for _ in range(200):
        top = float(bf16(np.array([np.ldexp(1.0 + rng.random(), int(rng.integers(-30, 30)))]))[0])
        E = row_exponent(np.array([top]))
        lo = np.ldexp(1.0, E - 17)
        s = np.concatenate([[top], bf16(np.exp2(rng.uniform(np.log2(lo), np.log2(top), size=15)))])
        s = np.maximum(s, bf16(lo))  # bf16 rounding stays at or above the floor
        assert not fold_inexact(s)
        for g in range(s.size):
            q = np.arange(-4, 4, dtype=np.float64)
            for pp in range(8):
                got = fold(q, np.full(8, pp), s[g], E)
                assert np.array_equal(got, q * s[g])


@pytest.mark.parametrize("set_len", [128, 1024, 8192])
def test_guard_bound_holds_on_wide_spreads(set_len):
    """Random magnitudes spread over 2^-60 .. 2^60 within every set and random
    slot offsets: the conversion error of every output stays within the
    guard's bound 4 sum_g |s_g| D_g."""
    rng = np.random.default_rng(20 + set_len)
    k = 8192
    for _ in range(12):
        x = bf16(rng.standard_normal(k) * np.exp2(rng.integers(-60, 60, size=k)))
        x[rng.random(k) < 0.05] = 0.0
        q = rng.integers(-4, 4, size=k).astype(np.float64)
        s = bf16(np.abs(rng.standard_normal(k // 128)) * np.exp2(rng.integers(-10, 10, size=k // 128)))
        y_fast, bound = emulate_sets(x, q, s, set_len, rng)
        assert abs(y_fast - exact(x, q, s)) <= bound * (1 + 1e-9) + 1e-300


def test_values_above_the_floor_convert_exactly():
    """The pre-test: every bf16 value of magnitude in [2^(e-7), 2^(e+15)),
    under exponent e and any slot offset p <= 7, has an exact fp16 operand --
    so a set whose smallest non-zero value is at least 2^(e-7) has D = 0."""
    rng = np.random.default_rng(14)
    for e in (-140, -30, -15, 0, 20, 100):
        mags = np.ldexp(1.0 + rng.random(4000), rng.integers(e - 7, e + 15, size=4000))
        x = bf16(mags * np.where(rng.random(4000) < 0.5, -1.0, 1.0))
        x = x[(np.abs(x) >= np.ldexp(1.0, e - 7)) & (np.abs(x) < np.ldexp(1.0, e + 15))]
        for p in range(8):
            assert error_mass(x, e, np.full(x.size, p)) == 0.0, (e, p)


@pytest.mark.parametrize("m,k,set_len", [(1, 8192, 128), (32, 8192, 1024), (16, 28672, 1024), (32, 28672, 1024),
                                         (1, 28672, 128), (512, 8192, 8192), (512, 28672, 28672)])
def test_synthetic_workloads_take_the_fast_path(m, k, set_len):
    """The layer workloads' activations (N(0,1) in bf16): even at the worst
    slot offset (p = 7) their conversion error, against the workloads'
    largest scale, stays far inside the budget, so no output is recomputed."""
    x = synth.bf16_bits_to_f32(synth.layer_x(m, k)).astype(np.float64)
    smax = 0.01 * 6 + 1e-4  # |N(0, 0.01)| + 1e-4 never reaches 6 sigma in these draws
    worst = 0.0
    for row in x:
        for b in range(0, k, set_len):
            seg = row[b:b + set_len]
            worst = max(worst, error_mass(seg, set_exponent(seg), np.full(seg.size, 7)))
    assert 4.0 * smax * worst <= BUDGET
