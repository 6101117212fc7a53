"""Pins for the mixed-precision oracle (CPU only).

"GPU矩阵乘法优化：共享内存Tiling技术实战", section 7.1: FP32 operands converted to half
precision before the matrix cores.  The oracle rounds the operands to fp16 or
bf16 (nearest, ties to even) and runs the FP64 GEMM oracle on them.  Pinned
here against: hand-worked values of each format (ties, the largest finite value
and overflow, subnormals, signed zero, inf, NaN); a brute-force nearest-value
search over every one of the 65536 bit patterns of each format, decoded from
sign/exponent/fraction by the formats' definitions; numpy's own float16
conversion; and GEMM cases whose results follow in closed form.  Planted
mistakes (truncation instead of rounding, ties away from zero, one operand left
unrounded) must each fail a pin.
"""
import numpy as np
import pytest

from fp32_gemm_08_amd.inputs import make_case
from oracle import gemm_full, gemm_lowp_rows, round_bf16, round_fp16, round_to

F32 = np.float32


def _decode_fp16(bits):
    s = (bits >> 15) & 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    sign = np.where(s == 1, -1.0, 1.0)
    val = np.where(e == 0, sign * f * 2.0 ** -24, sign * (1 + f / 1024.0) * np.exp2(e.astype(np.float64) - 15))
    return np.where(e == 31, np.nan, val)


def _decode_bf16(bits):
    s = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    sign = np.where(s == 1, -1.0, 1.0)
    val = np.where(e == 0, sign * f * 2.0 ** -133, sign * (1 + f / 128.0) * np.exp2(e.astype(np.float64) - 127))
    return np.where(e == 255, np.nan, val)


def _nearest_brute(x, decode, maxfin):
    """Nearest representable value, ties to the pattern with an even last bit;
    beyond the largest finite value by half a step or more: inf."""
    bits = np.arange(1 << 16, dtype=np.int64)
    vals = decode(bits)
    keep = np.isfinite(vals) & ((bits >> 15) == 0)          # non-negative finite patterns
    v, b = vals[keep], bits[keep]
    order = np.argsort(v)
    v, b = v[order], b[order]
    ax = np.abs(x.astype(np.float64))
    hi = np.clip(np.searchsorted(v, ax), 1, len(v) - 1)
    lo = hi - 1
    dlo, dhi = ax - v[lo], v[hi] - ax
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((b[hi] & 1) == 0))
    r = np.where(pick_hi, v[hi], v[lo])
    r = np.where(ax >= v[-1], v[-1], r)
    step_top = v[-1] - v[-2]
    r = np.where(ax >= maxfin + step_top / 2, np.inf, r)      # ties at the top go to the even "next" = inf
    return np.copysign(r, x.astype(np.float64))


def _sample(seed, n=200000, lo=-30, hi=20):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n) * np.exp2(rng.integers(lo, hi, n))
    with np.errstate(over="ignore"):
        return x.astype(F32)


# ---- rounding pins --------------------------------------------------------------------------------

FP16_CASES = [(1 + 2 ** -11, 1.0), (1 + 3 * 2 ** -11, 1 + 2 ** -9), (-(1 + 3 * 2 ** -11), -(1 + 2 ** -9)),
              (65504.0, 65504.0), (65519.99, 65504.0), (65520.0, np.inf), (-70000.0, -np.inf),
              (2 ** -24, 2 ** -24), (2 ** -25, 0.0), (3 * 2 ** -26, 2 ** -24), (2 ** -14, 2 ** -14),
              (0.1, 0.0999755859375), (1 / 3, 0.333251953125)]
BF16_CASES = [(1 + 2 ** -8, 1.0), (1 + 3 * 2 ** -8, 1 + 2 ** -6), (1 + 2 ** -8 + 2 ** -20, 1 + 2 ** -7),
              (-(1 + 3 * 2 ** -8), -(1 + 2 ** -6)), (0.1, 0.10009765625), (1 / 3, 0.333984375),
              (3.3895313892515355e38, 3.3895313892515355e38), (float(np.finfo(F32).max), np.inf),
              (1e-40, 9.183549615799121e-41)]


def pin_fp16_hand(rnd):
    x = np.array([c[0] for c in FP16_CASES], dtype=F32)
    want = np.array([c[1] for c in FP16_CASES], dtype=np.float64)
    got = rnd(x).astype(np.float64)
    sz = rnd(np.array([-0.0, 0.0], dtype=F32))
    special = rnd(np.array([np.inf, -np.inf, np.nan], dtype=F32))
    return (np.array_equal(got, want) and np.signbit(sz[0]) and not np.signbit(sz[1])
            and np.isposinf(special[0]) and np.isneginf(special[1]) and np.isnan(special[2]))


def pin_bf16_hand(rnd):
    x = np.array([c[0] for c in BF16_CASES], dtype=F32)
    want = np.array([c[1] for c in BF16_CASES], dtype=np.float64)
    got = rnd(x).astype(np.float64)
    special = rnd(np.array([np.inf, -np.inf, np.nan, -0.0], dtype=F32))
    return (np.array_equal(got, want) and np.isposinf(special[0]) and np.isneginf(special[1])
            and np.isnan(special[2]) and np.signbit(special[3]))


def pin_fp16_brute(rnd):
    x = _sample(1, lo=-28, hi=17)
    want = _nearest_brute(x, _decode_fp16, 65504.0)
    return np.array_equal(rnd(x).astype(np.float64), want)


def pin_bf16_brute(rnd):
    x = _sample(2, lo=-140, hi=128)
    x = x[np.isfinite(x)]
    want = _nearest_brute(x, _decode_bf16, float(_decode_bf16(np.array([0x7F7F]))[0]))
    return np.array_equal(rnd(x).astype(np.float64), want)


def pin_fp16_numpy(rnd):
    x = _sample(3)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).astype(F32)
    return np.array_equal(rnd(x).view(np.uint32), want.view(np.uint32))


def pin_tie_grid(rnd_fp16, rnd_bf16):
    # exact midpoints between consecutive representable values: every one is a
    # tie and must go to the neighbour with the even last bit
    k = np.arange(0, 1024, dtype=np.float64)
    mid16 = (1 + (k + 0.5) / 1024).astype(F32)               # between 1 + k/1024 and 1 + (k+1)/1024
    even16 = 1 + (k + (k % 2)) / 1024
    k7 = np.arange(0, 128, dtype=np.float64)
    mid_b = (1 + (k7 + 0.5) / 128).astype(F32)
    even_b = 1 + (k7 + (k7 % 2)) / 128
    return (np.array_equal(rnd_fp16(mid16).astype(np.float64), even16)
            and np.array_equal(rnd_bf16(mid_b).astype(np.float64), even_b))


@pytest.mark.parametrize("pin,rnd", [(pin_fp16_hand, round_fp16), (pin_bf16_hand, round_bf16),
                                     (pin_fp16_brute, round_fp16), (pin_bf16_brute, round_bf16),
                                     (pin_fp16_numpy, round_fp16)],
                         ids=["fp16_hand", "bf16_hand", "fp16_brute", "bf16_brute", "fp16_numpy"])
def test_rounding_pins(pin, rnd):
    assert pin(rnd)


def test_tie_grid():
    assert pin_tie_grid(round_fp16, round_bf16)


# ---- GEMM pins -----------------------------------------------------------------------------------

@pytest.mark.parametrize("precision", ["fp16", "bf16"])
def test_representable_inputs_equal_fp32_oracle(precision):
    # small integers are exact in both formats: the mixed-precision result is the FP32 one, bit for bit
    case = make_case(37, 29, 50, trans_b=True, alpha=1.5, beta=-0.5, dist="int2", seed=7, lda=53)
    D, S, _ = gemm_lowp_rows(precision, 37, 29, 50, 1.5, case.A, case.B, True, -0.5, case.C)
    D32, S32 = gemm_full(37, 29, 50, 1.5, case.A, case.B, True, -0.5, case.C)
    assert np.array_equal(D, D32) and np.array_equal(S, S32)


@pytest.mark.parametrize("precision,tie,down", [("fp16", 1 + 2 ** -11, 1.0), ("bf16", 1 + 2 ** -8, 1.0),
                                                ("fp16", 1 + 3 * 2 ** -11, 1 + 2 ** -9),
                                                ("bf16", 1 + 3 * 2 ** -8, 1 + 2 ** -6)])
def test_closed_form_product(precision, tie, down):
    # A = tie everywhere, B = 2 everywhere: D = K * r(tie) * 2 in closed form
    M, N, K = 3, 4, 5
    A = np.full((M, K), tie, dtype=F32)
    B = np.full((K, N), 2.0, dtype=F32)
    D, S, _ = gemm_lowp_rows(precision, M, N, K, 1.0, A, B, False, 0.0, None)
    assert np.all(D == K * down * 2.0) and np.all(S == K * down * 2.0)


def test_both_operands_rounded():
    # A exact, B = 1 + 2^-9 (exact in fp16, not in bf16): only B's rounding shows
    A = np.ones((2, 3), dtype=F32)
    B = np.full((3, 2), 1 + 2 ** -9, dtype=F32)
    D16, _, _ = gemm_lowp_rows("fp16", 2, 2, 3, 1.0, A, B, False, 0.0, None)
    Db, _, _ = gemm_lowp_rows("bf16", 2, 2, 3, 1.0, A, B, False, 0.0, None)
    assert np.all(D16 == 3 * (1 + 2 ** -9)) and np.all(Db == 3.0)


def test_round_to_rejects_unknown():
    with pytest.raises(ValueError):
        round_to("fp8", np.zeros(2, F32))


# ---- planted mistakes ----------------------------------------------------------------------------

def _trunc_bf16(x):                     # truncation instead of rounding
    u = np.ascontiguousarray(x, dtype=F32).view(np.uint32)
    return (u & np.uint32(0xFFFF0000)).view(F32)


def _ties_away_fp16(x):                 # ties away from zero instead of to even
    xd = np.asarray(x, dtype=F32).astype(np.float64)
    out = xd.copy()
    fin = np.isfinite(xd) & (xd != 0)
    a = np.abs(xd[fin])
    e = np.maximum(np.floor(np.log2(a)), -14.0)
    step = np.exp2(e - 10.0)
    q = np.floor(a / step + 0.5) * step
    out[fin] = np.copysign(np.where(q > 65504.0, np.inf, q), xd[fin])
    return out.astype(F32)


def _no_subnormal_fp16(x):              # flushes fp16 subnormals to zero
    r = round_fp16(x)
    return np.where(np.abs(r) < 2 ** -14, np.copysign(0.0, r), r).astype(F32)


def _no_overflow_fp16(x):               # saturates instead of overflowing to inf
    r = round_fp16(x)
    return np.where(np.isinf(r) & np.isfinite(x), np.copysign(65504.0, x), r).astype(F32)


@pytest.mark.parametrize("mutant,pins", [
    (_trunc_bf16, [pin_bf16_hand, pin_bf16_brute]),
    (_ties_away_fp16, [pin_fp16_hand, pin_fp16_brute, pin_fp16_numpy]),
    (_no_subnormal_fp16, [pin_fp16_hand, pin_fp16_brute, pin_fp16_numpy]),
    (_no_overflow_fp16, [pin_fp16_hand, pin_fp16_brute, pin_fp16_numpy]),
], ids=["trunc_bf16", "ties_away_fp16", "no_subnormal_fp16", "no_overflow_fp16"])
def test_planted_rounding_mistake_is_caught(mutant, pins):
    with np.errstate(all="ignore"):
        results = [p(mutant) for p in pins]
    assert not all(results), f"{mutant.__name__} passed {[p.__name__ for p in pins]}"
