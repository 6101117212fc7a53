"""Pins for the transpose oracle (CPU only).

The operation is the one of "现代 CUDA 工具箱实战：从朴素代码到硬件极限的优化之路",
section 代码实现: the output element at (j, i) is the input element at (i, j).
Each pin below checks the oracle against something other than itself: a
hand-written example, a closed form (index-encoded values), a brute force over
plain Python lists, the independent FP64 GEMM oracle (I * X^T with X integer
valued is exact), the involution T(T(X)) = X, and bit patterns that arithmetic
would disturb.  The same pins are run against deliberately wrong transposes to
show that each plausible mistake fails at least one of them.
"""
import numpy as np
import pytest

from fp32_gemm_08_amd import inputs
from oracle import gemm_full, transpose

# (rows, cols, ld_src): square, ragged, single row/column, padded storage.
SHAPES = [(1, 1, 1), (2, 3, 3), (3, 2, 5), (7, 13, 16), (16, 16, 16), (64, 65, 70), (65, 64, 64),
          (1, 33, 40), (33, 1, 4)]


def _bits(x):
    return np.ascontiguousarray(x).view(np.uint32)


def pin_hand_example(tr):
    # [[1 2 3]      [[1 4]
    #  [4 5 6]]  ->  [2 5]
    #                [3 6]]   written out from the definition.
    src = np.array([[1, 2, 3, -1], [4, 5, 6, -1]], dtype=np.float32)  # ld 4, padding -1
    out = tr(src, 2, 3)
    return out.shape == (3, 2) and np.array_equal(out, np.array([[1, 4], [2, 5], [3, 6]], np.float32))


def pin_index_encoding(tr):
    # src(i, j) = i*cols + j, exact in float32 below 2^24; dst(j, i) must hold it.
    for rows, cols, ld in SHAPES:
        src = np.full((rows, ld), np.nan, dtype=np.float32)
        src[:, :cols] = np.arange(rows * cols, dtype=np.float32).reshape(rows, cols)
        want = np.add.outer(np.arange(cols), cols * np.arange(rows)).astype(np.float32)
        out = tr(src, rows, cols)
        if out.shape != (cols, rows) or not np.array_equal(out, want):
            return False
    return True


def pin_brute_force(tr):
    # Plain Python lists, no numpy indexing.
    rng = np.random.default_rng(11)
    for rows, cols, ld in SHAPES[:6]:
        src = rng.uniform(-1, 1, size=(rows, ld)).astype(np.float32)
        lst = src.tolist()
        want = [[lst[i][j] for i in range(rows)] for j in range(cols)]
        out = tr(src, rows, cols)
        if out.shape != (cols, rows) or out.tolist() != want:
            return False
    return True


def pin_gemm_identity(tr):
    # The FP64 GEMM oracle with transB: D = I_cols * op(B), op(B)(k, i) = X(i, k),
    # so D(j, i) = X(i, j) exactly for integer-valued X.
    for rows, cols, ld in SHAPES:
        case = inputs.make_case(cols, rows, cols, trans_b=True, dist="int2", seed=rows * 100 + cols,
                                ldb=ld)
        X = case.B                                    # rows x ld storage of the N x K operand
        eye = np.eye(cols, dtype=np.float32)
        D, _ = gemm_full(cols, rows, cols, 1.0, eye, X, True, 0.0, None)
        out = tr(X, rows, cols)
        if out.shape != (cols, rows) or not np.array_equal(out.astype(np.float64), D):
            return False
    return True


def pin_involution(tr):
    for rows, cols, ld in SHAPES:
        src = inputs.make_transpose_input(rows, cols, seed=3, ld_src=ld)
        back = tr(tr(src, rows, cols), cols, rows)
        if back.shape != (rows, cols) or not np.array_equal(_bits(back), _bits(src[:, :cols])):
            return False
    return True


def pin_special_bits(tr):
    src = inputs.make_transpose_input(40, 50, seed=4, ld_src=53, specials=True)
    out = tr(src, 40, 50)
    want = src[:, :50].view(np.uint32).T
    return out.shape == (50, 40) and np.array_equal(_bits(out), want)


def pin_degenerate(tr):
    src = np.zeros((0, 5), dtype=np.float32)
    if tr(src, 0, 5).shape != (5, 0):
        return False
    src = np.zeros((4, 1), dtype=np.float32)
    return tr(src, 4, 0).shape == (0, 4)


PINS = [pin_hand_example, pin_index_encoding, pin_brute_force, pin_gemm_identity, pin_involution,
        pin_special_bits, pin_degenerate]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    assert pin(transpose)


# ---- planted mistakes: each must fail at least one pin -----------------------------------------

def _no_transpose(src, rows, cols):           # forgets the transposition
    return np.array(src[:rows, :cols]).reshape(cols, rows)


def _reads_padding(src, rows, cols):          # uses the storage width as cols
    return transpose(src, rows, src.shape[1])


def _off_by_one(src, rows, cols):             # shifts the column index
    out = transpose(src, rows, cols)
    return np.roll(out, 1, axis=0) if cols > 1 else out


def _via_float_math(src, rows, cols):         # passes the values through arithmetic (x*1 + 0)
    with np.errstate(invalid="ignore"):
        return transpose(src, rows, cols) * np.float32(1.0) + np.float32(0.0)


MUTANTS = [_no_transpose, _reads_padding, _off_by_one, _via_float_math]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_planted_mistake_is_caught(mutant):
    failed = []
    for pin in PINS:
        try:
            ok = pin(mutant)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"{mutant.__name__} passed every pin"
