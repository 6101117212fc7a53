"""Helpers for the GPU parity tests: run the C-ABI on device copies of seeded
inputs, with canary guard bands around C, and compare with the FP64 oracle."""
import sys

import numpy as np

import fp32_gemm_08_amd as lib

CANARY = np.float32(-7777.25)
GUARD_ROWS = 2
ALGOS = ["naive", "naive_wg", "lds_tiled", "lds_tiled_nopad", "regblock", "mfma", "mfma_32", "mfma_128x64", "auto"]


def say(*msg):
    print("[gpu-case]", *msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def run_case(case, algo, c_fill=np.nan, ldc_pad=0, guard=True, stream=None, a_offset=0, b_offset=0):
    """Run one GEMM through sgemm_f32_algo; returns (status, D storage (M, ldc))
    and checks the guard rows / padding columns of C stayed untouched.

    a_offset / b_offset shift the operand base address by that many floats
    (misaligned base pointers)."""
    torch = torch_mod()
    dev = torch.device("cuda", 0)
    M, N, K = case.M, case.N, case.K
    ldc = case.ldc + ldc_pad
    Cst = np.full((M, ldc), CANARY, dtype=np.float32)
    if case.C is not None:
        Cst[:, :N] = case.C[:, :N]
    else:
        Cst[:, :N] = c_fill
    g = GUARD_ROWS if guard else 0
    full = np.full((M + 2 * g, ldc), CANARY, dtype=np.float32)
    full[g:g + M] = Cst
    dA = torch.from_numpy(np.concatenate([np.zeros(a_offset, np.float32), case.A.ravel()])).to(dev)
    dB = torch.from_numpy(np.concatenate([np.zeros(b_offset, np.float32), case.B.ravel()])).to(dev)
    dC = torch.from_numpy(full.ravel().copy()).to(dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    algo_id = lib.ALGO[algo] if isinstance(algo, str) else int(algo)
    say(f"algo={algo} M={M} N={N} K={K} transB={int(case.trans_b)} alpha={case.alpha} beta={case.beta} "
        f"lda={case.lda} ldb={case.ldb} ldc={ldc} meta={case.meta}")
    st = lib.sgemm_f32_algo(algo_id, M, N, K, case.alpha,
                            dA.data_ptr() + 4 * a_offset, case.lda,
                            dB.data_ptr() + 4 * b_offset, case.ldb, int(case.trans_b), case.beta,
                            dC.data_ptr() + 4 * g * ldc, ldc, s.cuda_stream)
    torch.cuda.synchronize()
    out = dC.cpu().numpy().reshape(M + 2 * g, ldc)
    D = out[g:g + M]
    # guard rows and padding columns must still hold the canary
    if g:
        assert np.all(out[:g].view(np.uint32) == CANARY.view(np.uint32)), "write above C"
        assert np.all(out[g + M:].view(np.uint32) == CANARY.view(np.uint32)), "write below C"
    if ldc > N:
        assert np.all(D[:, N:].view(np.uint32) == CANARY.view(np.uint32)), "write into C padding"
    return st, D


def oracle_rows(o, case, rows=None):
    D, S, _ = o.gemm_rows(case.M, case.N, case.K, case.alpha, case.A, case.B, case.trans_b,
                          case.beta, case.C, rows=rows)
    return D, S


def sample_rows(M, n=24, seed=0, tile=128):
    """First/last rows, rows on both sides of tile boundaries, and random rows."""
    rng = np.random.default_rng(seed)
    rows = {0, M - 1, min(M - 1, tile - 1), min(M - 1, tile), M // 2, max(0, M - tile)}
    while len(rows) < min(n, M):
        rows.add(int(rng.integers(0, M)))
    return np.array(sorted(rows), dtype=np.int64)
