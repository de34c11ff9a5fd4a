"""Helpers shared by the GPU parity tests: move oracle-made inputs to the GPU
and bring results back as FP64 for comparison."""
import numpy as np
import torch

import oracle
import dense_matrix_unit_amd as dmu


def dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host_bf16_codes(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return oracle.decode_bf16(host_bf16_codes(t))
    return t.cpu().numpy().astype(np.float64)


def bf16(x) -> np.ndarray:
    return oracle.encode_bf16(np.asarray(x, np.float32))


def padded(x: np.ndarray, mult: int) -> torch.Tensor:
    """GPU copy of a 2-D array whose row stride is rounded up to `mult`
    elements (the ABI wants 16-byte-multiple leading dimensions)."""
    rows, cols = x.shape
    ld = (cols + mult - 1) // mult * mult
    big = np.zeros((rows, ld), x.dtype)
    big[:, :cols] = x
    return dev(big)[:, :cols]


def empty_padded(rows, cols, dtype, mult=8):
    ld = (cols + mult - 1) // mult * mult
    return torch.empty((rows, ld), dtype=dtype, device="cuda")[:, :cols]


def run_gemm_bf16(A, B, layout, out_dtype, C=None):
    M = A.shape[0]
    N = B.shape[1] if layout == dmu.B_ROW_MAJOR else B.shape[0]
    out = empty_padded(M, N, out_dtype)
    dmu.gemm_bf16(padded(A, 8), padded(B, 8), out, layout,
                  C=None if C is None else padded(C, 4))
    torch.cuda.synchronize()
    return out


def assert_within_bound(D, D_ref, S, bf16_out, what=""):
    ok = oracle.within_bound(D, D_ref, S, bf16_out)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        det = [(tuple(i), D[tuple(i)], D_ref[tuple(i)], S[tuple(i)]) for i in idx]
        raise AssertionError("%s: %d of %d outside the bound; first: %s"
                             % (what, (~ok).sum(), ok.size, det))


def round_out(D_ref, bf16_out):
    """Exact output expected for integer-valued problems: the FP64 result is
    an exact integer below 2^24, so FP32 holds it and BF16 RNE of it is unique."""
    f32 = D_ref.astype(np.float32)
    assert np.array_equal(f32.astype(np.float64), D_ref)
    if bf16_out:
        return oracle.decode_bf16(oracle.encode_bf16(f32))
    return f32.astype(np.float64)


def within_fp8_bound(D, Dref, S, bf16_out, loss_of_rows):
    """Element-wise |D - Dref| <= 1e-5 S (+ 2^-8 |Dref| for BF16 output) + the
    FP8 instructions' own loss.  The loss (an O(MNK) computation) is only
    evaluated for rows where the FP32 term alone is exceeded: the verdict is
    the same as with the loss everywhere, since it only adds to the bound.
    loss_of_rows(r) gives the loss of the rows r (indices into D).  Returns
    the mask of elements within the bound, and the full tolerance of those rows."""
    tol = 1e-5 * S
    if bf16_out:
        tol = tol + 2.0 ** -8 * np.abs(Dref)
    err = np.abs(D - Dref)
    ok = err <= tol
    rows = np.flatnonzero(~ok.all(axis=1))
    if rows.size:
        tol_rows = tol[rows] + loss_of_rows(rows)
        ok[rows] = err[rows] <= tol_rows
        tol = tol.copy()
        tol[rows] = tol_rows
    return ok, tol
