"""quantize_fp8_noalloc, the entry point that allocates nothing, against the
allocating quantize_fp8 through the C ABI: bit-identical codes and scales on
two calls in a row, the second with a smaller input (its scratch then holds
the first call's slots beyond the ones it writes), for contiguous and strided
tensors and the block shapes.  (Its size limit is checked on the CPU, in
test_abi.py: the call returns before launching anything.)"""
import numpy as np
import pytest
import torch

import dense_matrix_unit_amd as dmu
from dense_matrix_unit_amd import workloads as wl

pytestmark = pytest.mark.gpu


def both(X, fmt, block=None, ldq_extra=0):
    rows, cols = X.shape
    out = []
    for fn in (dmu.quantize_fp8, dmu.quantize_fp8_noalloc):
        ldq = (cols + ldq_extra + 15) // 16 * 16  # row strides are multiples of 16 bytes
        Qbig = torch.full((rows, ldq), 0xAA, dtype=torch.uint8, device="cuda")
        Q = Qbig[:, :cols]
        br, bc = (rows, cols) if block is None else block
        s = torch.full(((rows // br) * (cols // bc),), float("nan"), dtype=torch.float32,
                       device="cuda")
        fn(X, Q, s, fmt, block)
        torch.cuda.synchronize()
        out.append((Qbig.cpu().numpy(), s.cpu().numpy()))
    return out


def gpu(shape, seed, ld_extra=0, outliers=False):
    rows, cols = shape
    src = wl.normal_with_outlier_rows(shape, seed, frac=0.01)[0] if outliers else wl.normal(shape, seed)
    big = torch.zeros((rows, cols + ld_extra), dtype=torch.float32, device="cuda")
    big[:, :cols] = torch.from_numpy(src).cuda()
    return big[:, :cols]


@pytest.mark.parametrize("fmt", [dmu.E4M3, dmu.E5M2])
@pytest.mark.parametrize("first,second", [((4096, 4096), (300, 512)),
                                          ((2048, 8192), (1, 4)),
                                          ((1000, 1000), (64, 128))])
def test_noalloc_matches_quantize_fp8_twice(fmt, first, second):
    for shape, seed in ((first, 1), (second, 2)):
        (Qa, sa), (Qn, sn) = both(gpu(shape, seed), fmt)
        assert np.array_equal(Qa, Qn), shape
        assert np.array_equal(sa, sn) and np.isfinite(sa).all(), shape


@pytest.mark.parametrize("fmt", [dmu.E4M3, dmu.E5M2])
def test_noalloc_strided_rows_twice(fmt):
    # rows with a stride (ldx, ldq larger than cols): whole rows per scratch slot
    for shape, seed, extra in (((3000, 512), 3, 64), ((17, 96), 4, 32)):
        (Qa, sa), (Qn, sn) = both(gpu(shape, seed, extra), fmt, ldq_extra=extra)
        assert np.array_equal(Qa, Qn) and np.array_equal(sa, sn), shape


@pytest.mark.parametrize("block", [(1, 128), (128, 128)])
def test_noalloc_block_scales(block):
    for shape, seed in (((1024, 2048), 5), ((256, 384), 6)):
        (Qa, sa), (Qn, sn) = both(gpu(shape, seed, outliers=True), dmu.E4M3, block)
        assert np.array_equal(Qa, Qn) and np.array_equal(sa, sn), shape

