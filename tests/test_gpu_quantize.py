"""quantize_fp8 (HIP) must equal the oracle bit for bit: codes and scales."""
import numpy as np
import pytest
import torch

import oracle
import dense_matrix_unit_amd as dmu
from dense_matrix_unit_amd import workloads as wl
from gpu_helpers import dev

pytestmark = pytest.mark.gpu
FMTS = [dmu.E4M3, dmu.E5M2]
BLOCKS = [None, (1, 128), (128, 128)]


def nan_code(q):
    return (q & 0x7F) == 0x7F


def run_quant(X, fmt, block, ldq_pad=0):
    rows, cols = X.shape
    br, bc = (rows, cols) if block is None else block
    Qbig = torch.full((rows, cols + ldq_pad), 0x5A, dtype=torch.uint8, device="cuda")
    Q = Qbig[:, :cols]
    s = torch.full(((rows // br) * (cols // bc),), -7.0, dtype=torch.float32, device="cuda")
    dmu.quantize_fp8(dev(X) if not isinstance(X, torch.Tensor) else X, Q, s, fmt, block)
    torch.cuda.synchronize()
    if ldq_pad:
        assert torch.all(Qbig[:, cols:] == 0x5A)
    return Q.cpu().numpy(), s.cpu().numpy().reshape(rows // br, cols // bc)


def compare(X, fmt, block, Q, s):
    Qr, sr = oracle.quantize_fp8(X, fmt, *(block or (None, None)))
    both_nan = nan_code(Q) & nan_code(Qr)           # NaN sign is unspecified
    assert np.array_equal(np.where(both_nan, 0, Q), np.where(both_nan, 0, Qr))
    nan_s = np.isnan(s) & np.isnan(sr)
    assert np.array_equal(np.where(nan_s, 0, s).view(np.uint32), np.where(nan_s, 0, sr).view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", BLOCKS)
def test_bit_exact_small(fmt, block):
    X, _ = wl.normal_with_outlier_rows((384, 640), 3, frac=0.02)
    Q, s = run_quant(X, fmt, block)
    compare(X, fmt, block, Q, s)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", BLOCKS)
def test_bit_exact_wide_range_and_strides(fmt, block):
    # magnitudes over many binades so FP8 subnormals, ties and saturation occur
    rng = np.random.default_rng(5)
    X = (rng.standard_normal((256, 384)) * 2.0 ** rng.integers(-30, 30, (256, 384))).astype(np.float32)
    X[0, :8] = [0.0, -0.0, 1e-40, -1e-45, 3e38, -3e38, 2.0 ** -20, 448.0]
    Xbig = np.zeros((256, 400), np.float32)
    Xbig[:, :384] = X
    Xt = dev(Xbig)[:, :384]
    Q, s = run_quant(Xt, fmt, block, ldq_pad=16)
    compare(X, fmt, block, Q, s)


@pytest.mark.parametrize("fmt", FMTS)
def test_special_blocks(fmt):
    X = wl.normal((128, 512), 4)
    X[0, 3] = np.nan            # block (0,0) of 1x128: NaN
    X[1, 130] = np.inf          # block (1,1): Inf
    X[2, 256:384] = 0.0         # block (2,2): all zero
    X[2, 300] = -0.0
    X[3, 384:512] = -2.5        # all equal
    for block in [(1, 128), (128, 128), None]:
        Q, s = run_quant(X, fmt, block)
        compare(X, fmt, block, Q, s)


@pytest.mark.parametrize("fmt", FMTS)
def test_per_tensor_4096(fmt):
    X = wl.normal((4096, 4096), wl.SEED_A)
    Q, s = run_quant(X, fmt, None)
    compare(X, fmt, None, Q, s)


def test_block_sizes_of_block_scaled_workload():
    Xa, _ = wl.normal_with_outlier_rows((8192, 7168), wl.SEED_A)
    Q, s = run_quant(Xa, dmu.E4M3, (1, 128))
    compare(Xa, dmu.E4M3, (1, 128), Q, s)
    del Xa, Q, s
    Xb = wl.normal((7168, 7168), wl.SEED_B)
    Q, s = run_quant(Xb, dmu.E4M3, (128, 128))
    compare(Xb, dmu.E4M3, (128, 128), Q, s)


def test_per_tensor_calls_on_two_streams():
    # per-tensor quantisation keeps its amax partials in a workspace shared by
    # every stream of the GPU; calls alternating between two streams, each on
    # its own tensor (one 100x the other), must each get their own amax
    X1 = wl.normal((2048, 2048), 11)
    X2 = wl.normal((2048, 2048), 12) * np.float32(100.0)
    g1, g2 = torch.from_numpy(X1).cuda(), torch.from_numpy(X2).cuda()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for it in range(6):
        st, X = (s1, g1) if it % 2 == 0 else (s2, g2)
        Q = torch.empty((2048, 2048), dtype=torch.uint8, device="cuda")
        sc = torch.empty(1, dtype=torch.float32, device="cuda")
        with torch.cuda.stream(st):
            dmu.quantize_fp8(X, Q, sc, dmu.E4M3)
        outs.append((Q, sc))
    torch.cuda.synchronize()
    refs = [oracle.quantize_fp8(X, oracle.E4M3) for X in (X1, X2)]
    for it, (Q, sc) in enumerate(outs):
        Qr, sr = refs[it % 2]
        assert np.array_equal(Q.cpu().numpy(), Qr), it
        assert sc.item() == float(sr[0, 0]), it


@pytest.mark.parametrize("fmt", FMTS)
def test_per_tensor_every_walk(fmt):
    # A contiguous tensor that the grid can hold in registers takes the
    # one-pass kernel, a strided one the two-pass row walk, and a contiguous
    # one larger than 64 MB the two-pass flat walk; all must equal the oracle.
    X = wl.normal((1024, 1024), 21)
    Q, s = run_quant(X, fmt, None)                       # one pass
    compare(X, fmt, None, Q, s)
    Xbig = np.zeros((1024, 1040), np.float32)
    Xbig[:, :1024] = X
    Q, s = run_quant(dev(Xbig)[:, :1024], fmt, None)     # rows, two passes
    compare(X, fmt, None, Q, s)
    X = wl.normal((8192, 4096), 22)
    X[5000, 7] = 300.0                                   # amax far from the first rows
    Q, s = run_quant(X, fmt, None)                       # flat, two passes
    compare(X, fmt, None, Q, s)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(1, 16), (3, 64), (384, 640), (1000, 1008), (4096, 4096)])
def test_one_pass_fallback_when_workgroups_give_up(fmt, shape):
    # With a wait bound of 0 a waiting workgroup gives up at once and the last
    # one to arrive encodes its share from X (the path taken when the grid's
    # workgroups are not all resident); which workgroups give up depends on
    # timing, and the codes must not.  Then quantize_fp8_noalloc on the same
    # scratch: the one-pass kernel must have left its sync words cleared.
    X = wl.normal(shape, 23)
    X.flat[len(X.flat) // 2] = -77.0
    g = dev(X)
    for limit in (0, 0, 4096):
        Q = torch.full(shape, 0x5A, dtype=torch.uint8, device="cuda")
        sc = torch.full((1,), -7.0, dtype=torch.float32, device="cuda")
        dmu.probe_quantize_tensor_resident(g, Q, sc, fmt, spin_limit=limit)
        torch.cuda.synchronize()
        compare(X, fmt, None, Q.cpu().numpy(), sc.cpu().numpy().reshape(1, 1))
    Q = torch.full(shape, 0x5A, dtype=torch.uint8, device="cuda")
    sc = torch.full((1,), -7.0, dtype=torch.float32, device="cuda")
    dmu.quantize_fp8_noalloc(g, Q, sc, fmt)
    torch.cuda.synchronize()
    compare(X, fmt, None, Q.cpu().numpy(), sc.cpu().numpy().reshape(1, 1))


def test_one_pass_nonfinite_tensor():
    # NaN anywhere makes the amax NaN; an Inf (no NaN) makes it Inf; both keep
    # the integer encoder, on the one-pass kernel as on the two-pass walks
    for bad in (np.nan, np.inf, -np.inf):
        X = wl.normal((512, 512), 24)
        X[100, 200] = bad
        for fmt in FMTS:
            Q, s = run_quant(X, fmt, None)
            compare(X, fmt, None, Q, s)


@pytest.mark.parametrize("fmt", FMTS)
def test_one_pass_under_graph_replay(fmt):
    # The allocation-free entry point captured once in a HIP graph and replayed
    # on new contents of the same input buffer, with eager copies and
    # synchronisations between replays: the one-pass kernel keeps no state
    # across calls but what it clears itself, so every replay must match the
    # oracle, and so must an eager call after the replays.
    shape = (2048, 1024)
    Xs = [wl.normal(shape, 30 + k) * np.float32(10.0 ** (k - 1)) for k in range(3)]
    Xg = torch.from_numpy(Xs[0]).cuda()
    Q = torch.empty(shape, dtype=torch.uint8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    dmu.quantize_fp8_noalloc(Xg, Q, sc, fmt)      # outside the capture first
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dmu.quantize_fp8_noalloc(Xg, Q, sc, fmt)
    torch.cuda.synchronize()
    for rep in range(6):
        X = Xs[rep % 3]
        Xg.copy_(torch.from_numpy(X))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        compare(X, fmt, None, Q.cpu().numpy(), sc.cpu().numpy().reshape(1, 1))
    dmu.quantize_fp8_noalloc(Xg, Q, sc, fmt)
    torch.cuda.synchronize()
    compare(Xs[5 % 3], fmt, None, Q.cpu().numpy(), sc.cpu().numpy().reshape(1, 1))
