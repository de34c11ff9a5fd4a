"""The C-ABI library loads on the CPU host, exports every function the public
headers declare, and rejects bad arguments before launching anything (every
call below fails validation, so no GPU is touched)."""
import glob
import os
import re

import pytest

import dense_matrix_unit_amd as dmu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    lib = dmu.load_library()
    names = declared_functions()
    assert {"gemm_bf16", "gemm_fp8_scaled", "quantize_fp8", "dmu_status_string"} <= names
    for n in names:
        assert hasattr(lib, n), n
        assert n in dmu.SYMBOLS, n


def test_status_strings_and_version():
    lib = dmu.load_library()
    assert lib.dmu_version() >> 16 == 1
    for s in (0, -1, -2, -3, 7):
        assert lib.dmu_status_string(s)
    assert b"INVALID" in lib.dmu_status_string(-1)


FAKE = 1 << 20  # aligned, never dereferenced: every call below is rejected first


def call_bf16(**kw):
    a = dict(A=FAKE, lda=64, B=FAKE, ldb=64, b_layout=1, C=None, ldc=0, D=FAKE, ldd=64,
             d_dtype=0, M=64, N=64, K=64, stream=None)
    a.update(kw)
    return dmu.load_library().gemm_bf16(*a.values())


@pytest.mark.parametrize("kw", [
    dict(A=None), dict(B=None), dict(D=None), dict(M=0), dict(N=-1), dict(K=0), dict(K=12),
    dict(lda=32), dict(ldb=32), dict(ldd=32), dict(b_layout=2), dict(d_dtype=5),
    dict(A=FAKE + 2), dict(D=FAKE + 8), dict(lda=68), dict(C=FAKE, ldc=8),
    dict(C=FAKE, ldc=64, d_dtype=1), dict(b_layout=0, ldb=60),
])
def test_gemm_bf16_rejects(kw):
    assert call_bf16(**kw) == dmu.DMU_ERR_INVALID_ARG


def test_gemm_bf16_unsupported_huge_ld():
    assert call_bf16(lda=1 << 23, K=64) == dmu.DMU_ERR_UNSUPPORTED


def call_fp8(**kw):
    a = dict(A=FAKE, lda=128, fa=0, B=FAKE, ldb=128, fb=0, sa=FAKE, sb=FAKE, mode=0, C=None,
             ldc=0, D=FAKE, ldd=64, d_dtype=1, M=64, N=64, K=128, stream=None)
    a.update(kw)
    return dmu.load_library().gemm_fp8_scaled(*a.values())


@pytest.mark.parametrize("kw", [
    dict(A=None), dict(sa=None), dict(sb=None), dict(fa=2), dict(fb=-1), dict(mode=3),
    dict(K=8), dict(K=136, mode=1, lda=144, ldb=144), dict(lda=120), dict(ldb=136),
    dict(sa=FAKE + 2), dict(M=0),
])
def test_gemm_fp8_rejects(kw):
    assert call_fp8(**kw) == dmu.DMU_ERR_INVALID_ARG


def call_quant(**kw):
    a = dict(X=FAKE, rows=256, cols=256, ldx=256, fmt=0, br=1, bc=128, Q=FAKE, ldq=256,
             scales=FAKE, stream=None)
    a.update(kw)
    return dmu.load_library().quantize_fp8(*a.values())


@pytest.mark.parametrize("kw", [
    dict(X=None), dict(Q=None), dict(scales=None), dict(rows=0), dict(fmt=2), dict(ldx=128),
    dict(ldq=200), dict(br=3), dict(bc=100), dict(X=FAKE + 4), dict(ldx=258),
])
def test_quantize_rejects(kw):
    assert call_quant(**kw) == dmu.DMU_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(br=2, bc=128), dict(br=1, bc=64), dict(br=256, bc=128)])
def test_quantize_unsupported_blocks(kw):
    assert call_quant(**kw) == dmu.DMU_ERR_UNSUPPORTED


def test_python_binding_rejects_cpu_tensors():
    import torch

    A = torch.zeros(64, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        dmu.gemm_bf16(A, A, torch.zeros(64, 64))


def call_mx(**kw):
    a = dict(A=FAKE, lda=256, fa=0, B=FAKE, ldb=256, fb=0, sa=FAKE, ldsa=8, sb=FAKE, ldsb=8,
             C=None, ldc=0, D=FAKE, ldd=64, d_dtype=1, M=64, N=64, K=256, stream=None)
    a.update(kw)
    return dmu.load_library().gemm_mxfp8(*a.values())


@pytest.mark.parametrize("kw", [
    dict(A=None), dict(B=None), dict(sa=None), dict(sb=None), dict(D=None), dict(fa=2),
    dict(fb=-1), dict(K=96), dict(K=160, lda=160, ldb=160), dict(K=0), dict(lda=240),
    dict(ldsa=4), dict(ldsb=6), dict(ldsa=10), dict(sa=FAKE + 2), dict(sb=FAKE + 1),
    dict(A=FAKE + 8), dict(M=0), dict(N=0), dict(d_dtype=3), dict(ldd=60),
])
def test_gemm_mxfp8_rejects(kw):
    assert call_mx(**kw) == dmu.DMU_ERR_INVALID_ARG


def test_gemm_mxfp8_unsupported_huge_scale_ld():
    assert call_mx(ldsa=1 << 24) == dmu.DMU_ERR_UNSUPPORTED


def call_qmx(**kw):
    a = dict(X=FAKE, rows=64, cols=256, ldx=256, fmt=0, Q=FAKE, ldq=256, S=FAKE, lds=8,
             stream=None)
    a.update(kw)
    return dmu.load_library().quantize_mxfp8(*a.values())


@pytest.mark.parametrize("kw", [
    dict(X=None), dict(Q=None), dict(S=None), dict(rows=0), dict(cols=0), dict(cols=48, ldx=48,
    ldq=64), dict(cols=16, ldx=16, ldq=16), dict(fmt=2), dict(ldx=250), dict(ldq=240),
    dict(ldq=264), dict(lds=7), dict(X=FAKE + 4), dict(Q=FAKE + 8),
])
def test_quantize_mxfp8_rejects(kw):
    assert call_qmx(**kw) == dmu.DMU_ERR_INVALID_ARG


def call_mx4(**kw):
    a = dict(A=FAKE, lda=512, B=FAKE, ldb=512, sa=FAKE, ldsa=16, sb=FAKE, ldsb=16, C=None, ldc=0,
             D=FAKE, ldd=64, d_dtype=1, M=64, N=64, K=512, stream=None)
    a.update(kw)
    return dmu.load_library().gemm_mxfp4(*a.values())


@pytest.mark.parametrize("kw", [
    dict(A=None), dict(B=None), dict(sa=None), dict(sb=None), dict(D=None), dict(K=256),
    dict(K=768, lda=768, ldb=768), dict(lda=496), dict(lda=528), dict(ldsa=8), dict(ldsb=20),
    dict(sa=FAKE + 4), dict(sb=FAKE + 8), dict(A=FAKE + 8), dict(M=0), dict(d_dtype=2),
])
def test_gemm_mxfp4_rejects(kw):
    assert call_mx4(**kw) == dmu.DMU_ERR_INVALID_ARG


def call_qmx4(**kw):
    a = dict(X=FAKE, rows=64, cols=256, ldx=256, Q=FAKE, ldq=256, S=FAKE, lds=8, stream=None)
    a.update(kw)
    return dmu.load_library().quantize_mxfp4(*a.values())


@pytest.mark.parametrize("kw", [
    dict(X=None), dict(Q=None), dict(S=None), dict(rows=0), dict(cols=48, ldx=48, ldq=64),
    dict(ldq=272), dict(ldq=224), dict(lds=7), dict(X=FAKE + 4), dict(Q=FAKE + 8),
])
def test_quantize_mxfp4_rejects(kw):
    assert call_qmx4(**kw) == dmu.DMU_ERR_INVALID_ARG


def call_grouped(**kw):
    a = dict(A=FAKE, lda=64, B=FAKE, ldb=64, stride_b=64 * 64, off=FAKE, G=4, D=FAKE, ldd=64,
             d_dtype=1, max_m=256, N=64, K=64, stream=None)
    a.update(kw)
    return dmu.load_library().gemm_grouped_bf16(*a.values())


@pytest.mark.parametrize("kw", [
    dict(A=None), dict(B=None), dict(off=None), dict(D=None), dict(G=0), dict(G=70000),
    dict(K=12), dict(lda=60), dict(ldb=60), dict(stride_b=64 * 63), dict(stride_b=64 * 64 + 4),
    dict(off=FAKE + 4), dict(A=FAKE + 2), dict(max_m=0), dict(N=0), dict(d_dtype=7),
])
def test_gemm_grouped_rejects(kw):
    assert call_grouped(**kw) == dmu.DMU_ERR_INVALID_ARG


def call_bf16_fused(**kw):
    a = dict(A=FAKE, lda=64, B=FAKE, ldb=64, b_layout=1, bias=None, act=0, D=FAKE, ldd=64,
             d_dtype=2, d_scale=FAKE, M=64, N=64, K=64, stream=None)
    a.update(kw)
    return dmu.load_library().gemm_bf16_fused(*a.values())


@pytest.mark.parametrize("kw", [
    dict(A=None), dict(D=None), dict(act=4), dict(act=-1), dict(d_dtype=4), dict(d_scale=None),
    dict(d_scale=FAKE + 2), dict(bias=FAKE + 1), dict(ldd=56, N=56, d_dtype=2), dict(K=12),
    dict(b_layout=3), dict(M=0),
])
def test_gemm_bf16_fused_rejects(kw):
    assert call_bf16_fused(**kw) == dmu.DMU_ERR_INVALID_ARG


def call_fp8_fused(**kw):
    a = dict(A=FAKE, lda=128, fa=0, B=FAKE, ldb=128, fb=0, sa=FAKE, sb=FAKE, bias=None, act=2,
             D=FAKE, ldd=64, d_dtype=1, d_scale=None, M=64, N=64, K=128, stream=None)
    a.update(kw)
    return dmu.load_library().gemm_fp8_fused(*a.values())


@pytest.mark.parametrize("kw", [
    dict(sa=None), dict(sb=None), dict(fa=4), dict(K=8), dict(d_dtype=3), dict(act=9),
    dict(lda=120), dict(D=FAKE + 4),
])
def test_gemm_fp8_fused_rejects(kw):
    assert call_fp8_fused(**kw) == dmu.DMU_ERR_INVALID_ARG


def call_attention(**kw):
    a = dict(Q=FAKE, ldq=128, hq=128 * 256, K=FAKE, ldk=128, hk=128 * 256, V=FAKE, ldv=128,
             hv=128 * 256, O=FAKE, ldo=128, ho=128 * 256, lse=None, heads=2, Sq=256, Sk=256,
             d=128, scale=0.088, causal=0, stream=None)
    a.update(kw)
    return dmu.load_library().attention_bf16(*a.values())


@pytest.mark.parametrize("kw", [
    dict(Q=None), dict(K=None), dict(V=None), dict(O=None), dict(d=96), dict(d=256),
    dict(heads=0), dict(Sq=0), dict(Sk=-1), dict(causal=2), dict(causal=1, Sq=300),
    dict(scale=0.0), dict(scale=-1.0), dict(scale=float("inf")), dict(scale=float("nan")),
    dict(ldq=120), dict(ldk=100), dict(ldv=132), dict(ldo=64), dict(hq=-8), dict(hv=12),
    dict(Q=FAKE + 8), dict(O=FAKE + 2), dict(lse=FAKE + 2),
    # heads whose outputs overlap: stride 0, one row short of a whole head,
    # side by side in a row stride that cannot hold both
    dict(ho=0), dict(ho=128 * 255), dict(ho=128, ldo=192), dict(ho=64, ldo=256),
])
def test_attention_rejects(kw):
    assert call_attention(**kw) == dmu.DMU_ERR_INVALID_ARG


def test_attention_rejects_heads_past_32_bit_offsets():
    # Q's rows span 2^31 bytes; the output heads are laid out without overlap
    assert call_attention(ldq=1 << 16, Sq=1 << 15, ho=1 << 22) == dmu.DMU_ERR_UNSUPPORTED


def call_quantize(fn, **kw):
    a = dict(X=FAKE, rows=64, cols=128, ldx=128, fmt=0, br=64, bc=128, Q=FAKE, ldq=128, s=FAKE,
             stream=None)
    a.update(kw)
    return getattr(dmu.load_library(), fn)(*a.values())


@pytest.mark.parametrize("fn", ["quantize_fp8", "quantize_fp8_noalloc"])
@pytest.mark.parametrize("kw", [
    dict(X=None), dict(Q=None), dict(s=None), dict(rows=0), dict(fmt=2), dict(ldx=126),
    dict(ldq=120), dict(br=3), dict(X=FAKE + 4), dict(Q=FAKE + 8), dict(s=FAKE + 2),
])
def test_quantize_rejects(fn, kw):
    assert call_quantize(fn, **kw) == dmu.DMU_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,rc", [
    (dict(X=None), dmu.DMU_ERR_INVALID_ARG), (dict(Q=None), dmu.DMU_ERR_INVALID_ARG),
    (dict(s=None), dmu.DMU_ERR_INVALID_ARG), (dict(rows=0), dmu.DMU_ERR_INVALID_ARG),
    (dict(cols=120), dmu.DMU_ERR_INVALID_ARG), (dict(fmt=2), dmu.DMU_ERR_INVALID_ARG),
    (dict(spin=-1), dmu.DMU_ERR_INVALID_ARG), (dict(spin=(1 << 16) + 1), dmu.DMU_ERR_INVALID_ARG),
    (dict(X=FAKE + 4), dmu.DMU_ERR_INVALID_ARG),
])
def test_probe_quantize_resident_rejects(kw, rc):
    a = dict(X=FAKE, rows=256, cols=128, fmt=0, Q=FAKE, s=FAKE, spin=0, stream=None)
    a.update(kw)
    assert dmu.load_library().dmu_probe_quantize_tensor_resident(*a.values()) == rc
