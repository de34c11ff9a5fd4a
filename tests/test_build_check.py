"""The build's scan of hand-waited LDS reads (dense_matrix_unit_amd.build.
scan_lds_asm_waits) on small listings: it accepts reads whose registers are
used only after the covering s_waitcnt, and rejects a use or an overwrite
before it -- in any operand position and with operand modifiers -- and any
label or branch met while reads are pending."""
import pytest

from dense_matrix_unit_amd.build import scan_lds_asm_waits

HEAD = ["_Zkernel:\n"]


def listing(body):
    return HEAD + ["\t%s\n" % line for line in body]


GOOD = [
    "s_waitcnt lgkmcnt(0)",
    "ds_read_b64_tr_b16 v[8:9], v1 offset:0",
    "ds_read_b64_tr_b16 v[10:11], v1 offset:2048",
    "ds_read_b64_tr_b16 v[12:13], v2 offset:0",
    "ds_read_b64_tr_b16 v[14:15], v2 offset:2048",
    "s_waitcnt lgkmcnt(2)",
    "v_mfma_f32_32x32x16_bf16 v[20:35], v[8:11], v[40:43], v[20:35]",
    "s_waitcnt lgkmcnt(0)",
    "v_mfma_f32_32x32x16_bf16 v[20:35], v[12:15], v[40:43], v[20:35]",
]


def test_accepts_uses_after_their_wait():
    assert scan_lds_asm_waits(listing(GOOD)) == 4


def test_rejects_a_use_before_the_wait():
    bad = GOOD[:5] + ["s_waitcnt lgkmcnt(2)",
                      "v_mfma_f32_32x32x16_bf16 v[20:35], v[12:15], v[40:43], v[20:35]"]
    with pytest.raises(RuntimeError):
        scan_lds_asm_waits(listing(bad))


def test_rejects_a_copy_before_the_wait():
    bad = GOOD[:3] + ["v_mov_b32_e32 v50, v9"]
    with pytest.raises(RuntimeError):
        scan_lds_asm_waits(listing(bad))


def test_rejects_an_overwrite_before_the_wait():
    bad = GOOD[:3] + ["v_add_f32_e32 v10, v3, v4"]
    with pytest.raises(RuntimeError):
        scan_lds_asm_waits(listing(bad))


def test_a_new_function_starts_clean_and_empty_listing_is_an_error():
    assert scan_lds_asm_waits(listing(GOOD[:3]) + ["_Zother:\n", "\tv_mov_b32_e32 v50, v9\n"]) == 2
    with pytest.raises(RuntimeError):
        scan_lds_asm_waits(HEAD)


@pytest.mark.parametrize("use", [
    "v_add_f32_e64 v50, -v9, v3",            # negated source
    "v_add_f32_e64 v50, |v10|, v3",          # absolute value
    "v_fma_f32 v50, -|v11|, v3, v4",         # both
    "v_cvt_f32_f16_sdwa v50, sext(v8) dst_sel:DWORD src0_sel:WORD_0",
])
def test_rejects_modified_operands(use):
    with pytest.raises(RuntimeError):
        scan_lds_asm_waits(listing(GOOD[:3] + [use]))


@pytest.mark.parametrize("use", [
    "ds_write_b64 v1, v[8:9] offset:64",      # stored data
    "ds_write_b32 v9, v3",                    # address
    "buffer_store_dword v10, v2, s[0:3], 0 offen",
    "global_store_dwordx2 v[2:3], v[10:11], off",
    "ds_read_b64 v[8:9], v1",                 # a second read into a pending register
    "global_load_dword v11, v[2:3], off",
])
def test_rejects_memory_operands(use):
    with pytest.raises(RuntimeError):
        scan_lds_asm_waits(listing(GOOD[:3] + [use]))


def test_rejects_control_flow_while_pending():
    with pytest.raises(RuntimeError):
        scan_lds_asm_waits(listing(GOOD[:3]) + [".LBB0_2:\n"])
    with pytest.raises(RuntimeError):
        scan_lds_asm_waits(listing(GOOD[:3] + ["s_cbranch_scc1 .LBB0_2"]))
    # after the wait both are fine
    ok = GOOD + ["s_cbranch_scc1 .LBB0_2"]
    assert scan_lds_asm_waits(listing(ok) + [".LBB0_2:\n"]) == 4


def test_unrelated_registers_and_comments_pass():
    body = GOOD[:3] + ["v_add_f32_e64 v50, -v7, |v12|  ; v9 in a comment",
                       "v_mov_b32_e32 v90, v91"] + GOOD[3:]
    assert scan_lds_asm_waits(listing(body)) == 4
