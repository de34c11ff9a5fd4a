"""A bank-conflict model of shared memory (LDS), checked first against the
worked example of the vidyal.ai page, Step 3 ("bank conflicts and the XOR
swizzle"; tests/golden/bank_groups_step3.json), then applied to the 16-byte
fragment reads of this library's GEMM kernel (csrc/gemm.hip) and the 8-byte
transposing V reads of its attention kernel (csrc/attention.hip) on gfx950.

Model: memory is `banks` banks of 4 bytes, word w in bank w mod banks.  An
access by a group of lanes served together takes as many wavefronts as the
largest number of distinct words any one bank must deliver (lanes reading the
same word share it).  A wide access is served a group of lanes at a time, as
many lanes as the banks can feed at once, and the groups' wavefronts add up."""
import json
import os

import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bank_groups_step3.json")


def wavefronts(byte_addrs, access_bytes, banks, lanes_per_pass):
    """Wavefronts to serve one access: byte_addrs[l] is lane l's first byte,
    each lane reading access_bytes (a multiple of 4)."""
    total = 0
    for g in range(0, len(byte_addrs), lanes_per_pass):
        words_per_bank = {}
        for a in byte_addrs[g:g + lanes_per_pass]:
            for w in range(a // 4, (a + access_bytes) // 4):
                words_per_bank.setdefault(w % banks, set()).add(w)
        total += max(len(ws) for ws in words_per_bank.values())
    return total


def bank_group(byte_addr, banks):
    """16-byte bank group of an address (banks / 4 groups)."""
    return (byte_addr // 16) % (banks // 4)


# ---- the page's three layouts (64-byte rows of 4 chunks)
def page_offset(layout, row, chunk, row_bytes=64, pad=16):
    if layout == "pad":
        return row * (row_bytes + pad) + 16 * chunk
    if layout == "swz":
        return row * row_bytes + 16 * (chunk ^ ((row >> 1) & 3))
    return row * row_bytes + 16 * chunk


def test_model_reproduces_the_page_table():
    g = json.load(open(GOLDEN))
    for layout in ("none", "pad", "swz"):
        addrs = [page_offset(layout, r, 0) for r in range(8)]
        assert [bank_group(a, g["banks"]) for a in addrs] == \
            g["rows_0_7_chunk_0_bank_groups"][layout]
        # one 8 x 8 matrix: 8 rows of 16 bytes, served together
        assert wavefronts(addrs, 16, g["banks"], 8) == g["passes"][layout]


def test_model_reproduces_the_four_matrix_count():
    # four 8 x 8 matrices (rows 0-7, chunks 0-3) are four separate 8-row
    # accesses: 16 wavefronts plain, the minimum of 4 when padded or swizzled
    g = json.load(open(GOLDEN))
    got = {lay: sum(wavefronts([page_offset(lay, r, c) for r in range(8)], 16, g["banks"], 8)
                    for c in range(4)) for lay in ("none", "pad", "swz")}
    assert got["none"] == g["four_matrices_wavefronts"]["none"]
    assert got["pad"] == got["swz"] == g["four_matrices_wavefronts"]["minimum"]


# ---- gfx950: the GEMM kernel's LDS tile rows of 128 bytes (8 chunks of 16)
def kernel_offset(layout, row, chunk):
    """Byte offset of logical 16-byte chunk `chunk` of tile row `row`:
    swizzled (the kernel's layout: position chunk ^ ((row ^ row >> 3) & 7)),
    plain (128-byte rows) or padded (144-byte rows)."""
    if layout == "swz":
        return row * 128 + 16 * (chunk ^ ((row ^ (row >> 3)) & 7))
    if layout == "pad":
        return row * 144 + 16 * chunk
    return row * 128 + 16 * chunk


def fragment_read(layout, base_row, c0, c1):
    """One 16-byte-per-lane fragment read of a 32x32 MFMA operand: lane l reads
    tile row base_row + l % 32, logical chunk c0 (lanes 0-31) or c1 (lanes
    32-63) -- the kernel's BF16 step (c0, c1 = 2s, 2s+1) or one of the two
    reads of an FP8 step."""
    return [kernel_offset(layout, base_row + l % 32, c0 if l < 32 else c1) for l in range(64)]


# two readings of gfx950's LDS for 128-bit reads: 32 banks serving 8 lanes
# at a time, or 64 banks serving 16 lanes at a time
LDS_MODELS = [(32, 8), (64, 16)]


@pytest.mark.parametrize("banks,lanes", LDS_MODELS)
def test_kernel_fragment_reads_are_conflict_free_when_swizzled(banks, lanes):
    minimum = 64 * 16 // (banks * 4)
    for base_row in range(0, 256, 32):  # every 32-row block of a 256-row tile
        for s in range(4):               # BF16 steps: chunks 2s, 2s+1
            assert wavefronts(fragment_read("swz", base_row, 2 * s, 2 * s + 1), 16, banks,
                              lanes) == minimum
        for s in range(2):               # FP8 steps: two reads, chunks 4s+h, 4s+2+h
            for h in range(2):
                assert wavefronts(fragment_read("swz", base_row, 4 * s + h, 4 * s + 2 + h), 16,
                                  banks, lanes) == minimum


@pytest.mark.parametrize("banks,lanes", LDS_MODELS)
def test_kernel_fragment_reads_plain_and_padded(banks, lanes):
    # the ablation's two other layouts: plain 128-byte rows put every lane of
    # a pass in the same bank group (8-way); 144-byte rows spread them
    minimum = 64 * 16 // (banks * 4)
    for base_row in (0, 96, 224):
        for s in range(4):
            plain = wavefronts(fragment_read("plain", base_row, 2 * s, 2 * s + 1), 16, banks, lanes)
            pad = wavefronts(fragment_read("pad", base_row, 2 * s, 2 * s + 1), 16, banks, lanes)
            assert plain == 8 * minimum
            assert pad == minimum


def test_dma_writes_are_contiguous():
    # the direct global->LDS copies write 64 lanes x 16 bytes at consecutive
    # addresses: conflict-free in either model, whatever the layout (the
    # swizzle is applied to the global source offsets, not the LDS side)
    for banks, lanes in LDS_MODELS:
        assert wavefronts([16 * l for l in range(64)], 16, banks, lanes) == 64 * 16 // (banks * 4)


# ---- gfx950: the attention kernel's transposing reads of V (csrc/attention.hip)
def vswz(d, j):
    """Swizzle of V row j's 16-byte chunks: bits 2-3 of the chunk index flipped
    with the row (d = 128: j % 4; d = 64: bit 1 of j)."""
    return (j & 3) << 2 if d == 128 else ((j >> 1) & 1) << 2


def v_read(d, nt, ks, second, swizzled=True):
    """Byte addresses of one ds_read_b64_tr_b16 of V (8 bytes per lane): lane
    l = 32 h + 16 g + i reads row 4h + i/4 (+ 16 ks, + 8 for the step's second
    read) at 16-bit elements 4 (i % 4) .. +3 of columns 32 nt + 16 (g % 2)."""
    vrow = 2 * d
    out = []
    for lane in range(64):
        h, g, i = lane >> 5, lane >> 4, lane & 15
        chunk = 4 * nt + 2 * (g & 1) + ((i & 3) >> 1)
        if swizzled:
            chunk ^= vswz(d, i >> 2)
        out.append(16 * ks * vrow + (8 * vrow if second else 0) + (4 * h + (i >> 2)) * vrow +
                   (chunk << 4) + ((i & 1) << 3))
    return out


@pytest.mark.parametrize("d", [64, 128])
def test_attention_v_reads_conflict_free_with_64_banks(d):
    # 64 banks serve 32 lanes of 8 bytes at a time: 2 wavefronts at best
    for nt in range(d // 32):
        for ks in range(4):
            for second in (False, True):
                assert wavefronts(v_read(d, nt, ks, second), 8, 64, 32) == 2
                # without the swizzle the 4 rows' 64-byte runs share banks
                assert wavefronts(v_read(d, nt, ks, second, swizzled=False), 8, 64, 32) > 2


@pytest.mark.parametrize("d", [64, 128])
def test_attention_v_reads_with_32_banks(d):
    # 32 banks serve 16 lanes of 8 bytes (4 rows x 32 bytes): rows j and j+2
    # of the swizzle land 128 bytes apart, so the reads are 2-way conflicted
    # (8 wavefronts, against 4 at best and 16 without the swizzle).  gfx950's
    # LDS is the 64-bank case: 16-byte reads sustain more than 128 bytes per
    # clock per CU, which 32 banks of 4 bytes cannot deliver.
    for nt in range(d // 32):
        for ks in range(4):
            for second in (False, True):
                assert wavefronts(v_read(d, nt, ks, second), 8, 32, 16) == 8
                assert wavefronts(v_read(d, nt, ks, second, swizzled=False), 8, 32, 16) == 16


# ---- gfx950: the GEMM kernel's transposing reads of a row-major B slice
# (csrc/gemm.hip, B stored K x N): 64 K rows of 512 bytes (256 BF16 columns,
# 32 chunks of 16 bytes), chunk c of K row r at position c ^ ((r % 4) << 2)
def brow_read(wn, j, s, second, swizzled=True):
    """Byte addresses of one ds_read_b64_tr_b16 of sub-tile j of wave column
    wn at K step s (8 bytes per lane): lane l = 32 h + 16 g + i reads K row
    16 s + 8 h + i/4 (+ 4 for the second read) at 16-bit elements
    4 (i % 4) .. +3 of columns 128 wn + 32 j + 16 (g % 2)."""
    out = []
    for lane in range(64):
        h, g, i = lane >> 5, lane >> 4, lane & 15
        row = 16 * s + 8 * h + (4 if second else 0) + (i >> 2)
        chunk = (128 * wn + 32 * j) // 8 + 2 * (g & 1) + ((i & 3) >> 1)
        if swizzled:
            chunk ^= (row & 3) << 2
        out.append(row * 512 + (chunk << 4) + ((i & 1) << 3))
    return out


def test_row_major_b_reads_conflict_free_with_64_banks():
    # every read of every wave column, sub-tile and step: 2 wavefronts, the
    # minimum for 512 bytes; unswizzled, the 4 K rows of a 16-lane group share
    # one 64-byte bank run (512-byte rows)
    for wn in range(2):
        for j in range(4):
            for s in range(4):
                for second in (False, True):
                    assert wavefronts(brow_read(wn, j, s, second), 8, 64, 32) == 2
                    assert wavefronts(brow_read(wn, j, s, second, swizzled=False), 8, 64, 32) == 8


def test_row_major_b_reads_cover_the_fragment():
    # lane l of the two reads gets column l % 32 of the sub-tile and K values
    # 8 (l / 32) + 0..7 of the step, the K run its A fragment holds (one
    # 16-byte chunk per lane); each read's 16-lane group names 4 K rows x 16
    # columns, element e of lane i's 8 bytes being column 4 (i % 4) + e
    for wn in range(2):
        for j in range(4):
            for s in range(4):
                got = {}
                for second in (False, True):
                    addrs = brow_read(wn, j, s, second)
                    for lane in range(64):
                        g, i = lane >> 4, lane & 15
                        for e in range(4):
                            a = addrs[lane] + 2 * e
                            row, pos = a // 512, (a % 512) // 16
                            col = 8 * (pos ^ ((row & 3) << 2)) + (a % 16) // 2
                            # the transposed result: lane 16 g + t of the group
                            # receives column t of the 4 rows named by i / 4
                            t = 4 * (i & 3) + e
                            got.setdefault((16 * g + t, row), col)
                for lane in range(64):
                    rows = sorted(r for (l, r) in got if l == lane)
                    assert rows == [16 * s + 8 * (lane >> 5) + k for k in range(8)]
                    assert {got[(lane, r)] for r in rows} == {128 * wn + 32 * j + lane % 32}
