"""CPU checks of the C ABI: the library loads, exports every declared symbol,
rejects invalid arguments before touching the GPU, and its host-side
scheduler / LDS / bounds helpers (the same inline code the kernels run) obey
their contracts and the pages' printed examples."""
import json
import os
import re

import pytest

from tiled_dense_gemm_09_amd import tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "tg.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tg_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    syms = declared_symbols()
    assert set(syms) >= {"tg_gemm", "tg_gemm_bias_act", "tg_gemm_qkv"}
    for s in syms:
        assert hasattr(tg.lib, s), s
    assert set(syms) == set(tg.SYMBOLS)


def test_synchronising_build_loads_and_exports_the_same_symbols():
    # libtg_debugsync.so: the same sources with every pipeline wait a full
    # wait; a GPU test compares its outputs with libtg.so's bit for bit
    dbg = tg.load_library(tg.DEBUG_SYNC_PATH)
    for s in declared_symbols():
        assert hasattr(dbg, s), s
    assert dbg.tg_status_string(1) == b"TG_ERROR_INVALID_VALUE"
    assert dbg.tg_workspace_bytes() == 0


def test_status_strings():
    assert tg.lib.tg_status_string(0) == b"TG_SUCCESS"
    assert tg.lib.tg_status_string(1) == b"TG_ERROR_INVALID_VALUE"
    assert tg.lib.tg_status_string(99) == b"TG_UNKNOWN_STATUS"


FAKE_A = 0x7F0000000000
FAKE_B = 0x7F0010000000
FAKE_C = 0x7F0020000000


@pytest.mark.parametrize("args", [
    dict(dt=7),                       # unknown dtype
    dict(M=-1),                       # negative size
    dict(K=1 << 31),                  # too large
    dict(lda=31),                     # pitch shorter than the row
    dict(ldb=63),
    dict(ldc=10),
    dict(A=0),                        # NULL input
    dict(C=0),                        # NULL output
    dict(C=FAKE_A + 64),              # output overlaps A
    dict(act=5),                      # unknown activation
    dict(bias=FAKE_B + 1, act=1),     # misaligned bias
])
def test_invalid_arguments_launch_nothing(args):
    a = dict(dt=1, M=64, N=64, K=32, A=FAKE_A, lda=32, B=FAKE_B, ldb=64, C=FAKE_C, ldc=64,
             bias=0, act=0)
    a.update(args)
    if a["bias"] or a["act"]:
        st = tg.lib.tg_gemm_bias_act(a["dt"], a["M"], a["N"], a["K"], a["A"], a["lda"], a["B"],
                                     a["ldb"], a["bias"] or None, a["act"], a["C"], a["ldc"],
                                     None)
    else:
        st = tg.lib.tg_gemm(a["dt"], a["M"], a["N"], a["K"], a["A"], a["lda"], a["B"], a["ldb"],
                            a["C"], a["ldc"], None)
    assert st == 1


FAKE_R = 0x7F0030000000


@pytest.mark.parametrize("args", [
    dict(op=2),                       # unknown operand form
    dict(op=1, ldb=31),               # B stored [N,K]: pitch shorter than K
    dict(op=0, ldb=63),               # B [K,N]: pitch shorter than N
    dict(ldr=63),                     # residual pitch shorter than N
    dict(R=FAKE_R + 1),               # misaligned residual
    dict(R=FAKE_C + 128),             # residual overlapping C without being C
    dict(R=FAKE_C, ldr=72),           # C itself but with another pitch
    dict(op=1, C=FAKE_B + 64 * 16),   # C inside B's [N,K] extent
])
def test_invalid_extended_arguments_launch_nothing(args):
    a = dict(dt=2, M=64, N=64, K=32, A=FAKE_A, lda=32, B=FAKE_B, ldb=32, op=1, C=FAKE_C, ldc=64,
             bias=0, act=0, R=FAKE_R, ldr=64)
    a.update(args)
    st = tg.lib.tg_gemm_ex(a["dt"], a["M"], a["N"], a["K"], a["A"], a["lda"], a["B"], a["ldb"],
                           a["op"], a["bias"] or None, a["act"], a["R"] or None, a["ldr"], a["C"],
                           a["ldc"], None)
    assert st == 1


def test_extended_empty_problem_is_a_noop():
    assert tg.lib.tg_gemm_ex(1, 0, 64, 64, FAKE_A, 64, FAKE_B, 64, 1, None, 0, FAKE_C, 64,
                             FAKE_C, 64, None) == 0


FAKE_SA = 0x7F0040000000
FAKE_SB = 0x7F0050000000


@pytest.mark.parametrize("args", [
    dict(fa=3),                       # unknown 8-bit format
    dict(odt=7),                      # unknown output dtype
    dict(K=48),                       # K not a multiple of the 32-element scale block
    dict(lda=63),                     # A pitch (bytes) shorter than K
    dict(ldb=63),
    dict(ldsa=255),                   # scale pitch shorter than M
    dict(ldsb=255),
    dict(SA=0),                       # NULL scales
    dict(C=FAKE_A + 128),             # output overlapping A
    dict(C=FAKE_SB + 64),             # output overlapping the B scales
    dict(act=4),
])
def test_invalid_mx_arguments_launch_nothing(args):
    a = dict(fa=0, fb=1, M=256, N=256, K=64, A=FAKE_A, lda=64, SA=FAKE_SA, ldsa=256, B=FAKE_B,
             ldb=64, SB=FAKE_SB, ldsb=256, bias=0, act=0, odt=2, C=FAKE_C, ldc=256)
    a.update(args)
    st = tg.lib.tg_gemm_mx(a["fa"], a["fb"], a["M"], a["N"], a["K"], a["A"], a["lda"],
                           a["SA"] or None, a["ldsa"], a["B"], a["ldb"], a["SB"], a["ldsb"],
                           a["bias"] or None, a["act"], a["odt"], a["C"], a["ldc"], None)
    assert st == 1


@pytest.mark.parametrize("args,status", [
    (dict(dt=5), 1),                   # unknown dtype
    (dict(D=0), 1),                    # empty head dimension
    (dict(D=256), 2),                  # head dimension beyond the kernels
    (dict(S=-1), 1),
    (dict(Q=0), 1),                    # NULL input
    (dict(O=FAKE_A + 64), 1),          # output overlapping Q
    (dict(lse=FAKE_C + 2), 1),         # misaligned log-sum-exp
])
def test_invalid_attention_arguments_launch_nothing(args, status):
    a = dict(dt=2, B=1, H=2, S=128, D=128, Q=FAKE_A, K=FAKE_B, V=FAKE_SA, O=FAKE_C, lse=0)
    a.update(args)
    st = tg.lib.tg_attention_fwd(a["dt"], a["B"], a["H"], a["S"], a["D"], a["Q"] or None, a["K"],
                                 a["V"], a["O"], a["lse"] or None, 0.0, 0, None)
    assert st == status


def test_qkv_outputs_must_not_overlap():
    st = tg.lib.tg_gemm_qkv(2, 64, 64, 64, FAKE_A, 64, FAKE_B, FAKE_B + 2 ** 20, FAKE_B + 2 ** 21,
                            64, FAKE_C, FAKE_C + 128, FAKE_C + 2 ** 20, 64, None)
    assert st == 1


def test_empty_problem_is_a_noop():
    # M == 0 or N == 0 returns success without launching (no GPU needed)
    assert tg.lib.tg_gemm(1, 0, 64, 64, FAKE_A, 64, FAKE_B, 64, FAKE_C, 64, None) == 0
    assert tg.last_kernel() == "none"
    assert tg.lib.tg_gemm(2, 64, 0, 64, FAKE_A, 64, FAKE_B, 64, FAKE_C, 64, None) == 0


@pytest.mark.parametrize("grid", [
    (16, 16, 1), (32, 32, 1), (32, 16, 3), (64, 32, 3), (1, 1, 1), (4, 1, 1), (7, 13, 1),
    (3, 5, 3), (17, 9, 1), (1, 33, 3), (128, 128, 1)])
@pytest.mark.parametrize("group_m", [1, 4, 8, 16])
def test_scheduler_is_a_bijection(grid, group_m):
    tm_n, tn_n, nm = grid
    seen = set()
    for b in range(tm_n * tn_n * nm):
        mat, tm, tn = tg.schedule_tile(tm_n, tn_n, nm, group_m, b)
        assert 0 <= mat < nm and 0 <= tm < tm_n and 0 <= tn < tn_n
        seen.add((mat, tm, tn))
    assert len(seen) == tm_n * tn_n * nm
    with pytest.raises(ValueError):
        tg.schedule_tile(tm_n, tn_n, nm, group_m, tm_n * tn_n * nm)


def test_scheduler_keeps_each_xcd_on_a_compact_block():
    # 4096^3 with 256x256 tiles: 16 x 16 tiles, 8 XCDs, group of 8 tile-rows.
    # The 32 tiles an XCD runs at once (one per CU) should touch few row- and
    # column-panels: 8 rows x 4 columns here, versus up to 32 + 32 for the
    # plain row-major order.
    per_xcd = {}
    for b in range(256):
        _, tm, tn = tg.schedule_tile(16, 16, 1, 8, b)
        per_xcd.setdefault(b % 8, []).append((tm, tn))
    for tiles in per_xcd.values():
        rows = {t[0] for t in tiles}
        cols = {t[1] for t in tiles}
        assert len(rows) + len(cols) <= 12


def test_qkv_scheduler_reuses_x_panels_across_the_three_weights():
    # within one group the three matrices share the same tile rows
    rows_by_mat = {0: set(), 1: set(), 2: set()}
    for b in range(8 * 4 * 3):
        mat, tm, tn = tg.schedule_tile(8, 4, 3, 8, b)
        rows_by_mat[mat].add(tm)
    assert rows_by_mat[0] == rows_by_mat[1] == rows_by_mat[2] == set(range(8))


def test_lds_layout_matches_pitch_136_example():
    g = json.load(open(os.path.join(GOLDEN, "padded_layout_pitch136.json")))
    rows, cols = g["shape"]
    pitch, unit = g["strides_elements"]
    eb = g["element_bytes"]
    for r in range(rows):
        for c in (0, 1, 7, 8, 63, 127):
            assert tg.lds_offset(cols, r, c) == (r * pitch + c * unit) * eb


def _banks_16b(addrs, nbanks):
    """Max number of distinct 16-byte requests that share a 4-byte bank."""
    hits = {}
    for a in addrs:
        for w in range(4):
            bank = (a // 4 + w) % nbanks
            hits.setdefault(bank, set()).add(a)
    return max(len(v) for v in hits.values())


@pytest.mark.parametrize("cols", [64, 128])
@pytest.mark.parametrize("nbanks", [32, 64])
def test_fragment_reads_are_bank_conflict_free(cols, nbanks):
    # A 128-bit fragment read: consecutive rows, same 16-byte column chunk.
    # LDS serves nbanks * 4 bytes per cycle; the lanes of one cycle must hit
    # distinct banks.
    lanes_per_cycle = nbanks * 4 // 16
    for chunk in range(cols // 8):
        addrs = [tg.lds_offset(cols, r, chunk * 8) for r in range(lanes_per_cycle)]
        assert _banks_16b(addrs, nbanks) == 1


def test_unpadded_layout_would_conflict():
    # control for the check above: pitch = width (no padding) puts every row
    # of a fragment read on the same banks.
    addrs = [r * 64 * 2 for r in range(8)]
    assert _banks_16b(addrs, 32) == 8


# ---- XOR-swizzled LDS tiles of the asynchronous kernels.  Bank model of
# gfx950: 64 four-byte banks (256 bytes per pass); a 128-bit read is served
# 16 lanes per pass, a 64-bit (transposing) read 32 lanes per pass.  Each
# pass below is the set of addresses the kernels' lanes read together; a
# conflict-free pass touches every bank at most once.

NBANKS = 64


def _swz(layout, r):
    v = tg.lib.tg_lds_swizzle(layout, r)
    assert v >= 0
    return v


def _max_bank_load(pieces):
    """pieces: (byte address, length) per lane; the most lanes on one bank."""
    hits = {}
    for lane, (a, n) in enumerate(pieces):
        for w in range(n // 4):
            hits.setdefault((a // 4 + w) % NBANKS, set()).add(lane)
    return max(len(v) for v in hits.values())


def _a_pass(base_row, gran, swizzle=True):
    # 16 lanes read granule `gran` of rows base .. base+15 (64-byte rows)
    return [((base_row + i) * 64 + 16 * (gran ^ (_swz(0, base_row + i) if swizzle else 0)), 16)
            for i in range(16)]


def _b_pass(layout, row_bytes, rows, cols, swizzle=True):
    # lanes read 8 bytes (4 columns) at (row, col); granule col / 8, byte
    # (col % 8) * 2 within it
    out = []
    for r, c in zip(rows, cols):
        g = (c >> 3) ^ (_swz(layout, r) if swizzle else 0)
        out.append((r * row_bytes + 16 * g + (c & 7) * 2, 8))
    return out


def _b32_lanes(kk, h, col0):
    # 32x32x16 kernel, lanes 0..31 of a transposing B read: 16-lane group
    # g = lane / 16, jj = lane % 16 -> row 16 kk + 4 h + jj / 4, column
    # col0 + 16 g + 4 (jj % 4)
    rows, cols = [], []
    for lane in range(32):
        g, jj = lane >> 4, lane & 15
        rows.append(16 * kk + 4 * h + (jj >> 2))
        cols.append(col0 + 16 * g + 4 * (jj & 3))
    return rows, cols


def _b16_lanes(q0, h, col0):
    # 16x16x32 kernel, lanes of 16-lane groups q0 and q0 + 1 -> row 8 q + 4 h
    # + jj / 4, column col0 + 4 (jj % 4)
    rows, cols = [], []
    for q in (q0, q0 + 1):
        for jj in range(16):
            rows.append(8 * q + 4 * h + (jj >> 2))
            cols.append(col0 + 4 * (jj & 3))
    return rows, cols


@pytest.mark.parametrize("layout,granules", [(0, 4), (1, 16), (1, 32), (2, 8), (3, 32), (4, 24),
                                             (5, 16), (6, 8)])
def test_swizzles_permute_each_row(layout, granules):
    for r in range(64):
        s = _swz(layout, r)
        assert sorted(c ^ s for c in range(granules)) == list(range(granules))
    assert tg.lib.tg_lds_swizzle(7, 0) == -1 and tg.lib.tg_lds_swizzle(0, -1) == -1


def test_a_fragment_reads_are_bank_conflict_free():
    for base in range(0, 256, 16):
        for gran in range(4):
            assert _max_bank_load(_a_pass(base, gran)) == 1
    assert _max_bank_load(_a_pass(0, 0, swizzle=False)) == 4  # control


@pytest.mark.parametrize("bn", [64, 128, 256])
def test_b_transposing_reads_32x32_kernel_are_bank_conflict_free(bn):
    layout = 2 if bn == 64 else 1
    tj = bn // 64
    for kk in range(2):
        for h in range(2):
            for wave_n in range(2):
                for j in range(tj):
                    rows, cols = _b32_lanes(kk, h, wave_n * 32 * tj + 32 * j)
                    assert _max_bank_load(_b_pass(layout, 2 * bn, rows, cols)) == 1
    rows, cols = _b32_lanes(0, 0, 0)
    assert _max_bank_load(_b_pass(layout, 2 * bn, rows, cols, swizzle=False)) > 1  # control


def test_b_transposing_reads_16x16_kernel_are_bank_conflict_free():
    for q0 in (0, 2):
        for h in range(2):
            for col0 in range(0, 256, 16):
                rows, cols = _b16_lanes(q0, h, col0)
                assert _max_bank_load(_b_pass(3, 512, rows, cols)) == 1
    rows, cols = _b16_lanes(0, 0, 0)
    assert _max_bank_load(_b_pass(1, 512, rows, cols)) == 2  # without the row-bit-3 term


def test_b_transposing_reads_192_tile_kernel_are_bank_conflict_free():
    # 384-byte rows (192 columns): every 16-column fragment of either wave
    # column, both halves, both 32-lane passes
    for q0 in (0, 2):
        for h in range(2):
            for col0 in range(0, 192, 16):
                rows, cols = _b16_lanes(q0, h, col0)
                assert _max_bank_load(_b_pass(4, 384, rows, cols)) == 1
    rows, cols = _b16_lanes(0, 0, 0)
    assert _max_bank_load(_b_pass(4, 384, rows, cols, swizzle=False)) > 1  # control


def test_a_fragment_reads_of_64_deep_steps_are_bank_conflict_free():
    # 128-byte rows (64 k): 16 lanes read granule g of rows base .. base + 15
    for base in range(0, 256, 16):
        for gran in range(8):
            pieces = [((base + i) * 128 + 16 * (gran ^ _swz(6, base + i)), 16) for i in range(16)]
            assert _max_bank_load(pieces) == 1
    control = [((i) * 128 + 16 * 0, 16) for i in range(16)]
    assert _max_bank_load(control) == 8
    # the 64-byte-row swizzle does not cover 128-byte rows
    assert _max_bank_load([(i * 128 + 16 * (0 ^ _swz(0, i)), 16) for i in range(16)]) > 1


def test_b_transposing_reads_128_tile_kernel_are_bank_conflict_free():
    # 256-byte rows (128 columns): every 16-column fragment of either wave
    # column, both halves, both 32-lane passes, k rows 0..63 (the second
    # 32-deep slice of a 64-deep step starts at row 32)
    for q0 in (0, 2, 4, 6):
        for h in range(2):
            for col0 in range(0, 128, 16):
                rows, cols = _b16_lanes(q0, h, col0)
                assert _max_bank_load(_b_pass(5, 256, rows, cols)) == 1
    rows, cols = _b16_lanes(0, 0, 0)
    assert _max_bank_load(_b_pass(5, 256, rows, cols, swizzle=False)) > 1  # control
    # the 192-tile swizzle does not cover these rows
    assert _max_bank_load(_b_pass(4, 256, rows, cols)) > 1


def test_bounds_rule_matches_printed_example():
    g = json.load(open(os.path.join(GOLDEN, "oob_16x16.json")))
    rows, cols = g["shape"]
    r, c = g["coordinate"]
    assert r * g["strides_elements"][0] + c * g["strides_elements"][1] == g["linear_offset"]
    assert g["linear_offset"] < rows * cols  # inside the physical span ...
    assert tg.in_bounds(rows, cols, r, c) == g["in_bounds"]  # ... yet out of bounds
    assert tg.in_bounds(rows, cols, 15, 15) and not tg.in_bounds(rows, cols, 16, 0)
    assert not tg.in_bounds(rows, cols, -1, 0)
