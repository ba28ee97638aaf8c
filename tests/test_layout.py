"""Host checks of the pair kernels' LDS tile layout (no GPU): the chunk swizzle in
pair_common.h, read from the source, is a permutation of the 16 chunk positions for every row
and keeps every access shape of the block and triangle-update kernels free of LDS bank
conflicts under gfx950's rule: an access is served as two 32-lane halves, and a half is
conflict-free when its 16-byte slots are distinct modulo 512 bytes (16-byte accesses) or its
8-byte units distinct modulo 256 bytes (8-byte accesses)."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _swz():
    src = open(os.path.join(ROOT, "triangular_attention_amd", "csrc", "pair_common.h")).read()
    m = re.search(r"int swz\(int r\)\s*\{\s*return (.*?);\s*\}", src, re.S)
    assert m, "swz not found"
    expr = m.group(1)
    assert re.fullmatch(r"[r0-9&|^<>()\s+\-*]+", expr), expr   # integer arithmetic on r only
    return lambda r: eval(expr, {}, {"r": r}) & 15


def _byte(swz, row, chunk, half=0):
    return row * 256 + 16 * (chunk ^ swz(row)) + 8 * half


def _free16(addrs):
    return len({(a % 512) // 16 for a in addrs}) == len(addrs) == 32


def _free8(addrs):
    return len({(a % 256) // 8 for a in addrs}) == len(addrs) == 32


def test_swizzle_is_a_permutation_per_row():
    swz = _swz()
    for r in range(64):
        assert sorted(j ^ swz(r) for j in range(16)) == list(range(16))


def test_access_shapes_conflict_free():
    swz = _swz()
    for base in (0, 16, 32, 48):
        # MFMA operand reads: lane (g, c) reads row base + c, chunk 4s + g; halves g = 0, 1 / 2, 3
        for s in range(4):
            for gs in ((0, 1), (2, 3)):
                assert _free16([_byte(swz, base + c, 4 * s + g) for g in gs for c in range(16)])
        # transposing reads: rows base + 8g + kk (+4), chunks j0 and j0 + 1, both 8-byte halves
        for j0 in range(0, 16, 2):
            for extra in (0, 4):
                rows = [base + 8 * g + kk + extra for g in (0, 1) for kk in range(4)]
                assert _free8([_byte(swz, r, j, h) for r in rows for j in (j0, j0 + 1) for h in (0, 1)])
        # 8-byte reads or writes of one chunk of 16 rows, both halves
        for j in range(16):
            assert _free8([_byte(swz, base + c, j, h) for c in range(16) for h in (0, 1)])
        # 16-byte stores: 8 rows x 4 chunks (head-major D = 32), 16 rows x 2 chunks (D = 16),
        # 2 rows x 16 chunks (row-major loads)
        for r0 in (base, base + 8):
            for h in range(4):
                assert _free16([_byte(swz, r, 4 * h + dc) for r in range(r0, r0 + 8) for dc in range(4)])
        for h in range(8):
            assert _free16([_byte(swz, base + r, 2 * h + dc) for r in range(16) for dc in range(2)])
        for r0 in range(base, base + 16, 2):
            assert _free16([_byte(swz, r, j) for r in (r0, r0 + 1) for j in range(16)])


def _swz192():
    src = open(os.path.join(ROOT, "triangular_attention_amd", "csrc", "trimul.hip")).read()
    m = re.search(r"else return r \* MT \+ \(\(j \^ (.*?)\) << 3\);", src)
    assert m, "192-wide swizzle not found"
    expr = m.group(1)
    assert re.fullmatch(r"[r0-9&|^<>()\s]+", expr), expr
    return lambda r: eval(expr, {}, {"r": r})


def test_contraction_192_wide_tiles_conflict_free():
    """The [32 k][192] operand tiles of the per-channel products: chunks stay in their row, the
    transposing reads (rows 8g + 0..3 and + 4, two adjacent chunks, both halves) and the
    row-major stores (32 consecutive 16-byte chunks) are conflict-free."""
    f = _swz192()

    def addr(r, j, half=0):
        return r * 384 + 16 * (j ^ f(r)) + 8 * half

    assert all(0 <= (j ^ f(r)) < 24 and (j ^ f(r)) // 8 == j // 8 for r in range(32) for j in range(24))
    for base in (0, 16):
        for extra in (0, 4):
            rows = [base + 8 * g + kk + extra for g in (0, 1) for kk in range(4)]
            for j0 in range(0, 24, 2):
                assert _free8([addr(r, j, h) for r in rows for j in (j0, j0 + 1) for h in (0, 1)])
    for q0 in range(0, 32 * 24, 32):
        assert _free16([addr(q // 24, q % 24) for q in range(q0, q0 + 32)])
