"""Integer ranges inside the GEMM kernels, at worst-case inputs (CPU only).

A model, in Python integers, of what the det_gemm kernel (k_gemm8) and the
raw-digit kernel (k_partial) keep in fixed-width integers: the LDS cells, the
per-wave digit windows, their carry normalisation, the digit array the windows
are added into, and the raw-digit counters.  Every intermediate is checked
against the width that holds it, at the largest magnitudes the kernels can
see: every product at the largest significand product, all of one sign, in
every cell, for 1 to 128 epochs (K up to 2^19 in one launch).  The kernel
constants below restate the kernels' configuration (cell width, cells per
wave, adds between folds); the test fails if any of them leaves no headroom.
"""
import pytest

I64 = (-(1 << 63), (1 << 63) - 1)
I32 = (-(1 << 31), (1 << 31) - 1)
U32 = (0, (1 << 32) - 1)
ND = 18


def fits(v, rng):
    return rng[0] <= v <= rng[1]


class Grid:
    """One cell grid of k_gemm8: B-bit cells, W waves each folding CW
    consecutive cells, KFLUSH products per cell between folds, products
    |T| <= tmax, cells of `cell` width, the first reachable cell FIRST."""

    def __init__(self, name, B, W, ncell, first, kflush, tmax, cell):
        self.name, self.B, self.W, self.ncell, self.first = name, B, W, ncell, first
        self.kflush, self.tmax, self.cell = kflush, tmax, cell
        self.cw = ncell // W
        self.off = (B * first) & 31
        vb = 63 if cell == I64 else 31
        log2cw = max(0, (self.cw - 1).bit_length())
        self.wd = (self.off + B * (self.cw - 1) + vb + log2cw + 1 + 31) // 32


# f32: products |T| = |Px| * |Pw| * 2^(o mod 4) <= (2^24 - 1)^2 * 8, int64 cells,
# a fold every 4096 k; 16 waves, 128 cells from offset 0
F32 = Grid("f32 4-bit grid", B=4, W=16, ncell=128, first=0, kflush=4096,
           tmax=((1 << 24) - 1) ** 2 * 8, cell=I64)
# bf16: each operand's significand is shifted by its exponent mod 4 at decode
# (|x'|, |w'| <= 255 * 8), int32 cells, a fold every 512 k; 8 waves, 128 cells
# from cell 7 (offsets 32..538)
BF16 = Grid("bf16 4-bit grid", B=4, W=8, ncell=128, first=7, kflush=512,
            tmax=(255 * 8) ** 2, cell=I32)


def fold(grid, dg, cells, problems):
    """The fold of one wave: cell i at bit OFF + B*i of its window (digit 0 of
    the window at bit 0); 64-bit cells split into an unsigned low and a signed
    high word, each multiplied by 2^(bit mod 32) into the window digit; then
    the carry normalisation (all but the top digit into [0, 2^32))."""
    for i, v in enumerate(cells):
        bit = grid.off + grid.B * i
        scale = 1 << (bit & 31)
        if grid.cell == I64:
            lo, hi = v & 0xFFFFFFFF, v >> 32
            for j, part in ((bit >> 5, lo * scale), ((bit >> 5) + 1, hi * scale)):
                dg[j] += part
                if not fits(part, I64) or not fits(dg[j], I64):
                    problems.append(f"{grid.name}: window digit {j} leaves int64 in the fold")
        else:
            dg[bit >> 5] += v * scale
            if not fits(dg[bit >> 5], I64):
                problems.append(f"{grid.name}: window digit leaves int64 in the fold")
    for j in range(grid.wd - 1):
        carry = dg[j] >> 32
        dg[j] -= carry << 32
        dg[j + 1] += carry
        if not fits(dg[j + 1], I64):
            problems.append(f"{grid.name}: carry into window digit {j + 1} leaves int64")
    return dg


@pytest.mark.parametrize("grid", [F32, BF16], ids=lambda g: g.name)
@pytest.mark.parametrize("sign", [1, -1])
def test_cell_grid_worst_case(grid, sign):
    problems = []
    # every product of an epoch lands in the same cell at the largest
    # magnitude: that cell's value after kflush adds
    worst_cell = sign * grid.kflush * grid.tmax
    assert fits(worst_cell, grid.cell), f"{grid.name}: a cell overflows between folds"
    assert grid.cw * grid.W == grid.ncell and (grid.B * grid.cw) % 32 == 0
    for epochs in (1, 2, 8, 128):
        windows = []
        for wave in range(grid.W):
            dg = [0] * grid.wd
            for _ in range(epochs):
                fold(grid, dg, [worst_cell] * grid.cw, problems)
            windows.append(dg)
        # the windows' value is the exact sum of the cells they folded
        for wave, dg in enumerate(windows):
            want = sum(worst_cell * epochs << (grid.off + grid.B * i) for i in range(grid.cw))
            assert sum(d << (32 * j) for j, d in enumerate(dg)) == want
        # windows into the 18-digit array: wave v's digit 0 is accumulator
        # digit (B * (FIRST + v * CW)) / 32; digits past the last one join it
        D = [0] * ND
        for wave, dg in enumerate(windows):
            jb = (grid.B * (grid.first + wave * grid.cw)) >> 5
            dg = list(dg)
            for d in range(grid.wd - 1, 0, -1):
                if jb + d >= ND:
                    dg[d - 1] += dg[d] << 32
                    dg[d] = 0
            for d in range(grid.wd):
                if jb + d < ND:
                    D[jb + d] += dg[d]
        for j, v in enumerate(D):
            # the rounding reads digits within +-2^62; a K block's digits are
            # then added to the carried digits of up to 16 earlier blocks
            if not fits(16 * v, (-(1 << 62), 1 << 62)):
                problems.append(f"{grid.name}: digit {j} {v} leaves the rounding's +-2^62 at {epochs} epochs")
    assert problems == []


def test_raw_digit_counters_worst_case():
    # k_partial: unsigned 16-bit fields added into 32-bit counters, at most
    # 2^15 k per launch; f32 pairs two fields in one 64-bit counter, whose
    # 32-bit halves must not carry into each other
    per_launch = 1 << 15
    field_max = (1 << 16) - 1
    assert fits(per_launch * field_max, (0, (1 << 31) - 1))     # a pair half stays below 2^31
    assert fits(per_launch * field_max, U32)
    # digit j = (P[2j] - N[2j]) + 2^16 (P[2j+1] - N[2j+1]), each field the sum
    # of a low half and the previous slot's high half
    field = 2 * per_launch * field_max
    digit = field + (field << 16)
    # carried over the 16 launches of K = 2^19
    assert fits(16 * digit, (-(1 << 62), 1 << 62))


def test_bf16_cell_has_headroom_only_for_its_fold_interval():
    # the bf16 grid's int32 cells leave less than one more fold interval of
    # headroom: doubling the adds between folds would overflow them
    assert not fits(2 * BF16.kflush * BF16.tmax, I32)
    assert not fits(2 * F32.kflush * F32.tmax, I64)
