"""CPU model of the pipelined kernel's LDS tiles and operand reads (no GPU).

Each operand tile of a stage sits in LDS in its storage order: K-contiguous
(row-major A, column-major B: one LDS row per M row or N column, BK values
long) or outer-contiguous (column-major A, row-major B: one LDS row per k).
The 16-byte chunk c of LDS row r sits at physical chunk c ^ swz(r).  The
copies place logical chunk c of row r at r*ROWB + 16*(c ^ swz(r)); the
operand reads are `ds_read_b128` (K-contiguous) or two transposing
`ds_read_b64_tr_b16` (outer-contiguous; in each 16-lane group, lane i's
16-bit slot s receives element i % 4 of the 8 bytes addressed by lane
4*s + i/4, as probed on the device).

For every pipelined table entry, every wave position, k-step, operand and
lane, the model computes the addresses the kernel computes (the formulas of
`OpTile` and `OpReader` in csrc/kernels.hpp) and checks:

* the copy placement is a bijection onto the tile's LDS bytes;
* every operand register receives exactly the element the matrix
  instruction's documented lane layout asks for (32x32x16: lane l supplies
  outer index l % 32 at k = 8*(l/32) + 0..7 of the 16-deep step; 16x16x32:
  l % 16 at k = 8*(l/16) + 0..7 of the 32-deep step);
* gfx950's 64 banks of 4 bytes: each 16-lane group of a `ds_read_b128` and
  each 32-lane group of a `ds_read_b64` touches 64 distinct banks (no bank
  conflict), as the hardware counter SQ_LDS_BANK_CONFLICT also reads.

Planted mistakes must fail: a read that ignores the swizzle returns wrong
elements, and tiles without the swizzle conflict.
"""
import pytest

import dense_mixed_precision_amd as mp


class Tile:
    """One operand tile: BX outer indices (BM for A, BN for B) by BK."""

    def __init__(self, BX, BK, k_contig, nw, mi, swizzle=True):
        self.BX, self.BK, self.kc, self.mi, self.swizzle = BX, BK, k_contig, mi, swizzle
        self.rows = BX if k_contig else BK
        self.rowb = 2 * (BK if k_contig else BX)
        self.ch = self.rowb // 16
        assert self.rows * self.ch * 8 == BX * BK

    def swz(self, r):
        if not self.swizzle:
            return 0
        ch = self.ch
        if self.kc:
            return (r & 15) if ch == 16 else ((r >> 1) & 7) if ch == 8 else ((r >> 2) & 3)
        if self.mi == 32:
            return 4 * (r & 3) if ch >= 16 else 4 * ((r >> 1) & 1)
        return 2 * (r & 3) + 8 * ((r >> 3) & 1) if ch >= 16 else 2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1)

    def placement(self, read_swizzle=True):
        """LDS byte address -> (outer, k) of the element the copies put there."""
        lds = {}
        for r in range(self.rows):
            for c in range(self.ch):
                for e in range(8):
                    outer, k = (r, 8 * c + e) if self.kc else (8 * c + e, r)
                    addr = r * self.rowb + 16 * (c ^ self.swz(r)) + 2 * e
                    assert addr not in lds and 0 <= addr < self.rows * self.rowb
                    lds[addr] = (outer, k)
        assert len(lds) == self.BX * self.BK
        return lds


def banks_ok(addrs, width, group):
    """Lanes in groups of `group` consecutive lanes, each reading `width` bytes:
    every group must cover 64 distinct 4-byte banks."""
    for g0 in range(0, 64, group):
        banks = set()
        for a in addrs[g0:g0 + group]:
            for d in range(width // 4):
                b = (a // 4 + d) % 64
                if b in banks:
                    return False
                banks.add(b)
    return True


def check_operand(t, w_off, ks, f, read_swizzle=True, lds=None):
    """Values and banks of operand f of k-step ks for a wave whose part of the
    operand starts at outer index w_off.  Returns (values_ok, banks_ok)."""
    mi = t.mi
    kd = 16 if mi == 32 else 32
    lds = t.placement() if lds is None else lds
    want = [[(w_off + mi * f + l % mi, kd * ks + 8 * (l // mi) + e) for e in range(8)] for l in range(64)]
    sw_of = (lambda r: t.swz(r)) if read_swizzle else (lambda r: 0)
    if t.kc:
        addrs = []
        for l in range(64):
            row = w_off + (l & (mi - 1))
            off = row * t.rowb + f * mi * t.rowb + ((((kd // 8) * ks + l // mi) ^ sw_of(row)) * 16)
            addrs.append(off)
        got = [[lds.get(a + 2 * e) for e in range(8)] for a in addrs]
        return got == want, banks_ok(addrs, 16, 16)
    # outer-contiguous: two transposing 8-byte reads per operand
    p0 = []
    for l in range(64):
        g, q = l >> 4, l & 15
        if mi == 32:
            row_l = 8 * (g >> 1) + (q >> 2)
            col = w_off + 16 * (g & 1) + 4 * (q & 3)
        else:
            row_l = 8 * g + (q >> 2)
            col = w_off + 4 * (q & 3)
        c = col + mi * f
        p0.append(row_l * t.rowb + kd * ks * t.rowb + (((c >> 3) ^ sw_of(row_l)) * 16) + (c & 7) * 2)
    halves = []
    for part in (0, 1):
        addrs = [a + part * 4 * t.rowb for a in p0]
        vals = []
        for l in range(64):
            g0, i = 16 * (l // 16), l % 16
            vals.append([lds.get(addrs[g0 + 4 * s + i // 4] + 2 * (i % 4)) for s in range(4)])
        halves.append((vals, addrs))
    got = [halves[0][0][l] + halves[1][0][l] for l in range(64)]
    return got == want, all(banks_ok(a, 8, 32) for _, a in halves)


def tiles_of(c, swizzle=True):
    nw = c["waves_m"] * c["waves_n"] * c["k_groups"]
    ta = Tile(c["bm"], c["bk"], c["layout_a"] == mp.MPGEMM_ROW_MAJOR, nw, c["mfma_m"], swizzle)
    tb = Tile(c["bn"], c["bk"], c["layout_b"] == mp.MPGEMM_COL_MAJOR, nw, c["mfma_m"], swizzle)
    return ta, tb


def _pipe_ids():
    return [i for i in range(mp.mpgemm_num_configs()) if mp.mpgemm_config_info(i)["kind_name"] == "pipe"]


def _distinct_shapes():
    seen, out = set(), []
    for i in _pipe_ids():
        c = mp.mpgemm_config_info(i)
        key = (c["bm"], c["bn"], c["bk"], c["waves_m"], c["waves_n"], c["wave_m"], c["wave_n"], c["mfma_m"],
               c["layout_a"], c["layout_b"], c["k_groups"])
        if key not in seen:
            seen.add(key)
            out.append(i)
    return out


@pytest.mark.parametrize("cid", _distinct_shapes())
def test_operand_reads_get_the_instruction_layout_without_bank_conflicts(cid):
    c = mp.mpgemm_config_info(cid)
    ta, tb = tiles_of(c)
    kd = 16 if c["mfma_m"] == 32 else 32
    for t, nwav, wt in ((ta, c["waves_m"], c["wave_m"]), (tb, c["waves_n"], c["wave_n"])):
        lds = t.placement()
        for w in range(nwav):
            for ks in range(c["bk"] // kd):
                for f in range(wt // c["mfma_m"]):
                    vals, banks = check_operand(t, w * wt, ks, f, lds=lds)
                    assert vals, f"config {cid}: wrong elements (w_off {w * wt}, ks {ks}, f {f}, k-contig {t.kc})"
                    assert banks, f"config {cid}: bank conflict (w_off {w * wt}, ks {ks}, f {f}, k-contig {t.kc})"


def _first(pred):
    for i in _pipe_ids():
        c = mp.mpgemm_config_info(i)
        if pred(c):
            return c
    raise AssertionError("no such config")


@pytest.mark.parametrize("k_contig_a", [True, False])
def test_model_rejects_a_read_that_ignores_the_swizzle(k_contig_a):
    c = _first(lambda c: (c["layout_a"] == mp.MPGEMM_ROW_MAJOR) == k_contig_a and c["mfma_m"] == 32)
    ta, _ = tiles_of(c)
    assert check_operand(ta, 0, 0, 0)[0]
    assert not all(check_operand(ta, 0, ks, 0, read_swizzle=False)[0] for ks in range(c["bk"] // 16))


@pytest.mark.parametrize("k_contig_a", [True, False])
def test_model_sees_conflicts_without_the_swizzle(k_contig_a):
    c = _first(lambda c: (c["layout_a"] == mp.MPGEMM_ROW_MAJOR) == k_contig_a and c["mfma_m"] == 32
               and c["bm"] == 128)
    ta, _ = tiles_of(c, swizzle=False)
    vals, banks = check_operand(ta, 0, 0, 0)
    assert vals and not banks
