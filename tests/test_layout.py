"""Host checks of the scan kernel's LDS layouts (no GPU).

The [64][64] bf16 tiles are stored with their 16-byte units XOR-swizzled per
row: unit u of row r at position u ^ g(r).  K~ and -M^T tiles (read as
16-byte rows by 32 consecutive lanes) use g(r) = (r ^ ((r >> 3) & 3)) & 7; the
V tile (read by ds_read_b64_tr_b16 transpose loads) uses gv(r) with row bits
2, 0, 1 as unit bits 0, 1, 2.  These tests restate the index formulas of
path_fwd_bf16.hip and check that the copies put every unit where the reads
look for it, that the transpose loads assemble the PV operand the MFMA
needs, and that no read pattern puts two different words of one LDS pass on
the same bank, for the two bank models the kernel is laid out for (64 banks
of 4 bytes serving 32 lanes, 32 banks serving 16 lanes).
"""
import itertools

import numpy as np


def perm16(s):
    return s if (s < 4 or s >= 12) else (s + 4 if s < 8 else s - 4)


def permk(s):
    return (s & ~15) | perm16(s & 15)


def g_rows(r):
    return (r ^ ((r >> 3) & 3)) & 7


def g_v(r):
    return ((r >> 2) & 1) | ((r & 1) << 1) | (((r >> 1) & 1) << 2)


def dma_layout(tile, g):
    """global_load_lds of an 8-wave copy: wave w, lane i fills LDS bytes
    1024 w + 16 i .. +15 with global row 8 w + i // 8, unit (i % 8) ^ g(row)."""
    lds = np.zeros(64 * 64, dtype=tile.dtype)
    for w in range(8):
        for i in range(64):
            r = 8 * w + i // 8
            u = (i % 8) ^ g(r)
            lds[512 * w + 8 * i: 512 * w + 8 * i + 8] = tile[r, 8 * u: 8 * u + 8]
    return lds


def test_dma_places_unit_u_at_u_xor_g():
    rng = np.random.default_rng(0)
    tile = rng.integers(0, 1 << 15, size=(64, 64))
    for g in (g_rows, g_v):
        lds = dma_layout(tile, g)
        for r in range(64):
            for u in range(8):
                p = u ^ g(r)
                assert np.array_equal(lds[r * 64 + 8 * p: r * 64 + 8 * p + 8], tile[r, 8 * u: 8 * u + 8])


def vtr_byte_offsets(lane):
    """The 8 per-lane byte offsets of the PV transpose loads (par, load, dt)."""
    hh, hp, j = lane >> 5, (lane >> 4) & 1, lane & 15
    off = {}
    for par, ins, dt in itertools.product(range(2), range(2), range(2)):
        tok = permk(16 * par + 8 * hh + 4 * ins + (j >> 2))
        d = permk(32 * dt + 16 * hp + 4 * (j & 3))
        off[(par, ins, dt)] = (tok * 64 + (((d >> 3) ^ g_v(tok)) << 3) + (d & 7)) * 2
    return off


def transpose_load(lds, byte_off):
    """ds_read_b64_tr_b16 over 64 lanes: within each group of 16 lanes, lane
    i, element t is element i % 4 of the 8 bytes read by lane 4 t + i // 4."""
    out = np.zeros((64, 4), dtype=lds.dtype)
    for lane in range(64):
        grp, i = lane // 16, lane % 16
        for t in range(4):
            src = 16 * grp + 4 * t + i // 4
            out[lane, t] = lds[byte_off[src] // 2 + i % 4]
    return out


def test_transpose_loads_give_the_pv_operand():
    """O^T += V^T P^T: the A operand of k-step ks for rows dt is, in lane l,
    V^T[32 dt + l % 32][keys 16 ks + 8 (l // 32) .. +7] in the permuted key
    (k-slot) and d (row) orders."""
    rng = np.random.default_rng(1)
    V = rng.integers(0, 1 << 15, size=(64, 64))        # [token][d]
    lds = dma_layout(V, g_v)
    offs = [vtr_byte_offsets(l) for l in range(64)]
    for dt, ks in itertools.product(range(2), range(4)):
        base = 2048 * (ks >> 1)                          # rows 32 (ks >> 1) further: 4096 bytes
        halves = []
        for ins in range(2):
            bo = [base * 2 + offs[l][((ks & 1), ins, dt)] for l in range(64)]
            halves.append(transpose_load(lds, bo))
        got = np.concatenate(halves, axis=1)             # [lane][8]
        for lane in range(64):
            rho = 32 * dt + lane % 32
            for t in range(8):
                sigma = 16 * ks + 8 * (lane // 32) + t
                assert got[lane, t] == V[permk(sigma), permk(rho)], (dt, ks, lane, t)


def conflict_degree(byte_addrs, nbytes, lanes_per_pass, nbanks):
    worst = 1
    for p0 in range(0, 64, lanes_per_pass):
        banks = {}
        for lane in range(p0, p0 + lanes_per_pass):
            for w in range(nbytes // 4):
                word = byte_addrs[lane] // 4 + w
                banks.setdefault(word % nbanks, set()).add(word)
        worst = max(worst, max(len(v) for v in banks.values()))
    return worst


BANK_MODELS = [(32, 64), (16, 32)]                      # (lanes per pass, banks)


def test_transpose_loads_are_conflict_free():
    offs = [vtr_byte_offsets(l) for l in range(64)]
    for key in itertools.product(range(2), range(2), range(2)):
        addrs = [offs[l][key] for l in range(64)]
        for lanes, banks in BANK_MODELS:
            assert conflict_degree(addrs, 8, lanes, banks) == 1, (key, lanes, banks)


def test_row_reads_are_conflict_free():
    """K~ and -M^T operand reads: lane l reads 16 bytes, unit 2 ks + l // 32 of
    row 32 t + l % 32 (16 lanes, or 8 lanes of 16 bytes, per 128-byte pass)."""
    for ks, t in itertools.product(range(4), range(2)):
        addrs = []
        for l in range(64):
            r = 32 * t + l % 32
            u = 2 * ks + l // 32
            addrs.append((r * 64 + ((u ^ g_rows(r)) << 3)) * 2)
        for lanes, banks in [(16, 64), (8, 32)]:
            assert conflict_degree(addrs, 16, lanes, banks) == 1, (ks, t, lanes, banks)
