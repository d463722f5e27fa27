"""CPU model of the forward kernel's register and LDS layouts (no GPU).

The kernel's correctness rests on a few layout facts that a parity test only
shows indirectly; this module checks them one by one, the way
"FlashAttention：一次前向计算" (qingsen), section "back to the source", checks
load coordinates, swizzle addresses and MMA coverage on the host:

* the K and V tiles' LDS stores cover each element once (the V tile with its
  16-byte chunks swizzled by vswz, the K tile with padded rows);
* the 16-byte K-fragment reads (served 16 lanes at a time) and the
  ds_read_b64_tr_b16 transpose reads of V (served 32 lanes at a time) meet no
  bank conflict on a 64-bank, 4-byte-wide LDS, for d = 64 and 128;
* what those reads deliver is the operand the MFMA needs: K rows for
  S^T = K Q^T, and V^T with keys in the order in which the S^T accumulator,
  converted to bf16, supplies P^T for O^T += V^T P^T;
* the two half-waves that lane_pair_max / lane_pair_sum combine (lanes l and
  l ^ 32) hold complementary halves of one query's keys, and the causal mask's
  key index is the accumulator's;
* the bf16 epilogue's LDS staging of O (d = 128) returns every element at its
  own row and column, with conflict-free reads, 2-way writes, and store steps
  that each cover whole rows.

The swizzle and the K row pad are read from the kernel sources, so a change
there is checked here; the lane address formulas are the kernel's, restated.
"""
import os
import re
from collections import defaultdict

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "flashattention_forward_fa_amd", "csrc")
BANKS, BANK_BYTES = 64, 4
BLOCK_N = 64            # keys per K/V block


def _read(name):
    with open(os.path.join(CSRC, name)) as f:
        return f.read()


def _vswz_from_source():
    """The two branches of vswz<D> in fa_device.h, as Python functions."""
    src = _read("fa_device.h")
    body = src[src.index("int vswz(int r)"):]
    e128 = re.search(r"if constexpr \(D == 128\) return (.+?);", body).group(1)
    e64 = re.search(r"else return (.+?);", body).group(1)
    return {128: eval("lambda r: " + e128), 64: eval("lambda r: " + e64)}


def _k_pad_from_source():
    src = _read("fa_fwd_kernel.hip")
    return int(re.search(r"KS = D \+ (\d+);", src).group(1))


VSWZ = _vswz_from_source()
KPAD = _k_pad_from_source()


def conflicts(accesses, group):
    """Extra LDS cycles of one instruction: lanes are served `group` at a time;
    within a group, two lanes touching different 4-byte words of one bank
    conflict.  accesses: per lane (byte address, bytes)."""
    extra = 0
    for g0 in range(0, len(accesses), group):
        banks = defaultdict(set)
        for addr, nb in accesses[g0:g0 + group]:
            for word in range(addr // 4, (addr + nb) // 4):
                banks[word % BANKS].add(word)
        extra += max(len(s) for s in banks.values()) - 1
    return extra


# ----------------------------------------------------------------- stores

@pytest.mark.parametrize("D", [64, 128])
def test_swizzle_stays_in_row(D):
    nch = D // 8
    for r in range(256):
        assert 0 <= VSWZ[D](r) < nch, (D, r)


@pytest.mark.parametrize("D", [64, 128])
def test_v_store_covers_each_element_once(D):
    """Chunk cc of row `row` goes to row*D + ((cc ^ vswz(row)) << 3) (elements)."""
    seen = np.zeros(BLOCK_N * D, dtype=int)
    for row in range(BLOCK_N):
        for cc in range(D // 8):
            base = row * D + ((cc ^ VSWZ[D](row)) << 3)
            seen[base:base + 8] += 1
    assert np.all(seen == 1)


@pytest.mark.parametrize("D", [64, 128])
def test_k_store_covers_each_element_once(D):
    KS = D + KPAD
    seen = np.zeros(BLOCK_N * KS, dtype=int)
    for row in range(BLOCK_N):
        for cc in range(D // 8):
            base = row * KS + 8 * cc
            seen[base:base + 8] += 1
    used = np.concatenate([np.arange(r * KS, r * KS + D) for r in range(BLOCK_N)])
    assert np.all(seen[used] == 1) and seen.sum() == BLOCK_N * D


# ----------------------------------------------------------------- K reads

def k_read(D, lane, kt, ds):
    """Element offset of the 8 bf16 a lane reads for S^T = K Q^T: key row
    32*kt + lane%32, head-dim chunk 16*ds + 8*(lane/32)."""
    lq, g = lane & 31, lane >> 5
    return (32 * kt + lq) * (D + KPAD) + 16 * ds + 8 * g


@pytest.mark.parametrize("D", [64, 128])
def test_k_fragment_reads_conflict_free(D):
    for kt in range(BLOCK_N // 32):
        for ds in range(D // 16):
            acc = [(2 * k_read(D, l, kt, ds), 16) for l in range(64)]
            assert conflicts(acc, 16) == 0, (D, kt, ds)


@pytest.mark.parametrize("D", [64, 128])
def test_k_fragment_is_the_a_operand(D):
    """MFMA 32x32x16 A operand: lane l supplies A[m = l%32][k = 8*(l/32) + e].
    Here m is the key (row of S^T) and k the head-dim index within step ds."""
    KS = D + KPAD
    for kt in range(BLOCK_N // 32):
        for ds in range(D // 16):
            for l in range(64):
                off = k_read(D, l, kt, ds)
                row, col = divmod(off, KS)
                assert row == 32 * kt + (l & 31)
                assert col == 16 * ds + 8 * (l >> 5)


# ----------------------------------------------------------------- V transpose reads

def v_tr_addr(D, lane, ks, dt, h):
    """Element offset a lane passes to ds_read_b64_tr_b16 (kernel: v_off[dt][h],
    plus 16 rows per key step ks)."""
    g = lane >> 5
    row = 4 * g + ((lane & 15) >> 2) + 8 * h
    col = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)
    return 16 * ks * D + row * D + ((((col >> 3) ^ VSWZ[D](row)) << 3) | (col & 7))


def tr_read(lds, D, ks, dt, h):
    """Model of ds_read_b64_tr_b16 on an LDS image: in each 16-lane group, lane
    s addresses 4 consecutive bf16 (row s/4, columns 4*(s%4)..+3 of a 4 x 16
    block); lane i of the group receives element e = value at (row e, column i)."""
    out = np.zeros((64, 4), dtype=lds.dtype)
    for g0 in range(0, 64, 16):
        block = np.zeros((4, 16), dtype=lds.dtype)
        for s in range(16):
            a = v_tr_addr(D, g0 + s, ks, dt, h)
            block[s // 4, 4 * (s % 4):4 * (s % 4) + 4] = lds[a:a + 4]
        for i in range(16):
            out[g0 + i] = block[:, i]
    return out


@pytest.mark.parametrize("D", [64, 128])
def test_v_transpose_reads_conflict_free(D):
    for ks in range(BLOCK_N // 16):
        for dt in range(D // 32):
            for h in range(2):
                acc = [(2 * v_tr_addr(D, l, ks, dt, h), 8) for l in range(64)]
                assert conflicts(acc, 32) == 0, (D, ks, dt, h)


def s_key(lane, kt, i):
    """Key (within the block) of accumulator element i of S^T tile kt in a lane:
    32x32 accumulator rows 8*(i/4) + 4*(lane/32) + i%4; the lane's column is
    its query."""
    return 32 * kt + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)


def p_key(lane, ks, e):
    """Key of element e of the bf16 P^T operand pf[ks]: elements 8*(ks%2)+e of
    S^T tile ks/2 (the kernel's pack order)."""
    return s_key(lane, ks >> 1, 8 * (ks & 1) + e)


@pytest.mark.parametrize("D", [64, 128])
def test_v_transpose_reads_give_vt_in_p_key_order(D):
    """Store a V block (distinct values) with the kernel's swizzled layout, run the
    modelled transpose reads, and check that lane l, element e of the MFMA A
    operand (hi read for e >= 4) is V[key][d] with d = 32*dt + l%32 and key the
    one P^T supplies at the same position (MFMA k index 8*(l/32) + e)."""
    V = np.arange(BLOCK_N * D, dtype=np.int64).reshape(BLOCK_N, D)
    lds = np.full(BLOCK_N * D, -1, dtype=np.int64)
    for row in range(BLOCK_N):
        for cc in range(D // 8):
            base = row * D + ((cc ^ VSWZ[D](row)) << 3)
            lds[base:base + 8] = V[row, 8 * cc:8 * cc + 8]
    for ks in range(BLOCK_N // 16):
        for dt in range(D // 32):
            lo, hi = tr_read(lds, D, ks, dt, 0), tr_read(lds, D, ks, dt, 1)
            for l in range(64):
                a = np.concatenate([lo[l], hi[l]])
                for e in range(8):
                    key = 16 * ks + (p_key(l, ks, e) - 32 * (ks >> 1) - 16 * (ks & 1))
                    assert a[e] == V[key, 32 * dt + (l & 31)], (D, ks, dt, l, e)


def test_p_operand_keys_match_accumulator_and_mfma_k_order():
    """The P^T operand's key at (lane, e) depends only on the MFMA k index
    8*(lane/32) + e (so the A and B operands pair the same keys), and each 16-key
    step covers its 16 keys once."""
    for ks in range(BLOCK_N // 16):
        by_k = {}
        for l in range(64):
            for e in range(8):
                k = 8 * (l >> 5) + e
                by_k.setdefault(k, set()).add(p_key(l, ks, e))
        assert all(len(v) == 1 for v in by_k.values())
        assert sorted(next(iter(v)) for v in by_k.values()) == list(range(16 * ks, 16 * ks + 16))


def test_half_waves_hold_complementary_keys():
    """Lanes l and l ^ 32 own the same query (l % 32) and between them every key
    of a block exactly once: the in-lane reduction plus one exchange
    (lane_pair_max / lane_pair_sum) covers the whole row -- the CDNA analog of
    the page's four-lane groups (table 6: each key held by exactly one lane)."""
    for l in range(32):
        keys = [s_key(l, kt, i) for kt in range(BLOCK_N // 32) for i in range(16)]
        keys += [s_key(l ^ 32, kt, i) for kt in range(BLOCK_N // 32) for i in range(16)]
        assert sorted(keys) == list(range(BLOCK_N))


def test_mask_index_is_the_accumulator_key():
    """mask_block compares 32*kt + 8*(i>>2) + (i&3) against a limit that has the
    lane's 4*(lane/32) already subtracted: the same key as s_key."""
    src = _read("fa_fwd_kernel.hip")
    assert "if (32 * kt + 8 * (i >> 2) + (i & 3) > lim) s[kt][i] = -INFINITY;" in src
    assert "const int ln = fresh_lane();" in src
    assert "- kv0 - 4 * (ln >> 5);" in src
    for l in range(64):
        for kt in range(2):
            for i in range(16):
                assert 32 * kt + 8 * (i >> 2) + (i & 3) + 4 * (l >> 5) == s_key(l, kt, i)


def test_page_row_reduces_to_three_in_this_layout():
    """The page's table 7 row (first eight keys -4..3, the rest -5), laid out
    over the two half-waves: in-lane maxima -1 and 3, combined 3 on both."""
    row = np.full(BLOCK_N, -5.0)
    row[:8] = np.arange(-4, 4)
    m = [max(row[s_key(l, kt, i)] for kt in range(2) for i in range(16)) for l in (0, 32)]
    assert m == [-1.0, 3.0]
    assert max(m) == 3.0


@pytest.mark.parametrize("D", [64, 128])
def test_model_sees_conflicts_without_the_swizzle(D, monkeypatch):
    """The bank model is not vacuous: with the chunks unswizzled (row-major V)
    the transpose reads do conflict (measured on the GPU as 28% of LDS-active
    cycles with the earlier unswizzled layout), and so do unpadded K rows."""
    monkeypatch.setitem(VSWZ, D, lambda r: 0)
    extra = sum(conflicts([(2 * v_tr_addr(D, l, 0, dt, h), 8) for l in range(64)], 32)
                for dt in range(D // 32) for h in range(2))
    assert extra > 0
    monkeypatch.setattr(__import__(__name__), "KPAD", 0)
    assert sum(conflicts([(2 * k_read(D, l, 0, ds), 16) for l in range(64)], 16)
               for ds in range(D // 16)) > 0


# ----------------------------------------------------------------- O staging (bf16 epilogue)

def o_stage_write(D, lane, dt, i4):
    """Element offset of the 4 bf16 of O a lane writes into its wave's staging
    tile: row lq, head-dim columns 32*dt + 8*i4 + 4*g .. +3, the 16-byte chunk
    4*dt + i4 XOR-swizzled by the row."""
    lq, g = lane & 31, lane >> 5
    cpr = D // 8
    return lq * D + (((4 * dt + i4) ^ (lq & (cpr - 1))) << 3) + 4 * g


def o_stage_read(D, lane, it):
    """(row, chunk, element offset) of the 16 bytes a lane reads back in step it."""
    cpr = D // 8
    u = 64 * it + lane
    r, cc = divmod(u, cpr)
    return r, cc, r * D + ((cc ^ (r & (cpr - 1))) << 3)


@pytest.mark.parametrize("D", [128])
def test_o_staging_round_trip(D):
    """Every element of the 32 x D tile is written once and read back at its
    own row and column; the reads cover every row's chunks once."""
    tile = np.full(32 * D, -1, dtype=np.int64)
    for lane in range(64):
        lq, g = lane & 31, lane >> 5
        for dt in range(D // 32):
            for i4 in range(4):
                off = o_stage_write(D, lane, dt, i4)
                for e in range(4):
                    assert tile[off + e] == -1
                    tile[off + e] = lq * D + 32 * dt + 8 * i4 + 4 * g + e   # its (row, column)
    assert np.all(tile >= 0)
    seen = set()
    for it in range(32 * (D // 8) // 64):
        for lane in range(64):
            r, cc, off = o_stage_read(D, lane, it)
            assert 0 <= r < 32 and (r, cc) not in seen
            seen.add((r, cc))
            assert list(tile[off:off + 8]) == [r * D + 8 * cc + e for e in range(8)]
    assert len(seen) == 32 * (D // 8)


@pytest.mark.parametrize("D", [128])
def test_o_staging_banks(D):
    """Reads (16 bytes, 16 lanes at a time) are conflict-free; the 8-byte
    writes (32 lanes at a time, all in the same half of their chunks) cost
    one extra cycle per group: 2-way, the least for 32 half-chunk writes."""
    for it in range(32 * (D // 8) // 64):
        acc = [(2 * o_stage_read(D, l, it)[2], 16) for l in range(64)]
        assert conflicts(acc, 16) == 0
    for dt in range(D // 32):
        for i4 in range(4):
            acc = [(2 * o_stage_write(D, l, dt, i4), 8) for l in range(64)]
            assert conflicts(acc, 32) == 2


@pytest.mark.parametrize("D", [128])
def test_o_staged_stores_write_whole_rows(D):
    """Each read-back step's lanes hold whole rows in order: the lanes of a
    row are consecutive and their 16-byte pieces tile the row."""
    cpr = D // 8
    for it in range(32 * cpr // 64):
        rows = defaultdict(list)
        for lane in range(64):
            r, cc, _ = o_stage_read(D, lane, it)
            rows[r].append((lane, cc))
        assert len(rows) == 64 // cpr
        for r, lc in rows.items():
            lanes = [l for l, _ in lc]
            assert lanes == list(range(lanes[0], lanes[0] + cpr))
            assert [c for _, c in lc] == list(range(cpr))
