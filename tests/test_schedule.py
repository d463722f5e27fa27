"""CPU model of the fixed-length tile orders (the forward's decode_fixed and the
backward's bwd_decode, restated).  Forward: the workgroups t with one value of
t % 8 run on one XCD (round-robin dispatch), and when B*H is a multiple of 8 the
tiles they are given belong to that XCD's heads; longest first (causal), the
XCD's heads go in groups whose tiles run longest first before the next
group's.  Checked here: every (head, query tile) is given to exactly one
workgroup, each XCD keeps to its own heads, and inside each head group the
query-tile index never increases ("Flash Attention 4", section on tile
scheduling: LPT order, and the L2 sections of heads)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "flashattention_forward_fa_amd", "csrc", "fa_fwd_kernel.hip")
XCD = 8


def _head_group():
    with open(SRC) as f:
        return int(re.search(r"constexpr int kLptHeadGroup = (\d+);", f.read()).group(1))


GROUP = _head_group()


def decode(t, BH, nm, lpt):
    if BH % XCD == 0:
        x, u, HX = t % XCD, t // XCD, BH // XCD
        if lpt:
            gs = GROUP if HX % GROUP == 0 else HX
            grp, v = divmod(u, gs * nm)
            return x * HX + grp * gs + v % gs, nm - 1 - v // gs
        return x * HX + u // nm, u % nm
    if lpt:
        return t % BH, nm - 1 - t // BH
    return t // nm, t % nm


@pytest.mark.parametrize("BH", [1, 3, 8, 16, 24, 64, 72, 128, 256])
@pytest.mark.parametrize("nm", [1, 3, 16])
@pytest.mark.parametrize("lpt", [0, 1])
def test_every_tile_once_and_xcd_heads(BH, nm, lpt):
    seen = set()
    for t in range(BH * nm):
        bh, m = decode(t, BH, nm, lpt)
        assert 0 <= bh < BH and 0 <= m < nm
        assert (bh, m) not in seen
        seen.add((bh, m))
        if BH % XCD == 0:
            HX = BH // XCD
            assert bh // HX == t % XCD          # the XCD's own heads
    assert len(seen) == BH * nm


@pytest.mark.parametrize("BH", [64, 128, 256])
def test_groups_run_longest_first(BH):
    nm = 16
    HX = BH // XCD
    gs = GROUP if HX % GROUP == 0 else HX
    for x in range(XCD):
        order = [decode(x + XCD * u, BH, nm, 1) for u in range(HX * nm)]
        for g0 in range(0, len(order), gs * nm):
            block = order[g0:g0 + gs * nm]
            heads = {bh for bh, _ in block}
            assert len(heads) == gs                          # one group of heads at a time
            ms = [m for _, m in block]
            assert ms == sorted(ms, reverse=True)            # longest first inside it


# ----------------------------------------------------------------- backward

BSRC = os.path.join(ROOT, "flashattention_forward_fa_amd", "csrc", "fa_bwd_kernel.hip")


def _bwd_group():
    with open(BSRC) as f:
        return int(re.search(r"constexpr int kBwdHeadGroup = (\d+);", f.read()).group(1))


BGROUP = _bwd_group()


def bwd_decode_fixed(t, nbh, nm, reverse):
    """The backward's fixed-length order (bwd_decode without offsets)."""
    if nbh % XCD == 0:
        x, u, HX = t % XCD, t // XCD, nbh // XCD
        gs = BGROUP if HX % BGROUP == 0 else HX
        grp, v = divmod(u, gs * nm)
        m, bh = v // gs, x + XCD * (grp * gs + v % gs)
    else:
        m, bh = t // nbh, t % nbh
    return bh, (nm - 1 - m if reverse else m)


@pytest.mark.parametrize("nbh", [1, 6, 8, 16, 24, 64, 128])
@pytest.mark.parametrize("nm", [1, 5, 32])
@pytest.mark.parametrize("reverse", [False, True])
def test_bwd_every_tile_once(nbh, nm, reverse):
    seen = set()
    for t in range(nbh * nm):
        bh, m = bwd_decode_fixed(t, nbh, nm, reverse)
        assert 0 <= bh < nbh and 0 <= m < nm and (bh, m) not in seen
        seen.add((bh, m))
        if nbh % XCD == 0:
            assert bh % XCD == t % XCD              # the XCD's own pairs
    assert len(seen) == nbh * nm


def test_bwd_groups_heaviest_first():
    nbh, nm = 64, 32
    for reverse in (False, True):
        for x in range(XCD):
            order = [bwd_decode_fixed(x + XCD * u, nbh, nm, reverse) for u in range(nbh // XCD * nm)]
            for g0 in range(0, len(order), BGROUP * nm):
                block = order[g0:g0 + BGROUP * nm]
                assert len({bh for bh, _ in block}) == BGROUP
                ms = [m for _, m in block]
                assert ms == sorted(ms, reverse=reverse)   # dQ from the top, dK/dV from 0
