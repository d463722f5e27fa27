"""fa_bwd_noalloc (the backward with its row terms in the library's static
device array instead of a caller's workspace) against fa_bwd, through the C
ABI: two calls in a row, the second on a smaller problem, each bit for bit
equal to fa_bwd on the same inputs; and a problem past the array's size is
refused with FA_ERR_TOO_LARGE before anything is launched."""
import numpy as np
import pytest

from flashattention_forward_fa_amd import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import flashattention_forward_fa_amd as fa
    fa.load()


def _case(w, dout_seed):
    """Inputs on the device, the forward's O and LSE, a seeded dO, and fa_bwd's
    gradients (with a torch-allocated workspace)."""
    import torch
    import flashattention_forward_fa_amd as fa
    q, k, v, off = parity.to_device(w)
    ms = w.Nq if w.varlen else None
    o, lse = fa.attention(q, k, v, w.scale, w.causal, varlen_offsets=off, max_seqlen=ms)
    dout = torch.from_numpy(wl.make_dout(w, seed=dout_seed).view(np.int16)).view(
        torch.bfloat16).cuda()
    ref = fa.attention_bwd(q, k, v, o, lse, dout, w.scale, w.causal, varlen_offsets=off,
                           max_seqlen=ms)
    torch.cuda.synchronize()
    return (q, k, v, o, lse, dout, off), ref


def _noalloc(w, t):
    import torch
    import flashattention_forward_fa_amd as fa
    q, k, v, o, lse, dout, off = t
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    st = fa.fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, w.B, w.H, w.Nq, w.Nk, w.d,
                           w.scale, int(w.causal), off, w.kv_heads, None)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("which", ["fixed", "varlen"])
def test_noalloc_matches_fa_bwd_twice_second_smaller(which):
    import torch
    if which == "fixed":
        big = wl.make_fixed(2, 8, 700, 700, 128, seed=61, causal=True, Hkv=2)
        small = wl.make_fixed(1, 4, 200, 300, 128, seed=62, causal=True)
    else:
        big = wl.make_varlen(8, 64, seed=63, lengths=[500, 0, 129, 700], causal=True)
        small = wl.make_varlen(4, 64, seed=64, lengths=[33, 100], causal=False)
    for w, seed in ((big, 71), (small, 72)):
        t, ref = _case(w, seed)
        got = _noalloc(w, t)
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(g, r), f"{w.name} {name}"


def test_noalloc_refuses_problems_past_its_array():
    import torch
    import flashattention_forward_fa_amd as fa
    cap = fa.fa_bwd_noalloc_max_bytes()
    assert cap == 32 << 20
    x = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(16, dtype=torch.float32, device="cuda")
    H, Nq = 32, (cap // 4) // 32 + 1              # 4 * H * Nq just past the array
    st = fa.fa_bwd_noalloc(x, x, x, x, lse, x, x, x, x, 1, H, Nq, Nq, 128, 0.1, 1, None, 0, None)
    assert st == fa.FA_ERR_TOO_LARGE
    assert "scratch" in fa.fa_status_string(st)
