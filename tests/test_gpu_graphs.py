"""HIP graph capture: one forward call and one backward call recorded into a
torch CUDA graph (a hipGraph on ROCm) replay to the eager results bit for bit,
replay after replay, with other eager work and synchronisations between the
replays.  The library issues only kernel launches on the caller's stream (no
allocation, copy or memset), which is what makes its calls capturable."""
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


@pytest.mark.parametrize("case", ["fixed_causal_gqa", "varlen_causal"])
def test_captured_forward_and_backward_replay_bitwise(case):
    import torch
    import flashattention_forward_fa_amd as fa
    if case == "fixed_causal_gqa":
        w = wl.make_fixed(2, 4, 333, 333, 128, seed=71, causal=True, Hkv=2)
        lse_shape = (w.B, w.H, w.Nq)
    else:
        w = wl.make_varlen(8, 64, seed=72, lengths=[200, 0, 77, 300], causal=True)
        lse_shape = (w.H, w.total_tokens)
    q, k, v, off = parity.to_device(w)
    do = torch.from_numpy(wl.make_dout(w, seed=73).view(np.int16)).view(torch.bfloat16).cuda()
    o = torch.empty_like(q)
    lse = torch.empty(lse_shape, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty((fa.fa_bwd_workspace_size(w.B, w.H, w.Nq) // 4,), dtype=torch.float32,
                     device="cuda")
    opts = fa.fa_fwd_opts_default()
    opts.kv_heads = w.kv_heads

    def step():   # on torch's current stream (the capture stream while capturing)
        st = fa.fa_fwd_ex(q, k, v, o, lse, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, w.causal, off,
                          None, opts)
        assert st == fa.FA_OK, fa.fa_status_string(st)
        st = fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, w.B, w.H, w.Nq, w.Nk, w.d, w.scale,
                       w.causal, off, w.kv_heads)
        assert st == fa.FA_OK, fa.fa_status_string(st)

    outs = (o, lse, dq, dk, dv)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    side = torch.cuda.Stream()          # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        for t in outs:                  # eager work between replays: overwrite every output
            t.fill_(float(rep + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, exp in zip(("o", "lse", "dq", "dk", "dv"), outs, ref):
            assert torch.equal(got, exp), f"replay {rep}: {name}"
