"""flash_attention: the forward and backward as one differentiable torch
operation.  Its output and gradients must be, bit for bit, those of the direct
calls (attention, then attention_bwd on the saved O and LSE), which the other
GPU tests hold to the oracle."""
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


def _dout(w, seed):
    import torch
    return torch.from_numpy(wl.make_dout(w, seed=seed).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("case", ["fixed_causal_gqa", "fixed_full_d64", "varlen_causal"])
def test_autograd_matches_direct_calls(case):
    import torch
    import flashattention_forward_fa_amd as fa
    if case == "fixed_causal_gqa":
        w = wl.make_fixed(2, 4, 300, 300, 128, seed=61, causal=True, Hkv=2)
    elif case == "fixed_full_d64":
        w = wl.make_fixed(1, 2, 200, 330, 64, seed=62, causal=False)
    else:
        w = wl.make_varlen(8, 64, seed=63, lengths=[150, 0, 33, 260], causal=True)
    q, k, v, off = parity.to_device(w)
    ms = w.Nq if w.varlen else None
    do = _dout(w, seed=64)
    o_ref, lse_ref = fa.attention(q, k, v, w.scale, w.causal, varlen_offsets=off, max_seqlen=ms)
    ref = fa.attention_bwd(q, k, v, o_ref, lse_ref, do, w.scale, w.causal, varlen_offsets=off,
                           max_seqlen=ms)
    qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = fa.flash_attention(qg, kg, vg, w.scale, w.causal, varlen_offsets=off, max_seqlen=ms)
    o.backward(do)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    for got, exp, name in zip((qg.grad, kg.grad, vg.grad), ref, ("dq", "dk", "dv")):
        assert got.dtype == torch.bfloat16 and got.shape == exp.shape, name
        assert torch.equal(got, exp), name


def test_autograd_non_contiguous_upstream_gradient():
    """An upstream gradient that is a transposed view is made contiguous first."""
    import torch
    import flashattention_forward_fa_amd as fa
    w = wl.make_fixed(1, 2, 128, 128, 64, seed=65, causal=True)
    q, k, v, _ = parity.to_device(w)
    do = _dout(w, seed=66)
    do_t = do.transpose(1, 2).contiguous().transpose(1, 2)     # same values, other strides
    assert not do_t.is_contiguous()
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    fa.flash_attention(qa, ka, va, w.scale, True).backward(do)
    qb, kb, vb = (t.clone().requires_grad_(True) for t in (q, k, v))
    fa.flash_attention(qb, kb, vb, w.scale, True).backward(do_t)
    torch.cuda.synchronize()
    for a, b in ((qa.grad, qb.grad), (ka.grad, kb.grad), (va.grad, vb.grad)):
        assert torch.equal(a, b)
