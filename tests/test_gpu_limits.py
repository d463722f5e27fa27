"""The largest head counts the C ABI admits (H * d < 2^23, where a 256-row
tile's 32-bit buffer range is 2^32 - 64 KiB): forward and backward.

Every head holds the same seeded data (one head's Q, K, V, dO replicated on the
device), so every head's result is the oracle's result for that one head; the
first, second, middle and last heads are compared in full.  An offset that
overflowed would send the far heads to the wrong memory.
"""
import numpy as np
import pytest

import oracle
from flashattention_forward_fa_amd import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu
N = 300


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import flashattention_forward_fa_amd as fa
    fa.load()


def replicated(bits, H):
    """[N, d] bf16 bits -> a [1, N, H, d] bf16 device tensor, every head equal."""
    import torch
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return t[None, :, None, :].expand(1, t.shape[0], H, t.shape[1]).contiguous()


@pytest.mark.parametrize("H,d", [(65535, 128), (131071, 64)])
def test_largest_head_count(H, d):
    import torch
    import flashattention_forward_fa_amd as fa
    assert 256 * H * d * 2 < 2 ** 32 <= 256 * (H + 1) * d * 2
    base = wl.make_fixed(1, 1, N, N, d, seed=4321 + d, causal=True)
    dout_bits = wl.make_dout(base, seed=4322)
    q, k, v = (replicated(x[0, :, 0], H) for x in (base.q, base.k, base.v))
    o, lse = fa.attention(q, k, v, base.scale, True)
    qf, kf, vf = parity.inputs_f64(base)
    o_ref, lse_ref = oracle.attention(qf, kf, vf, base.scale, True)
    heads = [0, 1, H // 2, H - 1]
    for h in heads:
        parity.compare(o[0, :, h].double().cpu().numpy()[None, :, None], lse[0, h].double().cpu().numpy()[None, None],
                       o_ref, lse_ref, bf16_out=True, what=f"H={H} d={d} head {h}")
    if d == 128:
        do = replicated(dout_bits[0, :, 0], H)
        dq, dk, dv = fa.attention_bwd(q, k, v, o, lse, do, base.scale, True)
        torch.cuda.synchronize()
        ref = oracle.attention_bwd(qf, kf, vf, wl.bf16_to_f64(dout_bits), base.scale, True)
        for h in heads:
            got = tuple(t[0, :, h].double().cpu().numpy()[None, :, None] for t in (dq, dk, dv))
            parity.compare_grads(got, ref, f"backward H={H} head {h}")
        del do, dq, dk, dv
    del q, k, v, o, lse
    torch.cuda.empty_cache()
