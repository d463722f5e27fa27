"""The timeline build (FA_TRACE): the summary arithmetic on a synthetic
timeline (CPU), the plain library's refusal of a trace buffer (CPU), and on
the GPU a traced launch whose stamps are ordered phase boundaries and whose
O equals the plain library's."""
import ctypes

import numpy as np
import pytest

import flashattention_forward_fa_amd as fa
from flashattention_forward_fa_amd import trace


def _synthetic_wave(slot=2000, m_work=1500, stores=300, loads=200, soft=1400, blocks=10):
    ev, t = [(1, 0)], 100
    for _ in range(blocks):
        ev += [(2, t), (3, t + m_work)]
        t += slot
        ev += [(4, t), (5, t + stores), (6, t + stores + loads), (7, t + stores + loads + soft)]
        t += slot
    ev += [(8, t), (9, t + 50)]
    return ev


def test_summary_of_a_synthetic_timeline():
    st = trace.summarise([_synthetic_wave(), _synthetic_wave()], d=128)
    assert st["slot"] == 2000 and st["m_work"] == 1500 and st["m_wait"] == 500
    assert st["v_stores"] == 300 and st["v_loads"] == 200 and st["v_softmax"] == 1400
    assert st["v_work"] == 1900 and st["v_wait"] == 100
    assert st["mfma_per_block"] == 1024
    # start at 0, first M phase at 100; loop end at 100 + 20 slots, end 50 later
    assert st["prologue"] == 100 and st["epilogue"] == 50
    assert st["edge_share"] == 150 / (100 + 20 * 2000 + 50)


def test_stamps_decode():
    row = np.zeros(trace.EVENTS, dtype=np.uint64)
    row[0] = (np.uint64(1) << np.uint64(56)) | np.uint64(12345)
    row[1] = (np.uint64(2) << np.uint64(56)) | np.uint64(12400)
    waves = trace.phases(row.reshape(1, 1, -1))
    assert waves == [[(1, 12345), (2, 12400)]]


def test_plain_library_refuses_a_trace_buffer():
    opts = fa.fa_fwd_opts_default()
    assert opts.trace is None and opts.trace_workgroups == 0
    P = 1 << 20
    opts.trace = P
    opts.trace_workgroups = 4
    st = fa.fa_fwd_check(P, P, P, P, P, 1, 2, 64, 64, 128, 0.1, 1, None, opts)
    assert st == fa.FA_ERR_UNSUPPORTED


@pytest.mark.gpu
def test_traced_launch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from flashattention_forward_fa_amd import workloads as wl
    from tests import parity
    w = wl.make_fixed(1, 8, 1024, 1024, 128, seed=90, causal=True)
    stamps = trace.record(w, 8.0, workgroups=8, settle_s=0.05)
    waves = trace.phases(stamps)
    assert len(waves) == 16                       # waves 0 and 4 of 8 workgroups
    for ev in waves:
        codes = [c for c, _ in ev]
        t = [x for _, x in ev]
        assert codes[0] == 1 and codes[-1] == 9 and 8 in codes
        assert all(b >= a for a, b in zip(t, t[1:]))
        assert codes.count(2) == codes.count(3) and codes.count(4) == codes.count(7)
    st = trace.summarise(waves, w.d)
    assert st["slot"] > 0 and st["m_work"] >= st["mfma_per_block"] * 0.9
    # the traced build computes what the plain one does
    o_plain, l_plain = parity.run_gpu(w)
    lib = trace.load_trace_lib()
    q, k, v, _ = parity.to_device(w)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    opts = fa.FaFwdOpts()
    lib.fa_fwd_opts_default(ctypes.byref(opts))
    assert lib.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         w.B, w.H, w.Nq, w.Nk, w.d, w.scale, 1, None, None, ctypes.byref(opts)) == 0
    torch.cuda.synchronize()
    assert np.array_equal(o.double().cpu().numpy(), o_plain)
    assert np.array_equal(lse.double().cpu().numpy(), l_plain)
