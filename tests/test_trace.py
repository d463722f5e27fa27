"""The timeline build (FA_TRACE): the summary arithmetic on a synthetic
timeline (CPU), the plain library's refusal of a trace buffer (CPU), and on
the GPU a traced launch whose stamps are ordered phase boundaries and whose
O equals the plain library's."""
import ctypes

import numpy as np
import pytest

import flashattention_forward_fa_amd as fa
from flashattention_forward_fa_amd import trace


def _synthetic_workgroup(slot=2000, m_work=(1500, 1600), v_work=(1900, 1800), blocks=10):
    """Eight waves of a ping-pong workgroup: group 0 starts with M(0), group 1
    with V(-1); every phase starts at its slot's start."""
    waves = []
    for wv in range(8):
        g = wv // 4
        ev, t = [(1, 0)], 100
        kinds = (["M", "V"] if g == 0 else ["V", "M"]) * blocks
        for kind in kinds:
            if kind == "M":
                ev += [(2, t), (3, t + m_work[g])]
            else:
                ev += [(4, t), (7, t + v_work[g])]
            t += slot
        ev += [(8, t), (9, t + 50)]
        waves.append(ev)
    return waves


def test_summary_of_a_synthetic_timeline():
    st = trace.summarise([_synthetic_workgroup(), _synthetic_workgroup()], d=128)
    assert st["slot"] == 2000
    assert st["m_work_g0"] == 1500 and st["v_work_g0"] == 1900
    assert st["m_work_g1"] == 1600 and st["v_work_g1"] == 1800
    # slots alternate between (group 0 M, group 1 V): slowest 1800, and
    # (group 0 V, group 1 M): slowest 1900
    assert st["slowest_work"] == 1850 and st["overhead"] == 150
    assert st["mfma_per_block"] == 1024 and st["n_waves"] == 16
    # start at 0, first M phase at 100 (group 0) or 2100 (group 1); loop end
    # 20 slots after 100, end 50 later
    assert st["epilogue"] == 50
    assert st["edge_share"] == (4 * 150 + 4 * 2150) / (8 * (100 + 20 * 2000 + 50))


def test_summary_of_a_synthetic_timeline_one_group():
    waves = []
    for _ in range(4):
        ev, t = [(1, 0)], 100
        for _ in range(10):
            ev += [(2, t), (3, t + 700), (4, t + 720), (7, t + 1600)]
            t += 1700
        ev += [(8, t), (9, t + 50)]
        waves.append(ev)
    st = trace.summarise([waves], d=64)
    assert st["slot"] == 1700 and st["m_work_g0"] == 700 and st["v_work_g0"] == 880
    assert st["slowest_work"] == 1600 and st["overhead"] == 100


def test_stamps_decode():
    row = np.zeros(trace.EVENTS, dtype=np.uint64)
    row[0] = (np.uint64(1) << np.uint64(56)) | np.uint64(12345)
    row[1] = (np.uint64(2) << np.uint64(56)) | np.uint64(12400)
    wgs = trace.phases(row.reshape(1, 1, -1))
    assert wgs == [[[(1, 12345), (2, 12400)]]]


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
    wgs = trace.phases(stamps)
    assert len(wgs) == 8 and all(len(waves) == 8 for waves in wgs)   # every wave of 8 workgroups
    for ev in (ev for waves in wgs for ev in waves):
        codes = [c for c, _ in ev]
        t = [x for _, x in ev]
        assert codes[0] == 1 and codes[-1] == 9 and 8 in codes
        assert all(b >= a for a, b in zip(t, t[1:]))
        assert codes.count(2) == codes.count(3) and codes.count(4) == codes.count(7)
    st = trace.summarise(wgs, w.d)
    assert st["slot"] > 0 and st["slowest_work"] > 0 and st["m_work_g0"] > 0
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
