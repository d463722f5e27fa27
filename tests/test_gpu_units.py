"""GPU unit tests of the forward kernel's row reductions (lane_pair_max,
lane_pair_sum of fa_device.h), run in a test-only kernel that holds a score
block in the forward kernel's accumulator layout; and of the dispatch order the
XCD-aware tile orders rely on; and a measurement of the issue rates behind
the forward kernel's phase slot (printed).

The vectors are the page's ("FlashAttention：一次前向计算", qingsen, section
"how the max of one row is found across threads", table 7, and section "sum
reduces over the same lanes"): a 64-key row whose first eight scores are
-4 .. 3 and the rest -5 reduces to 3 on every lane; partial sums that the page
combines in two exchange steps ((1/2, 1, 1/4, 1/4) -> (3/4, 5/4) -> 2) reduce
to 2.  In this layout a row's keys sit on two lanes (l and l ^ 32) instead of
four, so the page's middle step is what each half-wave holds after its in-lane
sum, and one exchange gives 2."""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "kernels", "libfa_unit.so")


@pytest.fixture(scope="module")
def unit():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} missing: build it with tests/kernels/build.py")
    lib = ctypes.CDLL(LIB)
    lib.fa_unit_lane_reduce.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_unit_lane_reduce.restype = ctypes.c_int
    lib.fa_unit_xcd_of_workgroups.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_void_p]
    lib.fa_unit_xcd_of_workgroups.restype = ctypes.c_int
    lib.fa_unit_issue_rates.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_unit_issue_rates.restype = ctypes.c_int
    return lib


def _run(lib, S):
    import torch
    s = torch.from_numpy(np.ascontiguousarray(S, dtype=np.float32)).cuda()
    out = torch.empty(128, dtype=torch.float32, device="cuda")
    assert s.shape == (32, 64)
    assert lib.fa_unit_lane_reduce(s.data_ptr(), out.data_ptr(), None) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(64, 2)


def test_page_vectors(unit):
    rng = np.random.default_rng(7)
    S = rng.standard_normal((32, 64)).astype(np.float32)
    S[0] = -5.0
    S[0, :8] = np.arange(-4, 4)                   # table 7: max 3
    S[1] = 0.0
    S[1, [0, 8]] = [0.5, 0.25]                   # keys of the lower half-wave: 3/4
    S[1, [4, 12]] = [1.0, 0.25]                   # keys of the upper half-wave: 5/4
    got = _run(unit, S)
    for lane in (0, 32):
        assert got[lane, 0] == 3.0
        assert got[lane + 1, 1] == 2.0
    # every lane ends with its own row's maximum and sum
    for lane in range(64):
        row = S[lane & 31].astype(np.float64)
        assert got[lane, 0] == row.max()
        np.testing.assert_allclose(got[lane, 1], row.sum(), rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("big", [1, 0])
def test_workgroups_run_on_xcd_of_their_index_mod_8(unit, big):
    """The forward and backward tile orders give the workgroups b with one value
    of b mod 8 the tiles of one set of heads, so that the tiles reading one head's
    K/V share an XCD's L2.  That rests on the dispatcher sending consecutive
    workgroups round-robin over the 8 XCDs, so that b and b + 8 share one; the
    hardware register XCC_ID, read by every workgroup of grids of several
    dispatch rounds (workgroups of the d = 128 forward kernel's size and LDS, one
    per compute unit, and of the 256-thread kernels'), shows it.  The first
    workgroup's XCD depends on the launches before (the round-robin carries
    over from one launch to the next), which the orders do not need."""
    import torch
    n = 4096
    out = torch.full((n,), 0xFFFF, dtype=torch.int32, device="cuda")
    assert unit.fa_unit_xcd_of_workgroups(out.data_ptr(), n, big, None) == 0
    torch.cuda.synchronize()
    xcc = out.cpu().numpy().astype(np.int64)
    assert np.array_equal(xcc, (xcc[0] + np.arange(n)) % 8)


def test_issue_rates(unit):
    """Issue rates of the two waves of a SIMD, as the forward kernel's ping-pong
    pairs them (one wave streaming 32x32x16 MFMAs, the other independent
    v_fma_f32): cycles per MFMA and per v_fma_f32, each wave alone and side by
    side.  Printed for the design notes; asserted only where the hardware
    leaves no doubt (an MFMA takes its 8 passes, a wave64 v_fma_f32 at least
    the 4 cycles of a 16-lane SIMD and at most that of the matrix core's)."""
    import torch
    grid, iters = 256, 2000
    cycles = torch.zeros(grid * 8, dtype=torch.int64, device="cuda")
    sink = torch.zeros(grid * 512, dtype=torch.float32, device="cuda")
    rates = {}
    for name, ra, rb in (("mfma alone", 1, 0), ("fma alone", 0, 2), ("side by side", 1, 2)):
        for _ in range(2):   # the first launch warms the clocks and caches
            assert unit.fa_unit_issue_rates(cycles.data_ptr(), sink.data_ptr(), grid, iters, ra, rb,
                                            None) == 0
            torch.cuda.synchronize()
        c = cycles.cpu().numpy().astype(np.float64).reshape(grid, 8)
        rates[name] = (np.median(c[:, :4]) / (4 * iters), np.median(c[:, 4:]) / (32 * iters))
    mfma_alone = rates["mfma alone"][0]
    fma_alone = rates["fma alone"][1]
    mfma_side, fma_side = rates["side by side"]
    print(f"issue rates (shader cycles): v_mfma_f32_32x32x16_bf16 {mfma_alone:.1f} alone, "
          f"{mfma_side:.1f} beside a v_fma_f32 wave; v_fma_f32 {fma_alone:.2f} alone, "
          f"{fma_side:.2f} beside an MFMA wave", flush=True)
    assert 30.0 <= mfma_alone <= 40.0 and 30.0 <= mfma_side <= 40.0
    assert 4.0 <= fma_alone <= 32.0 and 4.0 <= fma_side <= 32.0
