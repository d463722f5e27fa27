"""Phase timeline of the forward kernel, from the timeline build of the library.

``libfa_trace.so`` (``python -m flashattention_forward_fa_amd.build --trace``)
is the library compiled with FA_TRACE: lane 0 of waves 0 and 4 (one per
ping-pong group) of the first workgroups records shader-clock stamps at every
phase boundary of the block loop into ``fa_fwd_opts.trace``.  This tool runs
one workload on that build after a settle phase, and summarises, per phase
over the steady-state blocks of the traced waves (medians, shader cycles):

  M phase   -- rescale, S = Q K^T, O += P V issued; then the wait at the barrier
  V phase   -- LDS writes of the staged K/V ("stores"), issue of the next
               global loads ("loads"), masking and softmax; then the barrier
  slot      -- one phase of the ping-pong: the SIMD's two waves are in
               opposite phases, so a block takes two slots per wave
  prologue  -- from the wave's start to its first M phase (Q fragments,
               first K/V block); epilogue -- from the end of the block loop to
               the end (normalisation, O and LSE stores); with their sum over
               the traced waves as a share of the waves' whole time

and the matrix-core share of a slot (the MFMA cycles one M phase issues).  The
stamps themselves wait for the wave's outstanding LDS and scalar operations,
so absolute phase lengths are a little above the untraced kernel's; and each
stamp is a global store, which the vector-memory counter counts like a load,
so a section that waits for the staged K/V loads ("LDS writes") also waits
for the stamps stored before it and reads long.

    python -m flashattention_forward_fa_amd.trace [--config 3] [--workgroups 256]
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

EVENTS = 1024          # kTraceEvents
NAMES = {1: "start", 2: "M begin", 3: "M end", 4: "V begin", 5: "V stored", 6: "V loaded",
         7: "V end", 8: "loop end", 9: "end"}
MFMA_CYCLES = 32       # one v_mfma_f32_32x32x16 (bf16 or fp16) on the matrix core


def load_trace_lib():
    import flashattention_forward_fa_amd as fa
    fa._bind_torch_hip_runtime()
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_trace.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} missing: build it with "
                           f"`python -m flashattention_forward_fa_amd.build --trace`")
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp,
                              ctypes.POINTER(fa.FaFwdOpts)]
    lib.fa_fwd_ex.restype = i
    lib.fa_fwd_opts_default.argtypes = [ctypes.POINTER(fa.FaFwdOpts)]
    return lib


def record(w, tau: float, workgroups: int, settle_s: float = 0.5):
    """Run workload w on the timeline build: settle, then one traced launch.
    Returns the raw stamps, shape [workgroups, 2, EVENTS] (uint64)."""
    import torch
    import flashattention_forward_fa_amd as fa
    from tests import parity
    lib = load_trace_lib()
    q, k, v, off = parity.to_device(w)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.H, w.total_tokens) if w.varlen else (w.B, w.H, w.Nq),
                      dtype=torch.float32, device="cuda")
    buf = torch.zeros(workgroups * 2 * EVENTS, dtype=torch.int64, device="cuda")
    opts = fa.FaFwdOpts()
    lib.fa_fwd_opts_default(ctypes.byref(opts))
    opts.rescale_threshold = tau
    opts.kv_heads = w.kv_heads
    stream = torch.cuda.current_stream().cuda_stream

    def launch(traced):
        opts.trace = buf.data_ptr() if traced else None
        opts.trace_workgroups = workgroups if traced else 0
        st = lib.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           w.B, w.H, w.Nq, w.Nk, w.d, w.scale, int(w.causal),
                           off.data_ptr() if off is not None else None, stream,
                           ctypes.byref(opts))
        if st != 0:
            raise fa.FaError(st, "fa_fwd_ex (trace build)")

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(10):
            launch(False)
        torch.cuda.synchronize()
    launch(True)
    torch.cuda.synchronize()
    return buf.cpu().numpy().view(np.uint64).reshape(workgroups, 2, EVENTS)


def phases(stamps):
    """Per traced wave, the list of (code, cycle) events in order."""
    out = []
    for wg in range(stamps.shape[0]):
        for wv in range(stamps.shape[1]):
            row = stamps[wg, wv]
            codes = (row >> np.uint64(56)).astype(np.int64)
            t = (row & np.uint64(0x00FFFFFFFFFFFFFF)).astype(np.int64)
            n = int(np.argmax(codes == 0)) if np.any(codes == 0) else len(codes)
            if n:
                out.append(list(zip(codes[:n].tolist(), t[:n].tolist())))
    return out


def summarise(waves, d: int):
    """Medians over steady-state phases (the first and last two of each wave's
    M and V phases dropped)."""
    m_work, m_wait, v_store, v_load, v_soft, v_wait, v_work, slots = ([] for _ in range(8))
    pro, epi = [], []
    edge = total = 0
    for ev in waves:
        codes = [c for c, _ in ev]
        if codes and codes[0] == 1 and codes[-1] == 9 and 2 in codes and 8 in codes:
            t_first_m = ev[codes.index(2)][1]
            t_loop_end = ev[len(codes) - 1 - codes[::-1].index(8)][1]
            pro.append(t_first_m - ev[0][1])
            epi.append(ev[-1][1] - t_loop_end)
            edge += pro[-1] + epi[-1]
            total += ev[-1][1] - ev[0][1]
        m_beg = [i for i, (c, _) in enumerate(ev) if c == 2]
        v_beg = [i for i, (c, _) in enumerate(ev) if c == 4]
        for a in m_beg[2:-2]:
            if a + 2 < len(ev) and ev[a + 1][0] == 3 and ev[a + 2][0] == 4:
                m_work.append(ev[a + 1][1] - ev[a][1])
                m_wait.append(ev[a + 2][1] - ev[a + 1][1])
        for a in v_beg[2:-2]:
            if a + 4 < len(ev) and [c for c, _ in ev[a:a + 5]] == [4, 5, 6, 7, 2]:
                v_store.append(ev[a + 1][1] - ev[a][1])
                v_load.append(ev[a + 2][1] - ev[a + 1][1])
                v_soft.append(ev[a + 3][1] - ev[a + 2][1])
                v_work.append(ev[a + 3][1] - ev[a][1])
                v_wait.append(ev[a + 4][1] - ev[a + 3][1])
        for x, y in zip(m_beg[2:-3], m_beg[3:-2]):
            slots.append((ev[y][1] - ev[x][1]) / 2.0)
    med = lambda x: float(np.median(x)) if x else float("nan")
    mfma = (d // 16) * 2 * MFMA_CYCLES + (d // 32) * 4 * MFMA_CYCLES   # QK + PV per 64-key block
    return {"slot": med(slots), "m_work": med(m_work), "m_wait": med(m_wait),
            "v_work": med(v_work), "v_stores": med(v_store), "v_loads": med(v_load),
            "v_softmax": med(v_soft), "v_wait": med(v_wait), "mfma_per_block": mfma,
            "n_slots": len(slots), "n_waves": len(waves), "prologue": med(pro),
            "epilogue": med(epi), "edge_share": edge / total if total else float("nan")}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--tau", type=float, default=8.0)
    ap.add_argument("--workgroups", type=int, default=256)
    args = ap.parse_args()
    import torch
    from flashattention_forward_fa_amd import workloads as wl
    torch.cuda.set_device(0)
    w = wl.config(args.config)
    st = summarise(phases(record(w, args.tau, args.workgroups)), w.d)
    print(f"workload {w.name}, tau {args.tau:g}: {st['n_waves']} traced waves, "
          f"{st['n_slots']} steady-state slots (medians, shader cycles)")
    print(f"  slot (one phase of the ping-pong)      {st['slot']:8.0f}")
    print(f"  M phase: work {st['m_work']:6.0f}   wait at barrier {st['m_wait']:6.0f}   "
          f"(MFMA issue per block {st['mfma_per_block']})")
    print(f"  V phase: work {st['v_work']:6.0f}   wait at barrier {st['v_wait']:6.0f}")
    print(f"           LDS writes {st['v_stores']:6.0f}   load issue {st['v_loads']:6.0f}   "
          f"mask + softmax {st['v_softmax']:6.0f}")
    print(f"  matrix-core share of a slot: {st['mfma_per_block'] / st['slot']:.3f}")
    print(f"  prologue {st['prologue']:6.0f}   epilogue {st['epilogue']:6.0f}   "
          f"(their share of the traced waves' time: {st['edge_share']:.3f})")


if __name__ == "__main__":
    main()
