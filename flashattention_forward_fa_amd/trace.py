"""Phase timeline of the forward kernel, from the timeline build of the library.

``libfa_trace.so`` (``python -m flashattention_forward_fa_amd.build --trace``)
is the library compiled with FA_TRACE: lane 0 of every wave of the first
workgroups records shader-clock stamps at the phase boundaries of the block
loop into ``fa_fwd_opts.trace``.  This tool runs one workload on that build
after a settle phase and summarises the steady-state blocks of the traced
workgroups (medians, shader cycles):

  M phase   -- rescale, S = Q K^T, O += P V issued
  V phase   -- LDS writes of the staged K/V, issue of the next global loads,
               masking and softmax
  per group -- the work of each phase for the waves of ping-pong group 0
               (waves 0-3) and group 1 (waves 4-7): the two groups are in
               opposite phases in every slot
  slot      -- one phase of the ping-pong (a block takes two slots per
               wave), set by the slowest of the eight waves' phase work plus
               the barrier: "overhead" is the slot minus that slowest work
  prologue  -- from the wave's start to its first M phase (Q fragments,
               first K/V block); epilogue -- from the end of the block loop to
               the end (normalisation, O and LSE stores); with their sum over
               the traced waves as a share of the waves' whole time

At d = 64 there is one group and no barrier between the phases of a block, so
a slot is one block (M then V).  The stamps sit only at phase boundaries,
where the wave has no LDS operation outstanding, so reading the clock (which
waits for them) leaves the phases' lengths nearly unchanged.

    python -m flashattention_forward_fa_amd.trace [--config 3] [--workgroups 64]
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
WAVES = 8              # kTraceWaves: stamp rows per traced workgroup
NAMES = {1: "start", 2: "M begin", 3: "M end", 4: "V begin", 7: "V end", 8: "loop end", 9: "end"}
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
    Returns the raw stamps, shape [workgroups, WAVES, EVENTS] (uint64)."""
    import torch
    import flashattention_forward_fa_amd as fa
    from tests import parity
    lib = load_trace_lib()
    q, k, v, off = parity.to_device(w)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.H, w.total_tokens) if w.varlen else (w.B, w.H, w.Nq),
                      dtype=torch.float32, device="cuda")
    buf = torch.zeros(workgroups * WAVES * EVENTS, dtype=torch.int64, device="cuda")
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
    return buf.cpu().numpy().view(np.uint64).reshape(workgroups, WAVES, EVENTS)


def phases(stamps):
    """Per traced workgroup, per wave, the list of (code, cycle) events in order
    (waves that recorded nothing are left out)."""
    out = []
    for wg in range(stamps.shape[0]):
        waves = []
        for wv in range(stamps.shape[1]):
            row = stamps[wg, wv]
            codes = (row >> np.uint64(56)).astype(np.int64)
            t = (row & np.uint64(0x00FFFFFFFFFFFFFF)).astype(np.int64)
            n = int(np.argmax(codes == 0)) if np.any(codes == 0) else len(codes)
            if n:
                waves.append(list(zip(codes[:n].tolist(), t[:n].tolist())))
        if waves:
            out.append(waves)
    return out


def _phase_list(ev):
    """(kind, begin, end) of each M and V phase of one wave, in order."""
    ph = []
    for (c0, t0), (c1, t1) in zip(ev, ev[1:]):
        if c0 == 2 and c1 == 3:
            ph.append(("M", t0, t1))
        elif c0 == 4 and c1 == 7:
            ph.append(("V", t0, t1))
    return ph


def summarise(workgroups, d: int):
    """Medians over the steady-state phases (the first and last three of each
    wave dropped).  workgroups: the output of phases()."""
    med = lambda x: float(np.median(x)) if len(x) else float("nan")
    group_m = {0: [], 1: []}
    group_v = {0: [], 1: []}
    slots, slowest, pro, epi = [], [], [], []
    edge = total = 0
    for waves in workgroups:
        for ev in waves:
            codes = [c for c, _ in ev]
            if codes and codes[0] == 1 and codes[-1] == 9 and 2 in codes and 8 in codes:
                t_first_m = ev[codes.index(2)][1]
                t_loop_end = ev[len(codes) - 1 - codes[::-1].index(8)][1]
                pro.append(t_first_m - ev[0][1])
                epi.append(ev[-1][1] - t_loop_end)
                edge += pro[-1] + epi[-1]
                total += ev[-1][1] - ev[0][1]
        lists = [_phase_list(ev) for ev in waves]
        pingpong = len(waves) == 8
        if pingpong:
            # phase k of every wave is slot k (group 1 starts with V(-1))
            n = min(len(p) for p in lists)
            for k in range(3, n - 3):
                work = [p[k][2] - p[k][1] for p in lists]
                for wv, p in enumerate(lists):
                    (group_m if p[k][0] == "M" else group_v)[wv // 4].append(work[wv])
                begin = np.median([p[k][1] for p in lists])
                nxt = np.median([p[k + 1][1] for p in lists])
                slots.append(nxt - begin)
                slowest.append(max(work))
        else:
            # one group: a slot is a block, M then V
            pairs = [[(p[i], p[i + 1]) for i in range(0, len(p) - 1, 2)
                      if p[i][0] == "M" and p[i + 1][0] == "V"] for p in lists]
            n = min(len(q) for q in pairs)
            for k in range(3, n - 3):
                for q in pairs:
                    group_m[0].append(q[k][0][2] - q[k][0][1])
                    group_v[0].append(q[k][1][2] - q[k][1][1])
                begin = np.median([q[k][0][1] for q in pairs])
                nxt = np.median([q[k + 1][0][1] for q in pairs])
                slots.append(nxt - begin)
                slowest.append(max(q[k][1][2] - q[k][0][1] for q in pairs))
    mfma = (d // 16) * 2 * MFMA_CYCLES + (d // 32) * 4 * MFMA_CYCLES   # QK + PV per 64-key block
    return {"slot": med(slots), "slowest_work": med(slowest),
            "overhead": med(np.array(slots) - np.array(slowest)) if slots else float("nan"),
            "m_work_g0": med(group_m[0]), "v_work_g0": med(group_v[0]),
            "m_work_g1": med(group_m[1]), "v_work_g1": med(group_v[1]),
            "mfma_per_block": mfma, "n_slots": len(slots),
            "n_waves": sum(len(w) for w in workgroups), "prologue": med(pro),
            "epilogue": med(epi), "edge_share": edge / total if total else float("nan")}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--tau", type=float, default=8.0)
    ap.add_argument("--workgroups", type=int, default=64)
    args = ap.parse_args()
    import torch
    from flashattention_forward_fa_amd import workloads as wl
    torch.cuda.set_device(0)
    w = wl.config(args.config)
    st = summarise(phases(record(w, args.tau, args.workgroups)), w.d)
    print(f"workload {w.name}, tau {args.tau:g}: {st['n_waves']} traced waves, "
          f"{st['n_slots']} steady-state slots (medians, shader cycles)")
    print(f"  slot {st['slot']:8.0f}   slowest wave's phase work {st['slowest_work']:6.0f}   "
          f"barrier and skew {st['overhead']:6.0f}")
    print(f"  group 0 (waves 0-3): M work {st['m_work_g0']:6.0f}   V work {st['v_work_g0']:6.0f}")
    if w.d == 128:
        print(f"  group 1 (waves 4-7): M work {st['m_work_g1']:6.0f}   V work {st['v_work_g1']:6.0f}")
    if w.d == 128:
        # per slot each SIMD's matrix core runs one wave's block of MFMAs
        print(f"  MFMA cycles per block per wave {st['mfma_per_block']}; matrix-core share of a "
              f"slot {st['mfma_per_block'] / st['slot']:.3f}")
    print(f"  prologue {st['prologue']:6.0f}   epilogue {st['epilogue']:6.0f}   "
          f"(their share of the traced waves' time: {st['edge_share']:.3f})")


if __name__ == "__main__":
    main()
