"""Per-workgroup phase timestamps of the one-launch decode kernels.

Runs the decode step of one workload through the profiling build of the
library (libloki_stamps.so: the same kernels with LOKI_PHASE_STAMPS defined,
see csrc/phase_stamps.h) and prints, for the last of a run of back-to-back
steps, each phase's duration over the workgroups, the workgroups' end times
and how many workgroups are in each phase every 5 us.

    python -m sparse_decode_attention_rotate_amd.build --stamps
    python phase_stamps.py --workload llama2_7b_f16 [--out FILE]

Phases (boundaries recorded by thread 0 of each workgroup with the constant
100 MHz clock): the one-workgroup-per-(b, kv) kernel -- rotation, scores,
selection (with the rest of the rotation), attention; the
one-workgroup-per-head kernel -- rotation, scores, selection, append wait,
attention.  The stamps cost a few global stores per workgroup; the step time
printed is that of the stamped build.
"""
import argparse
import ctypes
import os
import sys
import time

import numpy as np
import torch

import sparse_decode_attention_rotate_amd as loki
import workloads as W

PHASES = {1: ("fused", ["rotation", "scores", "selection", "attention"]),
          2: ("head", ["rotation", "scores", "selection", "append wait", "attention"])}
SLOTS = 16  # kStampSlots of csrc/phase_stamps.h (the last holds HW_ID)
MAX_WG = 8192


def to_device(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama2_7b_f16", choices=sorted(W.WORKLOADS))
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    path = os.path.join(os.path.dirname(loki.LIB_PATH), "libloki_stamps.so")
    if not os.path.exists(path):
        sys.exit(f"{path} not built: python -m sparse_decode_attention_rotate_amd.build --stamps")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p

    wl = W.get(args.workload)
    x = W.generate(wl)
    desc = loki.Desc(batch=wl.B, n_q_heads=wl.Hq, n_kv_heads=wl.Hkv, head_dim=wl.D,
                     seq_len=wl.S, seq_capacity=wl.capacity, panel_dim=wl.d,
                     dtype=loki.NAME_CODE[wl.dtype])
    plan = loki.decode_kernel(desc, wl.d, wl.k, wl.append)
    if plan not in PHASES:
        sys.exit(f"{args.workload} does not run as one launch (plan {plan})")
    kernel, names = PHASES[plan]
    q, P = to_device(x["q"], wl.dtype), torch.from_numpy(np.ascontiguousarray(x["P"])).cuda()
    rows = to_device(x["krot"], wl.dtype)
    kc0 = loki.empty_kcache(desc)
    loki.pack_kcache(rows, kc0, desc.with_seq_len(wl.capacity))
    del rows
    v0 = to_device(x["v"], wl.dtype)
    kcs, vcs = [kc0] + [kc0.clone() for _ in range(2)], [v0] + [v0.clone() for _ in range(2)]
    k_new = to_device(x["k_new"], wl.dtype) if wl.append else None
    v_new = to_device(x["v_new"], wl.dtype) if wl.append else None
    out = torch.empty((wl.B, wl.Hq, wl.D), dtype=torch.float32, device="cuda")
    ws = loki.empty_workspace(desc, wl.d, wl.k)
    cd = desc.c()
    st = vp(torch.cuda.current_stream().cuda_stream)

    def step(i):
        kc, vc = kcs[i % 3], vcs[i % 3]
        if wl.append:
            rc = lib.loki_decode_append(vp(q.data_ptr()), vp(k_new.data_ptr()), vp(v_new.data_ptr()),
                                        vp(kc.data_ptr()), vp(vc.data_ptr()), vp(P.data_ptr()),
                                        wl.d, wl.k, vp(out.data_ptr()), None, None,
                                        ctypes.byref(cd), vp(ws.data_ptr()),
                                        ctypes.c_size_t(ws.numel()), st)
        else:
            rc = lib.loki_decode(vp(q.data_ptr()), vp(kc.data_ptr()), vp(vc.data_ptr()),
                                 vp(P.data_ptr()), wl.d, wl.k, vp(out.data_ptr()), None, None,
                                 ctypes.byref(cd), vp(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
                                 st)
        if rc != 0:
            sys.exit(f"loki call failed: {rc}")

    t = time.time()
    while time.time() - t < 0.3:
        for i in range(20):
            step(i)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3

    buf = np.zeros(MAX_WG * SLOTS, np.uint64)
    fn = getattr(lib, f"loki_phase_stamps_{kernel}")
    fn.argtypes, fn.restype = [vp, ctypes.c_size_t], ctypes.c_int
    if fn(buf.ctypes.data_as(vp), MAX_WG) != 0:
        sys.exit("reading the stamps failed")
    s = buf.reshape(MAX_WG, SLOTS).astype(np.int64)
    used = s[:, 0] > 0
    used &= s[:, 0] >= s[used, 0].max() - 100_000  # the last launch (within 1 ms)
    nb = len(names) + 1
    ts = (s[used][:, :nb] - s[used][:, 0].min()) / 100.0  # us
    lines = [f"# python {' '.join(sys.argv)}",
             f"{args.workload}: {W.describe(wl)}",
             f"kernel {kernel}_kernel, {used.sum()} workgroups, {us:.2f} us/step "
             f"(stamped build, {args.steps} back-to-back steps, 3 cache copies cycled); "
             f"last step's span {ts[:, -1].max():.2f} us",
             f"  start      p50 {np.median(ts[:, 0]):6.2f} max {ts[:, 0].max():6.2f}"]
    for i, nm in enumerate(names):
        d = ts[:, i + 1] - ts[:, i]
        lines.append(f"  {nm:12s} dur p10 {np.percentile(d, 10):6.2f} p50 {np.median(d):6.2f} "
                     f"p90 {np.percentile(d, 90):6.2f} max {d.max():6.2f} | ends p50 "
                     f"{np.median(ts[:, i + 1]):7.2f} max {ts[:, i + 1].max():7.2f}")
    lines.append("  workgroups per phase every 5 us:")
    for tt in np.arange(0, ts[:, -1].max() + 5, 5.0):
        ph = [int(((ts[:, i] <= tt) & (ts[:, i + 1] > tt)).sum()) for i in range(len(names))]
        lines.append(f"   t={tt:6.1f} " + " ".join(f"{nm}:{c:4d}" for nm, c in zip(names, ph)))
    # by dispatch round (blocks of 256 workgroups, one per compute unit):
    # when each round's workgroups finish their phases
    blk = np.nonzero(used)[0]
    if len(blk) > 256:
        lines.append("  by dispatch round (blocks of 256 workgroups): p50 / max end of each phase")
        for r0 in range(0, blk.max() + 1, 256):
            m = (blk >= r0) & (blk < r0 + 256)
            if not m.any():
                continue
            cells = " ".join(f"{nm}: {np.median(ts[m, i + 1]):6.2f}/{ts[m, i + 1].max():6.2f}"
                             for i, nm in enumerate(names))
            lines.append(f"   blocks {r0:4d}-{min(r0 + 255, blk.max()):4d}  {cells}")
    # compute units: HW_ID (last slot) gives CU_ID [11:8], SH_ID [12],
    # SE_ID [15:13]; workgroup i runs on XCD i % 8
    hw = s[:, SLOTS - 1]
    cu = ((blk % 8) << 16) | (((hw[blk] >> 13) & 7) << 8) | (((hw[blk] >> 12) & 1) << 4) | \
        ((hw[blk] >> 8) & 15)
    ucu, cnt = np.unique(cu, return_counts=True)
    lines.append(f"  compute units used: {len(ucu)}; workgroups per compute unit: "
                 + ", ".join(f"{c} on {n}" for c, n in zip(*np.unique(cnt, return_counts=True))))
    if len(blk) > 256:
        same = np.mean([cu[i] == cu[i + 256] for i in range(len(blk) - 256)
                        if blk[i] + 256 == blk[i + 256]])
        lines.append(f"  workgroups w and w + 256 on one compute unit: {same:.2f} of the pairs")
        # on compute units holding two workgroups: the later-dispatched one's
        # stream end against the earlier one's
        first, second = [], []
        for c in ucu[cnt == 2]:
            w = np.sort(np.nonzero(cu == c)[0])
            first.append(ts[w[0], 2])
            second.append(ts[w[1], 2])
        if first:
            lines.append(f"  two per compute unit: scores end p50 {np.median(first):.2f} (first "
                         f"dispatched) / {np.median(second):.2f} (second)")
    extra = s[used][:, nb:SLOTS - 1]
    for j in range(extra.shape[1]):
        if (extra[:, j] > 0).all():
            e = (extra[:, j] - s[used][:, 0].min()) / 100.0
            lines.append(f"  slot {nb + j}: p50 {np.median(e):7.2f} max {e.max():7.2f}")
        elif (extra[:, j] > 0).any():
            lines.append(f"  slot {nb + j}: written by {(extra[:, j] > 0).sum()} workgroups")
    text = "\n".join(lines)
    print(text)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()
