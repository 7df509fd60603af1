"""Benchmark of one Loki decode step on one MI355X.

Workload (default): the Llama2-13B decode shape -- batch 16, 40 heads, head
dim 128, 4096 cached tokens, d = 32 leading principal components for scoring,
k = 512 tokens kept, fp16 storage -- on seeded synthetic inputs.

A step is the whole hot path: query rotation, low-dim scores of every cached
token, per-(batch, head) top-k, exact attention over the selected tokens.
Inputs are resident in HBM before timing starts; three independent copies of
the caches are cycled so that a step never finds its data in the 256 MB
Infinity Cache from an earlier step.  Before the W warm-up steps the step runs
untimed for about 0.2 s (--settle) so that the clocks are at steady state.
The timed step is the method's call loki_decode(q, Kcache_rot, V, P, d, k,
out): the optional index output is not requested.

Prints ONE JSON line.  value = algorithmic bytes per step / step time, where
the algorithmic bytes are, per step, B*Hkv*S*d elements for scoring plus
B*Hq*2*k*D elements for the selected keys and values.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
# the shape each workload stands for, in the metric's label
SHAPE_LABEL = {"llama2_13b_f16": "Llama2-13B shape", "llama2_7b_f16": "Llama2-7B shape",
               "single_head_f32": "single head, S=1024, fp32",
               "long_context_bf16": "long context S=32768 with append, bf16",
               "gqa_llama3_8b_bf16": "GQA Llama-3-8B shape, bf16"}


def metric_label(name):
    return ("Loki decode-attn µs/step & achieved HBM GB/s (% peak), "
            + SHAPE_LABEL.get(name, name))
KERNEL_SOURCES = {"score": "score.hip", "attend": "attend.hip", "topk": "topk.hip",
                  "rotate_query": "project.hip", "fused": "fused.hip", "head": "head.hip"}
KERNEL_NAMES = {"score": "score_panel_kernel", "attend": "attend_kernel", "topk": "topk_kernel",
                "rotate_query": "project_kernel", "fused": "fused_kernel", "head": "head_kernel"}
# one-launch plans of loki_decode_plan: the kernel that runs the step
PLAN_KERNEL = {1: "fused", 2: "head"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama2_13b_f16")
    ap.add_argument("--sets", type=int, default=0,
                    help="independent cache copies cycled (default: max(3, 1 + "
                         "ceil(512 MB / bytes one step reads)), so that every copy has "
                         "left the 256 MB Infinity Cache before it is read again; 3 for "
                         "steps that read less than 32 MB)")
    ap.add_argument("--settle", type=float, default=0.2,
                    help="seconds of untimed steps before the warm-up (steady clocks)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="budget of the CPU-oracle baseline sample")
    ap.add_argument("--no-workloads", action="store_true",
                    help="time only --workload (by default every workload is timed too and "
                         "reported under \"workloads\")")
    ap.add_argument("--parity-units", type=int, default=64,
                    help="(batch, head) units of each other workload checked against the oracle")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="after the run, 5 plain device-to-device copies of MB megabytes "
                         "(reference for the HBM byte counters of a profiler run)")
    return ap.parse_args()


def src_sha(name):
    p = os.path.join(ROOT, "sparse_decode_attention_rotate_amd", "csrc", name)
    h = hashlib.sha256(open(p, "rb").read())
    for hdr in ["loki_common.h", "loki_internal.h", "select_core.h", "attend_core.h"]:
        h.update(open(os.path.join(ROOT, "sparse_decode_attention_rotate_amd", "csrc", hdr),
                      "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """The counter record of `kernel` (HBM bytes per launch, read and written)
    from the committed rocprofv3 summary (profiles/hbm_traffic_<workload>.txt,
    lines "traffic {json}"), if the counters were taken on the current source
    of that kernel; else None."""
    p = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(p):
        return None
    for line in open(p):
        if line.startswith("traffic "):
            t = json.loads(line[len("traffic "):])
            if t.get("kernel") == kernel and t.get("src_sha") == src_sha(KERNEL_SOURCES[kernel]):
                return t
    return None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the Loki step here runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); sharding over several GPUs is described, not built.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_decode_attention_rotate_amd as loki
    import workloads as W

    wl = W.get(args.workload)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    t0 = time.time()
    x = W.generate(wl)
    print(f"[bench] generated {wl.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[wl.dtype]

    def up(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    desc = loki.Desc(batch=wl.B, n_q_heads=wl.Hq, n_kv_heads=wl.Hkv, head_dim=wl.D,
                     seq_len=wl.S, seq_capacity=wl.capacity, panel_dim=wl.d,
                     dtype=loki.NAME_CODE[wl.dtype])
    kc0 = loki.empty_kcache(desc)
    loki.pack_kcache(up(x["krot"]), kc0, desc.with_seq_len(wl.capacity))
    v0 = up(x["v"])
    if args.sets <= 0:
        # steps that read little are launch-bound: three copies are enough
        step_bytes = wl.algorithmic_bytes()
        args.sets = max(3, 1 + -(-(512 << 20) // step_bytes)) if step_bytes >= (32 << 20) else 3
    sets = [(kc0, v0)] + [(kc0.clone(), v0.clone()) for _ in range(args.sets - 1)]
    q = up(x["q"])
    P = torch.from_numpy(np.ascontiguousarray(x["P"])).to(dev)
    out = torch.empty((wl.B, wl.Hq, wl.D), dtype=torch.float32, device=dev)
    idx = torch.empty((wl.B, wl.Hq, wl.k), dtype=torch.int32, device=dev)
    ws = loki.empty_workspace(desc, wl.d, wl.k)
    k_new = up(x["k_new"]) if wl.append else None
    v_new = up(x["v_new"]) if wl.append else None
    stream = torch.cuda.current_stream()
    plan_code = loki.decode_kernel(desc, wl.d, wl.k, wl.append)
    one_launch = plan_code != 0
    vp = ctypes.c_void_p

    def make_calls(d_, st_=stream):
        cd = d_.c()
        calls = []
        for kc, vc in sets:
            if wl.append:
                calls.append((loki.lib.loki_decode_append,
                              (vp(q.data_ptr()), vp(k_new.data_ptr()), vp(v_new.data_ptr()),
                               vp(kc.data_ptr()), vp(vc.data_ptr()), vp(P.data_ptr()), wl.d,
                               wl.k, vp(out.data_ptr()), None, None, ctypes.byref(cd),
                               vp(ws.data_ptr()), ws.numel(), vp(st_.cuda_stream))))
            else:
                # the step of the method: loki_decode(q, Kcache_rot, V, P, d, k, out);
                # the optional index and score outputs are not requested
                calls.append((loki.lib.loki_decode,
                              (vp(q.data_ptr()), vp(kc.data_ptr()), vp(vc.data_ptr()),
                               vp(P.data_ptr()), wl.d, wl.k, vp(out.data_ptr()),
                               None, None, ctypes.byref(cd), vp(ws.data_ptr()),
                               ws.numel(), vp(st_.cuda_stream))))
        return cd, calls

    # pre-marshalled C-ABI arguments, one tuple per cache copy
    cdesc, calls = make_calls(desc)
    cdesc_sep, calls_sep = make_calls(desc.with_flags(loki.FLAG_SEPARATE_KERNELS))

    def step(i, which=calls):
        fn, a = which[i % len(which)]
        rc = fn(*a)
        if rc != 0:
            raise RuntimeError(f"decode failed: {loki.strerror(rc)} {loki.last_error()}")

    # the device first runs the step for about args.settle seconds so that its
    # clocks reach their steady state (a decode server runs continuously; a
    # 20-step warm-up alone leaves the timed steps a few percent slower), then
    # the W warm-up steps
    t_settle = time.time()
    i = 0
    while time.time() - t_settle < args.settle:
        for _ in range(50):
            step(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: K whole steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # spread: five more regions of K steps timed the same way (the value
    # above is the first region's)
    spread_us = []
    for _ in range(5):
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(args.steps):
            step(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        spread_us.append(ev0.elapsed_time(ev1) / args.steps * 1e3)
    spread_us.sort()
    spread = {"regions": len(spread_us), "median_us": round(spread_us[len(spread_us) // 2], 2),
              "p10_us": round(spread_us[0], 2), "p90_us": round(spread_us[-1], 2)}

    # the step replayed from a HIP graph: 8 captured steps per cache copy, in
    # the eager order (so that one graph launch's own cost is spread thin)
    graph = None
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        per_graph = 8 * len(sets)
        with torch.cuda.graph(g):
            _, calls_cap = make_calls(desc, torch.cuda.current_stream())
            for i in range(per_graph):
                step(i, calls_cap)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // per_graph)
        ev0.record(stream)
        for _ in range(reps):
            g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        graph = {"us_per_step": round(ev0.elapsed_time(ev1) / (reps * per_graph) * 1e3, 2),
                 "steps": reps * per_graph, "steps_per_graph": per_graph}
        del g
    except Exception as e:  # reported, not fatal: the eager timing stands
        graph = {"error": str(e)[:200]}

    # the step once more on the first cache copy, with its index sets, for the
    # oracle's check of sampled units (before any later measurement rewrites
    # a cache row)
    gpu = None
    if not args.no_cpu_baseline:
        idx_c = torch.empty((wl.B, wl.Hq, wl.k), dtype=torch.int32, device=dev)
        fn, a = calls[0]
        a = list(a)
        a[9 if wl.append else 7] = vp(idx_c.data_ptr())
        if fn(*a) != 0:
            raise RuntimeError(f"decode failed: {loki.last_error()}")
        torch.cuda.synchronize()
        gpu = {"out": out.cpu().numpy().astype("float64"), "idx": idx_c.cpu().numpy()}

    # ---- separate launches: whole step, then each kernel alone, K back-to-back
    # launches between two events on the launch stream (as a kernel trace sees them)
    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(args.steps):
            fn(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / args.steps * 1e3

    sep_step_us = timed(lambda i: step(i, calls_sep))
    lib = loki.lib
    qr = torch.empty((wl.B, wl.Hq, wl.D), dtype=torch.float32, device=dev)
    scores = torch.empty((wl.B, wl.Hq, wl.S), dtype=torch.float32, device=dev)
    sel = torch.empty((wl.B, wl.Hq, wl.k), dtype=torch.float32, device=dev)
    cd = ctypes.byref(cdesc)
    st = vp(stream.cuda_stream)
    P_, q_, qr_, sc_, idx_, sel_, out_, ws_ = (vp(t.data_ptr()) for t in
                                               (P, q, qr, scores, idx, sel, out, ws))
    kcs = [vp(kc.data_ptr()) for kc, _ in sets]
    vcs = [vp(vc.data_ptr()) for _, vc in sets]
    split = True  # panel_dim = d: the step uses the split attention variant

    def chk(rc):
        if rc != 0:
            raise RuntimeError(f"{loki.strerror(rc)} {loki.last_error()}")

    lib.loki_decode(q_, kcs[0], vcs[0], P_, wl.d, wl.k, out_, idx_, None,
                    ctypes.byref(cdesc_sep), ws_, ws.numel(), st)
    chk(lib.loki_rotate_query(q_, P_, qr_, cd, st))
    chk(lib.loki_score(qr_, kcs[0], wl.d, sc_, cd, st))
    chk(lib.loki_topk(sc_, wl.k, idx_, sel_, cd, st))
    per_kernel = {
        "rotate_query": timed(lambda i: lib.loki_rotate_query(q_, P_, qr_, cd, st)),
        "score": timed(lambda i: lib.loki_score(qr_, kcs[i % len(kcs)], wl.d, sc_, cd, st)),
        "topk": timed(lambda i: lib.loki_topk(sc_, wl.k, idx_, sel_, cd, st)),
        "attend": timed(lambda i: lib.loki_attend(qr_, kcs[i % len(kcs)], vcs[i % len(vcs)], idx_,
                                                  sel_ if split else None, wl.k, out_, cd, ws_,
                                                  ws.numel(), st)),
    }
    per_kernel = {n: round(u, 2) for n, u in per_kernel.items()}

    # dense decode attention over all S tokens on the same caches: the baseline
    # the pages measure Loki's attention speed-up against
    ws_full = loki.empty_workspace(desc, wl.D, wl.S)
    wsf_ = vp(ws_full.data_ptr())
    chk(lib.loki_full_attention(q_, kcs[0], vcs[0], P_, out_, cd, wsf_, ws_full.numel(), st))
    full_us = timed(lambda i: lib.loki_full_attention(q_, kcs[i % len(kcs)], vcs[i % len(vcs)], P_,
                                                      out_, cd, wsf_, ws_full.numel(), st))
    es_ = 4 if wl.dtype == "f32" else 2
    full_bytes = es_ * wl.B * wl.Hkv * wl.S * wl.D * 2
    # PCAAttn, the pages' variant attending with the d-dim scores over all S
    chk(lib.loki_pca_attention(q_, kcs[0], vcs[0], P_, wl.d, out_, cd, wsf_, ws_full.numel(), st))
    pca_us = timed(lambda i: lib.loki_pca_attention(q_, kcs[i % len(kcs)], vcs[i % len(vcs)], P_,
                                                    wl.d, out_, cd, wsf_, ws_full.numel(), st))
    pca_bytes = es_ * wl.B * wl.Hkv * wl.S * (wl.d + wl.D)
    pca = {"us_per_step": round(pca_us, 2), "kv_bytes_per_step": pca_bytes,
           "GBps": round(pca_bytes / (pca_us * 1e-6) / 1e9, 1),
           "loki_speedup": round(pca_us / (ms_per_step * 1e3), 3)}
    del ws_full

    # Exact-TopK, the pages' other baseline: scores over all D coordinates
    # (panel = the whole rotated key row), top-k, attention over the k rows
    exact = None
    if not wl.append:
        desc_x = loki.Desc(batch=wl.B, n_q_heads=wl.Hq, n_kv_heads=wl.Hkv, head_dim=wl.D,
                           seq_len=wl.S, seq_capacity=wl.capacity, panel_dim=wl.D,
                           dtype=loki.NAME_CODE[wl.dtype])
        kc_x = loki.empty_kcache(desc_x)
        loki.pack_kcache(up(x["krot"]), kc_x, desc_x.with_seq_len(wl.capacity))
        ws_x = loki.empty_workspace(desc_x, wl.D, wl.k)
        cdx = desc_x.c()
        kcx_, wsx_ = vp(kc_x.data_ptr()), vp(ws_x.data_ptr())
        chk(lib.loki_decode(q_, kcx_, vcs[0], P_, wl.D, wl.k, out_, None, None, ctypes.byref(cdx),
                            wsx_, ws_x.numel(), st))
        exact_us = timed(lambda i: lib.loki_decode(q_, kcx_, vcs[i % len(vcs)], P_, wl.D, wl.k, out_,
                                                   None, None, ctypes.byref(cdx), wsx_, ws_x.numel(),
                                                   st))
        exact_bytes = es_ * (wl.B * wl.Hkv * wl.S * wl.D + wl.B * wl.Hq * wl.k * wl.D)
        exact = {"us_per_step": round(exact_us, 2), "bytes_per_step": exact_bytes,
                 "GBps": round(exact_bytes / (exact_us * 1e-6) / 1e9, 1),
                 "loki_speedup": round(exact_us / (ms_per_step * 1e3), 3)}
        del kc_x, ws_x

    # prefill: the prompt's S keys of every (b, kv) projected by P into a cache
    # copy (the kernel alone; V rows are a plain copy).  Input: stored rows of
    # the same shape and distribution.
    k_rows = up(x["krot"][:, :, :wl.S])
    kc_p = loki.empty_kcache(desc)
    kr_, kcp_ = vp(k_rows.data_ptr()), vp(kc_p.data_ptr())
    chk(lib.loki_prefill(kr_, None, wl.S, 0, P_, kcp_, None, cd, st))
    prefill_us = timed(lambda i: lib.loki_prefill(kr_, None, wl.S, 0, P_, kcp_, None, cd, st))
    prefill_bytes = es_ * wl.B * wl.Hkv * wl.S * wl.D * 2
    # the same bytes moved by a plain device copy: the read+write ceiling
    cp_dst = torch.empty_like(k_rows)
    copy_us = timed(lambda i: cp_dst.copy_(k_rows))
    prefill = {"us_per_call": round(prefill_us, 2), "tokens": wl.S, "bytes_per_call": prefill_bytes,
               "GBps": round(prefill_bytes / (prefill_us * 1e-6) / 1e9, 1),
               "frac_hbm_peak": round(prefill_bytes / (prefill_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
               "copy_same_bytes_us": round(copy_us, 2),
               "frac_of_copy_rate": round(copy_us / prefill_us, 4)}
    # calibration: PCA of n_calib seeded synthetic keys per KV head (the
    # generator's spectrum) on the GPU, the offline step that yields P
    gcal = torch.Generator(device=dev)
    gcal.manual_seed(7)
    sig = torch.from_numpy(W.sigma(wl)).to(dev, torch.float32)
    keys_cal = (torch.randn((wl.Hkv, wl.n_calib, wl.D), generator=gcal, device=dev) * sig).to(tdt)
    if tuple(keys_cal.shape) != (wl.Hkv, wl.n_calib, wl.D) or not keys_cal.is_contiguous():
        raise RuntimeError("calibration keys must be [Hkv, n_calib, D] contiguous")
    P_cal = torch.empty_like(P)
    var_cal = torch.empty((wl.Hkv, wl.D), dtype=torch.float32, device=dev)
    nb = ctypes.c_size_t()
    chk(lib.loki_calibrate_workspace_bytes(cd, wl.n_calib, ctypes.byref(nb)))
    ws_cal = torch.empty(nb.value, dtype=torch.uint8, device=dev)
    cal_args = (vp(keys_cal.data_ptr()), wl.n_calib, vp(P_cal.data_ptr()), vp(var_cal.data_ptr()),
                cd, vp(ws_cal.data_ptr()), ws_cal.numel(), st)
    chk(lib.loki_calibrate(*cal_args))
    saved_steps, args.steps = args.steps, min(args.steps, 20)
    cal_us = timed(lambda i: lib.loki_calibrate(*cal_args))
    args.steps = saved_steps
    calibration = {"us_per_call": round(cal_us, 1), "keys_per_head": wl.n_calib,
                   "kv_heads": wl.Hkv,
                   "covariance_GFLOP": round(2.0 * wl.Hkv * wl.n_calib * wl.D * wl.D / 1e9, 3)}
    del k_rows, kc_p, cp_dst, keys_cal, ws_cal

    # the appending step on the same shape: one new token per (b, kv) written
    # at row S-1 of each cache copy, then the decode over the S tokens.  The new
    # key and value are seeded draws with the keys' per-coordinate spread; the
    # timing does not depend on their values beyond the selection.  Last, since
    # it rewrites row S-1 of the cycled copies.
    append_step = None
    if not wl.append:
        gnew = torch.Generator(device=dev)
        gnew.manual_seed(11)
        kn_t = (torch.randn((wl.B, wl.Hkv, wl.D), generator=gnew, device=dev) * sig).to(tdt)
        vn_t = torch.randn((wl.B, wl.Hkv, wl.D), generator=gnew, device=dev).to(tdt)
        kn_, vn_ = vp(kn_t.data_ptr()), vp(vn_t.data_ptr())

        def append_call(i, cd_):
            chk(lib.loki_decode_append(q_, kn_, vn_, kcs[i % len(kcs)], vcs[i % len(vcs)], P_,
                                       wl.d, wl.k, out_, None, None, cd_, ws_, ws.numel(), st))

        # the decode step timed again just before, under the same conditions
        dec_us = timed(lambda i: step(i))
        app_us = timed(lambda i: append_call(i, cd))
        app_sep_us = timed(lambda i: append_call(i, ctypes.byref(cdesc_sep)))
        append_step = {"us_per_step": round(app_us, 2),
                       "launch_plan": ("one kernel" if loki.decode_plan(desc, wl.d, wl.k, True)
                                       else "separate kernels"),
                       "decode_us_alongside": round(dec_us, 2),
                       "over_decode_us": round(app_us - dec_us, 2),
                       "separate_launches_us": round(app_sep_us, 2)}
        del kn_t, vn_t

    es = 4 if wl.dtype == "f32" else 2
    alg_bytes = wl.algorithmic_bytes()
    score_bytes = es * wl.B * wl.Hkv * wl.S * wl.d
    attend_bytes = es * wl.B * wl.Hq * 2 * wl.k * wl.D
    if one_launch:
        # the step is one kernel: K back-to-back launches timed above
        dom, dom_us, dom_bytes = PLAN_KERNEL[plan_code], ms_per_step * 1e3, alg_bytes
        kernels = {dom: round(dom_us, 2)}
    else:
        per_kernel_bytes = {"score": score_bytes, "attend": attend_bytes}
        dom = max(["score", "attend"], key=lambda n: per_kernel[n])
        dom_us, dom_bytes = per_kernel[dom], per_kernel_bytes[dom]
        kernels = per_kernel
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    trec = measured_traffic(wl.name, dom)
    traffic = trec.get("hbm_bytes_per_launch") if trec else None

    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": metric_label(wl.name),
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {**W.describe(wl), "algorithmic_bytes_per_step": alg_bytes,
                   "cache_copies_cycled": args.sets},
        "launch_plan": {0: "separate kernels", 1: "one kernel (one workgroup per (b, kv))",
                        2: "one kernel (one workgroup per query head)"}[plan_code],
        "spread": spread,
        "graph": graph,
        "kernel_us": kernels,
        "separate_launches": {"us_per_step": round(sep_step_us, 2), "kernel_us": per_kernel},
        "full_attention": {"us_per_step": round(full_us, 2), "kv_bytes_per_step": full_bytes,
                           "GBps": round(full_bytes / (full_us * 1e-6) / 1e9, 1),
                           "loki_speedup": round(full_us / (ms_per_step * 1e3), 3)},
        "exact_topk": exact,
        "pca_attention": pca,
        "prefill": prefill,
        "calibration": calibration,
        "append_step": append_step,
        "roofline": {"bound": "hbm", "kernel": KERNEL_NAMES[dom], "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "traffic_read": (round(trec["fetch_kib_per_launch"] * 1024 * trec["fetch_scale"])
                                      if trec else None),
                     "traffic_write": (round(trec["write_kib_per_launch"] * 1024 * trec["write_scale"])
                                       if trec else None),
                     "algorithmic_bytes_per_launch": dom_bytes,
                     "avg_launch_us": round(dom_us, 2)},
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_seconds, gpu)

    if not args.no_workloads:
        # every workload's step, timed the same way (the default one from the
        # figures above); the others after it, one at a time
        del x
        par = result.get("cpu_baseline", {}).get("parity")
        idx_h = gpu["idx"] if gpu is not None else None
        entries = {}
        for name in W.WORKLOADS:
            if name == wl.name:
                if idx_h is None:
                    continue
                entries[name] = time_workload(
                    name, args, headline=(ms_per_step * 1e3, spread, full_us, par, idx_h))
            else:
                entries[name] = time_workload(name, args)
        result["workloads"] = entries

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = n

    print(json.dumps(result), flush=True)


def unit_sample(n_units, n_max):
    """Up to n_max (batch, head) units spread evenly over the step."""
    import numpy as np
    if n_units <= n_max:
        return list(range(n_units))
    return sorted(set(np.linspace(0, n_units - 1, n_max).round().astype(int).tolist()))


def parity_check(wl, x, out, idx, heads):
    """The sampled units of a GPU step against the oracle: index sets within
    the tie band of the oracle's fp64 scores, outputs against the oracle's
    attention over the GPU's own sets (normwise per row, and elementwise with
    a floor of 1e-3 of the row's largest magnitude)."""
    import numpy as np
    from oracle import loki_oracle as oracle

    krot, v = x["krot"][:, :, :wl.S], x["v"][:, :, :wl.S]
    if wl.append:  # the cache after the step's own append (the oracle's rotation)
        kr, vr = oracle.append_rows(x["k_new"], x["v_new"], x["P"], wl.dtype)
        krot, v = krot.copy(), v.copy()
        krot[:, :, wl.S - 1] = kr
        v[:, :, wl.S - 1] = vr
    r = oracle.decode(x["q"], krot, v, x["P"], wl.d, wl.k, wl.dtype, heads=heads)
    Hq = wl.Hq
    swaps = band_ok = 0
    for u in heads:
        b, h = divmod(u, Hq)
        gi = idx[b, h]
        sc = r["scores"][b, h]
        ok = (len(np.unique(gi)) == wl.k and gi.min() >= 0 and gi.max() < wl.S and
              bool(np.all(np.diff(gi) > 0)))
        if ok and wl.k < wl.S:
            srt = np.sort(sc)[::-1]
            tau = 1e-3 * max(abs(srt[wl.k - 1]), 1e-3 * np.abs(sc).max())
            mask = np.zeros(wl.S, bool)
            mask[gi] = True
            ok = sc[mask].min() >= sc[~mask].max() - tau
            swaps += wl.k - len(np.intersect1d(gi, r["idx"][b, h]))
        band_ok += int(ok)
    ref = oracle.attend_given(x["q"], krot, v, x["P"], idx, wl.dtype, heads=heads)
    errs, elem = [], []
    for u in heads:
        b, h = divmod(u, Hq)
        g_, r_ = out[b, h], ref[b, h]
        top = max(np.abs(r_).max(), 1e-30)
        errs.append(np.abs(g_ - r_).max() / top)
        elem.append((np.abs(g_ - r_) / np.maximum(np.abs(r_), 1e-3 * top)).max())
    tol = OUT_TOL[wl.dtype]
    return {"units": len(heads), "index_sets_within_tie_band": band_ok,
            "swapped_tokens_within_band": int(swaps),
            "max_rel_out": float(f"{max(errs):.3e}"),
            "max_rel_out_elementwise_floor": float(f"{max(elem):.3e}"),
            "tolerance": tol, "ok": bool(band_ok == len(heads) and max(errs) < tol)}


def gather_rows(wl, idx):
    """Rows the attention of one step gathers: per (b, kv) the distinct
    tokens selected by its query heads (the union), and the nominal count
    (k per query head)."""
    import numpy as np
    g = wl.Hq // wl.Hkv
    union = 0
    for b in range(wl.B):
        for kv in range(wl.Hkv):
            union += np.unique(idx[b, kv * g:(kv + 1) * g]).size
    return union, wl.B * wl.Hq * wl.k


def time_workload(name, args, headline=None):
    """One workload's decode step timed as the headline is (cycled cache
    copies, settle, warm-up, K steps between events on the launch stream,
    two more regions for the spread), the dense attention over all S tokens on
    the same caches, and the step checked against the oracle on sampled units.
    With `headline` (the already measured figures of the default workload)
    only the entry is assembled."""
    import numpy as np
    import torch

    import sparse_decode_attention_rotate_amd as loki
    import workloads as W

    wl = W.get(name)
    es = 4 if wl.dtype == "f32" else 2
    score_bytes = es * wl.B * wl.Hkv * wl.S * wl.d
    desc = loki.Desc(batch=wl.B, n_q_heads=wl.Hq, n_kv_heads=wl.Hkv, head_dim=wl.D,
                     seq_len=wl.S, seq_capacity=wl.capacity, panel_dim=wl.d,
                     dtype=loki.NAME_CODE[wl.dtype])
    code = loki.decode_kernel(desc, wl.d, wl.k, wl.append)
    plan = {0: "separate kernels", 1: "one kernel (one workgroup per (b, kv))",
            2: "one kernel (one workgroup per query head)"}[code]
    if headline is not None:
        us, spread, dense_us, par, idx_h = headline
        sets_n = args.sets
    else:
        dev = torch.device("cuda:0")
        t0 = time.time()
        x = W.generate(wl)

        def up(a):
            if wl.dtype == "bf16":
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                    torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        kc0 = loki.empty_kcache(desc)
        loki.pack_kcache(up(x["krot"]), kc0, desc.with_seq_len(wl.capacity))
        v0 = up(x["v"])
        step_bytes = wl.algorithmic_bytes()
        sets_n = max(3, 1 + -(-(512 << 20) // step_bytes)) if step_bytes >= (32 << 20) else 3
        sets = [(kc0, v0)] + [(kc0.clone(), v0.clone()) for _ in range(sets_n - 1)]
        q, P = up(x["q"]), torch.from_numpy(np.ascontiguousarray(x["P"])).to(dev)
        out = torch.empty((wl.B, wl.Hq, wl.D), dtype=torch.float32, device=dev)
        idx = torch.empty((wl.B, wl.Hq, wl.k), dtype=torch.int32, device=dev)
        ws = loki.empty_workspace(desc, wl.d, wl.k)
        k_new = up(x["k_new"]) if wl.append else None
        v_new = up(x["v_new"]) if wl.append else None
        stream = torch.cuda.current_stream()
        st = ctypes.c_void_p(stream.cuda_stream)
        vp = ctypes.c_void_p
        cd = desc.c()
        calls = []
        for kc, vc in sets:
            if wl.append:
                calls.append((loki.lib.loki_decode_append,
                              [vp(q.data_ptr()), vp(k_new.data_ptr()), vp(v_new.data_ptr()),
                               vp(kc.data_ptr()), vp(vc.data_ptr()), vp(P.data_ptr()), wl.d,
                               wl.k, vp(out.data_ptr()), None, None, ctypes.byref(cd),
                               vp(ws.data_ptr()), ws.numel(), st]))
            else:
                calls.append((loki.lib.loki_decode,
                              [vp(q.data_ptr()), vp(kc.data_ptr()), vp(vc.data_ptr()),
                               vp(P.data_ptr()), wl.d, wl.k, vp(out.data_ptr()), None, None,
                               ctypes.byref(cd), vp(ws.data_ptr()), ws.numel(), st]))

        def step(i):
            fn, a = calls[i % len(calls)]
            rc = fn(*a)
            if rc != 0:
                raise RuntimeError(f"{name}: {loki.strerror(rc)} {loki.last_error()}")

        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)

        def region(fn, n):
            torch.cuda.synchronize()
            ev0.record(stream)
            for i in range(n):
                fn(i)
            ev1.record(stream)
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / n * 1e3

        t_settle = time.time()
        i = 0
        while time.time() - t_settle < args.settle:
            for _ in range(50):
                step(i)
                i += 1
            torch.cuda.synchronize()
        for i in range(args.warmup):
            step(i)
        us = region(step, args.steps)
        more = sorted([us] + [region(step, args.steps) for _ in range(2)])
        spread = {"regions": 3, "median_us": round(more[1], 2), "min_us": round(more[0], 2),
                  "max_us": round(more[2], 2)}
        # dense attention over all S tokens on the same caches (the pages'
        # baseline of the Loki speed-up)
        ws_full = loki.empty_workspace(desc, wl.D, wl.S)
        wsf, nf = vp(ws_full.data_ptr()), ws_full.numel()

        def dense(i):
            kc, vc = sets[i % len(sets)]
            rc = loki.lib.loki_full_attention(vp(q.data_ptr()), vp(kc.data_ptr()),
                                              vp(vc.data_ptr()), vp(P.data_ptr()),
                                              vp(out.data_ptr()), ctypes.byref(cd), wsf, nf, st)
            if rc != 0:
                raise RuntimeError(f"{name} dense: {loki.last_error()}")

        for i in range(min(args.warmup, 5)):
            dense(i)
        dense_us = region(dense, max(10, args.steps // 4))
        del ws_full
        # the step once more on copy 0 with its index sets, for the oracle
        fn, a = calls[0]
        a = list(a)
        a[9 if wl.append else 7] = vp(idx.data_ptr())
        if fn(*a) != 0:
            raise RuntimeError(f"{name}: {loki.last_error()}")
        torch.cuda.synchronize()
        out_h = out.cpu().numpy().astype(np.float64)
        idx_h = idx.cpu().numpy()
        del sets, kc0, v0, q, P, out, idx, ws, k_new, v_new, calls
        torch.cuda.empty_cache()
        heads = unit_sample(wl.B * wl.Hq, args.parity_units)
        par = parity_check(wl, x, out_h, idx_h, heads)
        print(f"[bench] {name}: {us:.2f} us/step, parity {par['ok']} "
              f"({time.time() - t0:.1f}s)", file=sys.stderr, flush=True)
        del x
    nominal_bytes = wl.algorithmic_bytes()
    entry = {"metric": metric_label(name), "config": W.describe(wl),
             "launch_plan": plan, "us_per_step": round(us, 2), "spread": spread,
             "cache_copies_cycled": sets_n}
    union_rows, nominal_rows = gather_rows(wl, idx_h)
    if wl.Hq != wl.Hkv:
        # the gather counts each distinct selected row of a KV group once
        alg = score_bytes + es * union_rows * 2 * wl.D
        entry["alg_bytes_union"] = alg
        entry["alg_bytes_nominal"] = nominal_bytes
        entry["union_rows_over_nominal"] = round(union_rows / nominal_rows, 4)
    else:
        alg = nominal_bytes
        entry["alg_bytes"] = alg
    gbs = alg / (us * 1e-6) / 1e9
    # HBM bytes per launch of the step's one-launch kernel from the committed
    # counter record of this workload, while it matches the kernel's source
    kern = PLAN_KERNEL.get(code)
    trec = measured_traffic(wl.name, kern) if kern else None
    entry["traffic"] = trec.get("hbm_bytes_per_launch") if trec else None
    entry["traffic_over_alg"] = round(entry["traffic"] / alg, 4) if entry["traffic"] else None
    entry.update({"GBps": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                  "target_us_at_70pct": round(alg / (0.7 * PEAK_HBM_GBS * 1e9) * 1e6, 2),
                  "dense_attention_us": round(dense_us, 2),
                  "loki_speedup_vs_dense": round(dense_us / us, 3), "parity": par})
    return entry


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def set_omp_threads(n):
    """Thread count of the OpenMP runtime the C oracle runs on (libgomp)."""
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
        return True
    except OSError:
        return False


# normwise output tolerance per storage dtype (fp32 vs 16-bit inputs)
OUT_TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def cpu_baseline(wl, x, budget_s, gpu=None):
    """The fp64 CPU oracle on the host cores, on a bounded sample of the same
    step: whole (batch, head) units, as many as fit the time budget.  With
    `gpu` (the step's output and index sets) the sampled units are also checked
    against the oracle: index sets within the tie band of the oracle's
    scores, outputs against the oracle's attention over the GPU's sets."""
    import numpy as np
    from oracle import loki_oracle as oracle

    n_units = wl.B * wl.Hq
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    krot, v = x["krot"][:, :, :wl.S], x["v"][:, :, :wl.S]
    if wl.append:  # the cache after the step's own append (the oracle's rotation)
        kr, vr = oracle.append_rows(x["k_new"], x["v_new"], x["P"], wl.dtype)
        krot, v = krot.copy(), v.copy()
        krot[:, :, wl.S - 1] = kr
        v[:, :, wl.S - 1] = vr
    # calibrate on a few units, then size the sample to the budget
    probe = list(range(min(n_units, max(threads, 8))))
    t = time.time()
    oracle.decode(x["q"], krot, v, x["P"], wl.d, wl.k, wl.dtype, heads=probe)
    per_unit = (time.time() - t) / len(probe)
    n = int(min(n_units, max(len(probe), budget_s / max(per_unit, 1e-9) / 3)))
    heads = list(range(n))
    # repeat the sample so that each of the 3 timed runs takes about budget/3
    reps = max(1, int(budget_s / 3 / max(per_unit * n, 1e-9)))
    times = []
    for _ in range(3):
        t = time.time()
        for _ in range(reps):
            r = oracle.decode(x["q"], krot, v, x["P"], wl.d, wl.k, wl.dtype, heads=heads)
        times.append((time.time() - t) / reps)
    sec = float(np.median(times))
    es = 4 if wl.dtype == "f32" else 2
    g = wl.Hq // wl.Hkv
    # algorithmic bytes of a unit: S*d per query head's KV head share plus 2*k*D
    unit_bytes = es * (wl.S * wl.d / g + 2 * wl.k * wl.D)
    res = {"value": round(unit_bytes * n / sec / 1e9, 4), "unit": "GB/s", "cores": threads,
           "kind": "oracle", "cpu_model": cpu_model(),
           "sample": f"{n} of {n_units} (batch, head) units of one step, fp64 C oracle, "
                     f"median of 3 runs of {reps} repetitions ({sec:.3f} s per repetition), "
                     f"OpenMP over units",
           "seconds": round(sec, 3)}
    # one thread, on the first units of the sample (a few seconds)
    if set_omp_threads(1):
        n1 = max(1, min(n, int(max(1.0, budget_s / 10) / max(per_unit * threads, 1e-9))))
        t = time.time()
        oracle.decode(x["q"], krot, v, x["P"], wl.d, wl.k, wl.dtype, heads=list(range(n1)))
        s1 = time.time() - t
        set_omp_threads(threads)
        res["one_thread"] = {"value": round(unit_bytes * n1 / s1 / 1e9, 4), "unit": "GB/s",
                             "units": n1, "seconds": round(s1, 3)}
    if gpu is not None:
        # the sampled units of the GPU's step against the oracle
        res["parity"] = parity_check(wl, x, gpu["out"], gpu["idx"], heads)
    return res


if __name__ == "__main__":
    main()
