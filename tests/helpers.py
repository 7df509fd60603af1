"""Shared helpers of the GPU parity tests: upload seeded inputs, run the HIP
path through the binding, and compare with the CPU oracle by the parity rules.

Parity rules
  * selected index sets: with s the oracle's fp64 low-dim scores of a
    (batch, head) and s_(k) its k-th largest value, tau = 1e-3 * max(|s_(k)|,
    1e-3 * max|s|); the GPU set G (k distinct in-range tokens) is accepted iff
    min_{t in G} s_t >= max_{u not in G} s_u - tau.  So G equals the oracle's
    set whenever the k-th and (k+1)-th scores differ by more than tau, and
    near-ties may swap only inside that band.
  * outputs: the oracle recomputes the attention on the GPU's own index sets;
    per (batch, head) the normwise relative error max|g - r| / max|r| must be
    below 1e-5 for fp32 storage and 2e-3 for fp16 / bf16 storage.  The
    elementwise error with a floor, max |g - r| / max(|r|, 1e-3 max|r|), is
    reported beside it.
"""
import numpy as np
import torch

import workloads as W
from oracle import loki_oracle as oracle

OUT_TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _loki():
    import sparse_decode_attention_rotate_amd as loki
    return loki


def log(msg):
    print(msg, flush=True)


def to_device(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


def make_desc(wl: W.Workload, dp: int = 32, scale: float = 0.0):
    loki = _loki()
    return loki.Desc(batch=wl.B, n_q_heads=wl.Hq, n_kv_heads=wl.Hkv, head_dim=wl.D,
                     seq_len=wl.S, seq_capacity=wl.capacity, panel_dim=dp,
                     dtype=loki.NAME_CODE[wl.dtype], softmax_scale=scale)


def upload(wl: W.Workload, x: dict, dp: int = 32):
    """Device copies: q, packed K cache, V cache, P (and k_new / v_new)."""
    loki = _loki()
    desc = make_desc(wl, dp)
    dev = {"desc": desc, "q": to_device(x["q"], wl.dtype), "P": torch.from_numpy(np.ascontiguousarray(x["P"])).cuda(),
           "v": to_device(x["v"], wl.dtype)}
    krot_rows = to_device(x["krot"], wl.dtype)
    dev["kcache"] = loki.empty_kcache(desc)
    loki.pack_kcache(krot_rows, dev["kcache"], desc.with_seq_len(wl.capacity))
    del krot_rows
    if wl.append:
        dev["k_new"] = to_device(x["k_new"], wl.dtype)
        dev["v_new"] = to_device(x["v_new"], wl.dtype)
    return dev


def run_decode(wl: W.Workload, dev: dict, d: int = None, k: int = None, separate=False):
    """One decode step; separate=True forces the per-phase launches."""
    d = wl.d if d is None else d
    k = wl.k if k is None else k
    loki = _loki()
    desc = dev["desc"]
    if separate:
        desc = desc.with_flags(loki.FLAG_SEPARATE_KERNELS)
    idx = torch.full((wl.B, wl.Hq, k), -7, dtype=torch.int32, device="cuda")
    if wl.append:
        out = loki.decode_append(dev["q"], dev["k_new"], dev["v_new"], dev["kcache"], dev["v"],
                                 dev["P"], d, k, desc, idx_out=idx)
    else:
        out = loki.decode(dev["q"], dev["kcache"], dev["v"], dev["P"], d, k, desc, idx_out=idx)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), idx.cpu().numpy()


def oracle_inputs_after_append(wl: W.Workload, x: dict):
    """The oracle's own cache after the append (its own rotation and rounding)."""
    if not wl.append:
        return x["krot"], x["v"]
    kr, vr = oracle.append_rows(x["k_new"], x["v_new"], x["P"], wl.dtype)
    krot = x["krot"].copy()
    v = x["v"].copy()
    krot[:, :, wl.S - 1] = kr
    v[:, :, wl.S - 1] = vr
    return krot, v


def check_index_sets(gpu_idx: np.ndarray, scores: np.ndarray, k: int, heads=None):
    """Margin rule; returns (number of rows checked, rows differing from the
    oracle set, total swapped tokens).  Raises AssertionError on a violation."""
    B, Hq, S = scores.shape
    units = range(B * Hq) if heads is None else heads
    n_diff = n_swaps = 0
    for u in units:
        b, h = divmod(int(u), Hq)
        g = gpu_idx[b, h]
        s = scores[b, h]
        assert g.shape == (k,)
        assert np.all((g >= 0) & (g < S)), f"({b},{h}) index out of range"
        assert len(np.unique(g)) == k, f"({b},{h}) repeated index"
        assert np.all(np.diff(g) > 0), f"({b},{h}) indices not ascending"
        if k == S:
            continue
        srt = np.sort(s)[::-1]
        tau = 1e-3 * max(abs(srt[k - 1]), 1e-3 * np.abs(s).max())
        mask = np.zeros(S, bool)
        mask[g] = True
        lo_in = s[mask].min()
        hi_out = s[~mask].max()
        assert lo_in >= hi_out - tau, (
            f"({b},{h}) selection outside the tie band: min in {lo_in!r} < max out {hi_out!r} - {tau!r}")
        ref = oracle.topk_rows(s[None], k)[0]
        sw = k - len(np.intersect1d(ref, g))
        n_diff += sw > 0
        n_swaps += sw
    return len(units), n_diff, n_swaps


def rel_err_rows(g: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Per (b, h) normwise relative error max|g-r| / max|r|."""
    num = np.abs(g - r).max(axis=-1)
    den = np.abs(r).max(axis=-1)
    return num / np.maximum(den, 1e-30)


def rel_err_elementwise(g: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Per (b, h) elementwise relative error with a floor: max over the row of
    |g-r| / max(|r|, 1e-3 * max|r|) (reported beside the normwise error)."""
    top = np.maximum(np.abs(r).max(axis=-1, keepdims=True), 1e-30)
    return (np.abs(g - r) / np.maximum(np.abs(r), 1e-3 * top)).max(axis=-1)


def full_parity(wl: W.Workload, x: dict, out_gpu, idx_gpu, d=None, k=None, heads=None):
    """End-to-end check; returns a dict of the achieved numbers."""
    d = wl.d if d is None else d
    k = wl.k if k is None else k
    krot, v = oracle_inputs_after_append(wl, x)
    # the step reads the S cached tokens; rows past S are spare capacity
    krot, v = krot[:, :, :wl.S], v[:, :, :wl.S]
    r = oracle.decode(x["q"], krot, v, x["P"], d, k, wl.dtype, heads=heads)
    n, n_diff, n_swaps = check_index_sets(idx_gpu, r["scores"], k, heads)
    ref = oracle.attend_given(x["q"], krot, v, x["P"], idx_gpu, wl.dtype, heads=heads)
    if heads is None:
        err = rel_err_rows(out_gpu, ref)
        elem = rel_err_elementwise(out_gpu, ref)
    else:
        rows = [divmod(int(u), wl.Hq) for u in heads]
        err = np.array([rel_err_rows(out_gpu[bh], ref[bh]) for bh in rows])
        elem = np.array([rel_err_elementwise(out_gpu[bh], ref[bh]) for bh in rows])
    if heads is None:
        assert np.all(np.isfinite(out_gpu))
    assert err.max() < OUT_TOL[wl.dtype], f"max rel err {err.max():.3e}"
    return {"rows": n, "rows_with_band_swaps": int(n_diff), "swapped_tokens": int(n_swaps),
            "max_rel_err": float(err.max()), "max_rel_err_elementwise_floor": float(elem.max())}
