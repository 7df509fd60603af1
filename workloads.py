"""Seeded synthetic workloads for the Loki decode step.

This module only draws inputs.  It holds no step of the decode itself (query
rotation, scoring, selection, attention are in the HIP library and, separately,
in the CPU oracle); it prepares the inputs the way two earlier stages would:

  * the offline calibration: P is the PCA basis of a separate calibration draw
    of keys (poster page, "Visual Insights", Figure 1 right: PCA on keys
    collected offline from a calibration set);
  * an earlier prefill: the cache holds the already-rotated keys K . P, computed
    once in fp64 from the stored P and rounded once to the storage dtype.

Synthetic keys stand in for a model's keys: K = (Z * sigma) U^T with U a
random orthonormal basis per KV head and sigma_i = exp(-i / tau), so that the
keys are low-rank in the sense the pages report (a minority of principal
components hold most of the variance).  Values are N(0, 1).  The pages run
their measurements on model activations over public datasets; those are not
used here, these draws stand in for them.

Seeding: numpy SeedSequence(entropy, spawn_key=(workload id, role, head[, b])).
Storage arrays: f32 -> float32, f16 -> float16, bf16 -> uint16 (raw bits).
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
import os
from typing import Dict, Optional

import numpy as np

ROLE_U, ROLE_CALIB, ROLE_K, ROLE_V, ROLE_Q, ROLE_HEAVY, ROLE_NEW = range(7)

NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # seed-tree id
    B: int
    Hq: int
    Hkv: int
    D: int
    S: int              # valid tokens attended this step (including an appended one)
    d: int              # leading principal components used for scoring
    k: int              # tokens kept per query head
    dtype: str          # storage dtype of q, K, V
    tau: float          # sigma_i = exp(-i / tau)
    n_calib: int        # calibration keys per KV head
    heavy_frac: float = 0.0   # fraction of prefilled tokens with scaled key norm
    heavy_scale: float = 4.0
    append: bool = False      # last token arrives through the append path
    spectrum: str = "std"     # "std": sigma is the std; "variance": sigma is the variance
    S_cap: int = 0            # cache capacity (0 -> S)

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def capacity(self) -> int:
        return self.S_cap if self.S_cap else self.S

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def algorithmic_bytes(self) -> int:
        """Bytes one step must move: per KV head S*d for scoring, per query head 2*k*D."""
        es = 4 if self.dtype == "f32" else 2
        return es * (self.B * self.Hkv * self.S * self.d + self.B * self.Hq * 2 * self.k * self.D)


# The five workloads: a single-head fp32 case, Llama2-7B and Llama2-13B shaped
# decode, a long-context bf16 case with heavy hitters and a per-step append,
# and a grouped-query Llama-3-8B shaped decode.
WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("single_head_f32", 0, B=1, Hq=1, Hkv=1, D=128, S=1024, d=32, k=128,
                 dtype="f32", tau=20.0, n_calib=4096),
        Workload("llama2_7b_f16", 1, B=8, Hq=32, Hkv=32, D=128, S=4096, d=32, k=1024,
                 dtype="f16", tau=40.0, n_calib=8192),
        Workload("llama2_13b_f16", 2, B=16, Hq=40, Hkv=40, D=128, S=4096, d=32, k=512,
                 dtype="f16", tau=40.0, n_calib=8192),
        Workload("long_context_bf16", 3, B=4, Hq=32, Hkv=32, D=128, S=32768, d=32, k=4096,
                 dtype="bf16", tau=40.0, n_calib=8192, heavy_frac=0.02, append=True),
        Workload("gqa_llama3_8b_bf16", 4, B=16, Hq=32, Hkv=8, D=128, S=16384, d=32, k=2048,
                 dtype="bf16", tau=40.0, n_calib=8192),
    ]
}


def custom(name="custom", wid=100, **kw) -> Workload:
    base = dict(B=1, Hq=1, Hkv=1, D=128, S=256, d=32, k=32, dtype="f32", tau=20.0,
                n_calib=1024)
    base.update(kw)
    return Workload(name, wid, **base)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def rng(entropy: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=entropy, spawn_key=tuple(key)))


def sigma(wl: Workload) -> np.ndarray:
    s = np.exp(-np.arange(wl.D, dtype=np.float64) / wl.tau)
    return np.sqrt(s) if wl.spectrum == "variance" else s


def basis(wl: Workload, kv: int, entropy: int = 0) -> np.ndarray:
    """Random orthonormal D x D basis (columns), sign-fixed QR of a Gaussian."""
    G = rng(entropy, wl.wid, ROLE_U, kv).standard_normal((wl.D, wl.D))
    Q, R = np.linalg.qr(G)
    return Q * np.sign(np.diag(R))


def draw_keys(g: np.random.Generator, n: int, U: np.ndarray, sig: np.ndarray) -> np.ndarray:
    Z = g.standard_normal((n, U.shape[0]))
    return (Z * sig) @ U.T


def pca_basis(keys: np.ndarray):
    """PCA of calibration keys: eigenvectors of the centred (1/n) covariance,
    eigenvalues descending; each column's largest-magnitude entry made positive.
    Returns (P fp64 [D, D] with principal directions as columns, variances)."""
    mu = keys.mean(axis=0)
    X = keys - mu
    C = (X.T @ X) / keys.shape[0]
    w, V = np.linalg.eigh(C)
    order = np.argsort(-w, kind="stable")
    w, V = w[order], V[:, order]
    lead = np.argmax(np.abs(V), axis=0)
    V = V * np.sign(V[lead, np.arange(V.shape[1])])
    return V, w


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def from_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64 (exact)."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def calibration(wl: Workload, entropy: int = 0):
    """Per KV head: (U, P32) where P32 is the stored fp32 PCA basis."""
    sig = sigma(wl)
    out = []
    for kv in range(wl.Hkv):
        U = basis(wl, kv, entropy)
        cal = draw_keys(rng(entropy, wl.wid, ROLE_CALIB, kv), wl.n_calib, U, sig)
        P, _ = pca_basis(cal)
        out.append((U, np.ascontiguousarray(P, dtype=np.float32)))
    return out


def generate(wl: Workload, entropy: int = 0, with_raw_keys: bool = False) -> Dict[str, np.ndarray]:
    """Draw one full set of inputs for one decode step.

    Returns storage arrays q [B,Hq,D], krot [B,Hkv,S_cap,D] (rotated keys,
    logical row-major), v [B,Hkv,S_cap,D], P [Hkv,D,D] float32; for appending
    workloads also k_new, v_new [B,Hkv,D] (unrotated key, value) and pos = S-1,
    with cache row pos left zero.  Rows >= S (spare capacity) are zero.
    With with_raw_keys the unrotated fp64 keys [B,Hkv,S,D] are returned as "k64"
    (small workloads only).
    """
    B, Hq, Hkv, D, S = wl.B, wl.Hq, wl.Hkv, wl.D, wl.S
    cap = wl.capacity
    st = NP_STORAGE[wl.dtype]
    sig = sigma(wl)
    cal = calibration(wl, entropy)
    n_prefill = S - 1 if wl.append else S

    krot = np.zeros((B, Hkv, cap, D), st)
    v = np.zeros((B, Hkv, cap, D), st)
    q = np.zeros((B, Hq, D), st)
    P = np.ascontiguousarray(np.stack([p for _, p in cal]))
    k64 = np.zeros((B, Hkv, S, D), np.float64) if with_raw_keys else None
    out: Dict[str, np.ndarray] = {}
    if wl.append:
        out["k_new"] = np.zeros((B, Hkv, D), st)
        out["v_new"] = np.zeros((B, Hkv, D), st)

    def one_head(kv: int, b: int) -> None:
        U, P32 = cal[kv]
        K = draw_keys(rng(entropy, wl.wid, ROLE_K, kv, b), n_prefill, U, sig)
        if wl.heavy_frac > 0:
            n_heavy = int(round(wl.heavy_frac * n_prefill))
            pos = rng(entropy, wl.wid, ROLE_HEAVY, kv, b).choice(n_prefill, n_heavy, replace=False)
            K[pos] *= wl.heavy_scale
        krot[b, kv, :n_prefill] = to_storage(K @ P32.astype(np.float64), wl.dtype)
        v[b, kv, :n_prefill] = to_storage(
            rng(entropy, wl.wid, ROLE_V, kv, b).standard_normal((n_prefill, D)), wl.dtype)
        if k64 is not None:
            k64[b, kv, :n_prefill] = K
        if wl.append:
            gnew = rng(entropy, wl.wid, ROLE_NEW, kv, b)
            kn = draw_keys(gnew, 1, U, sig)[0]
            out["k_new"][b, kv] = to_storage(kn, wl.dtype)
            out["v_new"][b, kv] = to_storage(gnew.standard_normal(D), wl.dtype)
            if k64 is not None:
                k64[b, kv, S - 1] = from_storage(out["k_new"][b, kv], wl.dtype)

    # every (b, kv) draws from its own seeded stream, so the thread order does
    # not change the result
    jobs = [(kv, b) for kv in range(Hkv) for b in range(B)]
    with cf.ThreadPoolExecutor(max_workers=_workers()) as ex:
        list(ex.map(lambda a: one_head(*a), jobs))
    for kv in range(Hkv):
        U = cal[kv][0]
        for j in range(wl.g):
            h = kv * wl.g + j
            for b in range(B):
                q[b, h] = to_storage(draw_keys(rng(entropy, wl.wid, ROLE_Q, h, b), 1, U, sig)[0],
                                     wl.dtype)
    out.update(q=q, krot=krot, v=v, P=P)
    if wl.append:
        out["pos"] = np.int64(S - 1)
    if k64 is not None:
        out["k64"] = k64
    return out


def softmax_scale(wl: Workload) -> float:
    return 1.0 / math.sqrt(wl.D)


def get(name: str) -> Workload:
    return WORKLOADS[name]


def describe(wl: Workload) -> Dict[str, object]:
    return {"workload": wl.name, "batch": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
            "head_dim": wl.D, "seq_len": wl.S, "d": wl.d, "k": wl.k, "dtype": wl.dtype,
            "append": wl.append}


__all__ = ["Workload", "WORKLOADS", "custom", "generate", "calibration", "pca_basis",
           "to_storage", "from_storage", "sigma", "basis", "rng", "softmax_scale", "get",
           "describe", "Optional"]
