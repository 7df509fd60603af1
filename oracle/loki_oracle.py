"""ctypes wrapper of the fp64 CPU oracle (oracle/loki_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product package.

Arrays are numpy arrays in a storage dtype named by a string:
  "f32" -> float32, "f16" -> float16, "bf16" -> uint16 holding bfloat16 bits,
  "f64" -> float64 (oracle-only, for exact-arithmetic pins).

Parity pins (tests that tie each oracle function to something other than
itself; see tests/test_oracle_pins.py):
  decode (d=D, k=S)  -> textbook softmax(q K^T / sqrt(D)) V on the UNROTATED
                        keys, and torch scaled_dot_product_attention (CPU fp64)
  decode (k=S, any d)-> same full attention; idx = all tokens
  decode (d=D, k<S)  -> exact top-k of q.K^T by numpy argsort, attention over it
  low-dim scores     -> P = identity / permutation: truncated dot over chosen
                        coordinates; general P: projection onto the leading
                        principal subspace built from numpy SVD of the
                        calibration draw
  top-k              -> numpy lexsort, rank-count definition, exhaustive
                        max-sum subset search (S <= 12), q = 0 tie rule
  attend             -> k=1 gives the argmax V row; q=0 gives mean(V[:k]);
                        convex-combination bounds; V outside idx irrelevant;
                        scaling V scales out; token permutation equivariance;
                        key centring invariance
  pca_attention      -> d=D: textbook full attention on the unrotated keys and
                        torch SDPA; any d: torch SDPA over the leading d
                        rotated coordinates (P = identity: over the leading d
                        raw coordinates) with the full-D softmax scale;
                        convexity and V scaling
  covariance         -> numpy.cov(bias=True); keys built from Hadamard columns
                        with an exactly known covariance Q diag(sigma^2) Q^T
  calibrate          -> that closed form (P = Q with the sign rule, variances
                        sigma^2); eigen-residual, orthonormality, order, signs
  append             -> fp64 projection equal to the prefilled rotation;
                        rounding equal to numpy float16 / torch bfloat16
  rounding           -> numpy float64->float16, torch float32->bfloat16 and
                        hand-made ties
  hand example       -> tests/golden/tiny_rotation_example.json (closed form)
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# LOKI_ORACLE_LIB names another build of the same source (the sanitizer tier
# of the tests runs the pins against an AddressSanitizer / UBSan build)
LIB_PATH = os.environ.get("LOKI_ORACLE_LIB") or os.path.join(HERE, "libloki_oracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}
NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "f64": np.float64}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from oracle import build as _b  # noqa: WPS433  (build the oracle library on first use)
            _b.build()
        L = ctypes.CDLL(LIB_PATH)
        vp, ip, dp = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        L.oracle_decode.argtypes = [ip] * 7 + [dp, ip] + [vp] * 4 + [vp, ip] + [vp] * 4
        L.oracle_decode.restype = ip
        L.oracle_attend_given.argtypes = [ip] * 6 + [dp, ip] + [vp] * 5 + [vp, ip, vp]
        L.oracle_attend_given.restype = ip
        L.oracle_pca_attention.argtypes = [ip] * 6 + [dp, ip] + [vp] * 4 + [vp, ip, vp]
        L.oracle_pca_attention.restype = ip
        L.oracle_covariance.argtypes = [ip] * 4 + [vp, vp]
        L.oracle_covariance.restype = ip
        L.oracle_append_rows.argtypes = [ip] * 4 + [vp] * 5
        L.oracle_append_rows.restype = ip
        L.oracle_rotate_queries.argtypes = [ip] * 5 + [vp] * 3
        L.oracle_rotate_queries.restype = ip
        L.oracle_topk_rows.argtypes = [vp, ip, ip, ip, vp]
        L.oracle_topk_rows.restype = None
        L.oracle_round_to_dtype.argtypes = [vp, ctypes.c_size_t, ip, vp]
        L.oracle_round_to_dtype.restype = None
        L.oracle_decode_dtype.argtypes = [vp, ctypes.c_size_t, ip, vp]
        L.oracle_decode_dtype.restype = None
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dt=None):
    a = np.ascontiguousarray(a if dt is None else a.astype(dt, copy=False))
    return a


def _check_storage(a, dtype):
    want = NP_STORAGE[dtype]
    if a.dtype != want:
        raise TypeError(f"storage dtype {dtype} expects numpy {want}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _heads(heads):
    if heads is None:
        return None, 0
    h = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    return h, int(h.size)


def decode(q, krot, v, P, d, k, dtype, scale=0.0, heads=None):
    """One Loki decode step in fp64.

    q [B,Hq,D], krot [B,Hkv,S,D] (rotated keys, logical row-major), v [B,Hkv,S,D],
    P [Hkv,D,D] (any float dtype; used exactly as fp64).
    Returns dict(out [B,Hq,D] f64, idx [B,Hq,k] i32, scores [B,Hq,S] f64, qr [B,Hq,D] f64).
    With `heads` (flattened b*Hq+h) only those units are computed.
    """
    q = _check_storage(q, dtype)
    krot = _check_storage(krot, dtype)
    v = _check_storage(v, dtype)
    B, Hq, D = q.shape
    _, Hkv, S, D2 = krot.shape
    assert D2 == D and v.shape == krot.shape and P.shape == (Hkv, D, D)
    P64 = _c(P, np.float64)
    out = np.zeros((B, Hq, D), np.float64)
    idx = np.full((B, Hq, k), -1, np.int32)
    scores = np.zeros((B, Hq, S), np.float64)
    qr = np.zeros((B, Hq, D), np.float64)
    hh, nh = _heads(heads)
    rc = lib().oracle_decode(B, Hq, Hkv, S, D, int(d), int(k), float(scale), DTYPE_CODE[dtype],
                             _ptr(q), _ptr(krot), _ptr(v), _ptr(P64), _ptr(hh), nh,
                             _ptr(out), _ptr(idx), _ptr(scores), _ptr(qr))
    if rc != 0:
        raise ValueError("oracle_decode: argument outside the method's domain")
    return {"out": out, "idx": idx, "scores": scores, "qr": qr}


def attend_given(q, krot, v, P, idx, dtype, scale=0.0, heads=None):
    """Exact attention over the given ascending/any-order index sets idx [B,Hq,k]."""
    q = _check_storage(q, dtype)
    krot = _check_storage(krot, dtype)
    v = _check_storage(v, dtype)
    B, Hq, D = q.shape
    _, Hkv, S, _ = krot.shape
    idx = _c(idx, np.int32)
    k = idx.shape[-1]
    P64 = _c(P, np.float64)
    out = np.zeros((B, Hq, D), np.float64)
    hh, nh = _heads(heads)
    rc = lib().oracle_attend_given(B, Hq, Hkv, S, D, k, float(scale), DTYPE_CODE[dtype],
                                   _ptr(q), _ptr(krot), _ptr(v), _ptr(P64), _ptr(idx),
                                   _ptr(hh), nh, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_attend_given: bad arguments or index out of range")
    return out


def pca_attention(q, krot, v, P, d, dtype, scale=0.0, heads=None):
    """PCAAttn in fp64: softmax over all S tokens of scale * (low-dim score),
    weighted sum of all S value rows.  Shapes as decode; returns out [B,Hq,D]."""
    q = _check_storage(q, dtype)
    krot = _check_storage(krot, dtype)
    v = _check_storage(v, dtype)
    B, Hq, D = q.shape
    _, Hkv, S, D2 = krot.shape
    assert D2 == D and v.shape == krot.shape and P.shape == (Hkv, D, D)
    P64 = _c(P, np.float64)
    out = np.zeros((B, Hq, D), np.float64)
    hh, nh = _heads(heads)
    rc = lib().oracle_pca_attention(B, Hq, Hkv, S, D, int(d), float(scale), DTYPE_CODE[dtype],
                                    _ptr(q), _ptr(krot), _ptr(v), _ptr(P64), _ptr(hh), nh,
                                    _ptr(out))
    if rc != 0:
        raise ValueError("oracle_pca_attention: argument outside the method's domain")
    return out


def covariance(keys, dtype):
    """Centred (1/n) covariance [Hkv, D, D] fp64 of calibration keys [Hkv, n, D]."""
    keys = _check_storage(keys, dtype)
    Hkv, n, D = keys.shape
    cov = np.zeros((Hkv, D, D), np.float64)
    if lib().oracle_covariance(Hkv, n, D, DTYPE_CODE[dtype], _ptr(keys), _ptr(cov)) != 0:
        raise ValueError("oracle_covariance: bad arguments")
    return cov


def calibrate(keys, dtype):
    """PCA of calibration keys [Hkv, n, D] (poster page, "Visual Insights",
    Figure 1 right): per KV head the eigenvectors of the centred covariance as
    the columns of P, variances descending (equal ones keep their eigh order),
    each column's largest-magnitude entry (the first such) made positive.
    Returns (P [Hkv, D, D] fp64, variances [Hkv, D] fp64)."""
    cov = covariance(keys, dtype)
    Hkv, D, _ = cov.shape
    P = np.zeros((Hkv, D, D))
    var = np.zeros((Hkv, D))
    for kv in range(Hkv):
        w, V = np.linalg.eigh(cov[kv])
        order = np.argsort(-w, kind="stable")
        w, V = w[order], V[:, order]
        lead = np.argmax(np.abs(V), axis=0)
        V = V * np.where(V[lead, np.arange(D)] < 0, -1.0, 1.0)
        P[kv], var[kv] = V, w
    return P, var


def append_rows(k_new, v_new, P, dtype):
    """Rotate new keys [B,Hkv,D] by P in fp64, round once to dtype; copy v_new."""
    k_new = _check_storage(k_new, dtype)
    v_new = _check_storage(v_new, dtype)
    B, Hkv, D = k_new.shape
    P64 = _c(P, np.float64)
    kr = np.zeros_like(k_new)
    vr = np.zeros_like(v_new)
    rc = lib().oracle_append_rows(B, Hkv, D, DTYPE_CODE[dtype], _ptr(k_new), _ptr(v_new),
                                  _ptr(P64), _ptr(kr), _ptr(vr))
    if rc != 0:
        raise ValueError("oracle_append_rows: bad arguments")
    return kr, vr


def rotate_queries(q, P, Hkv, dtype):
    q = _check_storage(q, dtype)
    B, Hq, D = q.shape
    P64 = _c(P, np.float64)
    qr = np.zeros((B, Hq, D), np.float64)
    rc = lib().oracle_rotate_queries(B, Hq, Hkv, D, DTYPE_CODE[dtype], _ptr(q), _ptr(P64),
                                     _ptr(qr))
    if rc != 0:
        raise ValueError("oracle_rotate_queries: bad arguments")
    return qr


def topk_rows(s, k):
    """Top-k (score desc, index asc) of each row of s [..., S]; ascending indices."""
    s = _c(s, np.float64)
    S = s.shape[-1]
    rows = s.reshape(-1, S)
    idx = np.zeros((rows.shape[0], k), np.int32)
    lib().oracle_topk_rows(_ptr(rows), rows.shape[0], S, int(k), _ptr(idx))
    return idx.reshape(s.shape[:-1] + (k,))


def round_to(x, dtype):
    x = _c(x, np.float64)
    dst = np.zeros(x.shape, NP_STORAGE[dtype])
    lib().oracle_round_to_dtype(_ptr(x), x.size, DTYPE_CODE[dtype], _ptr(dst))
    return dst


def to_f64(a, dtype):
    a = _check_storage(a, dtype)
    dst = np.zeros(a.shape, np.float64)
    lib().oracle_decode_dtype(_ptr(a), a.size, DTYPE_CODE[dtype], _ptr(dst))
    return dst
