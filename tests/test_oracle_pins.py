"""Pins of the fp64 CPU oracle against things other than itself (CPU only).

Each test ties one part of the oracle to a textbook or library result, a
closed form, an invariant the method implies, or brute force on tiny inputs.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _orthonormal(D, seed):
    G = np.random.default_rng(seed).standard_normal((D, D))
    Q, R = np.linalg.qr(G)
    return Q * np.sign(np.diag(R))


def _case(B=2, Hq=2, Hkv=2, S=64, D=16, seed=0):
    """fp64 inputs with a random orthonormal P per KV head; keys also unrotated."""
    g = np.random.default_rng(seed)
    P = np.stack([_orthonormal(D, seed * 100 + i) for i in range(Hkv)])
    K = g.standard_normal((B, Hkv, S, D))
    V = g.standard_normal((B, Hkv, S, D))
    q = g.standard_normal((B, Hq, D))
    krot = np.einsum("bhsi,hij->bhsj", K, P)
    return q, K, krot, V, P


def _full_attention(q, K, V, mask=None):
    """softmax(q K^T / sqrt(D)) V per (b, h), written from the textbook definition."""
    B, Hq, D = q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            z = K[b, h // g] @ q[b, h] / math.sqrt(D)
            if mask is not None:
                z = np.where(mask[b, h], z, -np.inf)
            w = np.exp(z - z.max())
            out[b, h] = (w / w.sum()) @ V[b, h // g]
    return out


# ---------------------------------------------------------------- rounding

def test_rounding_f16_matches_numpy(oracle):
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.standard_normal(20000) * 10.0 ** g.integers(-9, 5, 20000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2 ** -24, 2 ** -25,
                  3 * 2 ** -26, 2 ** -14, 2 ** -14 - 2 ** -25]),
    ])
    # exact midpoints between consecutive fp16 values (ties to even)
    h = g.integers(0, 0x7bff, 5000).astype(np.uint16).view(np.float16).astype(np.float64)
    h2 = (g.integers(0, 0x7bff, 5000).astype(np.uint16) + 1).view(np.float16).astype(np.float64)
    x = np.concatenate([x, 0.5 * (h + np.nextafter(h.astype(np.float16),
                                                    np.float16(np.inf)).astype(np.float64)), h2])
    got = oracle.round_to(x, "f16").view(np.uint16)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_rounding_bf16_matches_torch_on_f32_exact_values(oracle):
    g = np.random.default_rng(2)
    x32 = (g.standard_normal(50000) * 10.0 ** g.integers(-30, 30, 50000)).astype(np.float32)
    bits = g.integers(0, 2 ** 31, 20000, dtype=np.uint32).view(np.float32)
    bits = bits[np.isfinite(bits)]
    x32 = np.concatenate([x32, bits, -bits])
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_to(x32.astype(np.float64), "bf16")
    assert np.array_equal(got, ref)


def test_rounding_bf16_single_rounding_ties(oracle):
    one = 1.0
    cases = [
        (one + 2 ** -8, 0x3F80),                  # tie -> even (1.0)
        (one + 3 * 2 ** -8, 0x3F82),              # tie -> even (1 + 2^-6)
        (one + 2 ** -8 + 2 ** -40, 0x3F81),       # just above a tie: up (no double rounding)
        (-(one + 2 ** -8 + 2 ** -40), 0xBF81),
        (2.0 ** -133, 0x0001),                    # smallest subnormal
        (2.0 ** -134, 0x0000),                    # tie between 0 and 2^-133 -> even (0)
        (3 * 2.0 ** -135, 0x0001),                # above the tie
        (0.0, 0x0000),
        (-0.0, 0x8000),
    ]
    x = np.array([c[0] for c in cases])
    got = oracle.round_to(x, "bf16")
    assert [hex(v) for v in got] == [hex(c[1]) for c in cases]


def test_dtype_decoding(oracle):
    g = np.random.default_rng(3)
    h = g.integers(0, 2 ** 16, 10000).astype(np.uint16)
    h = h[np.isfinite(h.view(np.float16))]
    got = oracle.to_f64(h.view(np.float16), "f16")
    assert np.array_equal(got, h.view(np.float16).astype(np.float64))
    b = g.integers(0, 2 ** 16, 10000).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(f)
    got = oracle.to_f64(b[keep], "bf16")
    assert np.array_equal(got, f[keep].astype(np.float64))


# ------------------------------------------------------- full attention pins

@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (3, 1)])
def test_d_full_k_full_equals_textbook_attention(oracle, Hq, Hkv):
    q, K, krot, V, P = _case(B=2, Hq=Hq, Hkv=Hkv, S=50, D=16, seed=Hq * 7 + Hkv)
    S, D = K.shape[2], K.shape[3]
    r = oracle.decode(q, krot, V, P, d=D, k=S, dtype="f64")
    ref = _full_attention(q, K, V)
    np.testing.assert_allclose(r["out"], ref, rtol=0, atol=1e-12)
    assert np.array_equal(r["idx"], np.broadcast_to(np.arange(S), r["idx"].shape))
    # library routine: torch SDPA on CPU fp64 over the unrotated keys
    g = Hq // Hkv
    Kq = torch.from_numpy(np.repeat(K, g, axis=1))
    Vq = torch.from_numpy(np.repeat(V, g, axis=1))
    sd = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None, :], Kq, Vq)[:, :, 0, :].numpy()
    np.testing.assert_allclose(r["out"], sd, rtol=0, atol=1e-12)


@pytest.mark.parametrize("d", [1, 3, 8, 15])
def test_k_full_any_d_equals_full_attention(oracle, d):
    q, K, krot, V, P = _case(S=40, D=16, seed=10 + d)
    r = oracle.decode(q, krot, V, P, d=d, k=40, dtype="f64")
    np.testing.assert_allclose(r["out"], _full_attention(q, K, V), rtol=0, atol=1e-12)


@pytest.mark.parametrize("k", [1, 5, 17])
def test_d_full_equals_exact_topk(oracle, k):
    q, K, krot, V, P = _case(S=60, D=16, seed=20 + k)
    r = oracle.decode(q, krot, V, P, d=16, k=k, dtype="f64")
    B, Hq, _ = q.shape
    mask = np.zeros((B, Hq, 60), bool)
    for b in range(B):
        for h in range(Hq):
            s = K[b, h] @ q[b, h]
            top = np.sort(np.argsort(-s, kind="stable")[:k])
            assert np.array_equal(r["idx"][b, h], top)
            mask[b, h, top] = True
    np.testing.assert_allclose(r["out"], _full_attention(q, K, V, mask), rtol=0, atol=1e-12)
    Kq, Vq = torch.from_numpy(K), torch.from_numpy(V)
    sd = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None, :], Kq, Vq,
        attn_mask=torch.from_numpy(mask)[:, :, None, :])[:, :, 0, :].numpy()
    np.testing.assert_allclose(r["out"], sd, rtol=0, atol=1e-12)


# ------------------------------------------------------------ low-dim score

def test_lowdim_scores_identity_and_permutation_bases(oracle):
    g = np.random.default_rng(30)
    D, S, d = 16, 33, 5
    K = g.standard_normal((1, 1, S, D))
    V = g.standard_normal((1, 1, S, D))
    q = g.standard_normal((1, 1, D))
    for perm in [np.arange(D), g.permutation(D)]:
        P = np.zeros((1, D, D))
        P[0, perm, np.arange(D)] = 1.0          # krot[:, j] = k[:, perm[j]]
        krot = K[:, :, :, perm]
        r = oracle.decode(q, krot, V, P, d=d, k=7, dtype="f64")
        ref = (q[0, 0, perm[:d]] * K[0, 0][:, perm[:d]]).sum(axis=1)
        np.testing.assert_allclose(r["scores"][0, 0], ref, rtol=0, atol=1e-13)


def test_lowdim_scores_are_projection_onto_principal_subspace(oracle):
    """Score = q^T Pi_d k with Pi_d the projector on the leading d principal
    directions, built here from numpy SVD of the calibration draw."""
    wl = W.custom(D=32, S=100, d=6, k=10, tau=6.0, n_calib=4000)
    U = W.basis(wl, 0)
    sig = W.sigma(wl)
    cal = W.draw_keys(W.rng(0, wl.wid, W.ROLE_CALIB, 0), wl.n_calib, U, sig)
    P, _ = W.pca_basis(cal)
    K = W.draw_keys(W.rng(0, 999, 1), wl.S, U, sig)
    q = W.draw_keys(W.rng(0, 999, 2), 1, U, sig)[0]
    V = np.random.default_rng(3).standard_normal((wl.S, wl.D))
    r = oracle.decode(q[None, None], (K @ P)[None, None], V[None, None], P[None], d=wl.d,
                      k=wl.k, dtype="f64")
    X = cal - cal.mean(axis=0)
    _, _, Vt = np.linalg.svd(X, full_matrices=False)
    Pi = Vt[:wl.d].T @ Vt[:wl.d]
    ref = K @ (Pi @ q)
    np.testing.assert_allclose(r["scores"][0, 0], ref, rtol=1e-9, atol=1e-12)


# ------------------------------------------------------------------ top-k

def _rank_count_select(s, k):
    S = len(s)
    sel = []
    for t in range(S):
        rank = sum(1 for u in range(S) if s[u] > s[t]) + sum(1 for u in range(t) if s[u] == s[t])
        if rank < k:
            sel.append(t)
    return sel


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_lexsort_and_rank_count(oracle, seed):
    g = np.random.default_rng(40 + seed)
    S = int(g.integers(1, 90))
    k = int(g.integers(1, S + 1))
    s = g.integers(-4, 5, S).astype(np.float64)      # many ties
    idx = oracle.topk_rows(s[None], k)[0]
    order = np.lexsort((np.arange(S), -s))           # primary: -s, secondary: index
    assert list(idx) == sorted(order[:k].tolist())
    assert list(idx) == _rank_count_select(list(s), k)


def test_topk_exhaustive_max_sum_subset(oracle):
    g = np.random.default_rng(50)
    for _ in range(40):
        S = int(g.integers(1, 11))
        k = int(g.integers(1, S + 1))
        s = g.integers(-3, 4, S).astype(np.float64)
        best = None
        for sub in itertools.combinations(range(S), k):   # lexicographic order
            tot = sum(s[list(sub)])
            if best is None or tot > best[0]:
                best = (tot, sub)
        idx = oracle.topk_rows(s[None], k)[0]
        assert tuple(idx.tolist()) == best[1]


def test_topk_signed_zero_is_a_tie(oracle):
    s = np.array([-0.0, 0.0, -0.0, -1.0, 0.0])
    assert oracle.topk_rows(s[None], 2)[0].tolist() == [0, 1]
    assert oracle.topk_rows(s[None], 4)[0].tolist() == [0, 1, 2, 4]


# ------------------------------------------------------ structural / special

def test_k1_returns_argmax_value_row(oracle):
    q, K, krot, V, P = _case(S=30, D=8, seed=60)
    r = oracle.decode(q, krot, V, P, d=3, k=1, dtype="f64")
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            t = int(np.argmax(r["scores"][b, h]))
            assert r["idx"][b, h, 0] == t
            assert np.array_equal(r["out"][b, h], V[b, h, t])


def test_zero_query_ties_to_first_k_and_mean(oracle):
    q, K, krot, V, P = _case(S=30, D=8, seed=61)
    q[:] = 0.0
    r = oracle.decode(q, krot, V, P, d=3, k=7, dtype="f64")
    assert np.array_equal(r["idx"], np.broadcast_to(np.arange(7), r["idx"].shape))
    np.testing.assert_allclose(r["out"], V[:, :, :7].mean(axis=2), rtol=0, atol=1e-15)


def test_structure_convexity_support_scaling(oracle):
    q, K, krot, V, P = _case(S=80, D=16, seed=62)
    r = oracle.decode(q, krot, V, P, d=4, k=9, dtype="f64")
    for b in range(2):
        for h in range(2):
            sel = V[b, h, r["idx"][b, h]]
            assert np.all(r["out"][b, h] >= sel.min(axis=0) - 1e-15)
            assert np.all(r["out"][b, h] <= sel.max(axis=0) + 1e-15)
    V2 = V.copy()
    for b in range(2):
        for h in range(2):
            outside = np.setdiff1d(np.arange(80), r["idx"][b, h])
            V2[b, h, outside] = 1e3
    r2 = oracle.decode(q, krot, V2, P, d=4, k=9, dtype="f64")
    assert np.array_equal(r2["out"], r["out"])
    r3 = oracle.decode(q, krot, V * 4.0, P, d=4, k=9, dtype="f64")
    assert np.array_equal(r3["out"], r["out"] * 4.0)


# ------------------------------------------------------------- PCAAttn pins

def _sdpa(q, K, V, scale):
    """torch scaled_dot_product_attention (CPU fp64), one query row per (b, h)."""
    B, Hq, _ = q.shape
    g = Hq // K.shape[1]
    Kq = torch.from_numpy(np.ascontiguousarray(np.repeat(K, g, axis=1)))
    Vq = torch.from_numpy(np.ascontiguousarray(np.repeat(V, g, axis=1)))
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.ascontiguousarray(q))[:, :, None, :], Kq, Vq,
        scale=scale)[:, :, 0, :].numpy()


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2)])
def test_pca_attention_full_d_is_full_attention(oracle, Hq, Hkv):
    q, K, krot, V, P = _case(B=2, Hq=Hq, Hkv=Hkv, S=45, D=16, seed=90 + Hq)
    out = oracle.pca_attention(q, krot, V, P, 16, "f64")
    np.testing.assert_allclose(out, _full_attention(q, K, V), rtol=0, atol=1e-12)


@pytest.mark.parametrize("d", [1, 4, 11])
def test_pca_attention_is_attention_over_leading_coordinates(oracle, d):
    """Any d: SDPA over the leading d rotated coordinates of query and keys, with
    the full-dimension scale; with P = identity, over the leading d raw ones."""
    q, K, krot, V, P = _case(B=2, Hq=4, Hkv=2, S=60, D=16, seed=95 + d)
    D = 16
    qr = np.einsum("bhi,hij->bhj", q, np.repeat(P, 2, axis=0))
    out = oracle.pca_attention(q, krot, V, P, d, "f64")
    ref = _sdpa(qr[..., :d], krot[..., :d], V, 1.0 / math.sqrt(D))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    eye = np.broadcast_to(np.eye(D), P.shape).copy()
    out_i = oracle.pca_attention(q, K, V, eye, d, "f64")
    np.testing.assert_allclose(out_i, _sdpa(q[..., :d], K[..., :d], V, 1.0 / math.sqrt(D)),
                               rtol=0, atol=1e-12)
    # a given scale replaces 1/sqrt(D)
    out_s = oracle.pca_attention(q, krot, V, P, d, "f64", scale=0.7)
    np.testing.assert_allclose(out_s, _sdpa(qr[..., :d], krot[..., :d], V, 0.7), rtol=0,
                               atol=1e-12)


def test_pca_attention_structure(oracle):
    q, K, krot, V, P = _case(S=50, D=16, seed=99)
    out = oracle.pca_attention(q, krot, V, P, 5, "f64")
    assert np.all(out >= V.min(axis=2) - 1e-15) and np.all(out <= V.max(axis=2) + 1e-15)
    np.testing.assert_array_equal(oracle.pca_attention(q, krot, V * 2.0, P, 5, "f64"), out * 2.0)
    q0 = np.zeros_like(q)
    np.testing.assert_allclose(oracle.pca_attention(q0, krot, V, P, 5, "f64"), V.mean(axis=2),
                               rtol=0, atol=1e-15)


# --------------------------------------------------------- calibration pins

def test_covariance_matches_numpy_cov(oracle):
    g = np.random.default_rng(120)
    keys = g.standard_normal((3, 200, 16)) * np.linspace(2.0, 0.1, 16) + 5.0
    C = oracle.covariance(keys, "f64")
    for kv in range(3):
        np.testing.assert_allclose(C[kv], np.cov(keys[kv].T, bias=True), rtol=0, atol=1e-12)
    k16 = keys.astype(np.float16)
    C16 = oracle.covariance(k16, "f16")
    np.testing.assert_allclose(C16[1], np.cov(k16[1].astype(np.float64).T, bias=True), rtol=0,
                               atol=1e-12)


@pytest.mark.parametrize("D", [16, 128])
def test_calibrate_closed_form_hadamard(oracle, D):
    """Keys x_t = Z[t] diag(sigma) Q^T + mu with Z = columns 1..D of a 256 x 256
    Hadamard matrix (entries +-1, zero column sums, Z^T Z = 256 I): the centred
    covariance is exactly Q diag(sigma^2) Q^T, so P = Q (sign rule applied) and
    the variances are sigma^2, whatever the offset mu."""
    from scipy.linalg import hadamard
    Z = hadamard(256).astype(np.float64)[:, 1:D + 1]
    Q = _orthonormal(D, 121 + D)
    sig = np.linspace(3.0, 0.5, D)
    mu = np.random.default_rng(122).standard_normal(D) * 4.0
    keys = (Z * sig) @ Q.T + mu
    P, var = oracle.calibrate(keys[None], "f64")
    np.testing.assert_allclose(var[0], sig ** 2, rtol=0, atol=1e-11)
    lead = np.argmax(np.abs(Q), axis=0)
    Qs = Q * np.sign(Q[lead, np.arange(D)])
    np.testing.assert_allclose(P[0], Qs, rtol=0, atol=1e-9)


def test_calibrate_eigen_properties(oracle):
    g = np.random.default_rng(123)
    keys = g.standard_normal((2, 500, 32)) * np.exp(-np.arange(32) / 8.0)
    P, var = oracle.calibrate(keys, "f64")
    C = oracle.covariance(keys, "f64")
    for kv in range(2):
        np.testing.assert_allclose(C[kv] @ P[kv], P[kv] * var[kv], rtol=0, atol=1e-12)
        np.testing.assert_allclose(P[kv].T @ P[kv], np.eye(32), rtol=0, atol=1e-12)
        assert np.all(np.diff(var[kv]) <= 0)
        lead = np.argmax(np.abs(P[kv]), axis=0)
        assert np.all(P[kv][lead, np.arange(32)] > 0)


def test_token_permutation_equivariance(oracle):
    q, K, krot, V, P = _case(B=1, Hq=1, Hkv=1, S=70, D=16, seed=63)
    perm = np.random.default_rng(64).permutation(70)
    r = oracle.decode(q, krot, V, P, d=5, k=11, dtype="f64")
    rp = oracle.decode(q, krot[:, :, perm], V[:, :, perm], P, d=5, k=11, dtype="f64")
    assert sorted(perm[rp["idx"][0, 0]].tolist()) == r["idx"][0, 0].tolist()
    np.testing.assert_allclose(rp["out"], r["out"], rtol=0, atol=1e-13)


def test_key_centring_invariance(oracle):
    """Subtracting a mean key shifts all scores of a query by one constant, so the
    selection and the softmax are unchanged."""
    q, K, krot, V, P = _case(B=1, Hq=1, Hkv=1, S=70, D=16, seed=65)
    mu = np.random.default_rng(66).standard_normal(16) * 3.0
    krot_c = np.einsum("bhsi,hij->bhsj", K - mu, P)
    r = oracle.decode(q, krot, V, P, d=5, k=11, dtype="f64")
    rc = oracle.decode(q, krot_c, V, P, d=5, k=11, dtype="f64")
    assert np.array_equal(r["idx"], rc["idx"])
    np.testing.assert_allclose(rc["out"], r["out"], rtol=0, atol=1e-12)


def test_gqa_mapping_matches_replicated_heads(oracle):
    q, K, krot, V, P = _case(B=2, Hq=6, Hkv=2, S=40, D=8, seed=67)
    r = oracle.decode(q, krot, V, P, d=3, k=6, dtype="f64")
    rr = oracle.decode(q, np.repeat(krot, 3, axis=1), np.repeat(V, 3, axis=1),
                       np.repeat(P, 3, axis=0), d=3, k=6, dtype="f64")
    assert np.array_equal(r["idx"], rr["idx"])
    assert np.array_equal(r["out"], rr["out"])


def test_rotation_preserves_full_scores(oracle):
    """(q P).(k P) = q.k for orthonormal P (fp64)."""
    q, K, krot, V, P = _case(S=25, D=16, seed=68)
    qr = oracle.rotate_queries(q, P, 2, "f64")
    for b in range(2):
        for h in range(2):
            np.testing.assert_allclose(krot[b, h] @ qr[b, h], K[b, h] @ q[b, h], rtol=0,
                                       atol=1e-12)
    r = oracle.decode(q, krot, V, P, d=16, k=25, dtype="f64")
    np.testing.assert_allclose(r["qr"], qr, rtol=0, atol=0)


def test_heads_subset_matches_full_run(oracle):
    q, K, krot, V, P = _case(B=3, Hq=4, Hkv=2, S=30, D=8, seed=69)
    r = oracle.decode(q, krot, V, P, d=3, k=5, dtype="f64")
    rs = oracle.decode(q, krot, V, P, d=3, k=5, dtype="f64", heads=[1, 6, 11])
    for u in [1, 6, 11]:
        b, h = divmod(u, 4)
        assert np.array_equal(rs["out"][b, h], r["out"][b, h])
        assert np.array_equal(rs["idx"][b, h], r["idx"][b, h])


def test_attend_given_matches_decode_on_its_own_idx(oracle):
    q, K, krot, V, P = _case(S=45, D=16, seed=70)
    r = oracle.decode(q, krot, V, P, d=4, k=9, dtype="f64")
    out = oracle.attend_given(q, krot, V, P, r["idx"], "f64")
    assert np.array_equal(out, r["out"])
    mask = np.zeros((2, 2, 45), bool)
    for b in range(2):
        for h in range(2):
            mask[b, h, r["idx"][b, h]] = True
    np.testing.assert_allclose(out, _full_attention(q, K, V, mask), rtol=0, atol=1e-12)


def test_domain_errors(oracle):
    q, K, krot, V, P = _case(S=10, D=8, seed=71)
    for d, k in [(0, 3), (9, 3), (3, 0), (3, 11)]:
        with pytest.raises(ValueError):
            oracle.decode(q, krot, V, P, d=d, k=k, dtype="f64")


# ----------------------------------------------------------------- append

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_append_rotation_and_rounding(oracle, dtype):
    wl = W.custom(B=2, Hq=2, Hkv=2, D=32, S=20, d=8, k=4, dtype=dtype, tau=8.0, n_calib=500,
                  append=True)
    x = W.generate(wl)
    kr, vr = oracle.append_rows(x["k_new"], x["v_new"], x["P"], dtype)
    kn64 = W.from_storage(x["k_new"], dtype)
    ref = np.einsum("bhi,hij->bhj", kn64, x["P"].astype(np.float64))
    if dtype == "bf16":
        # exact bf16 rounding of the fp64 product, via fp64 -> bits by hand-free route:
        # compare decoded values: |got - ref| <= half an ulp, ties impossible here
        got = W.from_storage(kr, dtype)
        ulp = 2.0 ** (np.floor(np.log2(np.abs(ref))) - 7)
        assert np.all(np.abs(got - ref) <= 0.5 * ulp)
    else:
        assert np.array_equal(kr, W.to_storage(ref, dtype))
    assert np.array_equal(vr, x["v_new"])
    # decode after the append equals decode on a cache prefilled with that row
    krot = x["krot"].copy()
    V = x["v"].copy()
    krot[:, :, -1] = kr
    V[:, :, -1] = vr
    r = oracle.decode(x["q"], krot, V, x["P"], d=wl.d, k=wl.k, dtype=dtype)
    assert r["idx"].min() >= 0


# ------------------------------------------------------------ golden example

def test_hand_derived_example():
    from oracle import loki_oracle as oracle
    ex = json.load(open(os.path.join(GOLDEN, "tiny_rotation_example.json")))
    c = 1.0 / math.sqrt(2.0)
    P = np.array([[[c, c], [c, -c]]])
    for case in ex["cases"]:
        q = np.array(case["q"])[None, None]
        K = np.array(case["K"])[None, None]
        V = np.array(case["V"])[None, None]
        krot = K @ P[0]
        r = oracle.decode(q, krot, V, P, d=case["d"], k=case["k"], dtype="f64")
        np.testing.assert_allclose(r["scores"][0, 0], case["expected_scores"], rtol=0,
                                   atol=1e-14)
        assert r["idx"][0, 0].tolist() == case["expected_idx"]
        z = np.array(case["expected_unscaled_logits"]) / math.sqrt(2.0)
        w = np.exp(z - z.max())
        w /= w.sum()
        exp_out = w @ V[0, 0, case["expected_idx"]]
        np.testing.assert_allclose(r["out"][0, 0], exp_out, rtol=0, atol=1e-14)


# ------------------------------------------------------- generator pins

def test_generator_basis_is_orthonormal_and_sorted():
    wl = W.get("llama2_13b_f16").replace(Hkv=2, Hq=2, B=1)
    for kv, (U, P32) in enumerate(W.calibration(wl)):
        assert np.abs(U.T @ U - np.eye(128)).max() < 1e-12
        P = P32.astype(np.float64)
        assert np.abs(P.T @ P - np.eye(128)).max() < 1e-5
        cal = W.draw_keys(W.rng(0, wl.wid, W.ROLE_CALIB, kv), wl.n_calib, U, W.sigma(wl))
        X = cal - cal.mean(axis=0)
        rq = ((X @ P) ** 2).mean(axis=0)                       # per-column variance
        assert np.all(np.diff(rq) <= 1e-9 * rq[0])


def test_generator_spectrum_rank_at_90_percent():
    """Diagnostic of the key generator: principal components holding 90% of the
    key variance (the pages report about 80 of 128 for real models)."""
    for spectrum, lo, hi in [("std", 40, 52), ("variance", 75, 90)]:
        wl = W.get("llama2_13b_f16").replace(spectrum=spectrum)
        var = W.sigma(wl) ** 2
        frac = np.cumsum(var) / var.sum()
        rank = int(np.searchsorted(frac, 0.9) + 1)
        assert lo <= rank <= hi, (spectrum, rank)


def test_generator_is_seeded_and_shapes():
    wl = W.custom(B=2, Hq=4, Hkv=2, D=16, S=30, d=4, k=5, dtype="f16", tau=5.0, n_calib=200,
                  heavy_frac=0.1, append=True, S_cap=40)
    a, b = W.generate(wl), W.generate(wl)
    for key in a:
        assert np.array_equal(a[key], b[key])
    assert a["krot"].shape == (2, 2, 40, 16) and a["q"].shape == (2, 4, 16)
    assert not a["krot"][:, :, 29:].any()          # appended row + spare capacity are empty
    c = W.generate(wl, entropy=1)
    assert not np.array_equal(a["krot"], c["krot"])
