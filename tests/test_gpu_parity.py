"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Per-kernel tests isolate each step (layout, query rotation, append, scores,
top-k on fixed scores, attention on fixed index sets); end-to-end tests run
loki_decode / loki_decode_append on seeded inputs spanning several tiles with
ragged tails, the degenerate cases, and the five full-size workloads.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import loki_oracle as oracle
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_decode_attention_rotate_amd as loki
    return loki


def _small(dtype="f16", **kw):
    base = dict(B=2, Hq=4, Hkv=2, D=128, S=3000, d=32, k=300, dtype=dtype, tau=40.0,
                n_calib=2048)
    base.update(kw)
    return W.custom(name="small", wid=200, **base)


# ------------------------------------------------------------------ layout

@pytest.mark.parametrize("dtype,dp,D", [("f16", 32, 128), ("bf16", 16, 128), ("f32", 32, 128),
                                        ("f16", 128, 128), ("f32", 8, 64), ("bf16", 64, 64),
                                        ("bf16", 32, 96), ("f32", 64, 96)])
def test_pack_unpack_layout(L, dtype, dp, D):
    wl = _small(dtype, D=D, S=77, S_cap=100)
    H.log(f"pack/unpack {dtype} dp={dp} D={D}")
    x = W.generate(wl)
    desc = H.make_desc(wl, dp)
    rows = H.to_device(x["krot"][:, :, :77], dtype)
    cache = L.empty_kcache(desc)
    L.pack_kcache(rows, cache, desc)
    back = L.unpack_kcache(cache, 77, desc)
    torch.cuda.synchronize()
    assert np.array_equal(H.to_host(back, dtype), x["krot"][:, :, :77])
    # documented layout: per (b, kv) [S_cap, dp] panel then [S_cap, D - dp]
    flat = H.to_host(cache, dtype).reshape(wl.B * wl.Hkv, 100 * D)
    src = x["krot"][:, :, :77].reshape(wl.B * wl.Hkv, 77, D)
    for hd in range(wl.B * wl.Hkv):
        panel = flat[hd, :100 * dp].reshape(100, dp)
        rest = flat[hd, 100 * dp:].reshape(100, D - dp)
        assert np.array_equal(panel[:77], src[hd, :, :dp])
        assert np.array_equal(rest[:77], src[hd, :, dp:])


# --------------------------------------------------------------- rotation

@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("f32", 4, 4, 128), ("f16", 8, 2, 128),
                                            ("bf16", 6, 3, 128), ("f16", 6, 3, 96)])
def test_rotate_query(L, dtype, Hq, Hkv, D):
    wl = _small(dtype, Hq=Hq, Hkv=Hkv, B=5, S=64, k=8, D=D)
    H.log(f"rotate {dtype} Hq={Hq} Hkv={Hkv}")
    x = W.generate(wl)
    dev = H.upload(wl, x)
    qr = L.rotate_query(dev["q"], dev["P"], dev["desc"]).cpu().numpy().astype(np.float64)
    ref = oracle.rotate_queries(x["q"], x["P"], Hkv, dtype)
    q64 = W.from_storage(x["q"], dtype)
    P = x["P"].astype(np.float64)
    g = Hq // Hkv
    bound = np.stack([np.abs(q64[:, h]) @ np.abs(P[h // g]) for h in range(Hq)], axis=1)
    assert np.all(np.abs(qr - ref) <= 2 * D * 2.0 ** -24 * bound + 1e-30)


# ----------------------------------------------------------------- append

def _ulp(r: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the f16 / bf16 values at |r| (subnormal spacing below the
    smallest normal)."""
    mant, emin = {"f16": (10, -14), "bf16": (7, -126)}[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** emin)))
    return 2.0 ** (e - mant)


@pytest.mark.parametrize("dtype,dp,D", [("f32", 32, 128), ("f16", 32, 128), ("bf16", 32, 128),
                                        ("f16", 128, 128), ("bf16", 16, 128), ("bf16", 32, 96)])
def test_append_row(L, dtype, dp, D):
    wl = _small(dtype, S=50, S_cap=64, k=5, append=True, B=3, Hq=4, Hkv=4, D=D)
    H.log(f"append {dtype} dp={dp}")
    x = W.generate(wl)
    dev = H.upload(wl, x, dp)
    desc = dev["desc"]
    pos = 49
    L.append(dev["k_new"], dev["v_new"], dev["P"], dev["kcache"], dev["v"], pos, desc)
    rows = L.unpack_kcache(dev["kcache"], 64, desc.with_seq_len(64))
    torch.cuda.synchronize()
    _check_appended(dtype, x, H.to_host(rows, dtype), H.to_host(dev["v"], dtype), pos)


def _check_appended(dtype, x, got, v_got, pos):
    """Row pos of the K cache (unpacked rows `got`) and of the V cache
    `v_got` against the oracle's append; every other row unchanged."""
    kr, vr = oracle.append_rows(x["k_new"], x["v_new"], x["P"], dtype)
    g = W.from_storage(got[:, :, pos], dtype)
    r = W.from_storage(kr, dtype)
    frac_exact = np.mean(g == r)
    H.log(f"  appended elements equal to the oracle's rounding: {frac_exact:.5f}")
    D = g.shape[-1]
    kn = W.from_storage(x["k_new"], dtype)
    mag = np.einsum("bhi,hij->bhj", np.abs(kn), np.abs(x["P"].astype(np.float64)))
    if dtype == "f32":
        # the stored value is the fp32 product itself: fp32 dot-product error bound
        assert np.all(np.abs(g - r) <= 2 * D * 2.0 ** -24 * mag)
    else:
        # fp32 product rounded once to f16 / bf16: one unit in the last place
        # plus the fp32 dot-product error (which matters only under cancellation)
        assert np.all(np.abs(g - r) <= _ulp(r, dtype) + 2 * D * 2.0 ** -24 * mag)
        assert frac_exact > 0.99
    assert np.array_equal(v_got[:, :, pos], vr)
    keep = np.ones(got.shape[2], bool)
    keep[pos] = False
    assert np.array_equal(got[:, :, keep], x["krot"][:, :, keep])
    assert np.array_equal(v_got[:, :, keep], x["v"][:, :, keep])


# ----------------------------------------------------------------- prefill

def _oracle_prefill(k_rows, v_rows, P, dtype):
    """The oracle's append applied to every token of k_rows [B, Hkv, n, D]."""
    B, Hkv, n, D = k_rows.shape
    kt = np.ascontiguousarray(k_rows.transpose(0, 2, 1, 3).reshape(B * n, Hkv, D))
    vt = np.ascontiguousarray(v_rows.transpose(0, 2, 1, 3).reshape(B * n, Hkv, D))
    kr, _ = oracle.append_rows(kt, vt, P, dtype)
    return np.ascontiguousarray(kr.reshape(B, n, Hkv, D).transpose(0, 2, 1, 3))


def _raw(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32 if a.dtype.itemsize == 4 else np.uint16)


def _random_bits(g, shape, dtype):
    bits = g.integers(0, 1 << 16, shape, dtype=np.uint32).astype(np.uint16)
    if dtype == "f32":
        return (bits.astype(np.uint32) * 65537).view(np.float32)
    return bits if dtype == "bf16" else bits.view(np.float16)


@pytest.mark.parametrize("dtype,D,dp,n,pos", [
    ("f16", 128, 32, 1100, 37), ("bf16", 128, 16, 1100, 0), ("f32", 128, 32, 700, 5),
    ("f16", 128, 128, 64, 0), ("bf16", 128, 64, 1, 1199), ("bf16", 128, 32, 600, 600),
    ("f16", 64, 16, 300, 3), ("f32", 64, 8, 513, 0), ("bf16", 96, 32, 500, 7),
    ("f32", 96, 32, 130, 1)])
def test_prefill(L, dtype, D, dp, n, pos):
    S_cap = 1200
    wl = _small(dtype, D=D, S=n, S_cap=S_cap, Hq=3, Hkv=3, d=min(32, D), k=1)
    H.log(f"prefill {dtype} D={D} dp={dp} n={n} pos={pos}")
    x = W.generate(wl, with_raw_keys=True)
    k_rows = W.to_storage(x["k64"], dtype)
    v_rows = x["v"][:, :, :n]
    g = np.random.default_rng(11)
    k_init = _random_bits(g, (wl.B, wl.Hkv, S_cap, D), dtype)
    v_init = _random_bits(g, (wl.B, wl.Hkv, S_cap, D), dtype)
    desc = H.make_desc(wl, dp)
    kcache = L.empty_kcache(desc)
    L.pack_kcache(H.to_device(k_init, dtype), kcache, desc.with_seq_len(S_cap))
    vcache = H.to_device(v_init, dtype)
    P = torch.from_numpy(x["P"]).cuda()
    L.prefill(H.to_device(k_rows, dtype), P, kcache, desc, v_rows=H.to_device(v_rows, dtype),
              vcache=vcache, pos=pos)
    rows = L.unpack_kcache(kcache, S_cap, desc.with_seq_len(S_cap))
    torch.cuda.synchronize()
    got = H.to_host(rows, dtype)
    inside = np.zeros(S_cap, bool)
    inside[pos:pos + n] = True
    # rows outside [pos, pos + n) keep their bits, in both caches
    assert np.array_equal(_raw(got[:, :, ~inside]), _raw(k_init[:, :, ~inside]))
    vg = H.to_host(vcache, dtype)
    assert np.array_equal(_raw(vg[:, :, ~inside]), _raw(v_init[:, :, ~inside]))
    assert np.array_equal(_raw(vg[:, :, inside]), _raw(np.ascontiguousarray(v_rows)))
    ref = _oracle_prefill(k_rows, v_rows, x["P"], dtype)
    gk = W.from_storage(got[:, :, inside], dtype)
    rk = W.from_storage(ref, dtype)
    frac_exact = np.mean(gk == rk)
    H.log(f"  elements equal to the oracle's rounding: {frac_exact:.5f}")
    # fp32-accurate product (fp32 dot-product error bound), rounded once: for
    # f16 / bf16 one unit in the last place more
    kn = W.from_storage(k_rows, dtype)
    mag = np.einsum("bhti,hij->bhtj", np.abs(kn), np.abs(x["P"].astype(np.float64)))
    bound = 2 * D * 2.0 ** -24 * mag + (0.0 if dtype == "f32" else _ulp(rk, dtype))
    ratio = np.abs(gk - rk) / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    H.log(f"  worst |gpu - oracle| / bound = {ratio[worst]:.3f} at {worst}: "
          f"gpu {gk[worst]!r} oracle {rk[worst]!r} magnitude {mag[worst]:.3e}")
    assert np.all(ratio <= 1.0)
    if dtype != "f32":
        assert frac_exact > 0.99


@pytest.mark.parametrize("dtype,g", [("f16", 4), ("bf16", 1)])
def test_prefill_then_decode(L, dtype, g):
    """A cache filled by loki_prefill decodes like the oracle's own prefill."""
    wl = _small(dtype, B=2, Hq=2 * g, Hkv=2, S=2500, S_cap=2600, d=32, k=256)
    H.log(f"prefill + decode {dtype} g={g}")
    x = W.generate(wl, with_raw_keys=True)
    k_rows = W.to_storage(x["k64"], dtype)
    desc = H.make_desc(wl, 32)
    dev = {"desc": desc, "q": H.to_device(x["q"], dtype), "P": torch.from_numpy(x["P"]).cuda(),
           "kcache": L.empty_kcache(desc), "v": torch.zeros((wl.B, wl.Hkv, 2600, wl.D),
                                                           dtype=desc.torch_dtype, device="cuda")}
    L.prefill(H.to_device(k_rows, dtype), dev["P"], dev["kcache"], desc,
              v_rows=H.to_device(np.ascontiguousarray(x["v"][:, :, :wl.S]), dtype),
              vcache=dev["v"])
    out, idx = H.run_decode(wl, dev)
    krot = np.zeros_like(x["krot"])
    krot[:, :, :wl.S] = _oracle_prefill(k_rows, x["v"][:, :, :wl.S], x["P"], dtype)
    res = H.full_parity(wl, dict(x, krot=krot), out, idx)
    H.log(f"  {res}")


@pytest.mark.parametrize("name", ["llama2_13b_f16", "gqa_llama3_8b_bf16"])
def test_prefill_full_size(L, name):
    """Full-size prefill (launch sizes as timed), checked on sampled token rows."""
    wl = W.get(name)
    dtype, B, Hkv, S, D = wl.dtype, wl.B, wl.Hkv, wl.S, wl.D
    H.log(f"prefill full size {name}")
    g = np.random.default_rng(2024)
    P = np.stack([W.basis(wl, kv).astype(np.float32) for kv in range(Hkv)])
    desc = H.make_desc(wl, 32)
    k_dev = torch.empty((B, Hkv, S, D), dtype=desc.torch_dtype, device="cuda")
    # seeded keys, generated on the host one batch row at a time
    for b in range(B):
        kb = W.to_storage(g.standard_normal((Hkv, S, D)) * W.sigma(wl)[None, None, :], dtype)
        k_dev[b].copy_(H.to_device(kb, dtype))
    kcache = L.empty_kcache(desc)
    L.prefill(k_dev, torch.from_numpy(P).cuda(), kcache, desc)
    rows = L.unpack_kcache(kcache, S, desc)
    bs = torch.from_numpy(g.integers(0, B, 512)).cuda()
    ts = torch.from_numpy(g.integers(0, S, 512)).cuda()
    got = H.to_host(rows[bs, :, ts].contiguous(), dtype)     # [512, Hkv, D]
    k_in = H.to_host(k_dev[bs, :, ts].contiguous(), dtype)
    torch.cuda.synchronize()
    kr, _ = oracle.append_rows(k_in, k_in, P, dtype)
    gk, rk = W.from_storage(got, dtype), W.from_storage(kr, dtype)
    mag = np.einsum("nhi,hij->nhj", np.abs(W.from_storage(k_in, dtype)), np.abs(P.astype(np.float64)))
    bound = 2 * D * 2.0 ** -24 * mag + _ulp(rk, dtype)
    frac_exact = np.mean(gk == rk)
    H.log(f"  sampled elements equal to the oracle's rounding: {frac_exact:.5f}")
    assert np.all(np.abs(gk - rk) <= bound)
    assert frac_exact > 0.99


# ------------------------------------------------------------------ scores

@pytest.mark.parametrize("dtype,g,d,dp", [("f16", 1, 32, 32), ("bf16", 4, 32, 32),
                                          ("f32", 2, 32, 32), ("f16", 8, 20, 32),
                                          ("f16", 1, 48, 32), ("bf16", 1, 16, 16),
                                          ("f32", 1, 128, 128), ("f16", 3, 32, 32)])
def test_scores(L, dtype, g, d, dp):
    wl = _small(dtype, Hq=2 * g, Hkv=2, S=2500, k=50)
    H.log(f"scores {dtype} g={g} d={d} dp={dp}")
    x = W.generate(wl)
    dev = H.upload(wl, x, dp)
    desc = dev["desc"]
    qr_dev = L.rotate_query(dev["q"], dev["P"], desc)
    s = L.score(qr_dev, dev["kcache"], d, desc).cpu().numpy().astype(np.float64)
    r = oracle.decode(x["q"], x["krot"], x["v"], x["P"], d, 50, dtype)
    k64 = W.from_storage(x["krot"], dtype)
    qr = r["qr"]
    # fp32 bound: error of the fp32 query rotation plus the fp32 dot product
    mag = np.stack([np.einsum("bj,btj->bt", np.abs(qr[:, h, :d]), np.abs(k64[:, h // g, :, :d]))
                    for h in range(wl.Hq)], axis=1)
    assert np.all(np.abs(s - r["scores"]) <= 4 * (128 + d) * 2.0 ** -24 * mag + 1e-30)


# ------------------------------------------------------------------- top-k

def _topk_cases():
    g = np.random.default_rng(123)
    cases = []
    for S, k in [(1, 1), (7, 3), (64, 64), (1000, 125), (4096, 512), (5000, 1), (8192, 1024),
                 (8193, 4000), (20000, 2500), (32768, 4096), (40000, 5000)]:
        cases.append((f"normal-{S}-{k}", g.standard_normal((3, S)).astype(np.float32), k))
    cases.append(("ties", g.integers(-3, 4, (4, 3000)).astype(np.float32), 700))
    cases.append(("all-equal", np.full((2, 2048), 0.5, np.float32), 100))
    z = g.choice(np.array([0.0, -0.0, 1.0, -1.0], np.float32), (2, 1500))
    cases.append(("signed-zero", z, 900))
    hh = g.standard_normal((2, 32768)).astype(np.float32)
    hh[:, g.choice(32768, 655, replace=False)] *= 16.0
    cases.append(("heavy", hh, 4096))
    cases.append(("tiny-range", (1.0 + g.integers(0, 4, (2, 5000)) * 2.0 ** -23).astype(np.float32), 1234))
    # exact duplicates of the k-th value scattered before and after it
    dup = g.standard_normal((3, 4096)).astype(np.float32)
    for row in dup:
        kth = np.sort(row)[::-1][511]
        row[g.choice(4096, 6, replace=False)] = kth
    cases.append(("dup-at-threshold", dup, 512))
    cases.append(("dup-at-threshold-16k", np.tile(dup[:, :4096], (1, 4)) * 1.0, 2048))
    # a few huge outliers squeeze the bulk into few linear bins: the crowded
    # threshold bin is refined once (1e3, 1e4) or, still crowded, resolved by
    # radix passes (1e7); with duplicates of the k-th value as well
    for scale_out, S, k in [(1e3, 4096, 512), (1e4, 32768, 4096), (1e7, 32768, 4096),
                            (1e4, 16384, 2048)]:
        o = g.standard_normal((3, S)).astype(np.float32)
        pos = g.choice(S, max(1, S // 1000), replace=False)
        o[:, pos] = (np.sign(g.standard_normal(pos.size)) * scale_out).astype(np.float32)
        cases.append((f"outliers-{scale_out:g}-{S}-{k}", o, k))
    od = cases[-1][1].copy()
    for row in od:
        kth = np.sort(row)[::-1][2047]
        row[g.choice(16384, 9, replace=False)] = kth
    cases.append(("outliers-dup-at-threshold", od, 2048))
    return cases


@pytest.mark.parametrize("name,s,k", _topk_cases(), ids=[c[0] for c in _topk_cases()])
def test_topk_bit_exact(L, name, s, k):
    H.log(f"topk {name} S={s.shape[1]} k={k}")
    rows, S = s.shape
    desc = L.Desc(batch=1, n_q_heads=rows, n_kv_heads=1, head_dim=128, seq_len=S,
                  seq_capacity=S, panel_dim=32, dtype=L.F16)
    sd = torch.from_numpy(s).cuda().reshape(1, rows, S)
    idx = L.topk(sd, k, desc).cpu().numpy()[0]
    ref = oracle.topk_rows(s.astype(np.float64), k)
    assert np.array_equal(idx, ref)


def test_topk_selected_scores_out(L):
    g = np.random.default_rng(11)
    s = g.standard_normal((4, 3000)).astype(np.float32)
    s[:, 5] = -0.0
    desc = L.Desc(batch=2, n_q_heads=2, n_kv_heads=2, head_dim=128, seq_len=3000,
                  seq_capacity=3000, panel_dim=32, dtype=L.F16)
    sd = torch.from_numpy(s).cuda().reshape(2, 2, 3000)
    sel = torch.empty((2, 2, 700), dtype=torch.float32, device="cuda")
    idx = L.topk(sd, 700, desc, sel_out=sel).cpu().numpy().reshape(4, 700)
    got = sel.cpu().numpy().reshape(4, 700)
    ref = np.take_along_axis(s, idx, axis=1)
    ref[ref == 0] = 0.0
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------- attention alone

@pytest.mark.parametrize("dtype,D,k,g", [("f16", 128, 300, 1), ("bf16", 128, 128, 2),
                                         ("f32", 128, 1, 1), ("f32", 64, 257, 1),
                                         ("f16", 64, 640, 4), ("bf16", 128, 1000, 1),
                                         ("bf16", 96, 500, 2), ("f32", 96, 700, 1)])
def test_attend_given_index_sets(L, dtype, D, k, g):
    wl = _small(dtype, D=D, Hq=2 * g, Hkv=2, S=1500, k=k)
    H.log(f"attend {dtype} D={D} k={k} g={g}")
    x = W.generate(wl)
    dev = H.upload(wl, x)
    rg = np.random.default_rng(7)
    idx = np.stack([np.stack([rg.choice(1500, k, replace=False) for _ in range(wl.Hq)])
                    for _ in range(wl.B)]).astype(np.int32)
    qr = L.rotate_query(dev["q"], dev["P"], dev["desc"])
    out = L.attend(qr, dev["kcache"], dev["v"], torch.from_numpy(idx).cuda(), dev["desc"])
    out = out.cpu().numpy().astype(np.float64)
    ref = oracle.attend_given(x["q"], x["krot"], x["v"], x["P"], idx, dtype)
    err = H.rel_err_rows(out, ref)
    H.log(f"  max rel err {err.max():.2e}")
    assert err.max() < H.OUT_TOL[dtype]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_attend_with_low_dim_partial_logits(L, dtype):
    """Per-step pipeline score -> topk (sel_out) -> attend(sel_scores): only the
    key coordinates beyond the panel are read, same result."""
    wl = _small(dtype, S=2000, k=250, tau=20.0 if dtype == "f32" else 40.0)
    x = W.generate(wl)
    dev = H.upload(wl, x)
    desc = dev["desc"]
    qr = L.rotate_query(dev["q"], dev["P"], desc)
    sc = L.score(qr, dev["kcache"], 32, desc)
    sel = torch.empty((wl.B, wl.Hq, 250), dtype=torch.float32, device="cuda")
    idx = L.topk(sc, 250, desc, sel_out=sel)
    out = L.attend(qr, dev["kcache"], dev["v"], idx, desc, sel_scores=sel)
    out = out.cpu().numpy().astype(np.float64)
    ref = oracle.attend_given(x["q"], x["krot"], x["v"], x["P"], idx.cpu().numpy(), dtype)
    err = H.rel_err_rows(out, ref)
    H.log(f"  max rel err {err.max():.2e}")
    assert err.max() < H.OUT_TOL[dtype]


def test_attend_skips_out_of_range_indices(L):
    wl = _small("f16", S=600, k=64)
    x = W.generate(wl)
    dev = H.upload(wl, x)
    rg = np.random.default_rng(8)
    idx = np.stack([np.stack([rg.choice(600, 64, replace=False) for _ in range(4)])
                    for _ in range(2)]).astype(np.int32)
    bad = idx.copy()
    bad[:, :, 5] = -3
    bad[:, :, 9] = 600
    qr = L.rotate_query(dev["q"], dev["P"], dev["desc"])
    out = L.attend(qr, dev["kcache"], dev["v"], torch.from_numpy(bad).cuda(), dev["desc"])
    out = out.cpu().numpy().astype(np.float64)
    keep = np.delete(idx, [5, 9], axis=2)
    ref = oracle.attend_given(x["q"], x["krot"], x["v"], x["P"], keep, "f16")
    assert H.rel_err_rows(out, ref).max() < 2e-3


# --------------------------------------------------------------- end to end

E2E = {
    "f16-ragged": dict(dtype="f16"),
    "bf16-ragged": dict(dtype="bf16"),
    "f32-ragged": dict(dtype="f32", tau=20.0),
    "gqa4-bf16": dict(dtype="bf16", Hq=8, Hkv=2, S=5000, k=700),
    "gqa8-f16": dict(dtype="f16", Hq=16, Hkv=2, S=2100, k=130),
    "gqa3-generic": dict(dtype="f16", Hq=6, Hkv=2, S=1100, k=100),
    # grouped heads inside the one-launch kernel (g = 2, 4; their scores and
    # index lists fit its LDS budget)
    "gqa2-fused-f16": dict(dtype="f16", B=3, Hq=8, Hkv=4, S=3000, k=300),
    "gqa4-fused-bf16": dict(dtype="bf16", B=2, Hq=8, Hkv=2, S=1800, k=200),
    "gqa2-fused-f32": dict(dtype="f32", B=2, Hq=4, Hkv=2, S=2222, k=222, tau=20.0),
    "gqa4-fused-k1": dict(dtype="f16", B=2, Hq=8, Hkv=2, S=1000, k=1),
    "d-below-panel": dict(dtype="f16", d=20),
    "d-above-panel": dict(dtype="f16", d=48),
    "d-full": dict(dtype="f16", d=128),
    "k-full": dict(dtype="f16", S=700, k=700),
    "k-one": dict(dtype="bf16", k=1),
    "seq-one": dict(dtype="f16", S=1, k=1, d=8),
    "cap-above-seq": dict(dtype="f16", S=1900, S_cap=2600, k=200),
    "d64-head": dict(dtype="f16", D=64, d=16, tau=20.0),
    # head dimension 96 (keys of 96 coordinates, the other lanes of a row idle)
    "d96-f16": dict(dtype="f16", D=96),
    "d96-bf16-gqa4": dict(dtype="bf16", D=96, Hq=8, Hkv=2, S=5000, k=700),
    "d96-f32": dict(dtype="f32", D=96, S=2100, k=210, tau=20.0),
    "d96-long": dict(dtype="bf16", D=96, B=1, Hq=8, Hkv=8, S=20000, k=2500, heavy_frac=0.02),
    "long-11k": dict(dtype="bf16", B=1, Hq=2, Hkv=2, S=11000, k=1375),
    "long-30k": dict(dtype="bf16", B=1, Hq=2, Hkv=2, S=30000, k=3000, heavy_frac=0.02),
    "long-40k": dict(dtype="f16", B=1, Hq=1, Hkv=1, S=40000, k=5000),
    # grouped heads whose selections cover at least half of the tokens
    # (g*k >= S/2): shared rows, several attention splits per head
    "gqa2-wide-f16": dict(dtype="f16", B=2, Hq=8, Hkv=4, S=5100, k=1300),
    "gqa4-wide-900": dict(dtype="bf16", B=2, Hq=8, Hkv=2, S=900, k=300),
    "gqa4-wide-f32": dict(dtype="f32", B=1, Hq=8, Hkv=2, S=4500, k=600, tau=20.0),
    "gqa4-k-full": dict(dtype="f16", B=1, Hq=4, Hkv=1, S=1500, k=1500),
    # 256 query rows (a workgroup per compute unit): the separate path's
    # attention takes each row's k selected tokens in one split of 1024 or
    # 2048 rows (ragged), with no merge
    "rows256-k900": dict(dtype="f16", B=8, Hq=32, Hkv=32, S=2000, k=900),
    "rows256-k1500": dict(dtype="bf16", B=8, Hq=32, Hkv=32, S=2600, k=1500),
}


@pytest.mark.parametrize("separate", [False, True], ids=["default", "separate"])
@pytest.mark.parametrize("case", list(E2E), ids=list(E2E))
def test_decode_end_to_end(L, case, separate):
    wl = _small(**E2E[case])
    x = W.generate(wl)
    dev = H.upload(wl, x)
    plan = L.decode_plan(dev["desc"], wl.d, wl.k, wl.append)
    if "fused" in case:
        assert plan, f"{case} is meant to take the one-launch kernel"
    H.log(f"decode {case} separate={separate} one_launch={plan}: {W.describe(wl)}")
    out, idx = H.run_decode(wl, dev, separate=separate)
    res = H.full_parity(wl, x, out, idx)
    H.log(f"  {res}")


@pytest.mark.parametrize("dtype,B,nh,S,k", [("f16", 2, 4, 3000, 300), ("bf16", 8, 40, 2000, 300)],
                         ids=["512-threads", "256-threads-helpers"])
def test_provisional_range_far_from_later_scores(L, dtype, B, nh, S, k):
    """The one-launch kernel bins every score with a range taken from its first
    batch of scores.  Here the first 1100 tokens score almost alike (a range
    thousands of times narrower than the rest) and every later token scores
    up to a thousand times further out, on both sides: the clamped binning
    must stay monotone, and the selection exact up to the tie band."""
    wl = _small(dtype, B=B, Hq=nh, Hkv=nh, S=S, k=k)
    x = W.generate(wl)
    K = W.from_storage(x["krot"], dtype)
    g = np.random.default_rng(17)
    K[:, :, :1100, :32] = K[:, :, :1, :32] * (1.0 + 1e-3 * g.standard_normal((B, nh, 1100, 1)))
    K[:, :, 1100:S, :32] *= g.choice([1.0, 30.0, 1000.0], size=(B, nh, S - 1100, 1))
    x["krot"] = W.to_storage(K, dtype)
    dev = H.upload(wl, x)
    assert L.decode_plan(dev["desc"], wl.d, wl.k)
    H.log(f"provisional binning range {dtype} B={B} heads={nh}")
    out, idx = H.run_decode(wl, dev)
    res = H.full_parity(wl, x, out, idx)
    H.log(f"  {res}")


# The one-launch kernel with one query head per workgroup and its whole row of
# scores in LDS (rows up to 32768 tokens, grouped heads of any size): 512
# threads up to 16384 tokens (two workgroups per compute unit), 1024 above;
# helpers for single-head rows when the heads leave workgroup slots free (a
# multiple of 8 heads, k >= 256); grouped heads padded to whole blocks of 8
# (b, kv) units; binning over mean +- 6 sd above 16384 tokens.
HEAD_CASES = {
    "g1-pairs-20k-heavy": dict(dtype="bf16", B=2, Hq=8, Hkv=8, S=20000, k=2500, heavy_frac=0.02),
    "g1-pairs-512thr": dict(dtype="f16", B=1, Hq=8, Hkv=8, S=9000, k=300),
    "g1-small-k-no-pairs": dict(dtype="f16", B=1, Hq=8, Hkv=8, S=9000, k=100),
    "g1-32768-heavy": dict(dtype="bf16", B=1, Hq=8, Hkv=8, S=32768, k=4096, heavy_frac=0.02),
    "g1-odd-heads": dict(dtype="f16", B=1, Hq=5, Hkv=5, S=12345, k=1234),
    "g1-k-eq-S": dict(dtype="f16", B=1, Hq=8, Hkv=8, S=4500, k=4500),
    "g1-k1": dict(dtype="bf16", B=1, Hq=8, Hkv=8, S=5000, k=1),
    "g4-xcd-padding": dict(dtype="bf16", B=3, Hq=12, Hkv=3, S=6000, k=800),
    "g4-16k": dict(dtype="bf16", B=2, Hq=8, Hkv=2, S=16384, k=2048),
    "g2-f32": dict(dtype="f32", B=2, Hq=4, Hkv=2, S=7000, k=700, tau=20.0),
    "g16-f16": dict(dtype="f16", B=1, Hq=16, Hkv=1, S=5000, k=400),
    "g8-cap-above-seq": dict(dtype="f16", B=1, Hq=16, Hkv=2, S=4700, S_cap=5000, k=500),
    "g2-16k": dict(dtype="bf16", B=2, Hq=4, Hkv=2, S=16384, k=2048),
    "g6": dict(dtype="f16", B=1, Hq=12, Hkv=2, S=7000, k=900),
    "g3-odd-group": dict(dtype="bf16", B=2, Hq=6, Hkv=2, S=9000, k=1000),
}


@pytest.mark.parametrize("case", list(HEAD_CASES), ids=list(HEAD_CASES))
def test_decode_head_kernel(L, case):
    wl = _small(**HEAD_CASES[case])
    x = W.generate(wl)
    dev = H.upload(wl, x)
    assert L.decode_plan(dev["desc"], wl.d, wl.k), f"{case} is meant to take one launch"
    H.log(f"decode (one head per workgroup) {case}: {W.describe(wl)}")
    out, idx = H.run_decode(wl, dev)
    res = H.full_parity(wl, x, out, idx)
    H.log(f"  {res}")


HEAD_APPEND = {
    "g1-pairs-append": dict(dtype="bf16", B=2, Hq=8, Hkv=8, S=20000, S_cap=20100, k=2500,
                            heavy_frac=0.02),
    "g1-pairs-append-selected": dict(dtype="f16", B=1, Hq=8, Hkv=8, S=9000, S_cap=9000, k=600,
                                     selected=True),
    "g4-append-selected": dict(dtype="bf16", B=2, Hq=8, Hkv=2, S=6000, S_cap=6100, k=700,
                               selected=True),
    "g4-append-in-first-batch": dict(dtype="bf16", B=2, Hq=8, Hkv=2, S=4200, S_cap=4300, k=300,
                                     selected=True),
    "g1-32768-append": dict(dtype="bf16", B=1, Hq=8, Hkv=8, S=32768, S_cap=32768, k=4096,
                            heavy_frac=0.02),
}


@pytest.mark.parametrize("case", list(HEAD_APPEND), ids=list(HEAD_APPEND))
def test_decode_append_head_kernel(L, case):
    kw = dict(HEAD_APPEND[case])
    selected = kw.pop("selected", False)
    wl = _small(append=True, **kw)
    assert L.decode_plan(H.make_desc(wl, 32), wl.d, wl.k, True)
    H.log(f"decode_append (one head per workgroup) {case}: {W.describe(wl)}")
    _decode_append_check(L, wl, separate=False, selected=selected)


def test_head_kernel_ties_radix_passes(L):
    """Panel coordinates drawn from 12 distinct rows: every score is tied with
    hundreds of others, the bin of the k-th score cannot be split, and the
    selection resolves it by radix passes and the lower-index rule."""
    wl = _small("f16", B=1, Hq=8, Hkv=8, S=9000, k=1000)
    x = W.generate(wl)
    K = W.from_storage(x["krot"], "f16")
    g = np.random.default_rng(23)
    pick = g.integers(0, 12, size=(wl.B, wl.Hkv, wl.S))
    for b in range(wl.B):
        for h in range(wl.Hkv):
            K[b, h, :wl.S, :32] = K[b, h, pick[b, h], :32]
    x["krot"] = W.to_storage(K, "f16")
    dev = H.upload(wl, x)
    assert L.decode_plan(dev["desc"], wl.d, wl.k)
    out, idx = H.run_decode(wl, dev)
    res = H.full_parity(wl, x, out, idx)
    H.log(f"  ties: {res}")
    # exact ties must follow the lower-index rule exactly: the GPU's fp32
    # scores of equal rows are equal, so the sets match the oracle's
    r = oracle.decode(x["q"], x["krot"], x["v"], x["P"], wl.d, wl.k, "f16")
    s = oracle.decode(x["q"], x["krot"], x["v"], x["P"], wl.d, wl.k, "f16")["scores"]
    for h in range(wl.Hq):
        srt = np.sort(s[0, h])[::-1]
        if srt[wl.k - 1] - srt[wl.k] > 1e-3 * abs(srt[wl.k - 1]):
            assert np.array_equal(idx[0, h], r["idx"][0, h])


@pytest.mark.parametrize("dtype,B,nh,S,k", [("bf16", 2, 8, 20000, 2500), ("f16", 1, 8, 9000, 700)])
def test_head_kernel_helpers_match_solo(L, dtype, B, nh, S, k):
    """Helpers of the one-head-per-workgroup kernel against the solo heads:
    the same index sets, outputs equal up to fp32 summation order and
    bit-identical from launch to launch."""
    wl = _small(dtype, B=B, Hq=nh, Hkv=nh, S=S, k=k)
    x = W.generate(wl)
    dev = H.upload(wl, x)
    ws = L.empty_workspace(dev["desc"], wl.d, wl.k)
    out_solo, idx_solo = _decode_with(L, wl, dev, L.FLAG_NO_HELPERS, ws)
    first = None
    for rep in range(3):
        out, idx = _decode_with(L, wl, dev, 0, ws)
        assert np.array_equal(idx, idx_solo)
        assert H.rel_err_rows(out, out_solo).max() < 1e-5
        if first is None:
            first = out
        else:
            assert np.array_equal(out, first), f"launch {rep} differs from launch 0"
    res = H.full_parity(wl, x, out, idx)
    H.log(f"  head helpers {dtype}: {res}")


def test_launch_plan(L):
    """Which workloads take the one-launch kernel."""
    expect = {"single_head_f32": True, "llama2_7b_f16": True, "llama2_13b_f16": True,
              "long_context_bf16": True, "gqa_llama3_8b_bf16": True}
    for name, one in expect.items():
        wl = W.get(name)
        desc = H.make_desc(wl, 32)
        assert L.decode_plan(desc, wl.d, wl.k, wl.append) == one, name
        assert not L.decode_plan(desc.with_flags(L.FLAG_SEPARATE_KERNELS), wl.d, wl.k)
    wl = _small("f16", S=3000, k=300)
    assert not L.decode_plan(H.make_desc(wl, 32), 20, 300)      # d != dp
    assert L.decode_plan(H.make_desc(wl, 32), 32, 300, True)    # append: the same kernel


def _decode_append_check(L, wl, separate, selected=False):
    x = W.generate(wl)
    P = x["P"].astype(np.float64)
    qf = W.from_storage(x["q"], wl.dtype)[:, ::wl.g]          # first query of each group
    qr = np.einsum("bhi,hij->bhj", qf, P)
    if selected:
        # the new key along that query: its score is the largest of the row,
        # so the attention gathers the appended row
        x["k_new"] = W.to_storage(2.0 * qf, wl.dtype)
    # stale contents in row S-1 of both caches (a key scoring far below every
    # other token, large values): reading the row before the append shows in
    # the selection or the output
    xs = dict(x, krot=x["krot"].copy(), v=x["v"].copy())
    xs["krot"][:, :, wl.S - 1] = W.to_storage(-8.0 * np.sign(qr), wl.dtype)
    xs["v"][:, :, wl.S - 1] = W.to_storage(np.full((wl.B, wl.Hkv, wl.D), 50.0), wl.dtype)
    dev = H.upload(wl, xs)
    out, idx = H.run_decode(wl, dev, separate=separate)
    res = H.full_parity(wl, x, out, idx)
    H.log(f"  {res}")
    rows = L.unpack_kcache(dev["kcache"], wl.capacity, dev["desc"].with_seq_len(wl.capacity))
    torch.cuda.synchronize()
    _check_appended(wl.dtype, x, H.to_host(rows, wl.dtype), H.to_host(dev["v"], wl.dtype),
                    wl.S - 1)


@pytest.mark.parametrize("separate", [False, True], ids=["default", "separate"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_decode_append_end_to_end(L, dtype, separate):
    wl = _small(dtype, S=2600, S_cap=3000, k=333, append=True, heavy_frac=0.02)
    H.log(f"decode_append {dtype} separate={separate}")
    _decode_append_check(L, wl, separate)


@pytest.mark.parametrize("separate", [False, True], ids=["default", "separate"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_append_head_dim_96(L, dtype, separate):
    wl = _small(dtype, D=96, S=3100, S_cap=3200, k=300, append=True)
    H.log(f"decode_append D=96 {dtype} separate={separate}")
    _decode_append_check(L, wl, separate, selected=True)


@pytest.mark.parametrize("separate", [False, True], ids=["default", "separate"])
def test_decode_append_grouped_heads(L, separate):
    """An appending step of grouped heads (g = 4, S above the limit of the
    one-workgroup-per-(b, kv) kernel: the per-head kernel by default), with a
    new key certain to be selected."""
    wl = _small("bf16", B=2, Hq=8, Hkv=2, S=4500, S_cap=4600, k=600, append=True,
                heavy_frac=0.02)
    H.log(f"decode_append grouped heads separate={separate}")
    _decode_append_check(L, wl, separate, selected=True)


def test_decode_append_grouped_heads_wide_tiles(L):
    """The separate path's appending step with grouped heads in its widest
    score tiles: g = 4 and 128 (b, kv) units of 8195 tokens give 2048-token
    tiles of the rotating score kernel (S * units / 1024 above 1024 tokens),
    four whole tiles and a 3-token tail (S not a multiple of 4), and the
    new key certain to be selected."""
    wl = _small("bf16", B=16, Hq=32, Hkv=8, S=8195, S_cap=8200, k=800, append=True)
    H.log("decode_append grouped heads, 2048-token score tiles (separate)")
    _decode_append_check(L, wl, True, selected=True)


# One-launch appends: the new token's score enters the selection in the first
# panel batch or after it (512 threads: 1024 tokens per batch, 256 threads:
# 512), with helper workgroups, through the large-k selection, in GQA groups,
# and at the smallest sizes.
APPEND_FUSED = {
    "g1-512-past-first-batch": dict(dtype="f16", B=2, Hq=4, Hkv=4, S=1025, S_cap=1100, k=100),
    "g1-512-in-first-batch": dict(dtype="f16", B=2, Hq=4, Hkv=4, S=1024, S_cap=1100, k=100),
    "g1-512-selected": dict(dtype="f16", B=2, Hq=4, Hkv=4, S=1500, S_cap=1500, k=100,
                            selected=True),
    "g1-256-helpers": dict(dtype="bf16", B=8, Hq=40, Hkv=40, S=513, S_cap=600, k=300),
    "g1-256-helpers-selected": dict(dtype="bf16", B=8, Hq=40, Hkv=40, S=900, S_cap=900, k=300,
                                    selected=True),
    "g1-256-large-k": dict(dtype="f16", B=8, Hq=40, Hkv=40, S=2000, S_cap=2048, k=600,
                           selected=True),
    "g2-f32": dict(dtype="f32", B=2, Hq=8, Hkv=4, S=700, S_cap=800, k=64, selected=True),
    "g4-bf16": dict(dtype="bf16", B=2, Hq=16, Hkv=4, S=1800, S_cap=1800, k=200),
    "g4-bf16-selected": dict(dtype="bf16", B=2, Hq=16, Hkv=4, S=1800, S_cap=1800, k=200,
                             selected=True),
    "S1": dict(dtype="f16", B=2, Hq=4, Hkv=4, S=1, S_cap=8, k=1),
    "k-eq-S": dict(dtype="f16", B=2, Hq=8, Hkv=4, S=300, S_cap=320, k=300),
}


@pytest.mark.parametrize("case", list(APPEND_FUSED), ids=list(APPEND_FUSED))
def test_decode_append_one_launch(L, case):
    kw = dict(APPEND_FUSED[case])
    selected = kw.pop("selected", False)
    wl = _small(append=True, **kw)
    desc = H.make_desc(wl, 32)
    assert L.decode_plan(desc, wl.d, wl.k, True), f"{case} is meant to take the one-launch kernel"
    H.log(f"decode_append one launch {case}: {W.describe(wl)}")
    _decode_append_check(L, wl, separate=False, selected=selected)


def test_softmax_scale_argument(L):
    wl = _small("f16", S=900, k=90)
    x = W.generate(wl)
    dev = H.upload(wl, x)
    dev["desc"] = H.make_desc(wl, 32, scale=0.3)
    out, idx = H.run_decode(wl, dev)
    ref = oracle.attend_given(x["q"], x["krot"], x["v"], x["P"], idx, "f16", scale=0.3)
    assert H.rel_err_rows(out, ref).max() < 2e-3


def test_zero_query_ties_to_first_tokens(L):
    wl = _small("f16", S=1000, k=100)
    x = W.generate(wl)
    x["q"][:] = 0
    dev = H.upload(wl, x)
    out, idx = H.run_decode(wl, dev)
    assert np.array_equal(idx, np.broadcast_to(np.arange(100, dtype=np.int32), idx.shape))
    ref = W.from_storage(x["v"], "f16")[:, :, :100].mean(axis=2)
    ref = np.repeat(ref, 2, axis=1)
    assert H.rel_err_rows(out, ref).max() < 1e-5


def test_repeat_runs_are_bit_identical(L):
    wl = _small("bf16", S=4096, k=512, B=4, Hq=8, Hkv=8)
    x = W.generate(wl)
    dev = H.upload(wl, x)
    o1, i1 = H.run_decode(wl, dev)
    for _ in range(5):
        o2, i2 = H.run_decode(wl, dev)
        assert np.array_equal(o1, o2) and np.array_equal(i1, i2)


# ------------------------------------------- helpers (one-launch path)

def _decode_with(L, wl, dev, flags, ws):
    desc = dev["desc"].with_flags(flags)
    idx = torch.full((wl.B, wl.Hq, wl.k), -7, dtype=torch.int32, device="cuda")
    out = L.decode(dev["q"], dev["kcache"], dev["v"], dev["P"], wl.d, wl.k, desc, idx_out=idx,
                   workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), idx.cpu().numpy()


@pytest.mark.parametrize("dtype,B,nh,S,k", [("f16", 12, 40, 2048, 512), ("bf16", 2, 4, 3000, 333),
                                            ("f32", 3, 8, 1500, 256)])
def test_helpers_match_solo_units(L, dtype, B, nh, S, k):
    """Units of a partial round shared with helper workgroups (12 x 40 units:
    32 helpers on 256 compute units; the smaller shapes: every unit paired):
    the solo path's index sets, its outputs up to fp32 summation order,
    bit-identical outputs from launch to launch on one workspace, oracle parity."""
    wl = _small(dtype, B=B, Hq=nh, Hkv=nh, S=S, k=k)
    x = W.generate(wl)
    dev = H.upload(wl, x)
    ws = L.empty_workspace(dev["desc"], wl.d, wl.k)
    out_solo, idx_solo = _decode_with(L, wl, dev, L.FLAG_NO_HELPERS, ws)
    first = None
    for rep in range(4):
        out, idx = _decode_with(L, wl, dev, 0, ws)
        assert np.array_equal(idx, idx_solo)
        assert H.rel_err_rows(out, out_solo).max() < 1e-5
        if first is None:
            first = out
        else:
            assert np.array_equal(out, first), f"launch {rep} differs from launch 0"
    res = H.full_parity(wl, x, out, idx)
    H.log(f"  helpers {dtype} B={B} heads={nh}: {res}")


@pytest.mark.parametrize("dtype,B,Hq,Hkv,S,k", [("f16", 4, 8, 8, 4096, 1024),
                                               ("bf16", 2, 8, 4, 2500, 250),
                                               ("f16", 3, 4, 4, 8000, 700),
                                               ("f32", 2, 4, 2, 1500, 200)])
def test_per_head_kernel_flag(L, dtype, B, Hq, Hkv, S, k):
    """Shapes the one-workgroup-per-(b, kv) kernel takes, run with
    LOKI_FLAG_PER_HEAD_KERNEL through the one-workgroup-per-head kernel (its
    8-, 16- and 32-key register variants): plan 2, the default plan's index
    sets, its outputs up to fp32 summation order, oracle parity."""
    wl = _small(dtype, B=B, Hq=Hq, Hkv=Hkv, S=S, k=k)
    x = W.generate(wl)
    dev = H.upload(wl, x)
    ws = L.empty_workspace(dev["desc"], wl.d, wl.k)
    flag = L.FLAG_PER_HEAD_KERNEL
    assert L.decode_kernel(dev["desc"].with_flags(flag), wl.d, wl.k) == 2
    out0, idx0 = _decode_with(L, wl, dev, 0, ws)
    out1, idx1 = _decode_with(L, wl, dev, flag, ws)
    assert np.array_equal(idx0, idx1)
    assert H.rel_err_rows(out1, out0).max() < 1e-5
    res = H.full_parity(wl, x, out1, idx1)
    H.log(f"  per-head flag {dtype} B={B} Hq={Hq} Hkv={Hkv} S={S}: {res}")


# A head and its helper share out the panel stream (default): each streams one
# half of the passes and the two hand their scores over through the
# workspace; a half not published in time is scored by the member needing it.
SHARED_CASES = {
    "bf16-20000-heavy": dict(dtype="bf16", B=2, Hq=8, Hkv=8, S=20000, k=2500, heavy_frac=0.02),
    "f16-512thr-ragged": dict(dtype="f16", B=1, Hq=8, Hkv=8, S=12345, k=1234),
    "bf16-32768-append": dict(dtype="bf16", B=1, Hq=8, Hkv=8, S=32768, S_cap=32768, k=4096,
                              append=True),
    "f16-d96-append": dict(dtype="f16", B=1, Hq=8, Hkv=8, D=96, S=9001, S_cap=9100, k=900,
                           append=True),
    "f32-lpt8": dict(dtype="f32", B=1, Hq=8, Hkv=8, S=6000, k=700, tau=20.0),
}


@pytest.mark.parametrize("case", list(SHARED_CASES), ids=list(SHARED_CASES))
def test_head_kernel_shared_stream(L, case):
    """The shared stream against each member streaming the whole panel, and
    against members that never wait for each other (every half that is late
    scored by the member needing it): the same index sets and outputs, bit
    for bit, launch after launch on one workspace; oracle parity."""
    kw = dict(SHARED_CASES[case])
    wl = _small(**kw)
    H.log(f"shared stream {case}: {W.describe(wl)}")
    x = W.generate(wl)
    dev = H.upload(wl, x)
    assert L.decode_plan(dev["desc"], wl.d, wl.k, wl.append)
    ws = L.empty_workspace(dev["desc"], wl.d, wl.k)

    def run(flags):
        desc = dev["desc"].with_flags(flags)
        idx = torch.full((wl.B, wl.Hq, wl.k), -7, dtype=torch.int32, device="cuda")
        if wl.append:
            out = L.decode_append(dev["q"], dev["k_new"], dev["v_new"], dev["kcache"], dev["v"],
                                  dev["P"], wl.d, wl.k, desc, idx_out=idx, workspace=ws)
        else:
            out = L.decode(dev["q"], dev["kcache"], dev["v"], dev["P"], wl.d, wl.k, desc,
                           idx_out=idx, workspace=ws)
        torch.cuda.synchronize()
        return out.cpu().numpy(), idx.cpu().numpy()

    ref_out, ref_idx = run(L.FLAG_NO_SHARED_STREAM)
    for flags in (0, 0, L.FLAG_SHARED_NO_WAIT, 0, L.FLAG_SHARED_NO_WAIT):
        out, idx = run(flags)
        assert np.array_equal(idx, ref_idx), f"flags {flags}: index sets differ"
        assert np.array_equal(out.view(np.uint32), ref_out.view(np.uint32)), \
            f"flags {flags}: outputs differ"
    H.log(f"  {H.full_parity(wl, x, out.astype(np.float64), idx)}")


@pytest.mark.parametrize("fill", ["random", "ones"])
def test_head_kernel_shared_stream_dirty_workspace(L, fill):
    """The hand-over flags need no initialisation: a workspace full of
    garbage (or of 0xff bytes) gives the clean workspace's results, bit for
    bit, from the first launch on."""
    wl = _small("bf16", B=2, Hq=8, Hkv=8, S=12000, k=1500)
    x = W.generate(wl)
    dev = H.upload(wl, x)
    out_c, idx_c = _decode_with(L, wl, dev, 0, L.empty_workspace(dev["desc"], wl.d, wl.k))
    n = L.workspace_bytes(dev["desc"], wl.d, wl.k)
    g = torch.Generator(device="cuda").manual_seed(11)
    ws = (torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=g)
          if fill == "random" else torch.full((n,), 255, dtype=torch.uint8, device="cuda"))
    for _ in range(2):
        out, idx = _decode_with(L, wl, dev, 0, ws)
        assert np.array_equal(idx, idx_c) and np.array_equal(out, out_c)
    H.log(f"  shared stream, dirty workspace ({fill}): {H.full_parity(wl, x, out, idx)}")


@pytest.mark.parametrize("fill", ["random", "ones"])
def test_helpers_with_dirty_workspace(L, fill):
    """The pair flags need no initialisation: a workspace full of garbage (or
    of 0xff bytes) gives correct results from the first launch on."""
    wl = _small("f16", B=2, Hq=8, Hkv=8, S=1500, k=300)
    x = W.generate(wl)
    dev = H.upload(wl, x)
    n = L.workspace_bytes(dev["desc"], wl.d, wl.k)
    g = torch.Generator(device="cuda").manual_seed(7)
    ws = (torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=g)
          if fill == "random" else torch.full((n,), 255, dtype=torch.uint8, device="cuda"))
    for _ in range(2):
        out, idx = _decode_with(L, wl, dev, 0, ws)
        res = H.full_parity(wl, x, out, idx)
    H.log(f"  dirty workspace ({fill}): {res}")


@pytest.mark.parametrize("separate", [False, True], ids=["default", "separate"])
def test_concurrent_streams_distinct_workspaces(L, separate):
    """Two streams (default priority), each with its own workspace and
    outputs, stepping at the same time over the same caches: the library keeps
    no state between calls beyond each workspace's launch tags, so every step
    equals the step run alone, bit for bit (12 x 40 units: helpers active)."""
    wl = _small("f16", B=12, Hq=40, Hkv=40, S=2048, k=512)
    x = W.generate(wl)
    dev = H.upload(wl, x)
    flags = L.FLAG_SEPARATE_KERNELS if separate else 0
    H.log(f"concurrent streams separate={separate}")
    ref_out, ref_idx = _decode_with(L, wl, dev, flags, L.empty_workspace(dev["desc"], wl.d, wl.k))
    desc = dev["desc"].with_flags(flags)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [L.empty_workspace(dev["desc"], wl.d, wl.k) for _ in streams]
    torch.cuda.synchronize()
    results = []
    for _ in range(6):
        for s, ws in zip(streams, wss):
            with torch.cuda.stream(s):
                idx = torch.full((wl.B, wl.Hq, wl.k), -7, dtype=torch.int32, device="cuda")
                out = L.decode(dev["q"], dev["kcache"], dev["v"], dev["P"], wl.d, wl.k, desc,
                               idx_out=idx, workspace=ws)
                results.append((out, idx))
    torch.cuda.synchronize()
    for n, (out, idx) in enumerate(results):
        assert np.array_equal(idx.cpu().numpy(), ref_idx), f"step {n}: index sets differ"
        assert np.array_equal(out.cpu().numpy().astype(np.float64), ref_out), f"step {n}: outputs differ"


# ------------------------------------------------ dense decode attention

@pytest.mark.parametrize("dtype,Hq,Hkv,S,D", [("f16", 4, 4, 3000, 128), ("bf16", 8, 2, 1111, 128),
                                             ("f32", 2, 2, 700, 128), ("f16", 4, 4, 1, 128),
                                             ("bf16", 4, 2, 2500, 96)])
def test_full_attention(L, dtype, Hq, Hkv, S, D):
    """Dense attention over every cached token: the oracle's decode with
    d = D, k = S (pinned to textbook softmax(q K^T / sqrt(D)) V)."""
    wl = _small(dtype, Hq=Hq, Hkv=Hkv, S=S, k=min(S, 300), d=min(S, 32), D=D)
    H.log(f"full attention {dtype} Hq={Hq} Hkv={Hkv} S={S}")
    x = W.generate(wl)
    dev = H.upload(wl, x)
    out = L.full_attention(dev["q"], dev["kcache"], dev["v"], dev["P"], dev["desc"])
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    ref = oracle.decode(x["q"], x["krot"], x["v"], x["P"], wl.D, S, dtype)["out"]
    assert H.rel_err_rows(out, ref).max() < H.OUT_TOL[dtype]


@pytest.mark.parametrize("dtype,B,Hq,Hkv,S", [("bf16", 2, 2, 1, 5000), ("f16", 1, 2, 2, 70000)])
def test_full_attention_many_splits(L, dtype, B, Hq, Hkv, S):
    """Dense attention whose rows are split into more partials than one
    batch of the merge (10 splits of 512 tokens) and than one block of it
    (137 splits: more than head_dim, ragged last batch)."""
    wl = _small(dtype, B=B, Hq=Hq, Hkv=Hkv, S=S, k=300, d=32)
    H.log(f"full attention {dtype} B={B} Hq={Hq} Hkv={Hkv} S={S}")
    x = W.generate(wl)
    dev = H.upload(wl, x)
    out = L.full_attention(dev["q"], dev["kcache"], dev["v"], dev["P"], dev["desc"])
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    ref = oracle.decode(x["q"], x["krot"], x["v"], x["P"], wl.D, S, dtype)["out"]
    err = H.rel_err_rows(out, ref)
    H.log(f"  max rel err {err.max():.3e}")
    assert err.max() < H.OUT_TOL[dtype]


# ----------------------------------------------------------------- PCAAttn

@pytest.mark.parametrize("dtype,Hq,Hkv,S,d,dp,D", [
    ("f16", 4, 4, 3000, 32, 32, 128), ("bf16", 8, 2, 2600, 20, 32, 128),
    ("f32", 2, 2, 1500, 48, 32, 128), ("f16", 4, 2, 700, 128, 32, 128),
    ("bf16", 2, 2, 513, 7, 16, 128), ("f16", 4, 4, 1100, 16, 16, 64),
    ("f16", 4, 2, 1700, 32, 32, 96)])
def test_pca_attention(L, dtype, Hq, Hkv, S, d, dp, D):
    """PCAAttn: softmax over all tokens of the scaled low-dimensional scores."""
    wl = _small(dtype, Hq=Hq, Hkv=Hkv, S=S, D=D, k=min(S, 300), d=min(d, 32))
    H.log(f"pca attention {dtype} Hq={Hq} Hkv={Hkv} S={S} d={d} dp={dp} D={D}")
    x = W.generate(wl)
    dev = H.upload(wl, x, dp)
    out = L.pca_attention(dev["q"], dev["kcache"], dev["v"], dev["P"], d, dev["desc"])
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    ref = oracle.pca_attention(x["q"], x["krot"], x["v"], x["P"], d, dtype)
    err = H.rel_err_rows(out, ref)
    H.log(f"  max rel err {err.max():.3e}")
    assert np.all(np.isfinite(out))
    assert err.max() < H.OUT_TOL[dtype]


def test_pca_attention_full_size(L):
    """Llama2-13B shape (the launch the bench times), sampled query heads."""
    wl = W.get("llama2_13b_f16")
    H.log("pca attention full size llama2_13b_f16")
    x = W.generate(wl)
    dev = H.upload(wl, x, wl.d)
    out = L.pca_attention(dev["q"], dev["kcache"], dev["v"], dev["P"], wl.d, dev["desc"])
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    heads = np.random.default_rng(5).choice(wl.B * wl.Hq, 48, replace=False)
    ref = oracle.pca_attention(x["q"], x["krot"], x["v"], x["P"], wl.d, wl.dtype, heads=heads)
    for u in heads:
        b, h = divmod(int(u), wl.Hq)
        assert H.rel_err_rows(out[b, h][None], ref[b, h][None]).max() < H.OUT_TOL[wl.dtype]
    assert np.all(np.isfinite(out))


# ------------------------------------------------------------- calibration

@pytest.mark.parametrize("dtype,Hkv,n,D,offset", [
    ("f16", 40, 8192, 128, 0.0), ("bf16", 3, 5000, 128, 3.0), ("f32", 2, 3000, 64, 1.0),
    ("f16", 2, 100, 128, 0.5), ("bf16", 3, 4000, 96, 1.0)])
def test_calibrate(L, dtype, Hkv, n, D, offset):
    """PCA of calibration keys on the GPU against the oracle's fp64 PCA."""
    wl = _small(dtype, Hq=Hkv, Hkv=Hkv, D=D, S=64, k=8)
    H.log(f"calibrate {dtype} Hkv={Hkv} n={n} D={D} offset={offset}")
    keys = np.stack([W.draw_keys(W.rng(0, wl.wid, 1, kv), n, W.basis(wl, kv), W.sigma(wl))
                     for kv in range(Hkv)]) + offset
    keys = W.to_storage(keys, dtype)
    desc = H.make_desc(wl, min(32, D))
    P, var = L.calibrate(H.to_device(keys, dtype), desc)
    torch.cuda.synchronize()
    P = P.cpu().numpy().astype(np.float64)
    var = var.cpu().numpy().astype(np.float64)
    Pr, vr = oracle.calibrate(keys, dtype)
    lam0 = vr[:, :1]
    # eigenvalues: fp32-level error relative to the largest
    assert np.all(np.abs(var - vr) <= 1e-5 * lam0), np.abs(var - vr).max()
    # eigenvectors, up to sign: a vector is fixed only as far as its eigenvalue
    # gap allows (perturbation of the matrix / gap)
    gap = np.minimum(np.abs(np.diff(vr, prepend=np.inf, axis=1)),
                     np.abs(np.diff(vr, append=-np.inf, axis=1)))
    err = np.minimum(np.linalg.norm(P - Pr, axis=1), np.linalg.norm(P + Pr, axis=1))
    tol = 1e-5 + 1e-5 * lam0 / np.maximum(gap, 1e-300)
    worst = np.unravel_index(np.argmax(err / tol), err.shape)
    H.log(f"  worst eigenvector err/tol {err[worst] / tol[worst]:.3f} at {worst}, "
          f"max eigenvalue err {np.abs(var - vr).max() / lam0.max():.2e}")
    assert np.all(err <= tol)
    # the GPU's own output: orthonormal columns, signs by the first largest entry
    for kv in range(Hkv):
        assert np.abs(P[kv].T @ P[kv] - np.eye(D)).max() < 1e-5
        lead = np.argmax(np.abs(P[kv]), axis=0)
        assert np.all(P[kv][lead, np.arange(D)] > 0)
        assert np.all(np.diff(var[kv]) <= 0)


# ------------------------------------------------------------- Exact-TopK

@pytest.mark.parametrize("dtype,g", [("f16", 1), ("bf16", 4)])
def test_exact_topk_full_panel(L, dtype, g):
    """The pages' Exact-TopK baseline: panel_dim = d = D, so the selection
    ranks the exact scores q . k_t and the attention reuses them."""
    wl = _small(dtype, B=2, Hq=4 * g if g > 1 else 4, Hkv=4, S=2500, k=300, d=128)
    H.log(f"exact top-k {dtype} g={g}")
    x = W.generate(wl)
    dev = H.upload(wl, x, dp=128)
    out, idx = H.run_decode(wl, dev)
    res = H.full_parity(wl, x, out, idx)
    H.log(f"  {res}")


# ---------------------------------------------------- the five workloads

@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_full_size(L, name):
    wl = W.get(name)
    H.log(f"workload {name}: generating")
    x = W.generate(wl)
    dev = H.upload(wl, x)
    H.log(f"workload {name}: decode on GPU (one launch: "
          f"{L.decode_plan(dev['desc'], wl.d, wl.k, wl.append)})")
    out, idx = H.run_decode(wl, dev)
    outs, idxs = None, None
    if not wl.append:  # the appending workload would append twice
        outs, idxs = H.run_decode(wl, dev, separate=True)
    del dev
    torch.cuda.empty_cache()
    H.log(f"workload {name}: oracle")
    res = H.full_parity(wl, x, out, idx)
    H.log(f"  {name}: {res}")
    if outs is not None:
        res = H.full_parity(wl, x, outs, idxs)
        H.log(f"  {name} (separate launches): {res}")


# ----------------------------------------------------- output dtype, score output

OUT16_CASES = {
    "one-launch-g1-helpers": dict(dtype="f16", B=2, Hq=4, Hkv=4, S=1500, k=300),
    "one-launch-g4": dict(dtype="bf16", B=2, Hq=16, Hkv=4, S=1800, k=200),
    "head-kernel-g2": dict(dtype="bf16", B=2, Hq=4, Hkv=2, S=6000, k=1100),
    "head-kernel-f32": dict(dtype="f32", B=2, Hq=4, Hkv=4, S=5000, k=300),
    "separate-split-k": dict(dtype="bf16", B=2, Hq=4, Hkv=2, S=6000, k=1100, separate=True),
    "separate-f32": dict(dtype="f32", B=2, Hq=4, Hkv=4, S=5000, k=300, separate=True),
    "append-one-launch": dict(dtype="f16", B=2, Hq=4, Hkv=4, S=1200, S_cap=1300, k=200,
                              append=True),
}
TORCH16 = {"f16": torch.float16, "bf16": torch.bfloat16}


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("odt", ["f16", "bf16"])
@pytest.mark.parametrize("case", list(OUT16_CASES), ids=list(OUT16_CASES))
def test_out_dtype(L, case, odt):
    """A 16-bit output is the fp32 output of the same step rounded once to
    nearest-even (torch's conversion), bit for bit."""
    kw = dict(OUT16_CASES[case])
    flags = L.FLAG_SEPARATE_KERNELS if kw.pop("separate", False) else 0
    wl = _small(**kw)
    H.log(f"out_dtype {odt} {case}: {W.describe(wl)}")
    x = W.generate(wl)
    outs = {}
    for name, dt in (("f32", L.F32), (odt, L.NAME_CODE[odt])):
        dev = H.upload(wl, x)   # fresh caches: the appending step rewrites row S-1
        desc = dev["desc"].with_out_dtype(dt).with_flags(flags)
        if wl.append:
            outs[name] = L.decode_append(dev["q"], dev["k_new"], dev["v_new"], dev["kcache"],
                                         dev["v"], dev["P"], wl.d, wl.k, desc)
        else:
            outs[name] = L.decode(dev["q"], dev["kcache"], dev["v"], dev["P"], wl.d, wl.k, desc)
    torch.cuda.synchronize()
    assert outs[odt].dtype == TORCH16[odt]
    assert torch.equal(_bits(outs[odt]), _bits(outs["f32"].to(TORCH16[odt])))


@pytest.mark.parametrize("odt", ["f16", "bf16"])
@pytest.mark.parametrize("which", ["full", "pca"])
def test_out_dtype_all_tokens(L, which, odt):
    wl = _small("bf16", B=2, Hq=8, Hkv=4, S=1700, k=100)
    x = W.generate(wl)
    dev = H.upload(wl, x)
    fn = (lambda desc: L.full_attention(dev["q"], dev["kcache"], dev["v"], dev["P"], desc)) \
        if which == "full" else \
        (lambda desc: L.pca_attention(dev["q"], dev["kcache"], dev["v"], dev["P"], wl.d, desc))
    o32 = fn(dev["desc"])
    o16 = fn(dev["desc"].with_out_dtype(L.NAME_CODE[odt]))
    torch.cuda.synchronize()
    assert torch.equal(_bits(o16), _bits(o32.to(TORCH16[odt])))


@pytest.mark.parametrize("append", [False, True], ids=["decode", "decode_append"])
def test_decode_scores_out(L, append):
    """scores_out holds the low-dimensional scores the selection ranked: the
    returned sets are exactly their top k (ties to the lower index), and they
    equal loki_score's on the same caches up to fp32 rounding (the step may
    rotate the query inside its score kernel, with another summation order)."""
    wl = _small("f16", B=2, Hq=8, Hkv=4, S=1500, S_cap=1600, k=150, append=append)
    x = W.generate(wl)
    dev = H.upload(wl, x)
    desc = dev["desc"]
    assert L.decode_plan(desc, wl.d, wl.k, append)   # one launch without scores_out
    sc = torch.full((wl.B, wl.Hq, wl.S), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((wl.B, wl.Hq, wl.k), -7, dtype=torch.int32, device="cuda")
    if append:
        out = L.decode_append(dev["q"], dev["k_new"], dev["v_new"], dev["kcache"], dev["v"],
                              dev["P"], wl.d, wl.k, desc, idx_out=idx, scores_out=sc)
    else:
        out = L.decode(dev["q"], dev["kcache"], dev["v"], dev["P"], wl.d, wl.k, desc,
                       idx_out=idx, scores_out=sc)
    qr = L.rotate_query(dev["q"], dev["P"], desc)
    s2 = L.score(qr, dev["kcache"], wl.d, desc)
    torch.cuda.synchronize()
    assert torch.isfinite(sc).all()
    scale = s2.abs().amax(dim=-1, keepdim=True)
    assert ((sc - s2).abs() <= 1e-5 * scale).all()
    s = sc.cpu().numpy().astype(np.float64)
    g = idx.cpu().numpy()
    for b in range(wl.B):
        for h in range(wl.Hq):
            assert np.array_equal(g[b, h], oracle.topk_rows(s[b, h][None], wl.k)[0])
    res = H.full_parity(wl, x, out.cpu().numpy().astype(np.float64), g)
    H.log(f"  scores_out {res}")


# ------------------------------------------------------------ graph capture

GRAPH_CASES = {
    "one-launch-g1": dict(dtype="f16", B=2, Hq=4, Hkv=4, S=1500, k=300),
    "head-kernel-pairs": dict(dtype="bf16", B=1, Hq=8, Hkv=8, S=12000, k=1500),
    "head-kernel-g4-append": dict(dtype="bf16", B=2, Hq=8, Hkv=2, S=6000, S_cap=6100, k=700,
                                  append=True),
    "one-launch-g4": dict(dtype="bf16", B=2, Hq=16, Hkv=4, S=1800, k=200),
    "separate-split-k": dict(dtype="bf16", B=2, Hq=4, Hkv=2, S=6000, k=1100, separate=True),
    "append-one-launch": dict(dtype="f16", B=2, Hq=4, Hkv=4, S=1200, S_cap=1300, k=200,
                              append=True),
}


@pytest.mark.parametrize("helpers", [True, False], ids=["helpers", "no-helpers"])
@pytest.mark.parametrize("case", list(GRAPH_CASES), ids=list(GRAPH_CASES))
def test_decode_graph_replay(L, case, helpers):
    """The step captured into a HIP graph (torch.cuda.CUDAGraph) and replayed
    several times, with eager work and synchronisations between the replays:
    every replay equals the eager step bit for bit.  A replay reuses the
    captured launch tag of the helper pairs; the second workgroup of a pair
    clears the pair's flag, so every replay pairs afresh."""
    kw = dict(GRAPH_CASES[case])
    flags = (L.FLAG_SEPARATE_KERNELS if kw.pop("separate", False) else 0) | \
        (0 if helpers else L.FLAG_NO_HELPERS)
    wl = _small(**kw)
    H.log(f"graph replay {case} helpers={helpers}: {W.describe(wl)}")
    x = W.generate(wl)
    dev = H.upload(wl, x)
    desc = dev["desc"].with_flags(flags)
    out = torch.empty((wl.B, wl.Hq, wl.D), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.B, wl.Hq, wl.k), dtype=torch.int32, device="cuda")
    ws = L.empty_workspace(desc, wl.d, wl.k)

    def step(stream=None):
        if wl.append:
            L.decode_append(dev["q"], dev["k_new"], dev["v_new"], dev["kcache"], dev["v"],
                            dev["P"], wl.d, wl.k, desc, out=out, idx_out=idx, workspace=ws,
                            stream=stream)
        else:
            L.decode(dev["q"], dev["kcache"], dev["v"], dev["P"], wl.d, wl.k, desc, out=out,
                     idx_out=idx, workspace=ws, stream=stream)

    step()
    torch.cuda.synchronize()
    out_e, idx_e = out.clone(), idx.clone()
    res = H.full_parity(wl, x, out_e.cpu().numpy().astype(np.float64), idx_e.cpu().numpy())
    H.log(f"  eager {res}")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)                      # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()                          # the capture stream is the current stream here
    for rep in range(4):
        out.fill_(float("nan"))
        idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out_e), f"replay {rep}: outputs differ"
        assert torch.equal(idx, idx_e), f"replay {rep}: index sets differ"
        # an eager step on the same workspace between replays (a fresh tag)
        out.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        assert torch.equal(out, out_e), f"eager step after replay {rep}: outputs differ"
