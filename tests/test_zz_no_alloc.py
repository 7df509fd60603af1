"""loki_decode_noalloc: the decode step with the library's fixed per-GPU
scratch in place of a caller's workspace, through the C ABI, against
loki_decode with a workspace on the same inputs.

Both run the same kernels on the same data, so the index sets must be equal
and the outputs equal bit for bit; each call is also checked against the
oracle by the parity rules.  Two calls in a row share the scratch, the second
with a smaller input, so whatever the first left there must not leak into the
second.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_decode_attention_rotate_amd as loki
    return loki


def _case(**kw):
    base = dict(B=2, Hq=4, Hkv=2, D=128, S=3000, d=32, k=300, dtype="f16", tau=40.0,
                n_calib=2048)
    base.update(kw)
    return W.custom(name="noalloc", wid=210, **base)


def _pair(L, wl, separate):
    """(out, idx) of loki_decode_noalloc and of loki_decode, same inputs."""
    x = W.generate(wl)
    dev = H.upload(wl, x)
    desc = dev["desc"].with_flags(L.FLAG_SEPARATE_KERNELS if separate else 0)
    cd = desc.c()
    vp = ctypes.c_void_p
    st = vp(torch.cuda.current_stream().cuda_stream)
    res = []
    for fn in ("noalloc", "workspace"):
        out = torch.full((wl.B, wl.Hq, wl.D), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((wl.B, wl.Hq, wl.k), -7, dtype=torch.int32, device="cuda")
        args = [vp(dev["q"].data_ptr()), vp(dev["kcache"].data_ptr()), vp(dev["v"].data_ptr()),
                vp(dev["P"].data_ptr()), wl.d, wl.k, vp(out.data_ptr()), vp(idx.data_ptr()),
                None, ctypes.byref(cd)]
        if fn == "noalloc":
            rc = L.lib.loki_decode_noalloc(*args, st)
        else:
            ws = L.empty_workspace(desc, wl.d, wl.k)
            rc = L.lib.loki_decode(*args, vp(ws.data_ptr()), ws.numel(), st)
        assert rc == 0, f"{fn}: {L.strerror(rc)} {L.last_error()}"
        torch.cuda.synchronize()
        res.append((out.cpu().numpy().astype(np.float64), idx.cpu().numpy()))
    return x, res


# pairs of calls in a row: a larger step, then a smaller one on the same scratch
SEQUENCES = {
    "one-launch": [dict(B=12, Hq=40, Hkv=40, S=2048, k=512), dict(B=2, Hq=4, Hkv=4, S=900, k=90)],
    "separate": [dict(dtype="bf16", B=2, Hq=8, Hkv=2, S=9000, k=1500),
                 dict(dtype="bf16", B=1, Hq=4, Hkv=1, S=5000, k=600)],
    "gqa-separate-f32": [dict(dtype="f32", B=2, Hq=8, Hkv=2, S=6000, k=700, tau=20.0),
                         dict(dtype="f32", B=1, Hq=2, Hkv=2, S=1500, k=100, tau=20.0)],
}


@pytest.mark.parametrize("separate", [False, True], ids=["default", "separate"])
@pytest.mark.parametrize("seq", list(SEQUENCES), ids=list(SEQUENCES))
def test_noalloc_matches_workspace_call(L, seq, separate):
    for n, kw in enumerate(SEQUENCES[seq]):
        wl = _case(**kw)
        H.log(f"noalloc {seq} call {n} separate={separate}: {W.describe(wl)}")
        x, ((o_n, i_n), (o_w, i_w)) = _pair(L, wl, separate)
        assert np.array_equal(i_n, i_w), f"call {n}: index sets differ"
        assert np.array_equal(o_n, o_w), f"call {n}: outputs differ"
        res = H.full_parity(wl, x, o_n, i_n)
        H.log(f"  {res}")


def test_noalloc_refuses_oversized_step(L):
    """A step whose workspace exceeds the fixed scratch is refused before any
    launch, with LOKI_EWORKSPACE, and leaves its outputs untouched."""
    wl = _case(B=64, Hq=64, Hkv=64, S=8192, k=8, dtype="f16")
    desc = H.make_desc(wl, 32)
    assert L.workspace_bytes(desc, wl.d, wl.k) > L.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((wl.B, wl.Hq, wl.D), dtype=torch.float16, device="cuda")
    out = torch.full((wl.B, wl.Hq, wl.D), 3.0, dtype=torch.float32, device="cuda")
    dummy = torch.zeros(16, dtype=torch.float16, device="cuda")
    vp = ctypes.c_void_p
    rc = L.lib.loki_decode_noalloc(vp(q.data_ptr()), vp(dummy.data_ptr()), vp(dummy.data_ptr()),
                                   vp(dummy.data_ptr()), wl.d, wl.k, vp(out.data_ptr()), None,
                                   None, ctypes.byref(desc.c()),
                                   vp(torch.cuda.current_stream().cuda_stream))
    assert rc == -3, L.strerror(rc)
    assert "scratch" in L.last_error()
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
