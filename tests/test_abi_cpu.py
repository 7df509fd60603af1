"""The C-ABI library loads and validates arguments (CPU only: no kernel is launched).

Every call here fails validation before anything is enqueued, so no GPU is
touched; the compute paths are covered by the gpu-marked tests.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "loki.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(loki_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    import sparse_decode_attention_rotate_amd as loki
    return loki


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ["loki_decode", "loki_decode_append", "loki_append", "loki_rotate_query",
              "loki_score", "loki_topk", "loki_attend", "loki_pack_kcache", "loki_unpack_kcache",
              "loki_workspace_bytes", "loki_kcache_elems", "loki_strerror", "loki_last_error",
              "loki_decode_plan", "loki_full_attention", "loki_prefill", "loki_pca_attention",
              "loki_calibrate_workspace_bytes", "loki_calibrate"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    declared = _declared_functions()
    assert sorted(L.EXPORTS) == declared
    for n in declared:
        assert hasattr(L.lib, n)
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(loki_\w+)", out))
    assert set(declared) <= exported


def test_header_flags_match_binding(L):
    src = open(HEADER).read()
    flags = dict(re.findall(r"#define\s+LOKI_(FLAG_\w+)\s+(\d+)u", src))
    assert flags == {"FLAG_SEPARATE_KERNELS": "1", "FLAG_NO_HELPERS": "2",
                     "FLAG_NO_SHARED_STREAM": "4", "FLAG_SHARED_NO_WAIT": "8",
                     "FLAG_PER_HEAD_KERNEL": "16"}
    for name, v in flags.items():
        assert getattr(L, name) == int(v)


def _desc(L, **kw):
    base = dict(batch=2, n_q_heads=4, n_kv_heads=2, head_dim=128, seq_len=100,
                seq_capacity=128, panel_dim=32, dtype=L.F16)
    base.update(kw)
    return L.Desc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), -1), (dict(n_q_heads=3), -1), (dict(n_kv_heads=0), -1),
    (dict(head_dim=80), -2), (dict(head_dim=256), -2), (dict(dtype=7), -1),
    (dict(seq_len=0), -1), (dict(seq_capacity=50), -1), (dict(panel_dim=24), -1),
    (dict(panel_dim=4), -1), (dict(panel_dim=256), -1),
    (dict(n_q_heads=34, n_kv_heads=2), -2), (dict(out_dtype=3), -1), (dict(out_dtype=-1), -1),
])
def test_desc_validation(L, kw, code):
    n = ctypes.c_size_t()
    rc = L.lib.loki_workspace_bytes(ctypes.byref(_desc(L, **kw).c()), 32, 10, ctypes.byref(n))
    assert rc == code
    assert L.last_error() != ""
    assert L.strerror(rc) in ("invalid argument", "unsupported configuration")


def test_workspace_and_cache_sizes(L):
    d = _desc(L)
    assert L.kcache_elems(d) == 2 * 2 * 128 * 128
    ws = L.workspace_bytes(d, 32, 10)
    assert ws >= 8 * (128 + 100 + 10 + 10) * 4
    with pytest.raises(L.LokiError):
        L.workspace_bytes(d, 0, 10)
    with pytest.raises(L.LokiError):
        L.workspace_bytes(d, 32, 101)
    with pytest.raises(L.LokiError):
        L.workspace_bytes(d, 129, 10)
    assert L.workspace_bytes(d, 32, 300 if False else 100) > ws


def test_decode_rejects_bad_arguments_before_launch(L):
    d = _desc(L)
    cd = ctypes.byref(d.c())
    fake = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first
    odd = ctypes.c_void_p(0x10004)
    f = L.lib.loki_decode
    # null pointers
    assert f(None, fake, fake, fake, 32, 10, fake, None, None, cd, fake, 1 << 30, None) == -1
    assert f(fake, fake, fake, fake, 32, 10, None, None, None, cd, fake, 1 << 30, None) == -1
    # misaligned
    assert f(odd, fake, fake, fake, 32, 10, fake, None, None, cd, fake, 1 << 30, None) == -1
    assert "aligned" in L.last_error()
    # d, k domain
    assert f(fake, fake, fake, fake, 0, 10, fake, None, None, cd, fake, 1 << 30, None) == -1
    assert f(fake, fake, fake, fake, 129, 10, fake, None, None, cd, fake, 1 << 30, None) == -1
    assert f(fake, fake, fake, fake, 32, 0, fake, None, None, cd, fake, 1 << 30, None) == -1
    assert f(fake, fake, fake, fake, 32, 101, fake, None, None, cd, fake, 1 << 30, None) == -1
    # workspace too small
    assert f(fake, fake, fake, fake, 32, 10, fake, None, None, cd, fake, 16, None) == -3
    # scores_out misaligned
    assert f(fake, fake, fake, fake, 32, 10, fake, None, odd, cd, fake, 1 << 30, None) == -1
    assert "scores_out" in L.last_error()
    # desc null
    assert f(fake, fake, fake, fake, 32, 10, fake, None, None, None, fake, 1 << 30, None) == -1


def test_other_entry_points_validate(L):
    d = _desc(L)
    cd = ctypes.byref(d.c())
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10004)
    lib = L.lib
    assert lib.loki_append(fake, fake, fake, fake, fake, 128, cd, None) == -1   # pos >= S_cap
    assert lib.loki_append(fake, fake, fake, fake, fake, -1, cd, None) == -1
    assert lib.loki_append(None, fake, fake, fake, fake, 0, cd, None) == -1
    assert lib.loki_rotate_query(fake, None, fake, cd, None) == -1
    assert lib.loki_score(fake, fake, 0, fake, cd, None) == -1
    assert lib.loki_score(fake, fake, 129, fake, cd, None) == -1
    assert lib.loki_topk(fake, 0, fake, None, cd, None) == -1
    assert lib.loki_topk(fake, 101, fake, None, cd, None) == -1
    assert lib.loki_attend(fake, fake, fake, fake, None, 10, fake, cd, fake, 8, None) == -3
    assert lib.loki_pack_kcache(fake, 129, fake, cd, None) == -1
    assert lib.loki_unpack_kcache(fake, -1, fake, cd, None) == -1
    assert lib.loki_decode_append(fake, None, fake, fake, fake, fake, 32, 10, fake, None, None,
                                  cd, fake, 1 << 30, None) == -1
    fa = lib.loki_full_attention
    assert fa(fake, fake, fake, fake, None, cd, fake, 1 << 30, None) == -1  # out NULL
    assert fa(odd, fake, fake, fake, fake, cd, fake, 1 << 30, None) == -1   # misaligned q
    assert fa(fake, fake, fake, fake, fake, None, fake, 1 << 30, None) == -1  # desc NULL
    assert fa(fake, fake, fake, fake, fake, cd, fake, 16, None) == -3       # workspace
    pa = lib.loki_pca_attention
    assert pa(fake, fake, fake, fake, 0, fake, cd, fake, 1 << 30, None) == -1    # d = 0
    assert pa(fake, fake, fake, fake, 129, fake, cd, fake, 1 << 30, None) == -1  # d > D
    assert pa(fake, fake, fake, fake, 32, None, cd, fake, 1 << 30, None) == -1   # out NULL
    assert pa(fake, fake, fake, fake, 32, fake, cd, fake, 16, None) == -3        # workspace
    assert pa(fake, fake, fake, fake, 32, fake, None, fake, 1 << 30, None) == -1  # desc NULL
    nb = ctypes.c_size_t()
    assert lib.loki_calibrate_workspace_bytes(cd, 5000, ctypes.byref(nb)) == 0
    D, Hkv = d.head_dim, d.n_kv_heads
    assert nb.value >= Hkv * 3 * (D * D + D) * 4                        # 3 chunks of 2048 keys
    assert lib.loki_calibrate_workspace_bytes(cd, 0, ctypes.byref(nb)) == -1
    cal = lib.loki_calibrate
    assert cal(fake, 0, fake, None, cd, fake, 1 << 30, None) == -1      # n = 0
    assert cal(None, 10, fake, None, cd, fake, 1 << 30, None) == -1     # keys NULL
    assert cal(fake, 10, fake, odd, cd, fake, 1 << 30, None) == -1      # misaligned variances
    assert cal(fake, 5000, fake, None, cd, fake, 1024, None) == -3      # workspace
    pf = lib.loki_prefill
    assert pf(fake, None, 129, 0, fake, fake, None, cd, None) == -1     # past S_cap
    assert pf(fake, None, 100, 29, fake, fake, None, cd, None) == -1    # pos + n past S_cap
    assert pf(fake, None, -1, 0, fake, fake, None, cd, None) == -1
    assert pf(fake, None, 4, -1, fake, fake, None, cd, None) == -1
    assert pf(None, None, 4, 0, fake, fake, None, cd, None) == -1       # k_rows NULL
    assert pf(fake, fake, 4, 0, fake, fake, None, cd, None) == -1       # v_rows without vcache
    assert pf(fake, None, 4, 0, fake, odd, None, cd, None) == -1        # misaligned cache
    assert pf(fake, None, 4, 0, fake, fake, None, None, None) == -1     # desc NULL
    assert pf(fake, fake, 0, 128, fake, fake, fake, cd, None) == 0      # empty: nothing to do


def test_binding_has_no_cpu_path(L):
    """Product calls take device tensors only."""
    import torch
    d = _desc(L)
    q = torch.zeros((2, 4, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="device memory"):
        L.decode(q, q, q, q, 32, 10, d, workspace=torch.zeros(1), out=torch.zeros((2, 4, 128)))


@pytest.mark.parametrize("D", [64, 96, 128])
def test_head_dims_built(L, D):
    """head_dim 64, 96 and 128 are in the domain: sizing calls succeed."""
    n = ctypes.c_size_t()
    rc = L.lib.loki_workspace_bytes(ctypes.byref(_desc(L, head_dim=D).c()), 32, 10, ctypes.byref(n))
    assert rc == 0 and n.value > 0
    e = ctypes.c_size_t()
    assert L.lib.loki_kcache_elems(ctypes.byref(_desc(L, head_dim=D).c()), ctypes.byref(e)) == 0
    assert e.value == 2 * 2 * 128 * D
