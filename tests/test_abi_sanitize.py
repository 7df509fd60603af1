"""Sanitizer tier for the C ABI's host code (CPU only, no GPU).

loki_api.hip is rebuilt with AddressSanitizer + UndefinedBehaviorSanitizer on
its host pass only (device code is built as usual) and linked, with the other
built kernel objects, into a small host program.  The program drives every
argument check the header documents: each descriptor field out of range,
missing and misaligned pointers for every entry point, workspaces and the
fixed no-alloc scratch too small.  None of these reaches a launch, so no GPU
is needed; any out-of-bounds access or undefined behaviour in the validation
code aborts the program.
"""
import glob
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_decode_attention_rotate_amd")
CSRC = os.path.join(PKG, "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]

DRIVER = r"""
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include "loki.h"
static loki_desc base() {
  loki_desc d;
  memset(&d, 0, sizeof d);
  d.batch = 2; d.n_q_heads = 4; d.n_kv_heads = 2; d.head_dim = 128; d.seq_len = 100;
  d.seq_capacity = 128; d.panel_dim = 32; d.dtype = LOKI_F16;
  return d;
}
int main() {
  int bad = 0;
  for (int c = -6; c <= 1; c++) if (!loki_strerror(c)) bad++;
  size_t n = 0;
  loki_desc d = base();
  if (loki_workspace_bytes(&d, 32, 10, &n) != LOKI_OK || n == 0) bad++;
  if (loki_kcache_elems(&d, &n) != LOKI_OK) bad++;
  struct { int field; int value; int code; } cases[] = {
    {0, 0, LOKI_EINVAL}, {1, 3, LOKI_EINVAL}, {2, 0, LOKI_EINVAL}, {3, 80, LOKI_EUNSUPPORTED},
    {4, 0, LOKI_EINVAL}, {5, 50, LOKI_EINVAL}, {6, 24, LOKI_EINVAL}, {7, 9, LOKI_EINVAL}};
  for (auto& c : cases) {
    loki_desc e = base();
    int32_t* f[] = {&e.batch, &e.n_q_heads, &e.n_kv_heads, &e.head_dim, &e.seq_len,
                    &e.seq_capacity, &e.panel_dim, &e.dtype};
    *f[c.field] = c.value;
    if (loki_workspace_bytes(&e, 32, 10, &n) != c.code || loki_last_error()[0] == 0) {
      printf("field %d value %d\n", c.field, c.value);
      bad++;
    }
  }
  if (loki_workspace_bytes(NULL, 32, 10, &n) != LOKI_EINVAL) bad++;
  if (loki_workspace_bytes(&d, 0, 10, &n) != LOKI_EINVAL) bad++;
  if (loki_workspace_bytes(&d, 32, 101, &n) != LOKI_EINVAL) bad++;
  alignas(16) static char buf[1 << 16];
  float* fb = (float*)buf;
  if (loki_decode(NULL, buf, buf, fb, 32, 10, buf, NULL, NULL, &d, buf, sizeof buf, NULL) != LOKI_EINVAL) bad++;
  if (loki_decode(buf + 4, buf, buf, fb, 32, 10, buf, NULL, NULL, &d, buf, sizeof buf, NULL) != LOKI_EINVAL) bad++;
  if (loki_decode(buf, buf, buf, fb, 32, 10, buf, NULL, NULL, &d, buf, 16, NULL) != LOKI_EWORKSPACE) bad++;
  if (loki_decode_append(buf, NULL, buf, buf, buf, fb, 32, 10, buf, NULL, NULL, &d, buf, sizeof buf, NULL) != LOKI_EINVAL) bad++;
  if (loki_attend(fb, buf, buf, NULL, NULL, 10, buf, &d, buf, sizeof buf, NULL) != LOKI_EINVAL) bad++;
  if (loki_topk(fb, 0, (int32_t*)buf, NULL, &d, NULL) != LOKI_EINVAL) bad++;
  if (loki_append(buf, buf, fb, buf, buf, 128, &d, NULL) != LOKI_EINVAL) bad++;
  if (loki_prefill(buf, NULL, 10, 120, fb, buf, NULL, &d, NULL) != LOKI_EINVAL) bad++;
  if (loki_pack_kcache(buf, 129, buf, &d, NULL) != LOKI_EINVAL) bad++;
  if (loki_calibrate(buf, 0, fb, NULL, &d, buf, sizeof buf, NULL) != LOKI_EINVAL) bad++;
  loki_desc big = base();
  big.batch = 64; big.n_q_heads = 64; big.n_kv_heads = 64; big.seq_len = 8192; big.seq_capacity = 8192;
  if (loki_decode_noalloc(buf, buf, buf, fb, 32, 8, buf, NULL, NULL, &big, NULL) != LOKI_EWORKSPACE) bad++;
  printf("%s %d\n", bad ? "FAIL" : "ok", bad);
  return bad ? 1 : 0;
}
"""


def test_abi_validation_under_host_sanitizers():
    objs = [o for o in glob.glob(os.path.join(PKG, "_build", "*.hip.o"))
            if not o.endswith("loki_api.hip.o")]
    if not objs:
        pytest.skip("kernel objects not built (run __graft_entry__.build())")
    d = tempfile.mkdtemp(prefix="abi_san_")
    api = os.path.join(d, "api_san.o")
    drv = os.path.join(d, "driver.cpp")
    exe = os.path.join(d, "abi_san")
    open(drv, "w").write(DRIVER)
    host_san = [f for s in SAN for f in ("-Xarch_host", s)]
    r = subprocess.run(["hipcc", "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                        *host_san, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
                        os.path.join(CSRC, "loki_api.hip"), "-o", api],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run(["g++", "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"), drv, api,
                        *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                        "-o", exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert r.stdout.strip().endswith("ok 0")
