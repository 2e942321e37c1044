"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every .hip source is compiled as for the library (gfx950 device code
included, untouched) with the sanitizers on the host pass only, linked into
a separate library, and driven by a C program that is itself sanitized.  The
program calls each entry point's argument validation -- every check returns
before any HIP call -- and the host-only helpers that write caller buffers
(Hilbert order, central region, shift schedule, memory token count), with
every host array allocated on the heap at exactly the size the header
states, so a read or write one element past it is reported.  Needs no GPU.
"""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "sparse_window_attention_amd", "csrc")

DRIVER = r"""
#include "basa.h"
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static int fails = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL line %d: %s\n", __LINE__, #c); ++fails; } } while (0)

/* heap arrays of exactly n entries: any access past them is reported */
static int32_t* arr(int n, const int32_t* v) {
  int32_t* a = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  memcpy(a, v, sizeof(int32_t) * (size_t)n);
  return a;
}

#define FAKE ((void*)(uintptr_t)0x7F0000000000ull)
#define AT(i) ((void*)((uintptr_t)0x7F0000000000ull + (uintptr_t)(i) * (1ull << 32)))

int main(void) {
  const int32_t g2v[2] = {128, 128}, p2v[2] = {8, 8}, w2v[2] = {16, 16}, s2v[2] = {8, 0};
  const int32_t g3v[3] = {21, 30, 52}, p3v[3] = {3, 5, 4}, w3v[3] = {7, 10, 13}, s3v[3] = {3, 5, 6};
  int32_t *g2 = arr(2, g2v), *p2 = arr(2, p2v), *w2 = arr(2, w2v), *s2 = arr(2, s2v);
  int32_t *g3 = arr(3, g3v), *p3 = arr(3, p3v), *w3 = arr(3, w3v), *s3 = arr(3, s3v);

  CHECK(basa_mem_tokens(2, g2, p2) == 256);
  CHECK(basa_mem_tokens(3, g3, p3) == 546);
  CHECK(basa_mem_tokens(4, g3, p3) == -1);
  CHECK(basa_mem_tokens(2, g2, NULL) == -1);

  int32_t* sh = (int32_t*)malloc(3 * sizeof(int32_t));
  for (int b = 0; b < 8; ++b) CHECK(basa_shift_for_block(b, BASA_SCHED_FOUR_PHASE, 3, w3, sh) == BASA_OK);
  CHECK(sh[0] == 3 && sh[1] == 5 && sh[2] == 6);
  CHECK(basa_shift_for_block(1, BASA_SCHED_ALTERNATE, 2, w2, sh) == BASA_OK && sh[0] == 8 && sh[1] == 8);
  CHECK(basa_shift_for_block(-1, 1, 2, w2, sh) == BASA_ERR_INVALID_ARG);
  CHECK(basa_shift_for_block(0, 9, 2, w2, sh) == BASA_ERR_INVALID_ARG);
  free(sh);

  for (int side = 1; side <= 128; side *= 2) {
    int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)(side * side));
    CHECK(basa_hilbert_order(side, order) == BASA_OK);
    free(order);
  }
  CHECK(basa_hilbert_order(6, FAKE) == BASA_ERR_INVALID_ARG);
  CHECK(basa_hilbert_order(4, NULL) == BASA_ERR_INVALID_ARG);

  const int32_t regions[][4] = {{8, 8, 2, 2}, {10, 12, 3, 4}, {7, 6, 2, 3}, {1, 9, 1, 1}, {128, 128, 8, 8}};
  for (int i = 0; i < 5; ++i) {
    const int32_t* r = regions[i];
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(r[2] * r[3]));
    CHECK(basa_center_region(r[0], r[1], r[2], r[3], idx) == BASA_OK);
    free(idx);
  }
  CHECK(basa_center_region(8, 8, 9, 1, FAKE) == BASA_ERR_INVALID_ARG);

  /* window attention: every validation error, 2-D and 3-D geometry arrays */
  void *q = AT(0), *k = AT(1), *v = AT(2), *km = AT(3), *vm = AT(4), *o = AT(5);
  CHECK(basa_window_attn(NULL, k, v, NULL, NULL, 0, o, 1, 2, 128, 2, g2, w2, s2, -1.f, 0.f, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);
  CHECK(basa_window_attn(q, k, v, km, NULL, 256, o, 1, 2, 128, 2, g2, w2, s2, -1.f, 0.f, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);
  CHECK(basa_window_attn(q, k, v, NULL, NULL, 5, o, 1, 2, 128, 2, g2, w2, s2, -1.f, 0.f, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);
  CHECK(basa_window_attn(q, k, v, NULL, NULL, 0, q, 1, 2, 128, 2, g2, w2, s2, -1.f, 0.f, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);
  CHECK(basa_window_attn(q, k, v, NULL, NULL, 0, o, 1, 2, 96, 2, g2, w2, s2, -1.f, 0.f, BASA_BF16, 0, NULL) == BASA_ERR_UNSUPPORTED);
  const int32_t wb3v[3] = {7, 10, 12};   /* 12 does not divide 52 */
  int32_t* wb3 = arr(3, wb3v);
  CHECK(basa_window_attn(q, k, v, NULL, NULL, 0, o, 1, 2, 128, 3, g3, wb3, s3, -1.f, 0.f, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);
  free(wb3);
  CHECK(basa_window_attn(q, k, v, NULL, NULL, 0, o, 1, 2, 128, 3, g3, w3, s3, 0.f / 0.f, 0.f, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);
  CHECK(basa_window_attn(q, k, v, NULL, NULL, 0, o, 0, 2, 128, 3, g3, w3, s3, -1.f, 0.f, BASA_BF16, 0, NULL) == BASA_OK);
  CHECK(basa_window_attn_fwd(q, k, v, NULL, NULL, 0, o, NULL, 1, 2, 128, 2, g2, w2, s2, -1.f, 0.f, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);

  CHECK(basa_pool_kv(k, v, NULL, vm, 1, 2, 128, 2, g2, p2, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);
  CHECK(basa_pool_kv(k, v, km, k, 1, 2, 128, 3, g3, p3, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);

  CHECK(basa_full_attn(q, k, v, o, 1, 1, 0, 128, -1.f, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);
  CHECK(basa_dense_attn(q, k, v, o, 1, 1, 64, 0, 128, -1.f, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);
  CHECK(basa_dense_attn(q, k, v, k, 1, 1, 64, 64, 128, -1.f, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);

  int32_t* idx1 = arr(1, g2v);
  CHECK(basa_gather_kv(k, v, NULL, 1, km, vm, 1, 2, 128, 64, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);
  CHECK(basa_curve_attn(q, k, v, NULL, NULL, 0, o, 1, 2, 128, 64, NULL, 16, 0, -1.f, 0.f, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);
  CHECK(basa_curve_attn(q, k, v, NULL, NULL, 0, o, 1, 2, 128, 64, (int32_t*)FAKE, 48, 0, -1.f, 0.f, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);
  free(idx1);

  /* backward: workspace size, argument errors, the scratch-array limit */
  CHECK(basa_window_attn_bwd_workspace(1, 24, 128, 2, g2, p2) > 0);
  CHECK(basa_window_attn_bwd_workspace(1, 24, 128, 3, g3, NULL) > 0);
  void *dout = AT(6), *lse = AT(7), *dq = AT(8), *dk = AT(9), *dv = AT(10), *ws = AT(11);
  CHECK(basa_window_attn_bwd(q, k, v, km, vm, o, dout, (const float*)lse, dq, dk, dv, ws, 16, 1, 24,
                             128, 2, g2, w2, s2, p2, -1.f, 0.f, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);
  CHECK(basa_window_attn_bwd(q, k, v, km, vm, o, dout, (const float*)lse, dq, dk, dv, ws, 1ll << 30, 1, 24,
                             128, 3, g3, w3, s3, NULL, -1.f, 0.f, BASA_BF16, 0, NULL) == BASA_ERR_INVALID_ARG);
  const int32_t gu[2] = {512, 512}, wu[2] = {32, 32};
  int32_t *gU = arr(2, gu), *wU = arr(2, wu);
  CHECK(basa_window_attn_bwd_noalloc(q, k, v, km, vm, o, dout, (const float*)lse, dq, dk, dv, 1, 24, 128,
                                     2, gU, wU, s2, p2, -1.f, 0.f, BASA_BF16, 0, NULL) != BASA_OK);
  CHECK(basa_calib_mfma(NULL, 1, 1, NULL) == BASA_ERR_INVALID_ARG);
  CHECK(strlen(basa_last_error()) > 0);
  CHECK(strcmp(basa_status_string(99), "unknown status") == 0);

  free(g2); free(p2); free(w2); free(s2); free(g3); free(p3); free(w3); free(s3); free(gU); free(wU);
  printf("%s\n", fails ? "FAILED" : "ok");
  return fails ? 1 : 0;
}
"""

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _tool(path):
    if not os.path.exists(path):
        pytest.skip(f"{path} not available")
    return path


@pytest.mark.slow
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    hipcc = _tool("/opt/rocm/bin/hipcc")
    clang = _tool("/opt/rocm/llvm/bin/clang")
    objs = []
    procs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = tmp_path / (os.path.basename(src) + ".o")
        objs.append(str(obj))
        procs.append(subprocess.Popen(
            [hipcc, "--offload-arch=gfx950", "-mcode-object-version=5", "-O1", "-g",
             "-std=c++17", "-fPIC", *SAN, "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", "-c", src,
             "-o", str(obj)],
            stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for pr in procs:
        out, _ = pr.communicate(timeout=600)
        assert pr.returncode == 0, out
    lib = tmp_path / "libbasa_san.so"
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-mcode-object-version=5", "-shared", "-fPIC",
                        *SAN, "-o", str(lib), *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    src = tmp_path / "driver.c"
    src.write_text(DRIVER)
    exe = tmp_path / "driver"
    r = subprocess.run([clang, "-std=c99", "-O1", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", f"-I{INCLUDE}", str(src), "-o", str(exe),
                        str(lib), f"-Wl,-rpath,{tmp_path}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    log = r.stdout + r.stderr
    assert "AddressSanitizer" not in log and "runtime error" not in log, log
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), log
