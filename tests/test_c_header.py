"""The C ABI from C: include/basa.h compiles as strict C99 and as C++17 with
warnings as errors, and a C program linked against the built library gets
the host-only helpers' values and the argument errors (fake device pointers
are never dereferenced: validation returns first).  Needs no GPU.
"""
import os
import shutil
import subprocess

import pytest

import sparse_window_attention_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

PROGRAM = r"""
#include "basa.h"
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static int fails = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL line %d: %s\n", __LINE__, #c); ++fails; } } while (0)

int main(void) {
  CHECK(basa_version() == 100);
  CHECK(strcmp(basa_status_string(BASA_OK), "") != 0);

  const int32_t grid2[2] = {128, 128}, pool2[2] = {8, 8};
  CHECK(basa_mem_tokens(2, grid2, pool2) == 256);
  const int32_t grid3[3] = {21, 30, 52}, pool3[3] = {3, 5, 4};
  CHECK(basa_mem_tokens(3, grid3, pool3) == 7 * 6 * 13);
  const int32_t bad_pool[2] = {7, 8};
  CHECK(basa_mem_tokens(2, grid2, bad_pool) == -1);

  const int32_t win[2] = {16, 16};
  int32_t sh[2] = {-1, -1};
  CHECK(basa_shift_for_block(1, BASA_SCHED_FOUR_PHASE, 2, win, sh) == BASA_OK);
  CHECK(sh[0] == 8 && sh[1] == 0);
  CHECK(basa_shift_for_block(3, BASA_SCHED_FOUR_PHASE, 2, win, sh) == BASA_OK);
  CHECK(sh[0] == 8 && sh[1] == 8);
  CHECK(basa_shift_for_block(1, 7, 2, win, sh) == BASA_ERR_INVALID_ARG);
  CHECK(strlen(basa_last_error()) > 0);

  int32_t order[16];
  CHECK(basa_hilbert_order(4, order) == BASA_OK);
  int seen[16] = {0};
  for (int i = 0; i < 16; ++i) if (order[i] >= 0 && order[i] < 16) seen[order[i]]++;
  for (int i = 0; i < 16; ++i) CHECK(seen[i] == 1);
  for (int i = 1; i < 16; ++i) {
    const int dy = order[i] / 4 - order[i - 1] / 4, dx = order[i] % 4 - order[i - 1] % 4;
    CHECK(dy * dy + dx * dx == 1);
  }
  CHECK(basa_hilbert_order(3, order) == BASA_ERR_INVALID_ARG);

  /* argument errors come back before anything touches the device */
  const int32_t shift[2] = {0, 0};
  CHECK(basa_window_attn(NULL, NULL, NULL, NULL, NULL, 0, NULL, 1, 1, 128, 2, grid2, win,
                         shift, -1.0f, 0.0f, BASA_BF16, BASA_LAYOUT_BHND, NULL)
        == BASA_ERR_INVALID_ARG);
  CHECK(basa_pool_kv(NULL, NULL, NULL, NULL, 1, 1, 128, 2, grid2, pool2, BASA_BF16,
                     BASA_LAYOUT_BHND, NULL) == BASA_ERR_INVALID_ARG);

  printf("%s\n", fails ? "FAILED" : "ok");
  return fails ? 1 : 0;
}
"""


def _compiler(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} not available")
    return path


def test_header_compiles_as_c_and_cpp(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "basa.h"\nint main(void) { return basa_version() == 100 ? 0 : 1; }\n')
    for cc, std in ((_compiler("gcc"), "-std=c99"), (_compiler("g++"), "-std=c++17")):
        lang = ["-x", "c++"] if cc.endswith("g++") else []
        r = subprocess.run([cc, *lang, std, "-Wall", "-Wextra", "-Werror", "-pedantic",
                            "-fsyntax-only", f"-I{INCLUDE}", str(src)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_c_program_against_the_library(tmp_path):
    lib = S.library_path
    if not os.path.exists(lib):
        pytest.skip("library not built")
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(lib)
    r = subprocess.run([_compiler("gcc"), "-std=c99", "-Wall", "-Wextra", "-Werror",
                        f"-I{INCLUDE}", str(src), "-o", str(exe), lib,
                        f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
