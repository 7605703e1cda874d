"""The C ABI from a plain C program: include/muonh.h compiles as C99 with
warnings as errors, and a program linked against libmuonh.so creates and
queries plans and sees the documented host-side errors. No call here
reaches the HIP runtime (every call is a plan query or is rejected before
any device work), so this runs without a GPU."""
from __future__ import annotations

import shutil
import subprocess

import pytest

import orthogonalized_updates_amd as mh

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "muonh.h"

#define CHECK(c) do { if (!(c)) { printf("FAIL line %d: %s\n", __LINE__, #c); return 1; } } while (0)

int main(void) {
  CHECK(muonh_abi_version() == MUONH_ABI_VERSION);

  muonh_group_desc groups[2] = {{2048, 512, 3}, {300, 200, 2}};
  muonh_plan* plan = NULL;
  CHECK(muonh_plan_create(&plan, groups, 2, 0) == MUONH_OK);
  CHECK(plan != NULL);
  CHECK(muonh_plan_num_matrices(plan) == 5);
  CHECK(muonh_plan_num_params(plan) == 3LL * 2048 * 512 + 2LL * 300 * 200);
  CHECK(muonh_workspace_bytes(plan) > 0 && muonh_workspace_bytes(plan) % 256 == 0);

  /* host-side rejections: nothing is enqueued */
  uint32_t flags = 7u;
  CHECK(muonh_step_status(plan, NULL, 0, NULL, NULL) == MUONH_EINVAL);
  CHECK(muonh_step_status(plan, NULL, 0, NULL, &flags) == MUONH_EWORKSPACE);
  CHECK(flags == 7u);
  CHECK(strlen(muonh_last_error()) > 0);
  CHECK(muonh_step(plan, NULL, NULL, NULL, NULL, 0.02f, 0.95f, 5, NULL, 0, NULL) == MUONH_EINVAL);
  CHECK(muonh_read_update(plan, 5, NULL, NULL, 0, NULL) != MUONH_OK);

  /* W, G and M must not overlap: checked on host copies of the pointer
   * arrays (fake addresses, never dereferenced) */
  {
    const size_t bytes[5] = {2048u * 512u * 4u, 2048u * 512u * 4u, 2048u * 512u * 4u,
                             300u * 200u * 4u, 300u * 200u * 4u};
    char* base = (char*)(uintptr_t)((size_t)1 << 32);
    const void* w[5];
    const void* g[5];
    const void* m[5];
    size_t at = 0;
    int i;
    for (i = 0; i < 5; ++i) {
      w[i] = base + at;
      g[i] = base + ((size_t)1 << 30) + at;
      m[i] = base + ((size_t)2 << 30) + at;
      at += bytes[i];
    }
    CHECK(muonh_check_disjoint(plan, w, g, m) == MUONH_OK);
    CHECK(muonh_check_disjoint(plan, w, w, m) == MUONH_EALIAS);   /* G == W */
    CHECK(strstr(muonh_last_error(), "overlaps") != NULL);
    m[4] = (const char*)m[3] + 16;                                 /* overlapping M views */
    CHECK(muonh_check_disjoint(plan, w, g, m) == MUONH_EALIAS);
    CHECK(muonh_check_disjoint(NULL, w, g, m) == MUONH_EINVAL);
    CHECK(strcmp(muonh_status_string(MUONH_EALIAS), "unknown status") != 0);
  }
  muonh_plan_destroy(plan);

  muonh_plan* bad = NULL;
  muonh_group_desc zero = {0, 4, 1};
  CHECK(muonh_plan_create(&bad, &zero, 1, 0) == MUONH_ESHAPE && bad == NULL);
  CHECK(muonh_plan_create(&bad, groups, 1, MUONH_NS_FP32 | MUONH_NS_SPLIT_BF16) == MUONH_EINVAL);
  CHECK(strcmp(muonh_status_string(MUONH_OK), muonh_status_string(MUONH_EINVAL)) != 0);
  printf("c client ok\n");
  return 0;
}
"""


def test_header_and_library_work_from_c(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "client.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "client"
    lib_dir = mh.LIB_PATH.parent
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        f"-I{mh.HEADER_PATH.parent}", str(src), f"-L{lib_dir}", "-lmuonh",
                        f"-Wl,-rpath,{lib_dir}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c client ok" in r.stdout
