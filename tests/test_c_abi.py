"""The C ABI from a plain C caller: a C99 program (compiled with gcc
-pedantic -Werror) includes include/rope_kv_cache.h, links librkv.so and
calls the host-only entry points and the validation paths of the device
calls (null arguments, which return before any GPU work)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "rope_kv_cache_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "rope_kv_cache.h"

int main(void) {
  if (rkv_check_rope_capacity(4096, 4096) != RKV_OK) return 1;
  if (rkv_check_rope_capacity(4097, 4096) != RKV_ERR_CAPACITY) return 2;
  if (strstr(rkv_last_error(), "exceeds") == NULL) return 3;
  if (rkv_tokens_per_page() != 64) return 4;
  if (strcmp(rkv_status_string(RKV_ERR_ALIAS), "RKV_ERR_ALIAS") != 0) return 5;
  if (rkv_apply_rope_write_kv_packed_qkv(NULL, NULL, NULL, RKV_ROPE_NEOX, NULL) != RKV_ERR_NULL)
    return 6;
  if (rkv_dflash_target_kv_cache_update(NULL, NULL, NULL, NULL, NULL, NULL, NULL, -1, 1, 1, 128,
                                        128, 1, 1, RKV_ROPE_NEOX, NULL) != RKV_ERR_SHAPE)
    return 7;
  if (rkv_dflash_prepare_delta_metadata(NULL, NULL, 4, NULL, NULL, 0, NULL) != RKV_OK) return 8;
  if (rkv_dflash_build_linear_tree_metadata(NULL, NULL, 2, 8, NULL) != RKV_ERR_NULL) return 9;
  rkv_tensor t = {0};
  t.dtype = RKV_F8E4M3;
  if (rkv_apply_rope_write_kv_packed_qkv_qknorm(&t, &t, &t, NULL, NULL, 1e-6f, NULL, NULL,
                                                RKV_ROPE_GPTJ | RKV_ROUND_EXACT, NULL)
      != RKV_ERR_DTYPE)
    return 10;
  if (rkv_last_launch_groups_per_wave() != 0) return 11;   /* nothing was launched */
  printf("c abi ok\n");
  return 0;
}
"""


def test_c_caller(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "librkv.so")):
        pytest.skip("librkv.so is not built")
    src = tmp_path / "caller.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "caller"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src),
                    "-L", LIBDIR, "-lrkv", f"-Wl,-rpath,{LIBDIR}"], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    assert "c abi ok" in res.stdout
