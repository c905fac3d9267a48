"""The C ABI from a plain C caller: C99 programs (compiled with gcc
-pedantic -Werror) include include/rope_kv_cache.h and link librkv.so.
The first calls the host-only entry points and the validation paths of the
device calls (null arguments, which return before any GPU work).  The
second (GPU) allocates with the HIP runtime's C API, runs call 1 on a
quarter-turn table (cos 0, sin 1) and checks the exact result that the
rotation then has: each pair (x_u, x_v) becomes (-x_v, x_u), bit for bit,
in both arithmetic modes; V rows and untouched cache slots keep their bits."""
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


GPU_PROGRAM = r"""
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <hip/hip_runtime_api.h>
#include "rope_kv_cache.h"

#define HIPCHECK(x) do { if ((x) != hipSuccess) { fprintf(stderr, "hip error line %d\n", __LINE__); return 20; } } while (0)

static uint32_t lcg(uint32_t* s) { *s = *s * 1664525u + 1013904223u; return *s >> 8; }

/* a finite, nonzero fp16 value: biased exponent 1..29, random sign and mantissa */
static uint16_t rand_f16(uint32_t* s) {
  uint32_t r = lcg(s);
  return (uint16_t)((((r >> 5) & 1u) << 15) | ((1u + r % 29u) << 10) | ((r >> 6) & 0x3FFu));
}

enum { B = 2, S = 24, HQ = 3, HKV = 2, D = 128, R = 128, CAP = 40, H = HQ + 2 * HKV };
#define SENT 0x7E5A

static int run(int style) {
  const size_t nq = (size_t)B * S * H * D, nc = (size_t)B * 2 * HKV * CAP * D;
  uint16_t* in = malloc(nq * 2); uint16_t* out = malloc(nq * 2); uint16_t* cache = malloc(nc * 2);
  float* tab = malloc((size_t)S * R * 4);
  void *dq, *dc, *dt;
  size_t i;
  int b, s, h, d;
  uint32_t seed = 12345u + (uint32_t)style;
  rkv_status st;
  for (i = 0; i < nq; ++i) in[i] = rand_f16(&seed);
  for (i = 0; i < nc; ++i) cache[i] = SENT;
  for (s = 0; s < S; ++s)
    for (d = 0; d < R; ++d) tab[s * R + d] = d < R / 2 ? 0.0f : 1.0f;   /* cos 0, sin 1 */
  HIPCHECK(hipMalloc(&dq, nq * 2)); HIPCHECK(hipMalloc(&dc, nc * 2));
  HIPCHECK(hipMalloc(&dt, (size_t)S * R * 4));
  HIPCHECK(hipMemcpy(dq, in, nq * 2, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(dc, cache, nc * 2, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(dt, tab, (size_t)S * R * 4, hipMemcpyHostToDevice));
  {
    rkv_tensor tt = {0}, tq = {0}, tc = {0};
    tt.data = dt; tt.dtype = RKV_F32; tt.ndim = 3; tt.shape[0] = 1; tt.shape[1] = S; tt.shape[2] = R;
    tq.data = dq; tq.dtype = RKV_F16; tq.ndim = 4;
    tq.shape[0] = B; tq.shape[1] = S; tq.shape[2] = H; tq.shape[3] = D;
    tc.data = dc; tc.dtype = RKV_F16; tc.ndim = 5;
    tc.shape[0] = B; tc.shape[1] = 2; tc.shape[2] = HKV; tc.shape[3] = CAP; tc.shape[4] = D;
    st = rkv_apply_rope_write_kv_packed_qkv(&tt, &tq, &tc, style, NULL);
    if (st != RKV_OK) { fprintf(stderr, "%s: %s\n", rkv_status_string(st), rkv_last_error()); return 21; }
  }
  HIPCHECK(hipDeviceSynchronize());
  HIPCHECK(hipMemcpy(out, dq, nq * 2, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(cache, dc, nc * 2, hipMemcpyDeviceToHost));
  for (b = 0; b < B; ++b)
    for (s = 0; s < S; ++s)
      for (h = 0; h < H; ++h) {
        const uint16_t* x = in + (((size_t)b * S + s) * H + h) * D;
        const uint16_t* y = out + (((size_t)b * S + s) * H + h) * D;
        for (d = 0; d < D; ++d) {
          uint16_t want = x[d];
          if (h < HQ + HKV) {      /* rotated: (u, v) -> (-x_v, x_u) */
            int u = (style & 1) ? (d & ~1) : (d < R / 2 ? d : d - R / 2);
            int v = (style & 1) ? (d | 1) : u + R / 2;
            want = d == u ? (uint16_t)(x[v] ^ 0x8000u) : x[u];
          }
          if (y[d] != want) { fprintf(stderr, "qkv b%d s%d h%d d%d\n", b, s, h, d); return 30; }
        }
        if (h >= HQ) {             /* K rows (rotated, as in qkv) and V rows go to the cache */
          const int plane = h < HQ + HKV ? 0 : 1, kh = plane ? h - HQ - HKV : h - HQ;
          const uint16_t* c = cache + ((((size_t)b * 2 + plane) * HKV + kh) * CAP + s) * D;
          if (memcmp(c, y, D * 2) != 0) { fprintf(stderr, "cache b%d s%d h%d\n", b, s, h); return 31; }
        }
      }
  for (b = 0; b < B; ++b)          /* slots S..CAP-1 untouched */
    for (h = 0; h < 2 * HKV; ++h)
      for (s = S; s < CAP; ++s)
        for (d = 0; d < D; ++d)
          if (cache[(((size_t)b * 2 * HKV + h) * CAP + s) * D + d] != SENT) return 32;
  hipFree(dq); hipFree(dc); hipFree(dt);
  free(in); free(out); free(cache); free(tab);
  return 0;
}

int main(void) {
  const int styles[4] = {RKV_ROPE_NEOX, RKV_ROPE_GPTJ, RKV_ROPE_NEOX | RKV_ROUND_EXACT,
                         RKV_ROPE_GPTJ | RKV_ROUND_EXACT};
  int k, rc;
  for (k = 0; k < 4; ++k)
    if ((rc = run(styles[k])) != 0) { fprintf(stderr, "style %#x\n", styles[k]); return rc; }
  printf("c device ok\n");
  return 0;
}
"""


@pytest.mark.gpu
def test_c_caller_on_device(tmp_path):
    src = tmp_path / "device_caller.c"
    src.write_text(GPU_PROGRAM)
    exe = tmp_path / "device_caller"
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-D__HIP_PLATFORM_AMD__", "-isystem", os.path.join(rocm, "include"),
                    "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src),
                    "-L", LIBDIR, "-lrkv", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"],
                   check=True)
    print("[c-abi] running the C device caller", flush=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    assert "c device ok" in res.stdout
