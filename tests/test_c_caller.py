"""The C ABI from a plain C caller: include/gqla.h compiles as strict C11, a program links
libgqla.so, and the host-only entry points and argument checks behave as declared. No GPU:
every call here returns before touching a device."""
import os
import shutil
import subprocess

import pytest

import decode_attention_02_amd as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "gqla.h"

#define CHECK(cond) do { if (!(cond)) { printf("FAIL line %d: %s\n", __LINE__, #cond); return 1; } } while (0)

int main(void) {
  gqla_dims d;
  gqla_paged p;
  int32_t n = -1, path = -1;
  size_t ws = 1;
  float est[2] = {0.f, 0.f};
  memset(&d, 0, sizeof d);
  memset(&p, 0, sizeof p);
  d.batch = 32; d.num_heads = 32; d.num_groups = 8; d.latent_rank = 512; d.rope_dim = 64;
  d.nope_dim = 64; d.v_dim = 128; d.s_q = 1; d.block_size = 64; d.dtype = GQLA_BF16;
  p.max_blocks_per_seq = 128; p.max_ctx_len = 8192; p.num_blocks = 4096; p.num_splits = 0;

  CHECK(strstr(gqla_version(), "gfx950") != NULL);
  CHECK(gqla_cache_bytes_per_token(&d, GQLA_PATH_ABSORB) == 576 * 2);
  CHECK(gqla_cache_bytes_per_token(&d, GQLA_PATH_GQA) == 2048 * 2);

  CHECK(gqla_num_splits(&d, &p, GQLA_PATH_ABSORB, &n) == GQLA_OK);
  CHECK(n >= 1 && n <= 128);
  CHECK(gqla_workspace_bytes(&d, &p, GQLA_PATH_ABSORB, &ws) == GQLA_OK);
  CHECK((n == 1) == (ws == 0));
  CHECK(gqla_pick_path(&d, (int64_t)32 * 8192, 8192, &path, est) == GQLA_OK);
  CHECK(path == GQLA_PATH_ABSORB || path == GQLA_PATH_GQA);
  CHECK(est[0] > 0.f && est[1] > 0.f);   /* est_us is float[2]: {absorb, gqa} */

  /* Invalid dims: rejected with a message before anything is launched (no device here). */
  d.num_groups = 5;
  CHECK(gqla_absorb_query(&d, NULL, NULL, NULL, NULL, NULL) == GQLA_ERR_INVALID_ARG);
  CHECK(strlen(gqla_last_error()) > 0);
  CHECK(gqla_num_splits(&d, &p, GQLA_PATH_GQA, &n) == GQLA_ERR_INVALID_ARG);
  CHECK(strcmp(gqla_status_string(GQLA_ERR_INVALID_ARG), gqla_status_string(GQLA_OK)) != 0);
  printf("c caller ok: %d splits, %zu workspace bytes, path %d\n", (int)n, ws, (int)path);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_plain_c_program_links_and_calls_the_abi(tmp_path):
    src = tmp_path / "caller.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "caller"
    lib_dir = os.path.dirname(G.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), "-L", lib_dir, "-lgqla", f"-Wl,-rpath,{lib_dir}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c caller ok" in r.stdout
