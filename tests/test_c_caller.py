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


# The same caller against a build of the host side (argument checks, planning, the path
# model) with AddressSanitizer, so that an out-of-bounds access in the library's host code
# stops the program. The kernels' objects are linked uninstrumented; no call here reaches a
# device. A second program passes one float where gqla_pick_path writes two, and must be
# stopped: it shows that an overrun inside the library is caught.
OVERRUN = r"""
#include <string.h>
#include "gqla.h"
int main(void) {
  gqla_dims d;
  int32_t path = -1;
  float est = 0.f;
  memset(&d, 0, sizeof d);
  d.batch = 32; d.num_heads = 32; d.num_groups = 8; d.latent_rank = 512; d.rope_dim = 64;
  d.nope_dim = 64; d.v_dim = 128; d.s_q = 1; d.block_size = 64; d.dtype = GQLA_BF16;
  return gqla_pick_path(&d, (int64_t)32 * 8192, 8192, &path, &est) == GQLA_OK ? 0 : 3;
}
"""


def _asan_runtime():
    import glob
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


@pytest.mark.skipif(not os.path.exists("/opt/rocm/llvm/bin/clang") or _asan_runtime() is None,
                    reason="needs ROCm's clang and its AddressSanitizer runtime")
def test_c_caller_with_host_code_under_address_sanitizer(tmp_path):
    from decode_attention_02_amd import build as B
    host_srcs = ["gqla_api.cpp", "path_model.cpp"]
    kernel_objs = [os.path.join(B.BUILD, os.path.basename(s) + ".o") for s in B.sources()
                   if os.path.basename(s) not in host_srcs]
    if not all(os.path.exists(o) for o in kernel_objs):
        pytest.skip("build the library first (its kernel objects are linked as they are)")
    objs = []
    for name in host_srcs:
        obj = str(tmp_path / (name + ".o"))
        cmd = [B.hipcc()] + B.COMMON + ["-O1", "-g", "-Xarch_host", "-fsanitize=address",
                                        "-Xarch_host", "-fno-omit-frame-pointer",
                                        "-c", os.path.join(B.CSRC, name), "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        objs.append(obj)
    lib = tmp_path / "libgqla.so"
    link = [B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", str(lib)] + objs + kernel_objs + \
        ["-Xarch_host", "-fsanitize=address", "-shared-libasan"]
    subprocess.run(link, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
               LD_LIBRARY_PATH=os.path.dirname(_asan_runtime()) + ":" + os.environ.get("LD_LIBRARY_PATH", ""))
    results = {}
    for name, text in (("caller", PROGRAM), ("overrun", OVERRUN)):
        src = tmp_path / f"{name}.c"
        src.write_text(text)
        exe = tmp_path / name
        cc = ["/opt/rocm/llvm/bin/clang", "-std=c11", "-g", "-fno-omit-frame-pointer", "-shared-libasan",
              "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe), "-L", str(tmp_path), "-lgqla",
              f"-Wl,-rpath,{tmp_path}"]
        cc.insert(3, "-fsanitize" + "=address")
        subprocess.run(cc, check=True, capture_output=True, text=True)
        results[name] = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    ok = results["caller"]
    assert ok.returncode == 0 and "c caller ok" in ok.stdout, ok.stdout + ok.stderr
    bad = results["overrun"]
    assert bad.returncode != 0 and "stack-buffer-overflow" in bad.stderr, bad.stderr[-2000:]
