"""The C ABI from C (CPU only, no kernel is launched): include/fp8rl.h compiles as strict C99, and
a C program that takes the address of every declared function links against the built library
and gets the documented host-side results (version, workspace sizes, status strings, argument
validation statuses) through the C calling convention."""

import os
import re
import shutil
import subprocess

import pytest

from fp8_blockwise_quantization_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8rl.h")


def _declared():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(fp8rl_\w+)\s*\(", text)))


PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "fp8rl.h"

typedef void (*any_fn)(void);
static any_fn table[] = { %(table)s };

int main(void) {
  int n = (int)(sizeof(table) / sizeof(table[0]));
  for (int i = 0; i < n; ++i)
    if (!table[i]) return 10;
  /* host-only calls */
  printf("version %%d\n", fp8rl_version());
  printf("ws %%zu\n", fp8rl_workspace_bytes(FP8RL_OP_GROUPED_GEMM_FUSED_ACT, 32768, 1536, 2048, 128));
  printf("ws0 %%zu\n", fp8rl_workspace_bytes(FP8RL_OP_GEMM, 8192, 4096, 4096, 0));
  printf("str %%s\n", fp8rl_status_string(FP8RL_ERR_WORKSPACE));
  /* validation statuses (returned before any HIP call) */
  fp8rl_status s1 = fp8rl_gemm_w8a8_blockscaled(NULL, NULL, NULL, NULL, 64, 256, 256, NULL,
                                                FP8RL_OUT_BF16, 256, FP8RL_ACCUM_AUTO, NULL, 0,
                                                NULL);
  /* a fake, aligned device address: the shape check fails before anything is dereferenced */
  void* fake = (void*)(size_t)(1 << 20);
  fp8rl_status s2 = fp8rl_quant_weight_blk128((const uint16_t*)fake, 200, 256, 256,
                                              (uint8_t*)fake, 256, (float*)fake, NULL);
  fp8rl_status s3 = fp8rl_grouped_gemm_w8a8(NULL, NULL, NULL, NULL, NULL, 0, 64, 256, 256, NULL,
                                            FP8RL_OUT_BF16, FP8RL_ACCUM_AUTO, NULL, 0, NULL);
  printf("status %%d %%d %%d\n", (int)s1, (int)s2, (int)s3);
  printf("functions %%d\n", n);
  return 0;
}
"""


@pytest.fixture(scope="module")
def built(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lib = _lib.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("library not built")
    d = tmp_path_factory.mktemp("abi_c")
    names = _declared()
    src = d / "abi.c"
    src.write_text(PROGRAM % {"table": ", ".join(f"(any_fn){n}" for n in names)})
    exe = d / "abi"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-Wno-cast-function-type", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
           "-L", os.path.dirname(lib), "-l:" + os.path.basename(lib),
           "-Wl,-rpath," + os.path.dirname(lib)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe, names


def test_header_is_strict_c99_and_links(built):
    exe, names = built
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    out = dict(line.split(" ", 1) for line in res.stdout.strip().splitlines())
    assert int(out["functions"]) == len(names) == 23
    assert int(out["version"]) == _lib.lib().fp8rl_version()
    assert int(out["ws"]) == 4096 + 32768 * 2048 + 32768 * 16 * 4
    assert int(out["ws0"]) == 0
    assert out["str"] == "workspace too small"
    # NULL pointers, N not a multiple of 128, E < 1
    assert [int(v) for v in out["status"].split()] == [1, 2, 7]
