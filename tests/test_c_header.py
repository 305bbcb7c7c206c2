"""The boundary from plain C (no GPU needed): include/gqa_decode.h compiles as
C99 with warnings as errors, a C program links against libgqa_decode.so, and
the calls it makes (policies, workspace sizes, status strings and every
host-side refusal) behave as the header states.  Nothing here reaches a HIP
call: each refused call returns before any."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "decode_attention_08_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "gqa_decode.h"

#define CHECK(c) do { if (!(c)) { printf("failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void) {
  gqa_policy_t d, p;
  gqa_policy_default(&d);
  gqa_policy_pages(&p);
  CHECK(d.partition_size == 0 && p.partition_size == 512 && p.v1_max_ctx == 8192);
  CHECK(strncmp(gqa_status_string(GQA_OK), "GQA_OK", 6) == 0);
  CHECK(gqa_decode_workspace_size(4, 32, 8, 128, 200, &d) == 0);      /* nothing can split */
  CHECK(gqa_decode_workspace_size(4, 32, 8, 128, 4096, &d) > 0);
  CHECK(gqa_decode_workspace_size(4, 30, 8, 128, 4096, &d) == 0);     /* h_q % h_kv != 0 */

  /* fake, 256-byte aligned addresses: every call below is refused before any HIP call */
  char* a = (char*)0x100000;
  int32_t* bt = (int32_t*)0x200000;
  CHECK(gqa_decode(NULL, a, a, bt, bt, a, 2, 4, 8, 2, 128, 16, 0.1f, GQA_F16, a, 1 << 20, NULL, NULL)
        == GQA_ERR_NULL_PTR);
  CHECK(gqa_decode(a, a, a, bt, bt, a, 2, 4, 8, 3, 128, 16, 0.1f, GQA_F16, a, 1 << 20, NULL, NULL)
        == GQA_ERR_BAD_SHAPE);
  CHECK(gqa_decode(a, a, a, bt, bt, a, 2, 4, 8, 2, 96, 16, 0.1f, GQA_F16, a, 1 << 20, NULL, NULL)
        == GQA_ERR_UNSUPPORTED);
  CHECK(gqa_decode(a + 2, a, a, bt, bt, a, 2, 4, 8, 2, 128, 16, 0.1f, GQA_F16, a, 1 << 20, NULL,
                   NULL) == GQA_ERR_MISALIGNED);
  CHECK(gqa_decode(a, a, a, bt, bt, a, 2, 4096, 8, 2, 128, 16, 0.1f, GQA_F16, NULL, 0, &d, NULL)
        == GQA_ERR_WORKSPACE);
  gqa_policy_t bad = d;
  bad.flags = 64;
  CHECK(gqa_decode(a, a, a, bt, bt, a, 2, 4, 8, 2, 128, 16, 0.1f, GQA_F16, a, 1 << 20, &bad, NULL)
        == GQA_ERR_BAD_POLICY);
  CHECK(gqa_decode_contiguous(a, a, a, a, 2, 100, 8, 2, 128, 1.0f / 0.0f, GQA_BF16, a, 1 << 20,
                              NULL, NULL) == GQA_ERR_BAD_SCALE);
  CHECK(gqa_decode_xsplit(a, a, a, bt, bt, a, 0, 4, 8, 2, 128, 16, 0.1f, GQA_F16, NULL, 0, NULL,
                          NULL) == GQA_OK);                                /* nothing to do */
  gqa_policy_t fused = d;
  fused.flags = GQA_POLICY_FUSED_MERGE;
  CHECK(gqa_decode_noalloc(a, a, a, bt, bt, a, 2, 4, 8, 2, 128, 16, 0.1f, GQA_F16, &fused, NULL)
        == GQA_ERR_UNSUPPORTED);
  gqa_decode_args_t x;
  memset(&x, 0, sizeof x);
  x.layout = GQA_KV_PAGED;
  x.t_q = 0;
  CHECK(gqa_decode_ex(&x) == GQA_ERR_BAD_SHAPE);
  CHECK(gqa_decode_ex_workspace_size(&x) == 0);
  CHECK(GQA_NOALLOC_SCRATCH_BYTES == ((size_t)64 << 20));
  printf("ok\n");
  return 0;
}
"""


@pytest.fixture(scope="module")
def lib_built():
    if not os.path.exists(os.path.join(LIBDIR, "libgqa_decode.so")):
        import __graft_entry__
        __graft_entry__.build()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_is_c_and_refusals_from_c(tmp_path, lib_built):
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe),
           f"-L{LIBDIR}", "-lgqa_decode", f"-Wl,-rpath,{LIBDIR}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
