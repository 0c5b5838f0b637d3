"""The boundary as a C program sees it (no GPU): include/mq.h compiles as
strict C99 with warnings as errors, and a C program linked against libmq.so
gets the host-only answers (format tables, stride rule, launch plans, error
texts) without any device call."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "quantized_weight_prefill_q4_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "mq.h"

int main(void) {
    mq_gemm_plan_info p;
    int rc;
    if (mq_block_elems(MQ_Q4_K) != 256 || mq_block_bytes(MQ_Q4_K) != 144) return 1;
    if (mq_block_elems(MQ_Q8_0) != 32 || mq_block_bytes(MQ_Q6_K) != 210) return 2;
    if (mq_row_bytes(MQ_Q4_K, 3584) != 14 * 144) return 3;
    if (mq_f16cache_ld(4096) != 4160 || mq_f16cache_ld(3584) != 3584) return 4;
    if (mq_block_elems(5) != MQ_ERR_FORMAT) return 5;
    rc = mq_gemm_plan_query(0, 0, 2048, 18944, 3584, 0, &p);
    if (rc != MQ_OK || p.bm != 256 || p.bn != 256 || !p.has_kernel) return 6;
    if (p.dp_tiles != 512 || p.tail_tiles != 80 || p.split != 3) return 7;
    if (p.ws_bytes != mq_gemm_workspace_bytes(0, 2048, 18944, 3584, 0)) return 8;
    /* argument errors come back before any device work */
    if (mq_gemm_fused(MQ_Q4_K, 0, 256, 0, 0, 256, 64, 64, 256, 0, 0, 0, 0) != MQ_ERR_NULL) return 9;
    if (mq_dequant_to_f16(99, (void *)16, 1, 256, (uint16_t *)16, 256, 0) != MQ_ERR_FORMAT) return 10;
    if (strlen(mq_strerror(MQ_ERR_SCRATCH)) == 0) return 11;
    if (mq_gemm_fused_noalloc(MQ_Q4_K, (const uint16_t *)16, 3584, (const void *)16,
                              (float *)16, 18944, 2048, 18944, 3584, 16, 0) != MQ_ERR_SCRATCH)
        return 12;
    printf("ok\n");
    return 0;
}
"""


@pytest.fixture(scope="module")
def cc():
    c = shutil.which("gcc") or shutil.which("cc")
    if c is None:
        pytest.skip("no C compiler")
    return c


def test_header_is_strict_c99(cc, tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "mq.h"\nint main(void) { return MQ_OK; }\n')
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.join(ROOT, "include"), "-c", str(src), "-o",
                        str(tmp_path / "h.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_program_uses_the_host_side_of_the_library(cc, tmp_path):
    lib = os.path.join(PKG, "libmq.so")
    if not os.path.exists(lib):
        pytest.skip("libmq.so not built")
    src = tmp_path / "p.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "p"
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe), "-L", PKG, "-lmq", "-Wl,-rpath," + PKG],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
