"""The header is plain C: a C11 program that includes it, links the library and
calls the host-only entry points (no GPU needed) builds and runs."""
import os
import shutil
import subprocess

import pytest

import mla_tree_verify_02_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mla_tree_verify_02_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "mla_tree_verify.h"

int main(void)
{
    mtv_shape s = {1, 16, 8, 65552, 262144};
    int splits = 0, chunk = 0, groups = 0;
    int rc = mtv_plan_query(&s, 256, &splits, &chunk, &groups);
    printf("plan %d %d %d %d\n", rc, splits, chunk, groups);
    mtv_shape bad = {1, 65, 8, 65552, 262144};
    printf("bad %d\n", mtv_plan_query(&bad, 256, &splits, &chunk, &groups));
    printf("null %d\n", mla_tree_verify(&s, NULL, NULL, NULL, NULL, NULL, 0.07f, NULL, NULL,
                                         NULL, 0, NULL));
    uint64_t* counts = NULL;
    printf("check %d\n", mtv_check_inputs(&s, NULL, NULL, NULL, counts, NULL));
    printf("text %s\n", mtv_status_string(MTV_ERR_SHAPE));
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_uses_the_header_and_library(tmp_path):
    M.load()  # raises if the library was not built
    src = tmp_path / "caller.c"
    exe = tmp_path / "caller"
    src.write_text(PROGRAM)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    str(src), "-o", str(exe), "-L", PKG, "-lmla_tree_verify",
                    "-Wl,-rpath," + PKG], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True,
                         timeout=120).stdout.splitlines()
    plan = M.plan_query(M.make_shape(1, 16, 8, 65552, 262144), 256)
    assert out[0] == f"plan 0 {plan['splits']} {plan['chunk']} {plan['row_groups']}"
    assert out[1] == "bad -2"
    assert out[2] == "null -1"
    assert out[3] == "check -1"
    assert out[4] == "text " + M.status_string(-2)
