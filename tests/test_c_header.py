"""The public header compiles as strict C and agrees with the Python binding.

A small C program, compiled with gcc against include/csa2.h and linked with the built
libcsa2.so, prints the size and every field offset of the two argument structs and the
header's constants, and calls the entry points that need no GPU.  The Python binding's
ctypes structures and constants must match what the C compiler laid out.
"""
import os
import shutil
import subprocess

import pytest

import sparse_decode_attention_csa2_amd as csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RAGGED = [f[0] for f in csa2._Ragged._fields_]
DECODE = [f[0] for f in csa2._DecodeArgs._fields_]
CONSTS = {"CSA2_OK": csa2.OK, "CSA2_ERR_INVALID_ARG": csa2.ERR_INVALID_ARG,
          "CSA2_ERR_UNSUPPORTED": csa2.ERR_UNSUPPORTED, "CSA2_ERR_WORKSPACE_TOO_SMALL": csa2.ERR_WORKSPACE_TOO_SMALL,
          "CSA2_ERR_HIP": csa2.ERR_HIP, "CSA2_K_MAX": csa2.K_MAX, "CSA2_KEEP_MAX": csa2.KEEP_MAX,
          "CSA2_ROWS_PER_REQ_MAX": csa2.ROWS_PER_REQ_MAX, "CSA2_TOPK_ALL_MAX": csa2.TOPK_ALL_MAX,
          "CSA2_QP_BF16": csa2.QP_BF16, "CSA2_QP_MXFP8": csa2.QP_MXFP8, "CSA2_DECODE_EVENTS": csa2.DECODE_EVENTS,
          "CSA2_DQ_MAIN": csa2.DQ_MAIN, "CSA2_DQ_IDX": csa2.DQ_IDX, "CSA2_DQ_SWA": csa2.DQ_SWA}


def _program() -> str:
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "csa2.h"', "int main(void) {"]
    lines.append('  printf("sizeof ragged %zu\\n", sizeof(csa2_ragged));')
    lines.append('  printf("sizeof decode %zu\\n", sizeof(csa2_decode_args));')
    for f in RAGGED:
        lines.append(f'  printf("ragged {f} %zu\\n", offsetof(csa2_ragged, {f}));')
    for f in DECODE:
        lines.append(f'  printf("decode {f} %zu\\n", offsetof(csa2_decode_args, {f}));')
    for c in CONSTS:
        lines.append(f'  printf("const {c} %d\\n", (int)({c}));')
    lines += [
        '  printf("version %d\\n", (int)csa2_version());',
        '  printf("decode_null %d\\n", csa2_decode(NULL, NULL, 0, NULL));',
        '  printf("last_error_set %d\\n", csa2_last_error() != NULL && csa2_last_error()[0] != 0);',
        '  printf("ws_null %zu\\n", csa2_decode_workspace_size(NULL));',
        '  printf("status_ok %s\\n", csa2_status_string(CSA2_OK));',
        "  return 0;", "}"]
    return "\n".join(lines) + "\n"


@pytest.fixture(scope="module")
def c_output(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    if not os.path.exists(csa2.LIB_PATH):
        pytest.fail("libcsa2.so missing: build it first")
    d = tmp_path_factory.mktemp("cabi")
    src = d / "abi.c"
    exe = d / "abi"
    src.write_text(_program())
    libdir = os.path.dirname(csa2.LIB_PATH)
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           str(src), "-L", libdir, "-lcsa2", f"-Wl,-rpath,{libdir}", "-Wl,--allow-shlib-undefined", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, HIP_VISIBLE_DEVICES=os.environ.get("HIP_VISIBLE_DEVICES", ""))
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, env=env, timeout=120).stdout
    res = {}
    for line in out.splitlines():
        *key, val = line.split(" ")
        res[" ".join(key)] = val
    return res


def test_struct_layouts_match_the_binding(c_output):
    assert int(c_output["sizeof ragged"]) == csa2.ctypes.sizeof(csa2._Ragged)
    assert int(c_output["sizeof decode"]) == csa2.ctypes.sizeof(csa2._DecodeArgs)
    for f in RAGGED:
        assert int(c_output[f"ragged {f}"]) == getattr(csa2._Ragged, f).offset, f
    for f in DECODE:
        assert int(c_output[f"decode {f}"]) == getattr(csa2._DecodeArgs, f).offset, f


def test_constants_match_the_binding(c_output):
    for c, v in CONSTS.items():
        assert int(c_output[f"const {c}"]) == v, c


def test_entry_points_without_a_gpu(c_output):
    assert int(c_output["version"]) == csa2.version()
    assert int(c_output["decode_null"]) == csa2.ERR_INVALID_ARG
    assert c_output["last_error_set"] == "1"
    assert int(c_output["ws_null"]) == 0
    assert c_output["status_ok"] == "ok"
