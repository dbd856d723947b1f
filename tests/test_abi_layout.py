"""The ctypes mirrors of the C ABI structs match oscar.h field by field: a
small C program compiled against the header (gcc, host only) prints every
field's offset and each struct's size, and the mirrors must agree.  CPU only."""
import ctypes
import os
import shutil
import subprocess

import pytest

import bit_rotated_kv_attn_amd as hip

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STRUCTS = {"oscar_decode_args": hip.DecodeArgs, "oscar_demote_args": hip.DemoteArgs,
           "oscar_bf16_decode_args": hip.Bf16DecodeArgs}


@pytest.fixture(scope="module")
def c_layout(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "oscar.h"', "int main(void) {"]
    for cname, mirror in STRUCTS.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in mirror._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    d = tmp_path_factory.mktemp("abi")
    src, exe = d / "layout.c", d / "layout"
    src.write_text("\n".join(lines))
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    "-D__HIP_PLATFORM_AMD__", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    layout = {}
    for line in out:
        if line:
            parts = line.split()
            layout[tuple(parts[:-1])] = int(parts[-1])
    return layout


@pytest.mark.parametrize("cname", sorted(STRUCTS))
def test_mirror_matches_header(c_layout, cname):
    mirror = STRUCTS[cname]
    assert ctypes.sizeof(mirror) == c_layout[(cname, "size")]
    for f, _ in mirror._fields_:
        assert getattr(mirror, f).offset == c_layout[(cname, f)], f"{cname}.{f}"
