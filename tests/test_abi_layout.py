"""The ctypes structures of the binding have the layout the C compiler gives
the structures of include/ringattn.h (sizes and every field's offset), so a
field added or moved on one side cannot silently shift the other (CPU only:
compiles a small C program with the host compiler)."""

import ctypes
import os
import shutil
import subprocess

import pytest

from context_attention_diffusion_ringattn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

STRUCTS = {
    "ringattn_shape": _lib.Shape,
    "ringattn_plan": _lib.Plan,
    "ringattn_cp_config": _lib.CpConfig,
    "ringattn_cp_share": _lib.CpShare,
}


def c_layout(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ringattn.h"', "int main(void) {"]
    for cname, py in STRUCTS.items():
        lines.append(f'    printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in py._fields_:
            lines.append(f'    printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    lines += ["    return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    table = {}
    for line in out.splitlines():
        name, field, value = line.split()
        table[(name, field)] = int(value)
    return table


def test_struct_layouts_match_the_header(tmp_path):
    table = c_layout(tmp_path)
    for cname, py in STRUCTS.items():
        assert table[(cname, "size")] == ctypes.sizeof(py), cname
        for field, _ in py._fields_:
            assert table[(cname, field)] == getattr(py, field).offset, f"{cname}.{field}"
