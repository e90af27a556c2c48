"""The binding's ctypes structures have the C header's layout: a small C
program built against include/tree_attn.h prints the size and every field's
offset of each structure the binding passes by pointer, and they must match
ctypes' (a mismatch would make the library read or write the wrong fields
with no error)."""
import ctypes
import os
import shutil
import subprocess

import pytest

from prefix_tree_packed_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STRUCTS = {"ta_tree_desc": B._TreeDesc, "ta_attn_cfg": B._AttnCfg, "ta_plan_info": B._PlanInfo,
           "ta_pack_info": B._PackInfo, "ta_mlp_weights": B._MlpWeights}


def _c_layout(tmp_path):
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "tree_attn.h"', "int main(void) {"]
    for cname, cls in STRUCTS.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    got = {}
    for line in out.splitlines():
        name, field, value = line.split()
        got[(name, field)] = int(value)
    return got


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_ctypes_structures_match_the_header(tmp_path):
    c = _c_layout(tmp_path)
    for cname, cls in STRUCTS.items():
        assert c[(cname, "size")] == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert c[(cname, fname)] == getattr(cls, fname).offset, f"{cname}.{fname}"
