"""CPU check that the committed Python scripts name nothing unbound: every
name a function reads from the module scope is defined there or is a builtin
(a NameError on the GPU machine would otherwise show only when that line runs)."""
import builtins
import os
import symtable

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FILES = ["bench.py", "__graft_entry__.py", "gdn_inputs.py",
         os.path.join("gated_deltanet_recurrent_decode_amd", "__init__.py"),
         os.path.join("gated_deltanet_recurrent_decode_amd", "build.py"),
         os.path.join("oracle", "__init__.py")] + sorted(
    os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests")) if f.endswith(".py"))


def _unbound(path):
    src = open(path).read()
    top = symtable.symtable(src, path, "exec")
    module_names = {s.get_name() for s in top.get_symbols() if s.is_assigned() or s.is_imported()}
    module_names |= set(dir(builtins)) | {"__file__", "__name__", "__doc__"}
    missing = []

    def walk(t):
        for s in t.get_symbols():
            if s.is_global() and s.is_referenced() and s.get_name() not in module_names:
                missing.append(f"{t.get_name()}:{s.get_name()}")
        for c in t.get_children():
            walk(c)

    for c in top.get_children():
        walk(c)
    return missing


@pytest.mark.parametrize("name", FILES)
def test_no_unbound_names(name):
    assert _unbound(os.path.join(ROOT, name)) == []
