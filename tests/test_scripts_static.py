"""Static check of the driver scripts (bench.py, __graft_entry__.py): every
name a function reads that resolves to module scope must be defined there or
be a builtin.  Their GPU legs cannot run here, so a name left undefined in one
of them (a value computed in another function, say) would otherwise surface
only on a GPU.  Python's symtable does the scoping: names bound in enclosing
functions are free variables, everything else that is read and not bound
locally is looked up at module level."""
from __future__ import annotations

import builtins
import os
import subprocess
import symtable
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def undefined_globals(path):
    src = open(path).read()
    top = symtable.symtable(src, path, "exec")
    module_names = {s.get_name() for s in top.get_symbols() if s.is_assigned() or s.is_imported()}
    known = module_names | set(dir(builtins)) | {"__file__", "__name__", "__doc__"}
    missing = []

    def walk(table):
        for child in table.get_children():
            if child.get_type() == "function":
                for s in child.get_symbols():
                    if s.is_referenced() and s.is_global() and s.get_name() not in known:
                        missing.append(f"{child.get_name()}: {s.get_name()}")
            walk(child)

    walk(top)
    return missing


@pytest.mark.parametrize("script", ["bench.py", "__graft_entry__.py"])
def test_no_undefined_module_names(script):
    assert undefined_globals(os.path.join(ROOT, script)) == []


def test_the_check_sees_a_planted_mistake(tmp_path):
    p = tmp_path / "planted.py"
    p.write_text("X = 1\n\ndef f():\n    y = 2\n    return X + y\n\ndef g():\n    return y_from_f\n")
    assert undefined_globals(str(p)) == ["g: y_from_f"]


def test_bench_refuses_several_gpus():
    """bench.py --gpus 2 stops with a message before touching a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr
