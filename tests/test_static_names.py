"""Every name the Python files' functions read is defined somewhere: a local,
a parameter, an enclosing function's name, a module-level definition or
import, or a builtin.  The GPU tests only run on a GPU, so a stray name in
one (say, left behind by an edit of a neighbouring test) would otherwise
first show there; this finds it on the CPU."""
import builtins
import glob
import os
import symtable

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MODULES = sorted(glob.glob(os.path.join(ROOT, "tests", "*.py")) +
                 glob.glob(os.path.join(ROOT, "tests", "*", "*.py")) +
                 [os.path.join(ROOT, f) for f in (
                     "bench.py", "__graft_entry__.py", "kvgen/__init__.py", "oracle/__init__.py",
                     "fp8_kv_quantization_amd/__init__.py", "fp8_kv_quantization_amd/_build.py")])


def _undefined(path):
    src = open(path).read()
    top = symtable.symtable(src, path, "exec")
    module_names = {s.get_name() for s in top.get_symbols()
                    if s.is_assigned() or s.is_imported() or s.is_namespace()}
    known = module_names | set(dir(builtins)) | {"__file__", "__name__"}
    bad = []

    def walk(table):
        for child in table.get_children():
            for sym in child.get_symbols():
                if sym.is_referenced() and sym.is_global() and not sym.is_declared_global() \
                        and sym.get_name() not in known:
                    bad.append(f"{child.get_name()}:{sym.get_name()}")
            walk(child)

    walk(top)
    return bad


@pytest.mark.parametrize("path", MODULES, ids=[os.path.relpath(p, ROOT) for p in MODULES])
def test_no_undefined_names(path):
    assert _undefined(path) == []


def test_the_check_finds_a_stray_name(tmp_path):
    p = tmp_path / "m.py"
    p.write_text("import os\n\ndef f(a):\n    return os.sep + a + stray\n")
    assert _undefined(str(p)) == ["f:stray"]
