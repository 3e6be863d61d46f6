"""bench.py's GPU-only legs (the backward, MXFP8 and persistent lines), smoke() and the
binding's device-side helpers cannot run here, so a name that one of them reads but never
binds would surface only on the GPU.  This walks each top-level function and method of those files and checks that every name it loads is bound in the function (argument,
assignment, loop or comprehension target, import, nested definition) or at module level."""
import ast
import builtins
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bound_in(node):
    names = set()
    for x in ast.walk(node):
        if isinstance(x, ast.Name) and isinstance(x.ctx, (ast.Store, ast.Del)):
            names.add(x.id)
        elif isinstance(x, (ast.FunctionDef, ast.AsyncFunctionDef, ast.Lambda)):
            a = x.args
            names.update(p.arg for p in a.posonlyargs + a.args + a.kwonlyargs)
            if a.vararg:
                names.add(a.vararg.arg)
            if a.kwarg:
                names.add(a.kwarg.arg)
            if not isinstance(x, ast.Lambda):
                names.add(x.name)
        elif isinstance(x, ast.ClassDef):
            names.add(x.name)
        elif isinstance(x, (ast.Import, ast.ImportFrom)):
            names.update((a.asname or a.name).split(".")[0] for a in x.names)
        elif isinstance(x, ast.ExceptHandler) and x.name:
            names.add(x.name)
    return names


FILES = ["bench.py", "__graft_entry__.py"] + sorted(
    os.path.join("mixture_experts_layer_histogram_amd", f)
    for f in os.listdir(os.path.join(ROOT, "mixture_experts_layer_histogram_amd")) if f.endswith(".py"))


@pytest.mark.parametrize("path", FILES)
def test_functions_bind_every_name_they_read(path):
    tree = ast.parse(open(os.path.join(ROOT, path)).read())
    module = set(dir(builtins))
    for n in tree.body:                  # top-level bindings only, not those inside functions
        if isinstance(n, (ast.FunctionDef, ast.ClassDef)):
            module.add(n.name)
        elif not isinstance(n, ast.AsyncFunctionDef):
            module |= _bound_in(n)
    unbound = []
    funcs = [n for n in tree.body if isinstance(n, ast.FunctionDef)]
    funcs += [m for c in tree.body if isinstance(c, ast.ClassDef) for m in c.body if isinstance(m, ast.FunctionDef)]
    for f in funcs:                      # a nested function reads its enclosing function's names
        local = _bound_in(f)
        for x in ast.walk(f):
            if isinstance(x, ast.Name) and isinstance(x.ctx, ast.Load) and x.id not in local | module:
                unbound.append(f"{f.name}:{x.lineno}:{x.id}")
    assert not unbound, unbound
