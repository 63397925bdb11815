"""bench.py on the CPU: the multi-GPU refusal, the settle option, and a static
check that every name its functions read is bound (the GPU paths cannot run
here)."""
import ast
import builtins
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_settle_option_is_offered():
    r = subprocess.run([sys.executable, BENCH, "--help"], capture_output=True, text=True)
    assert r.returncode == 0
    assert "--settle-ms" in r.stdout


def _bound_names(fn):
    names = {a.arg for a in fn.args.args + fn.args.kwonlyargs}
    if fn.args.vararg:
        names.add(fn.args.vararg.arg)
    if fn.args.kwarg:
        names.add(fn.args.kwarg.arg)
    for node in ast.walk(fn):
        if isinstance(node, ast.Name) and isinstance(node.ctx, ast.Store):
            names.add(node.id)
        elif isinstance(node, (ast.FunctionDef, ast.Lambda)) and node is not fn:
            if isinstance(node, ast.FunctionDef):
                names.add(node.name)
            a = node.args
            names.update(x.arg for x in a.args + a.kwonlyargs)
            if a.vararg:
                names.add(a.vararg.arg)
        elif isinstance(node, (ast.Import, ast.ImportFrom)):
            names.update((x.asname or x.name).split(".")[0] for x in node.names)
        elif isinstance(node, ast.ExceptHandler) and node.name:
            names.add(node.name)
    return names


def test_no_unbound_names():
    tree = ast.parse(open(BENCH).read())
    module = set()
    for n in tree.body:
        if isinstance(n, (ast.FunctionDef, ast.ClassDef)):
            module.add(n.name)
        elif isinstance(n, ast.Assign):
            module.update(t.id for t in n.targets if isinstance(t, ast.Name))
        elif isinstance(n, (ast.Import, ast.ImportFrom)):
            module.update((x.asname or x.name).split(".")[0] for x in n.names)
    missing = []
    for fn in (n for n in tree.body if isinstance(n, ast.FunctionDef)):
        bound = _bound_names(fn) | module
        for node in ast.walk(fn):
            if (isinstance(node, ast.Name) and isinstance(node.ctx, ast.Load)
                    and node.id not in bound and not hasattr(builtins, node.id)):
                missing.append(f"{fn.name}:{node.lineno}:{node.id}")
    assert not missing, missing
