"""The CPU oracle and the HIP path share no code: the oracle includes only
system headers and never names the GPU package; the GPU package (kernels,
C ABI, binding, build script) never names the oracle; the input generator,
which both sides consume, imports neither; and bench.py imports the oracle only
inside its CPU-baseline and recall legs."""
import ast
import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "clustered_sparse_attention_kv_amd")


def read(p):
    with open(p) as f:
        return f.read()


def test_oracle_includes_only_system_headers_and_no_gpu_code():
    for p in glob.glob(os.path.join(ROOT, "oracle", "*.c")):
        for inc in re.findall(r'^\s*#\s*include\s*([<"].*?[>"])', read(p), re.M):
            assert inc.startswith("<"), (p, inc)
    for p in glob.glob(os.path.join(ROOT, "oracle", "*")):
        if os.path.isfile(p) and p.endswith((".c", ".py", ".h")):
            text = read(p)
            assert "clustered_sparse_attention_kv_amd" not in text and "csrc" not in text, p
            assert "kvcluster.h" not in text and "libkvcluster" not in text, p


def test_gpu_package_never_names_the_oracle():
    files = glob.glob(os.path.join(PKG, "*.py")) + glob.glob(os.path.join(PKG, "csrc", "*")) + \
        glob.glob(os.path.join(ROOT, "include", "*.h"))
    assert files
    for p in files:
        if os.path.isfile(p):
            text = read(p)
            assert not re.search(r"\boracle\b|orc_|liboracle", text), p


def test_input_generator_imports_neither_side():
    for p in glob.glob(os.path.join(ROOT, "synth", "*")):
        if os.path.isfile(p) and p.endswith((".c", ".py")):
            text = read(p)
            assert not re.search(r"\bimport oracle\b|from oracle|orc_|clustered_sparse_attention_kv_amd|kvcluster",
                                 text), p


def test_bench_imports_the_oracle_only_in_its_cpu_legs():
    tree = ast.parse(read(os.path.join(ROOT, "bench.py")))
    allowed = {"cpu_baseline", "recall_sample"}
    for node in ast.walk(tree):
        if isinstance(node, ast.FunctionDef):
            for sub in ast.walk(node):
                if isinstance(sub, (ast.Import, ast.ImportFrom)):
                    names = [a.name for a in sub.names] + ([sub.module] if isinstance(sub, ast.ImportFrom) else [])
                    if "oracle" in names:
                        assert node.name in allowed, node.name
    for node in tree.body:  # nothing at module level
        if isinstance(node, (ast.Import, ast.ImportFrom)):
            names = [a.name for a in node.names] + ([node.module] if isinstance(node, ast.ImportFrom) else [])
            assert "oracle" not in names
