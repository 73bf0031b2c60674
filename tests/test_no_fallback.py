"""The product path has no fallback: without the built library the binding
refuses to import, and nothing in the package reaches the oracle."""
import ast
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "ternary_weight_linear_bitlinear_amd")


def test_binding_refuses_to_import_without_library(tmp_path):
    """A copy of the package without libbitlinear.so raises ImportError at
    import instead of falling back to anything else."""
    dst = tmp_path / "ternary_weight_linear_bitlinear_amd"
    dst.mkdir()
    for name in ("__init__.py", "bitlinear.py"):
        shutil.copy(os.path.join(PKG, name), dst / name)
    code = ("import sys\n"
            "try:\n"
            "    import ternary_weight_linear_bitlinear_amd.bitlinear\n"
            "except ImportError as e:\n"
            "    print('refused:', e)\n"
            "    sys.exit(0)\n"
            "sys.exit(3)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "no fallback" in r.stdout


def test_package_never_imports_the_oracle():
    """No module of the package imports the oracle (only tests, smoke() and
    the benchmark's CPU baseline may)."""
    for name in os.listdir(PKG):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(PKG, name)).read())
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            else:
                continue
            assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), (name, mods)


def test_binding_refuses_a_stale_library(tmp_path):
    """The library records a digest of the sources it was built from; a copy
    of the package whose kernel sources differ from the built library's
    refuses to import instead of running (and timing) the old code."""
    pkg = tmp_path / "ternary_weight_linear_bitlinear_amd"
    shutil.copytree(PKG, pkg, ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    code = ("import sys\n"
            "try:\n"
            "    import ternary_weight_linear_bitlinear_amd.bitlinear\n"
            "except ImportError as e:\n"
            "    print('refused:', e)\n"
            "    sys.exit(4)\n"
            "print('loaded')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "loaded" in r.stdout, r.stdout + r.stderr
    with open(pkg / "csrc" / "gemm.hip", "a") as f:
        f.write("\n// an edit after the build\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 4, r.stdout + r.stderr
    assert "built from other sources" in r.stdout
