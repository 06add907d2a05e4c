"""The product path has no CPU or oracle fallback: a copy of the package
without libbasp.so fails to import its binding, and no package module
imports the oracle (no GPU)."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sequence_re_layout_amd")


def test_binding_raises_without_the_library(tmp_path):
    dst = tmp_path / "sequence_re_layout_amd"
    shutil.copytree(PKG, dst, ignore=shutil.ignore_patterns("*.so", "*.so.*", "__pycache__"))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n"
            "    from sequence_re_layout_amd import binding\n"
            "except ImportError as e:\n"
            "    print('IMPORT ERROR:', e); sys.exit(0)\n"
            "print('imported'); sys.exit(1)\n" % str(tmp_path))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                         cwd=str(tmp_path))
    assert res.returncode == 0, res.stdout + res.stderr
    assert "libbasp.so" in res.stdout


def test_build_modules_import_before_a_build(tmp_path):
    """A fresh checkout has no libbasp.so: the build entry point must still
    reach the build module (and the inputs and workload tables), while the
    binding refuses to load."""
    dst = tmp_path / "sequence_re_layout_amd"
    shutil.copytree(PKG, dst, ignore=shutil.ignore_patterns("*.so", "*.so.*", "__pycache__"))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from sequence_re_layout_amd import build, inputs, workloads\n"
            "assert callable(build.build) and workloads.BY_NAME\n"
            "try:\n"
            "    from sequence_re_layout_amd import binding\n"
            "except ImportError:\n"
            "    print('OK'); sys.exit(0)\n"
            "sys.exit(1)\n" % str(tmp_path))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                         cwd=str(tmp_path))
    assert res.returncode == 0 and "OK" in res.stdout, res.stdout + res.stderr


def test_package_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".cpp", ".hpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text and "oracle.c" not in text, f
