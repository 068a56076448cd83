"""The product path has no CPU fallback: importing the binding without its
built library raises ImportError naming the missing file."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = "fsdp_sharded_optimizer_flat_amd"


def test_import_without_library_raises(tmp_path):
    pkg = tmp_path / PKG
    pkg.mkdir()
    for f in os.listdir(os.path.join(ROOT, PKG)):
        if f.endswith(".py"):
            shutil.copy(os.path.join(ROOT, PKG, f), pkg / f)
    assert not (pkg / "libzero.so").exists()
    code = f"import sys; sys.path.insert(0, {str(tmp_path)!r}); import {PKG}"
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert res.returncode != 0
    assert "ImportError" in res.stderr and "libzero.so is missing" in res.stderr, res.stderr[-2000:]
