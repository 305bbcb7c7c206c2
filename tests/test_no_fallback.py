"""Without the built HIP library the package refuses to import (there is no CPU
or PyTorch fallback), checked on a copy of the package in a fresh process."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_import_fails_without_library(tmp_path):
    pkg = os.path.join(ROOT, "decode_attention_08_amd")
    dst = tmp_path / "decode_attention_08_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    r = subprocess.run([sys.executable, "-c", "import decode_attention_08_amd"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "not built" in r.stderr
