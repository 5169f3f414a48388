"""The kernel-source hash that ties a committed traffic summary to the
sources it was measured on must not depend on where the checkout lives (the
same tree runs from another path on another machine)."""
import os
import shutil
import subprocess
import sys

from recsys_ultra_long_amd import profiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_source_hash_is_location_independent(tmp_path):
    for d in ("recsys_ultra_long_amd", "include"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__", "_build"))
    out = subprocess.run([sys.executable, "-m", "recsys_ultra_long_amd.profiling", "hash"], cwd=tmp_path,
                         env={**os.environ, "PYTHONPATH": str(tmp_path)}, capture_output=True, text=True,
                         check=True).stdout.strip()
    assert out == profiling.source_hash()

