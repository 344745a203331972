"""The product path has no fallback: without librog.so the binding refuses to
load, loudly, and nothing under oracle/ is reachable from the package."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = "deterministic_collective_movement_amd"


def test_missing_library_fails_loudly(tmp_path):
    dst = tmp_path / PKG
    shutil.copytree(os.path.join(ROOT, PKG), dst,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n"
            "    import %s.rog\n"
            "except ImportError as e:\n"
            "    print('IMPORT-ERROR', e)\n"
            "else:\n"
            "    print('LOADED')\n") % (str(tmp_path), PKG)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                         cwd=str(tmp_path))
    assert "IMPORT-ERROR" in out.stdout and "librog.so is not built" in out.stdout, out.stdout + out.stderr


def test_package_never_imports_the_oracle():
    for dirpath, _, files in os.walk(os.path.join(ROOT, PKG)):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "rog_oracle" not in text, f


def test_oracle_never_includes_the_library():
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert ("import " + PKG) not in text and ("from " + PKG) not in text, f
            assert '#include "rog' not in text and "librog" not in text, f
