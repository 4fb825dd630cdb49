"""Host-side checks that the product path has no fallback: without the built
library the binding refuses to import, and nothing in the package reaches the
oracle."""

import os
import re
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "segment_causal_dit_amd")


def test_binding_without_library_fails_loudly(tmp_path):
    dst = tmp_path / "segment_causal_dit_amd"
    dst.mkdir()
    for f in os.listdir(PKG):
        if f.endswith(".py"):
            shutil.copy(os.path.join(PKG, f), dst / f)
    assert not (dst / "libsegcausal.so").exists()
    # the binding loads on first use of an entry point
    code = "import segment_causal_dit_amd as sc; sc.segcausal_joint_attn"
    r = subprocess.run([sys.executable, "-c", code], cwd=str(tmp_path), capture_output=True, text=True,
                       env=dict(os.environ, PYTHONPATH=str(tmp_path)), timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "not built" in r.stderr


def test_package_never_reaches_the_oracle():
    pat = re.compile(r"^\s*(import|from)\s+oracle\b|\boracle\.", re.M)
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not pat.search(text), os.path.join(dirpath, f)
