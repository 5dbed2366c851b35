"""The product path has one implementation, the HIP library: without libsage.so the
package refuses to run, and nothing in it reaches the CPU oracle."""
import os
import pathlib
import shutil
import subprocess
import sys

import pytest

PKG = pathlib.Path(__file__).resolve().parents[1] / "quantized_attention_04_amd"


def test_missing_library_raises(tmp_path):
    # a copy of the package's Python sources without the built library
    dst = tmp_path / "quantized_attention_04_amd"
    dst.mkdir()
    for f in PKG.glob("*.py"):
        shutil.copy(f, dst / f.name)
    code = ("import quantized_attention_04_amd as qa\n"
            "try:\n"
            "    qa.lib()\n"
            "except ImportError as e:\n"
            "    print('refused:', e)\n"
            "else:\n"
            "    raise SystemExit('loaded a library that was not built')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True, timeout=300,
                       env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode == 0, r.stderr
    assert "refused:" in r.stdout and "is missing" in r.stdout


def test_package_never_touches_the_oracle():
    for f in list(PKG.glob("*.py")) + list((PKG / "csrc").glob("*")):
        text = f.read_text(errors="ignore")
        assert "import oracle" not in text and "from oracle" not in text and "liboracle" not in text, f
