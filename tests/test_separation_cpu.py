"""The HIP path and the oracle stay apart, and the product fails loudly
without its library (CPU checks of the source tree).

* Nothing in the package (the binding, the build script, the HIP/C++
  sources) imports, includes or loads anything under ``oracle/``.
* The oracle and the input generator import nothing from the package.
* Importing the binding without ``libdflash.so`` raises instead of falling
  back to any other implementation.
"""

import os
import re
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_draft_select_amd")


def _files(top, exts):
    for dirpath, _, names in os.walk(top):
        if "_build" in dirpath or "__pycache__" in dirpath:
            continue
        for n in names:
            if n.endswith(exts):
                yield os.path.join(dirpath, n)


def test_package_never_reaches_the_oracle():
    py_import = re.compile(r"^\s*(import\s+oracle|from\s+oracle[\s.])", re.M)
    for p in _files(PKG, (".py",)):
        src = open(p).read()
        assert not py_import.search(src), p
        assert "oracle/" not in src and "oracle\\" not in src, p
    c_include = re.compile(r'#\s*include\s*[<"][^>"]*oracle', re.M)
    for p in _files(os.path.join(PKG, "csrc"), (".hip", ".hpp", ".cpp", ".h")):
        assert not c_include.search(open(p).read()), p


def test_oracle_and_generator_never_reach_the_package():
    pkg_import = re.compile(r"^\s*(import\s+block_draft_select_amd|from\s+block_draft_select_amd[\s.])", re.M)
    for top in ("oracle", "synth"):
        for p in _files(os.path.join(ROOT, top), (".py",)):
            src = open(p).read()
            assert not pkg_import.search(src), p
            assert "CDLL" not in src and "cdll" not in src, p  # no library loads
    for p in _files(os.path.join(ROOT, "synth"), (".py",)):
        assert not re.search(r"^\s*(import\s+oracle|from\s+oracle[\s.])", open(p).read(), re.M), p


def test_binding_without_library_raises(tmp_path):
    # a copy of the package without the built library
    dst = tmp_path / "block_draft_select_amd"
    dst.mkdir()
    for n in os.listdir(PKG):
        if n.endswith(".py"):
            shutil.copy(os.path.join(PKG, n), dst / n)
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n    import block_draft_select_amd\nexcept ImportError as e:\n    print('RAISED', e)\n"
            "else:\n    print('IMPORTED')\n") % str(tmp_path)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert "RAISED" in r.stdout and "libdflash.so" in r.stdout, r.stdout + r.stderr
