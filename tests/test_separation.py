"""The product and the oracle stay apart, and the product has no fallback
(CPU).

* No product source (the package's Python, its HIP/C++ sources, the public
  header) refers to the oracle, and no oracle source includes a product
  header or imports the product package.
* Neither shared library links the other; the oracle links no HIP runtime.
* The Python binding refuses to import when libggrms.so is missing, instead
  of computing anything some other way.
"""
import glob
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gated_group_rmsnorm_amd")


def _product_sources():
    pats = ["gated_group_rmsnorm_amd/*.py", "gated_group_rmsnorm_amd/csrc/*", "include/*"]
    return sorted(p for pat in pats for p in glob.glob(os.path.join(ROOT, pat)) if os.path.isfile(p))


def _oracle_sources():
    return sorted(p for ext in ("*.c", "*.h", "*.py")
                  for p in glob.glob(os.path.join(ROOT, "oracle", ext)))


def test_product_sources_do_not_refer_to_the_oracle():
    srcs = _product_sources()
    for name in ("ggrms_kernels.hpp", "ggrms_epilogue.hpp", "ggrms.h", "ggrms_tuning.h"):
        assert any(p.endswith(name) for p in srcs), name
    for p in srcs:
        text = open(p, errors="replace").read()
        assert not re.search(r"oracle", text, re.I), f"{os.path.relpath(p, ROOT)} mentions the oracle"


def test_oracle_sources_do_not_use_the_product():
    srcs = _oracle_sources()
    assert any(p.endswith("ggrms_oracle.c") for p in srcs)
    for p in srcs:
        text = open(p).read()
        for header in re.findall(r'#\s*include\s*[<"]([^>"]+)[>"]', text):
            assert header in ("math.h", "stdint.h", "string.h", "stddef.h", "ggrms_oracle.h"), \
                f"{os.path.relpath(p, ROOT)} includes {header}"
        assert "gated_group_rmsnorm_amd" not in text and "libggrms.so" not in text, p


def _needed(lib):
    out = subprocess.run(["readelf", "-d", lib], capture_output=True, text=True, check=True).stdout
    return re.findall(r"\(NEEDED\)\s+Shared library: \[([^\]]+)\]", out)


def test_libraries_do_not_link_each_other():
    import gated_group_rmsnorm_amd as g
    import oracle

    oracle.build(force=False)
    product = _needed(g.library_path())
    assert not any("oracle" in n for n in product), product
    assert any("amdhip64" in n for n in product), product  # the product is the HIP library
    olib = glob.glob(os.path.join(ROOT, "oracle", "*.so"))
    assert olib, "oracle library not built"
    for lib in olib:
        deps = _needed(lib)
        assert not any("ggrms" in n and "oracle" not in n for n in deps), deps
        assert not any("amdhip" in n or "hsa" in n for n in deps), deps


def test_binding_refuses_to_load_without_the_library(tmp_path):
    """A copy of the package without libggrms.so raises ImportError naming
    the missing library."""
    pkg = tmp_path / "gated_group_rmsnorm_amd"
    pkg.mkdir()
    for p in glob.glob(os.path.join(PKG, "*.py")):
        shutil.copy(p, pkg)
    r = subprocess.run([sys.executable, "-c", "import gated_group_rmsnorm_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=120,
                       env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libggrms.so" in r.stderr and "no non-HIP fallback" in r.stderr
