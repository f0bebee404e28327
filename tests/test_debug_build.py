"""Host-side checks of the debug build (no GPU needed).

libstreamkl_debug.so is the library compiled with -DSTREAMKL_DEBUG: every
global-memory access of the kernels, and the LDS accesses of their tile
loops, go through a bounds check (dbg_in in csrc/streamkl_device.h), and the
first violation is reported by streamkl_debug_take.  Here: the debug build
exports the release ABI plus streamkl_debug_take, the release build does not
export it, the header declares it only under STREAMKL_DEBUG, and dbg_in --
compiled for the host from the same header -- accepts exactly the accesses
that lie inside their buffer.
"""
import os
import re
import subprocess

import pytest

from attention_distillation_kl_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "streamkl.h")
CSRC = os.path.join(ROOT, "attention_distillation_kl_amd", "csrc")


def test_debug_library_exports_the_abi_and_the_take_call():
    dbg = _lib.load(_lib.DEBUG_LIB_PATH)
    for name in _lib.EXPORTS:
        assert hasattr(dbg, name), name
    assert hasattr(dbg, "streamkl_debug_take")
    assert dbg.streamkl_abi_version() == 1


def test_release_library_has_no_debug_export():
    assert not hasattr(_lib.load(), "streamkl_debug_take")


def test_header_declares_the_take_call_for_debug_builds_only():
    text = open(HEADER).read()
    m = re.search(r"#ifdef STREAMKL_DEBUG(.*?)#endif", text, flags=re.S)
    assert m and "unsigned streamkl_debug_take(void);" in m.group(1)
    outside = text[:m.start()] + text[m.end():]
    assert "streamkl_debug_take" not in outside


def test_site_codes_read_back():
    assert _lib.debug_site(0) == "none"
    assert _lib.debug_site((2 << 16) | 417) == "streamkl_bwd.h:417"
    assert _lib.debug_site(0xFFFFFFFF) == "device not readable"


DBG_IN_TEST = r"""
#include "streamkl_device.h"
#include <cstdio>
using streamkl::dbg_in;
int main() {
  const uintptr_t lo = 4096;
  int bad = 0;
  auto expect = [&](bool got, bool want, int line) {
    if (got != want) { std::printf("line %d: got %d\n", line, int(got)); ++bad; }
  };
  expect(dbg_in(lo, 16, lo, 64), true, __LINE__);            // first element
  expect(dbg_in(lo + 48, 16, lo, 64), true, __LINE__);       // last element, ends at the end
  expect(dbg_in(lo + 49, 16, lo, 64), false, __LINE__);      // runs one byte past the end
  expect(dbg_in(lo + 64, 16, lo, 64), false, __LINE__);      // starts at the end
  expect(dbg_in(lo + 64, 0, lo, 64), true, __LINE__);        // empty access at the end
  expect(dbg_in(lo - 16, 16, lo, 64), false, __LINE__);      // before the start
  expect(dbg_in(lo - 1, 1, lo, 64), false, __LINE__);
  expect(dbg_in(lo, 65, lo, 64), false, __LINE__);           // longer than the buffer
  expect(dbg_in(lo, 16, lo, 0), false, __LINE__);            // empty buffer
  expect(dbg_in(lo + 8, SIZE_MAX, lo, 64), false, __LINE__); // length wraps
  expect(dbg_in(UINTPTR_MAX - 7, 16, lo, 64), false, __LINE__);
  expect(dbg_in(lo + (uintptr_t(1) << 40), 4, lo, (size_t(1) << 40) + 4), true, __LINE__);  // past 4 GiB
  std::printf("%d bad\n", bad);
  return bad != 0;
}
"""


def test_bounds_arithmetic_on_the_host(tmp_path):
    src = tmp_path / "dbg_in_test.hip"
    exe = tmp_path / "dbg_in_test"
    src.write_text(DBG_IN_TEST)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    r = subprocess.run([hipcc, "-std=c++17", "--offload-host-only", "-x", "hip", "-I", CSRC,
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and "0 bad" in r.stdout, r.stdout
