"""The measurement library (include/qkceil.h) without a GPU: it loads,
exports what its header declares, and rejects invalid arguments on the host
before any launch (fake device addresses, never dereferenced)."""
import os
import re

import pytest

from attention_qk_norm_amd import ceiling
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qkceil.h")
A = 0x7F0000000000


def test_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = sorted(set(re.findall(r"^\s*int\s+(qkceil_\w+)\s*\(", text, re.M)))
    assert sorted(ceiling.EXPORTS) == declared
    L = ceiling.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name, value in (("OK", ceiling.OK), ("ERR_NULL", ceiling.ERR_NULL), ("ERR_SIZE", ceiling.ERR_SIZE),
                        ("ERR_ALIGN", ceiling.ERR_ALIGN), ("ERR_CONFIG", ceiling.ERR_CONFIG),
                        ("ERR_DEVICE", ceiling.ERR_DEVICE)):
        assert int(re.search(r"\bQKCEIL_%s\s*=\s*(-?\d+)" % name, text).group(1)) == value


@pytest.mark.parametrize("call", ["copy", "read", "write"])
def test_argument_checks(call):
    L = ceiling.lib()

    def run(src=A, dst=A + (1 << 30), n=1 << 20, vpl=4):
        if call == "copy":
            return L.qkceil_copy(src, dst, n, vpl, None)
        if call == "read":
            return L.qkceil_read(src, n, vpl, dst, None)
        return L.qkceil_write(dst, n, vpl, None)

    assert run(n=0) == ceiling.OK  # nothing to move: no launch
    for kw, want in [(dict(src=None), ceiling.ERR_NULL), (dict(dst=None), ceiling.ERR_NULL),
                     (dict(n=1000), ceiling.ERR_SIZE), (dict(n=(1 << 35) + 16), ceiling.ERR_SIZE),
                     (dict(src=A + 8), ceiling.ERR_ALIGN), (dict(dst=A + 4), ceiling.ERR_ALIGN),
                     (dict(vpl=3), ceiling.ERR_CONFIG), (dict(vpl=16), ceiling.ERR_CONFIG)]:
        if call == "write" and "src" in kw:
            continue  # the write stream has no source
        assert run(**kw) == want, kw
    assert L.qkceil_empty(0, None) == ceiling.ERR_CONFIG
    assert L.qkceil_clock(None, None) == ceiling.ERR_NULL
    assert L.qkceil_clock(A + 4, None) == ceiling.ERR_ALIGN
