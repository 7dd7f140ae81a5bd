"""C ABI checks that need no GPU: the library loads, exports every call the
header declares, the header is valid C with the struct layout the binding
assumes, and every argument check returns before any HIP call."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from post_weight_quantization_16_amd import _native as n

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptq.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gptq_[a-z_]+)\s*\(", src)))


def test_library_loads_and_exports_every_declared_call():
    L = n.lib()
    decl = _declared()
    assert set(decl) == set(n.EXPORTS)
    for name in decl:
        assert hasattr(L, name), name
    assert L.gptq_version().decode().startswith("gptq_mi355x")
    out = subprocess.run(["nm", "-D", "--defined-only", n.LIB_PATH], capture_output=True, text=True)
    for name in decl:
        assert re.search(rf"\bT {name}\b", out.stdout), name


def test_header_is_c_and_struct_layout_matches_binding():
    prog = r"""
#include <stdio.h>
#include <stddef.h>
#include "gptq.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu\n", sizeof(gptq_params), offsetof(gptq_params, bits),
         offsetof(gptq_params, group_size), offsetof(gptq_params, block_size),
         offsetof(gptq_params, percdamp), offsetof(gptq_params, act_order),
         offsetof(gptq_params, sym));
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "t.c")
        exe = os.path.join(td, "t")
        open(c, "w").write(prog)
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), c,
                        "-o", exe], check=True)
        got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    P = n.Params
    want = [ctypes.sizeof(P)] + [getattr(P, f).offset for f, _ in P._fields_]
    assert got == want


def _params(**kw):
    d = dict(bits=4, group_size=128, block_size=128, percdamp=0.01, act_order=0, sym=0)
    d.update(kw)
    return n.Params(**d)


FAKE = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation first


def _quant(p, W=FAKE, m=64, d=256, ld=256, ws=FAKE, ws_bytes=1 << 40, U=FAKE, wdt=n.BF16):
    L = n.lib()
    return L.gptq_quantize_layer(W, wdt, m, d, ld, U, None, None, ctypes.byref(p), FAKE, FAKE, FAKE,
                                 None, None, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(bits=5), n.ERR_INVALID_ARG),
    (dict(bits=1), n.ERR_INVALID_ARG),
    (dict(group_size=0), n.ERR_INVALID_ARG),
    (dict(group_size=-7), n.ERR_INVALID_ARG),
    (dict(percdamp=-0.1), n.ERR_INVALID_ARG),
    (dict(percdamp=float("nan")), n.ERR_INVALID_ARG),
    (dict(act_order=2), n.ERR_INVALID_ARG),
    (dict(block_size=64), n.ERR_UNSUPPORTED),
    (dict(group_size=48), n.ERR_UNSUPPORTED),
    (dict(group_size=16), n.ERR_UNSUPPORTED),
    (dict(group_size=96), n.ERR_UNSUPPORTED),
])
def test_quantize_rejects_bad_params(kw, code):
    assert _quant(_params(**kw)) == code
    assert n.last_error() != ""


def test_quantize_rejects_bad_shapes_and_pointers():
    p = _params()
    assert _quant(p, W=None) == n.ERR_INVALID_ARG
    assert _quant(p, U=None) == n.ERR_INVALID_ARG
    assert _quant(p, m=0) == n.ERR_INVALID_ARG
    assert _quant(p, d=0) == n.ERR_INVALID_ARG
    assert _quant(p, ld=100) == n.ERR_INVALID_ARG
    assert _quant(p, wdt=7) == n.ERR_INVALID_ARG
    assert _quant(p, ws=None) == n.ERR_WORKSPACE
    assert _quant(p, ws_bytes=1024) == n.ERR_WORKSPACE
    assert _quant(p, ws=ctypes.c_void_p((1 << 20) + 4)) == n.ERR_WORKSPACE
    assert "aligned" in n.last_error()


def test_group_sizes_accepted_by_validation_reach_workspace_check():
    """Supported combinations pass parameter checks (stopped by a short workspace)."""
    for g, d in [(128, 256), (64, 256), (32, 256), (256, 512), (-1, 300), (300, 300), (128, 300)]:
        assert _quant(_params(group_size=g), d=d, ld=d, ws_bytes=16) == n.ERR_WORKSPACE, (g, d)


def test_hessian_validation():
    L = n.lib()
    acc = L.gptq_hessian_accumulate
    assert acc(None, 64, FAKE, n.BF16, 10, 64, FAKE, 1 << 40, None) == n.ERR_INVALID_ARG
    assert acc(FAKE, 0, FAKE, n.BF16, 10, 64, FAKE, 1 << 40, None) == n.ERR_INVALID_ARG
    assert acc(FAKE, 64, FAKE, 9, 10, 64, FAKE, 1 << 40, None) == n.ERR_INVALID_ARG
    assert acc(FAKE, 64, FAKE, n.BF16, -1, 64, FAKE, 1 << 40, None) == n.ERR_INVALID_ARG
    assert acc(FAKE, 64, FAKE, n.BF16, 10, 32, FAKE, 1 << 40, None) == n.ERR_INVALID_ARG
    assert acc(FAKE, 64, None, n.BF16, 10, 64, FAKE, 1 << 40, None) == n.ERR_INVALID_ARG
    assert acc(FAKE, 64, FAKE, n.BF16, 10, 64, FAKE, 16, None) == n.ERR_WORKSPACE
    # zero tokens is a no-op that touches nothing
    assert acc(FAKE, 64, None, n.BF16, 0, 64, None, 0, None) == n.OK


def test_prepare_validation():
    L = n.lib()
    info = ctypes.c_int64(123)
    p = _params()
    prep = L.gptq_prepare_hinv
    assert prep(None, 64, ctypes.byref(p), FAKE, FAKE, None, FAKE, 1 << 40, ctypes.byref(info), None) == n.ERR_INVALID_ARG
    assert info.value == -1
    assert prep(FAKE, 64, None, FAKE, FAKE, None, FAKE, 1 << 40, None, None) == n.ERR_INVALID_ARG
    pa = _params(act_order=1)
    assert prep(FAKE, 64, ctypes.byref(pa), FAKE, None, None, FAKE, 1 << 40, None, None) == n.ERR_INVALID_ARG
    assert prep(FAKE, 64, ctypes.byref(p), FAKE, FAKE, None, FAKE, 8, None, None) == n.ERR_WORKSPACE


def test_workspace_sizes():
    L = n.lib()
    p = _params()
    ws = L.gptq_workspace_bytes
    assert ws(0, 0, 0, 10, None) == 0
    assert ws(9, 10, 10, 10, ctypes.byref(p)) == 0
    assert ws(2, 0, 64, 0, ctypes.byref(p)) == 0
    h = ws(0, 0, 4096, 131072, None)
    assert h > 0 and h % 256 == 0
    q = ws(2, 4096, 4096, 0, ctypes.byref(p))
    assert q >= 4096 * 4096 * 5  # fp32 working copy + codes
    assert ws(1, 0, 4096, 0, ctypes.byref(p)) >= 2 * 4096 * 4096 * 4
