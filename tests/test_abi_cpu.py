"""The C ABI without a GPU: the library loads, exports exactly what
include/*.h declares, and its host-only calls (version, error strings,
workspace sizing with its validation) behave."""
import ctypes as C
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        with open(h) as f:
            text = f.read()
        names |= set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text))
    return names


@pytest.fixture(scope="module")
def lib():
    from routed_fp8_expert_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from routed_fp8_expert_amd import build
        build.build()
    return binding


def test_exports_match_headers(lib):
    declared = _declared()
    assert len(declared) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert declared == exported
    L = lib.lib()
    for name in declared:
        assert getattr(L, name) is not None


def test_version_and_strings(lib):
    assert lib.moe_abi_version() == 5
    for status, text in [(0, "ok"), (-1, "invalid argument"), (-2, "unsupported shape"),
                         (-4, "workspace too small"), (-6, "device lost (sticky)"),
                         (-7, "too many ctxs on the device")]:
        assert lib.strerror(status) == text
    assert lib.strerror(-99) == "unknown status"


def _weights(lib, **kw):
    shape = dict(hidden=2048, n_experts=256, top_k=8, inter=512, shared_inter=512, fmt=0)
    shape.update(kw)
    c = lib.LayerWeightsC()
    c.struct_size = C.sizeof(lib.LayerWeightsC)
    c.hidden, c.n_experts, c.top_k = shape["hidden"], shape["n_experts"], shape["top_k"]
    c.inter, c.shared_inter, c.weight_format = shape["inter"], shape["shared_inter"], shape["fmt"]
    fake = 1 << 20   # host-side validation only looks at values and alignment
    for fam in (c.routed, c.shared):
        fam.gate_up = fam.down = fake
        fam.gate_up_scale = fam.down_scale = fake
        fam.gate_up_global = fam.down_global = fake
    c.routed.gate_up_stride = 2 * shape["inter"] * shape["hidden"]
    c.routed.down_stride = shape["inter"] * shape["hidden"]
    c.routed.gate_up_scale_stride = 64
    c.routed.down_scale_stride = 64
    c.router_w = fake
    return c


def _ws(lib, c, rows):
    return lib.lib().moe_workspace_bytes(C.byref(c), rows)


def test_workspace_sizing(lib):
    c = _weights(lib)
    one = _ws(lib, c, 1)
    assert one > 0
    # h for 8 routed + 1 shared entries of 512 floats (plus 8 replicas of it and
    # of the 256 logits for the single-launch layer) and small routing arrays
    h = 9 * 512 * 4
    assert 9 * h + 8 * 256 * 4 <= one <= 9 * h + 8 * 256 * 4 + 64 * 1024
    r64 = _ws(lib, c, 64)
    assert r64 >= (64 * 9) * 2048 * 4          # per-entry down outputs
    assert _ws(lib, c, 0) > 0
    assert _ws(lib, c, 1024) > 0


@pytest.mark.parametrize("kw,rows", [
    (dict(hidden=200), 1), (dict(inter=100), 1), (dict(top_k=0), 1), (dict(top_k=17), 1),
    (dict(n_experts=4, top_k=8), 1), (dict(n_experts=2048), 1), (dict(fmt=7), 1),
    (dict(hidden=16384), 1), ({}, -1), ({}, 1025), (dict(n_experts=1024), 1024),
    (dict(n_experts=512, top_k=10), 1024),
])
def test_workspace_rejects_bad_shapes(lib, kw, rows):
    assert _ws(lib, _weights(lib, **kw), rows) == 0


def test_workspace_rejects_misaligned_and_null(lib):
    c = _weights(lib)
    c.routed.gate_up = (1 << 20) + 8
    assert _ws(lib, c, 1) == 0
    c = _weights(lib)
    c.routed.down = None
    assert _ws(lib, c, 1) == 0
    c = _weights(lib)
    c.struct_size = 8
    assert _ws(lib, c, 1) == 0
    c = _weights(lib, fmt=1)
    c.routed.gate_up_global = None
    assert _ws(lib, c, 1) == 0
    assert lib.lib().moe_workspace_bytes(None, 1) == 0


def test_calls_without_ctx_are_rejected(lib):
    L = lib.lib()
    assert L.moe_ctx_status(None) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_route(None, None, None, 1, 0, None, None, None, 0, None) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward(None, None, None, 1, 0, None, None, None, None, 0, None, 0,
                               None) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_ctx_create(0, None) == lib.MOE_ERR_INVALID_ARG
