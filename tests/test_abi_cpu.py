"""The C ABI without a GPU: the library loads, exports every function the
header declares, sizes buffers, and rejects bad arguments before touching
the device."""
import ctypes
import os
import re

import pytest

from synth.workloads import LLAMA70B, LLAMA7B, TINY
from verification_verify_step_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "vstep.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vs_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(B.EXPORTS) == _declared()


def test_header_constants_match_binding():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define\s+(VS_[A-Z_0-9]+)\s+(-?\d+)", text))
    for name, val in defs.items():
        if hasattr(B, name):
            assert getattr(B, name) == int(val), name
    for name in ("VS_MAX_ROWS", "VS_MAX_SEQS", "VS_MAX_K", "VS_N_UNIFORMS", "VS_RESULT_INTS", "VS_MAX_PASS_ROWS"):
        assert name in defs and getattr(B, name) == int(defs[name]), name


def test_library_exports_every_symbol():
    L = B.lib()
    for name in _declared():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_sizes():
    w7 = B.vs_weight_bytes(LLAMA7B)
    # packed 7B weights: embed + 32 layers + head, bf16, plus small gains
    params = 32000 * 4096 * 2 + 32 * (4096 * 4096 * 4 + 3 * 4096 * 11008)
    assert params * 2 <= w7 <= params * 2 + 32 * 3 * 4096 * 4 + 200 * 256
    assert B.vs_weight_bytes(TINY) > 0 and B.vs_weight_bytes(LLAMA70B) > 130e9
    assert B.vs_workspace_bytes(LLAMA7B, 64, 8, 8192) > 0
    assert B.vs_kv_bytes(LLAMA7B, 100, 4, 50) >= 100 * 32 * 2 * 32 * 16 * 128 * 2


def test_bad_shapes_rejected():
    bad = LLAMA7B.__class__(**{**LLAMA7B.__dict__, "d_model": 4000})
    assert B.vs_weight_bytes(bad) == 0
    bad = LLAMA7B.__class__(**{**LLAMA7B.__dict__, "n_kv_heads": 5})
    assert B.vs_weight_bytes(bad) == 0
    bad = LLAMA7B.__class__(**{**LLAMA7B.__dict__, "exit_layer": 40})
    assert B.vs_weight_bytes(bad) == 0


def test_null_arguments_rejected_before_device_work():
    L = B.lib()
    assert L.vs_model_create(None, None, None, 1, 1, 1, None, None) == B.VS_E_INVAL
    cfg = B.vs_model_cfg.of(LLAMA7B)
    out = ctypes.c_void_p()
    rc = L.vs_model_create(ctypes.byref(cfg), None, None, 64, 1, 1024, None, ctypes.byref(out))
    assert rc == B.VS_E_INVAL and "null" in B.vs_last_error()
    bad = B.vs_model_cfg.of(LLAMA7B.__class__(**{**LLAMA7B.__dict__, "head_dim": 100}))
    rc = L.vs_model_create(ctypes.byref(bad), ctypes.c_void_p(1), ctypes.c_void_p(1), 64, 1, 1024, None,
                           ctypes.byref(out))
    assert rc == B.VS_E_SHAPE
    assert L.vs_draft(None, None, 1, None, None, 0, 1.0, None, None, None, None, None) == B.VS_E_INVAL
    assert L.vs_step(None, None, 1, None, None, 0, 1.0, None, None, None, None) == B.VS_E_INVAL
    with pytest.raises(B.VsError):
        B.vs_head(None, 1, 0, 0, None)
