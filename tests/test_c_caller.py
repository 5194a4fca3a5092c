"""The library driven from C.  tests/c/bsg_forward_demo (built by
__graft_entry__.build()) runs the layer's forward through the C ABI alone,
every device buffer from hipMalloc and no Python or torch in the process,
as a child process of the test; its output y is checked against the oracle
to the bf16 bar, and it checks by itself that an invalid call is refused."""
import os
import subprocess

import numpy as np
import pytest

from block_sparse_gemm_amd import synth
from tests.test_gpu_parity import check_float

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "bsg_forward_demo")


def test_forward_from_c(orc, tmp_path):
    if not os.path.exists(EXE):
        pytest.fail("tests/c/bsg_forward_demo is not built: run __graft_entry__.build()")
    cfg = synth.LayerConfig("c_caller", T=700, d=256, E=5, f=384, k=2)
    inp = synth.make_inputs(cfg, 31)
    np.ascontiguousarray(inp["logits"], np.float32).tofile(tmp_path / "logits.f32")
    for key, name in (("x", "x.bf16"), ("W1", "w1.bf16"), ("W2", "w2.bf16")):
        np.ascontiguousarray(inp[key].bits, np.uint16).tofile(tmp_path / name)
    print(f"[c caller] T={cfg.T} d={cfg.d} E={cfg.E} f={cfg.f} k={cfg.k}", flush=True)
    r = subprocess.run([EXE, str(tmp_path), str(cfg.T), str(cfg.d), str(cfg.E), str(cfg.f),
                        str(cfg.k)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    y = synth.bf16_bits_to_f32(np.fromfile(tmp_path / "y.bf16", dtype=np.uint16))
    y = y.reshape(cfg.T, cfg.d).astype(np.float64)
    rt = orc.route(inp["logits"], cfg.k)
    O = orc.make_layer(inp["x"].values, inp["W1"].values, inp["W2"].values, rt, cfg.k, cfg.E,
                       prec="bf16")
    report = {}
    check_float("y (C caller)", y, O.forward_tokens(np.arange(cfg.T)), "bf16", report)
