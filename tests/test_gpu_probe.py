"""The probe library (libmoe_expert_layer_probe.so: the same sources with MOE_PHASE_PROBE) adds
cycle stamps and nothing else: its forward and backward results are bitwise those of the product
library, and moe_probe_phases counts the tasks the GEMM launches ran."""
import ctypes
import os

import pytest
import torch

import moe_expert_layer_amd as mel
import synth
from moe_expert_layer_amd.build import PROBE_LIB_PATH
from synth import device as dv

pytestmark = pytest.mark.gpu

FIELDS, KINDS = 12, 8           # include/moe_expert_layer_probe.h
TASKS = 6                       # field index of the task count


def _probe_lib():
    if not os.path.exists(PROBE_LIB_PATH):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    for name, args in mel._SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_probe_phases.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.moe_probe_phases.restype = ctypes.c_int
    return lib


def _run(inp):
    d = dv.layer(inp)
    dout = dv.tensor(synth.make_dout(inp))
    out = mel.expert_forward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs)
    grads = mel.expert_backward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs, dout)
    torch.cuda.synchronize()
    return [out, *grads]


def test_probe_build_matches_the_product_and_counts_tasks():
    # large tiles (H % 256 == 0, F % 128 == 0) and 256-row dgrad tiles: every stamped kernel runs
    inp = synth.make_layer(T=700, H=512, F=512, E=8, k=2, dtype="bf16", seed=7)
    print(f"    probe vs product: T={inp.T} H={inp.H} F={inp.F} E={inp.E} k={inp.k}", flush=True)
    ref = _run(inp)
    product = mel.library()
    probe = _probe_lib()
    assert probe.moe_probe_phases(None, 1) == 0
    mel._lib = probe
    try:
        got = _run(inp)
    finally:
        mel._lib = product
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    buf = (ctypes.c_ulonglong * (KINDS * FIELDS))()
    assert probe.moe_probe_phases(ctypes.cast(buf, ctypes.c_void_p), 1) == 0
    tasks = [buf[kind * FIELDS + TASKS] for kind in range(KINDS)]
    # fc2, fc1, recompute, weight gradients, down dgrad, gate/up dgrad all ran tasks; MX none
    assert all(t > 0 for t in tasks[:6]) and tasks[6:] == [0, 0], tasks
