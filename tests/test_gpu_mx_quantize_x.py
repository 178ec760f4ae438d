"""The MX layer fed bfloat16 activations (MOE_FLAG_QUANTIZE_X): the library encodes x to OCP-MX on
its way into the gather of the execution path's step 6.

- The codes and block scales the encoder leaves in the workspace are bit-exact against the oracle's
  encoder applied to the same bfloat16 values: in token order when fc1 gathers its rows itself, and
  in the permuted row order when the permute runs as its own step (the encoding then rides on the
  permute's gather).
- The layer's output is bitwise that of the MX forward fed the host-encoded x, and within the MX bar
  (6e-2, whole tensor and per token) of the oracle's layer on those inputs.
"""
import dataclasses

import numpy as np
import pytest
import torch

import moe_expert_layer_amd as mel
import oracle
import synth
from synth import device as dv

pytestmark = pytest.mark.gpu

TOL = 6e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    mel.library()
    oracle.build()


def _host_encoded(inp):
    """The layer's inputs with x replaced by the oracle's OCP-MX encoding of the bfloat16 x."""
    xv = synth.bf16_bits_to_f32(inp.x_bf16).astype(np.float64)
    q, s = oracle.mx_quantize(xv)
    return dataclasses.replace(inp, x=q, x_scale=s), q, s


def _forward(d, x, x_scale, head=0, separate=False, ws=None):
    return mel.expert_forward_mx(x, x_scale, d.w_gate, d.wg_scale, d.w_up, d.wu_scale, d.w_down,
                                 d.wd_scale, d.expert_ids, d.probs, head_m_size=head, workspace=ws,
                                 separate_permute=separate)


def _workspace(inp, head=0, separate=False):
    flags = mel.FLAG_QUANTIZE_X | (mel.FLAG_SEPARATE_PERMUTE if separate else 0)
    p = mel.problem(inp.T, inp.H, inp.F, inp.E, inp.k, mel.MXFP8, head, flags)
    return torch.zeros(mel.workspace_size(p), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("T,H,F,E,k,separate", [
    (300, 1024, 1024, 5, 2, False),      # large tiles: fc1 gathers from the token-order encoding
    (300, 1024, 1024, 5, 2, True),       # large tiles, permute as its own step: encoded permuted rows
    (333, 256, 384, 6, 3, False),        # small tiles: always the permuted rows
    (97, 128, 128, 3, 1, False),
], ids=["large_gathered", "large_separate", "small", "small_k1"])
def test_encoded_rows_bit_exact_and_output_is_the_host_encoded_one(T, H, F, E, k, separate):
    inp = synth.make_layer(T=T, H=H, F=F, E=E, k=k, dtype="mxfp8", seed=T + H)
    enc, q, s = _host_encoded(inp)
    d = dv.layer(inp)
    ws = _workspace(inp, 0, separate)
    out = _forward(d, dv.tensor(inp.x_bf16), None, 0, separate, ws)
    codes, scales, permuted = mel.quantized_x(ws, T, H, F, E, k, 0, separate)
    torch.cuda.synchronize()
    # large tiles gather from the token-order encoding unless the permute is a step of its own
    assert permuted == (separate or H % 1024 != 0 or F % 1024 != 0)
    if not permuted:
        ref_q, ref_s = q, s
    else:
        _, _, perm, _ = oracle.route(inp.expert_ids, E)
        ref_q, ref_s = oracle.permute(q, perm, k), oracle.permute(s, perm, k)
    print(f"encoded rows: {codes.shape[0]} ({'permuted' if permuted else 'token order'})")
    assert np.array_equal(dv.host(scales), ref_s)
    assert np.array_equal(dv.host(codes), ref_q)
    # the layer on the host-encoded x: same bits
    ref_out = _forward(d, dv.tensor(q), dv.tensor(s), 0, separate)
    assert torch.equal(out, ref_out)
    # and the oracle's layer on those inputs
    ref, *_ = oracle.forward(enc)
    got = dv.host(out)
    err, row_err = oracle.inf_norm_rel(got, ref), oracle.row_inf_norm_rel(got, ref)
    print(f"T={T} H={H} F={F}: inf-norm rel err {err:.3e}, worst token {row_err:.3e}")
    assert err <= TOL and row_err <= TOL


def test_chunked_equals_unchunked_and_separate():
    inp = synth.make_layer(T=600, H=1024, F=1024, E=7, k=2, dtype="mxfp8", seed=5)
    d = dv.layer(inp)
    xb = dv.tensor(inp.x_bf16)
    base = _forward(d, xb, None, 0, False, _workspace(inp, 0, False))
    for head, sep in ((512, False), (256, False), (0, True), (512, True)):
        assert torch.equal(_forward(d, xb, None, head, sep, _workspace(inp, head, sep)), base)


def test_rejects_scale_with_bf16_x_and_flag_on_bf16_problem():
    lib = mel.library()
    prob = mel.problem(64, 128, 128, 4, 2, mel.BF16, 0, mel.FLAG_QUANTIZE_X)
    n = __import__("ctypes").c_size_t()
    assert lib.moe_workspace_size(__import__("ctypes").byref(prob), __import__("ctypes").byref(n)) == 1
    inp = synth.make_layer(T=64, H=128, F=128, E=4, k=2, dtype="mxfp8", seed=1)
    d = dv.layer(inp)
    with pytest.raises(ValueError):
        _forward(d, dv.tensor(inp.x_bf16), d.x_scale)


def test_mxfp8_full_size_from_bf16():
    """The MX workload at full size (T=16384, H=7168, F=2048, E=32, k=4) fed its bfloat16 x: the
    token-order encoding bit-exact on every row, the output bitwise that of the host-encoded call, and
    sampled tokens within the MX bar of the oracle."""
    print("[mx-bf16] generating the MX workload", flush=True)
    inp = synth.make_workload("mxfp8")
    enc, q, s = _host_encoded(inp)
    d = dv.layer(inp)
    ws = _workspace(inp, 0, False)
    out = _forward(d, dv.tensor(inp.x_bf16), None, 0, False, ws)
    codes, scales, permuted = mel.quantized_x(ws, inp.T, inp.H, inp.F, inp.E, inp.k)
    torch.cuda.synchronize()
    assert not permuted
    assert np.array_equal(dv.host(scales), s)
    assert np.array_equal(dv.host(codes), q)
    assert torch.equal(out, _forward(d, dv.tensor(q), dv.tensor(s)))
    assert torch.equal(out, _forward(d, dv.tensor(inp.x_bf16), None, 512, False, _workspace(inp, 512)))
    rng = np.random.default_rng(3)
    toks = np.sort(rng.choice(inp.T, 24, replace=False)).astype(np.int32)
    ref = oracle.forward_tokens(enc, toks)
    got = dv.host(out)[toks]
    err, row_err = oracle.inf_norm_rel(got, ref), oracle.row_inf_norm_rel(got, ref)
    print(f"[mx-bf16] full size: inf-norm rel err {err:.3e}, worst token {row_err:.3e}", flush=True)
    assert err <= TOL and row_err <= TOL
