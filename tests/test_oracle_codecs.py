"""Pins for the oracle's storage decoders and its OCP-MX encoder.

The pages name MX-FP8 as the reference project's matmul format (page 'MC2 通算融合架构总览', §1)
and per-row scale buffers (§5) but print no encoded value; the codec is OCP Microscaling Formats
v1.0 (E4M3 elements, E8M0 scales, blocks of 32).  Pins: torch's float8_e4m3fn / bfloat16 codecs
(independent library routines), the spec's anchor values, hand-derived blocks, and the input
generator's own (separately written) encoder.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_block_worked_example.json")


def test_bf16_decode_all_patterns():
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oracle.bf16_value(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_decode_all_codes_against_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_spec_anchors():
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6          # min normal
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9      # max subnormal
    assert oracle.e4m3_value(0x01) == 2.0 ** -9          # min subnormal
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0xB8) == -1.0
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.e8m0_value(254) == 2.0 ** 127
    assert math.isnan(oracle.e8m0_value(255))


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-448, 448, 4000), rng.standard_normal(4000),
                        rng.standard_normal(2000) * 1e-2, rng.standard_normal(2000) * 1e-3])
    # exact midpoints between neighbouring codes exercise ties-to-even
    vals = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = (vals[1:] + vals[:-1]) / 2
    v = np.concatenate([v, mids, -mids])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(x) for x in v], np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates_and_roundtrips():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(460.0) == 0x7E
    assert oracle.e4m3_encode(464.0) == 0x7E
    assert oracle.e4m3_encode(500.0) == 0x7E
    assert oracle.e4m3_encode(-1e9) == 0xFE
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c


def test_mx_worked_blocks():
    for b in json.load(open(GOLDEN))["blocks"]:
        q, s = oracle.mx_quantize(np.array(b["values"], np.float64)[None, :])
        assert int(s[0, 0]) == b["scale"], b["note"]
        assert q[0].tolist() == b["codes"], b["note"]


def test_mx_scale_rule_and_bounds():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((64, 32)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    q, s = oracle.mx_quantize(v)
    amax = np.abs(v).max(axis=1)
    assert np.array_equal(s[:, 0].astype(int), np.floor(np.log2(amax)).astype(int) - 8 + 127)
    deq = oracle.mx_decode(q, s)
    X = np.exp2(s[:, 0].astype(float) - 127)[:, None]
    assert np.all(np.abs(deq) <= 448 * X)
    # the block maximum lands in [256, 448] * X, so no block loses its top binade
    top = np.abs(deq).max(axis=1) / X[:, 0]
    assert np.all((top >= 256) & (top <= 448))
    # relative error of a normal-range, non-saturated element is at most half a step (2^-4)
    big = (np.abs(v) >= X * 2.0 ** -6) & (np.abs(v) <= X * 448)
    assert np.all(np.abs(deq - v)[big] <= np.abs(v)[big] * 2.0 ** -4 + 1e-300)
    # saturated elements come back as exactly +-448 X
    sat = np.abs(v) > X * 464
    assert np.all(np.abs(deq[sat]) == np.broadcast_to(448 * X, v.shape)[sat])


def test_generator_encoder_matches_oracle():
    rng = np.random.default_rng(9)
    v = (rng.standard_normal((96, 128)) * 0.02).astype(np.float32)
    v[3] = 0.0
    v[5, :32] *= 1e-30
    q_syn, s_syn = synth.mx_encode_blocks(v, axis=1)
    q_or, s_or = oracle.mx_quantize(v.astype(np.float64))
    assert np.array_equal(s_syn, s_or)
    assert np.array_equal(q_syn, q_or)
    # blocks along axis 0 (the weights' layout)
    q0, s0 = synth.mx_encode_blocks(v, axis=0)
    q1, s1 = oracle.mx_quantize(v.T.astype(np.float64))
    assert np.array_equal(q0, q1.T) and np.array_equal(s0, s1.T)
