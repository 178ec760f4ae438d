"""Parity at the workloads' full sizes, in the launch configuration the benchmark times.

The oracle cannot run these layers whole in seconds, so routing (cheap) is compared in full and
bit-exactly, the chunked mode is compared with the unchunked one bitwise, and the outputs are
compared on sampled tokens (rows) that the oracle computes one by one through the per-token
definition.  Samples always include the first and last row of expert groups (tile heads and ragged
tile tails) besides random ones.  The float metrics are the inf-norm relative error over the sample
and, per token, the row's inf-norm error relative to that row's largest output; both must meet the
dtype's bar.
"""
import numpy as np
import pytest
import torch

import moe_expert_layer_amd as mel
import oracle
import synth
from synth import device as dv

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "mxfp8": 6e-2}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    mel.library()
    oracle.build()


def _edge_tokens(perm, offsets, k, experts, rng, n_random):
    """Tokens owning the first and last permuted row of each listed expert group, plus random ones."""
    toks = set()
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            toks.add(int(perm[lo]) // k)
            toks.add(int(perm[hi - 1]) // k)
    T = perm.shape[0] // k
    toks.update(int(t) for t in rng.choice(T, size=n_random, replace=False))
    return np.array(sorted(toks), np.int32)


def _workspace(inp, head):
    code = {"bf16": mel.BF16, "mxfp8": mel.MXFP8}[inp.dtype]
    p = mel.problem(inp.T, inp.H, inp.F, inp.E, inp.k, code, head)
    return torch.empty(mel.workspace_size(p), dtype=torch.uint8, device="cuda")


def _layer_case(name, n_edge_experts, n_random):
    print(f"[fullsize] {name}: generating inputs", flush=True)
    inp = synth.make_workload(name)
    d = dv.layer(inp)
    print(f"[fullsize] {name}: T={inp.T} H={inp.H} F={inp.F} E={inp.E} k={inp.k}", flush=True)

    # routing, whole, bit-exact
    counts, offsets, perm, pos = oracle.route(inp.expert_ids, inp.E)
    g = mel.route(d.expert_ids, inp.E)
    assert np.array_equal(dv.host(g[0]), counts)
    assert np.array_equal(dv.host(g[1]), offsets)
    assert np.array_equal(dv.host(g[2]), perm)
    assert np.array_equal(dv.host(g[3]), pos)

    # the benchmark's launch configuration, unchunked and chunked by 512 rows: identical bits
    out = dv.forward(mel, d, 0, workspace=_workspace(inp, 0))
    out512 = dv.forward(mel, d, 512, workspace=_workspace(inp, 512))
    # and with the permute step as a kernel of its own instead of inside fc1's row copies
    sep = dv.forward(mel, d, 0, workspace=_workspace(inp, 0), separate_permute=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out512)
    assert torch.equal(out, sep)

    rng = np.random.default_rng(7)
    nonempty = [e for e in range(inp.E) if counts[e] > 0]
    experts = rng.choice(nonempty, size=min(n_edge_experts, len(nonempty)), replace=False)
    toks = _edge_tokens(perm, offsets, inp.k, experts, rng, n_random)
    print(f"[fullsize] {name}: oracle on {len(toks)} sampled tokens", flush=True)
    ref = oracle.forward_tokens(inp, toks)
    got = dv.host(out)[toks]
    err = oracle.inf_norm_rel(got, ref)
    row_err = oracle.row_inf_norm_rel(got, ref)
    print(f"[fullsize] {name}: inf-norm rel err over the sample {err:.3e}, worst token {row_err:.3e}",
          flush=True)
    assert np.isfinite(got).all()
    assert err <= TOL[inp.dtype]
    assert row_err <= TOL[inp.dtype]      # per token, against that token's own largest output


def test_mixtral_full_size():
    _layer_case("mixtral_bf16", n_edge_experts=8, n_random=16)


def test_finegrained_full_size():
    _layer_case("finegrained_bf16", n_edge_experts=24, n_random=16)


def test_mxfp8_full_size():
    _layer_case("mxfp8", n_edge_experts=12, n_random=12)


def test_ep_rank_full_size():
    print("[fullsize] ep_rank_bf16: generating inputs", flush=True)
    g = synth.make_workload("ep_rank_bf16")
    rows = dv.tensor(g.rows)
    args = (dv.tensor(g.group_offsets), dv.tensor(g.group_expert), dv.tensor(g.w_gate),
            dv.tensor(g.w_up), dv.tensor(g.w_down))
    y = mel.grouped_ffn(rows, *args)
    y512 = mel.grouped_ffn(rows, *args, head_m_size=512)
    torch.cuda.synchronize()
    assert torch.equal(y, y512)
    offs = np.asarray(g.group_offsets, np.int64)
    rng = np.random.default_rng(11)
    idx = set(int(i) for i in rng.choice(offs[-1], size=16, replace=False))
    for a, b in zip(offs[:-1], offs[1:]):
        if b > a:
            idx.update((int(a), int(b) - 1))
    idx = np.array(sorted(idx), np.int64)
    print(f"[fullsize] ep_rank_bf16: oracle on {len(idx)} sampled rows", flush=True)
    ref = oracle.grouped_ffn(g, row_index=idx)
    got = dv.host(y)[idx]
    err = oracle.inf_norm_rel(got, ref)
    row_err = oracle.row_inf_norm_rel(got, ref)
    print(f"[fullsize] ep_rank_bf16: inf-norm rel err over the sample {err:.3e}, worst row {row_err:.3e}",
          flush=True)
    assert err <= TOL["bf16"]
    assert row_err <= TOL["bf16"]
