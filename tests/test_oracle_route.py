"""Pins for the oracle's routing step (counts, offsets, stable permutation and its inverse).

Definition: page 'NPU Training Operators - MC2', section 执行路径, step 2 (torch.histc over the
flattened selected_experts with E bins on [0, E)), step 6 (permute) and step 10 (unpermute indices);
section 迁移检查 requires ids in [0, E).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "route_worked_example.json")


def test_worked_examples():
    for case in json.load(open(GOLDEN))["cases"]:
        counts, offsets, perm, pos = oracle.route(np.array(case["expert_ids"]), case["E"])
        assert counts.tolist() == case["counts"]
        assert offsets.tolist() == case["offsets"]
        assert perm.tolist() == case["perm"]
        assert pos.tolist() == case["pos"]


@pytest.mark.parametrize("T,k,E,seed", [(64, 2, 4, 0), (1000, 8, 128, 1), (4096, 2, 8, 2), (37, 3, 5, 3)])
def test_against_library_routines(T, k, E, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    counts, offsets, perm, pos = oracle.route(ids, E)
    flat = ids.ravel()
    # the pages' own counting call
    h = torch.histc(torch.from_numpy(flat).double(), bins=E, min=0, max=E)
    assert np.array_equal(counts, h.numpy().astype(np.int32))
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    assert np.array_equal(pos, inv)


def test_invariants_on_workload_routing():
    inp = synth.make_layer(T=2048, H=64, F=64, E=128, k=8, dtype="bf16", routing="zipf_gumbel",
                           zipf_s=1.1, n_zero=8)
    counts, offsets, perm, pos = oracle.route(inp.expert_ids, 128)
    M = 2048 * 8
    assert counts.sum() == M and offsets[-1] == M
    assert (counts == 0).sum() >= 8                      # the zero-weight experts stay empty
    assert np.array_equal(np.sort(perm), np.arange(M))   # a permutation
    assert np.array_equal(pos[perm], np.arange(M))
    flat = inp.expert_ids.ravel()
    for e in range(128):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)                  # stable: ascending slot index


def test_permute_gathers_token_rows():
    rng = np.random.default_rng(5)
    T, k, E, H = 50, 3, 6, 16
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = rng.standard_normal((T, H)).astype(np.float32)
    _, _, perm, pos = oracle.route(ids, E)
    xp = oracle.permute(x, perm, k)
    for p in range(T * k):
        assert np.array_equal(xp[p], x[perm[p] // k])
    for t in range(T):                                   # pos sends every slot back to its token
        for j in range(k):
            assert np.array_equal(xp[pos[t * k + j]], x[t])


@pytest.mark.parametrize("bad", [-1, 4, 1000])
def test_out_of_range_id_rejected(bad):
    ids = np.array([[0, 1], [2, bad]], np.int32)
    with pytest.raises(oracle.OracleError):
        oracle.route(ids, 4)
