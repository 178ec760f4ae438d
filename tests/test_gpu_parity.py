"""GPU parity of the HIP path against the CPU oracle at sizes the oracle finishes in seconds.

Every call goes through the C ABI (via the ctypes binding).  Bars: integer work (counts, offsets,
perm, pos, permute bytes) bit-exact; float outputs within max|gpu - oracle| / max|oracle|
<= 2e-2 for bfloat16 and 6e-2 for MX-FP8 (the stated bars) and 1e-5 for float32 (fp32 accumulation
over at most 14336 products of N(0,1) and N(0,0.02) values keeps that error near 1e-6; 1e-5 leaves
a tenfold margin).
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from synth import device as dv

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mel = pytest.importorskip("moe_expert_layer_amd")

TOL = {"f32": 1e-5, "bf16": 2e-2, "mxfp8": 6e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mel.library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------------------------------ route

@pytest.mark.parametrize("T,k,E,seed", [(64, 2, 4, 0), (4096, 2, 8, 1), (8192, 8, 128, 2),
                                         (16384, 4, 32, 3), (1, 1, 1, 4), (3000, 3, 1000, 5),
                                         (2049, 1, 2, 6), (0, 2, 4, 7)])
def test_route_bit_exact(T, k, E, seed):
    rng = np.random.default_rng(seed)
    ids = (np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T
           else np.zeros((0, k), np.int32))
    counts, offsets, perm, pos, ws = mel.route(dv.tensor(ids), E)
    oc, oo, op, opos = oracle.route(ids, E)
    assert np.array_equal(dv.host(counts), oc)
    assert np.array_equal(dv.host(offsets), oo)
    assert np.array_equal(dv.host(perm), op)
    assert np.array_equal(dv.host(pos), opos)
    assert mel.device_status(ws) == 0


def test_route_workload_routing_bit_exact():
    for name in ("finegrained_bf16", "mxfp8"):
        cfg = synth.WORKLOADS[name]
        inp = synth.make_layer(T=cfg["T"], H=32, F=32, E=cfg["E"], k=cfg["k"], dtype="f32",
                               routing=cfg["routing"],
                               **{kk: cfg[kk] for kk in ("zipf_s", "n_zero") if kk in cfg})
        counts, offsets, perm, pos, _ = mel.route(dv.tensor(inp.expert_ids), cfg["E"])
        oc, oo, op, opos = oracle.route(inp.expert_ids, cfg["E"])
        assert np.array_equal(dv.host(counts), oc) and np.array_equal(dv.host(offsets), oo)
        assert np.array_equal(dv.host(perm), op) and np.array_equal(dv.host(pos), opos)


def test_route_out_of_range_ids_flagged_and_dropped():
    rng = np.random.default_rng(9)
    T, k, E = 700, 2, 6
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    bad = rng.choice(T * k, 25, replace=False)
    ids.ravel()[bad[:10]] = E + 3
    ids.ravel()[bad[10:]] = -1
    counts, offsets, perm, pos, ws = mel.route(dv.tensor(ids), E)
    assert mel.device_status(ws) == 4            # MOE_ERR_EXPERT_ID_OUT_OF_RANGE
    flat = ids.ravel()
    ok = (flat >= 0) & (flat < E)
    assert np.array_equal(dv.host(counts), np.bincount(flat[ok], minlength=E))
    valid_slots = np.flatnonzero(ok)
    order = valid_slots[np.argsort(flat[ok], kind="stable")]
    p = dv.host(perm)
    assert np.array_equal(p[:ok.sum()], order)
    assert np.all(p[ok.sum():] == -1)
    ps = dv.host(pos)
    assert np.all(ps[~ok] == -1)
    assert np.array_equal(ps[order], np.arange(ok.sum()))


# ------------------------------------------------------------------------------------------ permute / unpermute

@pytest.mark.parametrize("dtype,H", [("f32", 256), ("bf16", 256), ("mxfp8", 256),
                                     ("bf16", 384), ("mxfp8", 7168), ("bf16", 8192)])
def test_permute_bit_exact(dtype, H):
    """Row widths whose 16-byte vectors divide a workgroup's 1024 (four per thread: 256, 8192) and
    ones that do not (one per thread: bf16 384 = 48 vectors, MX 7168 = 448), with a ragged end."""
    inp = synth.make_layer(T=300, H=H, F=128, E=7, k=3, dtype=dtype)
    _, _, perm, pos = oracle.route(inp.expert_ids, 7)
    d = dv.layer(inp)
    pos_d = dv.tensor(pos)
    if dtype == "mxfp8":
        xp, xsp = mel.permute(d.x, pos_d, 3, x_scale=d.x_scale)
        assert np.array_equal(dv.host(xsp), oracle.permute(inp.x_scale, perm, 3))
    else:
        xp = mel.permute(d.x, pos_d, 3)
    ref = oracle.permute(inp.x, perm, 3)
    got = xp.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else dv.host(xp)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dtype,k", [("bf16", 1), ("bf16", 2), ("bf16", 4), ("bf16", 8),
                                     ("f32", 1), ("f32", 2)])
def test_permute_unpermute_identity(dtype, k):
    """With the expert step replaced by the identity, unpermute(permute(x)) with probs 1/k gives x
    back bit for bit, and unit probs give k*x (power-of-two scalings and short exact sums)."""
    T, H, E = 257, 128, 8
    inp = synth.make_layer(T=T, H=H, F=64, E=E, k=k, dtype=dtype)
    d = dv.layer(inp)
    _, _, _, pos, _ = mel.route(d.expert_ids, E)
    xp = mel.permute(d.x, pos, k)
    x = dv.host(d.x)
    probs = torch.full((T, k), 1.0 / k, dtype=torch.float32, device="cuda")
    assert np.array_equal(dv.host(mel.unpermute(xp, pos, probs)), x)
    if k in (2, 4, 8) or (dtype == "f32" and k == 2):
        ones = torch.ones((T, k), dtype=torch.float32, device="cuda")
        assert np.array_equal(dv.host(mel.unpermute(xp, pos, ones)), np.float32(k) * x)


def test_unpermute_weighted_sum_matches_definition():
    rng = np.random.default_rng(4)
    T, k, H = 123, 4, 256
    y = rng.standard_normal((T * k, H)).astype(np.float32)
    perm = rng.permutation(T * k).astype(np.int32)
    pos = np.empty_like(perm)
    pos[perm] = np.arange(T * k, dtype=np.int32)
    probs = rng.random((T, k)).astype(np.float32)
    out = dv.host(mel.unpermute(dv.tensor(y), dv.tensor(pos), dv.tensor(probs)))
    ref = np.zeros((T, H))
    for j in range(k):
        ref += probs[:, j:j + 1].astype(np.float64) * y[pos.reshape(T, k)[:, j]]
    assert oracle.inf_norm_rel(out, ref) < 1e-6


@pytest.mark.parametrize("k,H", [(8, 4096), (12, 2176)])
def test_unpermute_bf16_many_slots_matches_definition(k, H):
    """bfloat16 unpermute with k >= 8 slots per token (one workgroup per row; k = 12 takes two
    batches of loads, H = 2176 gives rows of 272 vectors, more than one per lane for some lanes),
    some slots dropped (pos = -1): within one bfloat16 rounding of the fp64 weighted sum."""
    rng = np.random.default_rng(12)
    T = 97
    y_bits = synth.to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    perm = rng.permutation(T * k).astype(np.int32)
    pos = np.empty_like(perm)
    pos[perm] = np.arange(T * k, dtype=np.int32)
    pos[rng.random(T * k) < 0.1] = -1
    probs = rng.random((T, k)).astype(np.float32)
    out = dv.host(mel.unpermute(dv.tensor(y_bits), dv.tensor(pos), dv.tensor(probs)))
    y = synth.bf16_bits_to_f32(y_bits).astype(np.float64)
    ref = np.zeros((T, H))
    mag = np.zeros((T, H))                      # sum of |terms|: bounds the fp32 accumulation error
    pk = pos.reshape(T, k)
    for j in range(k):
        ok = pk[:, j] >= 0
        term = probs[ok, j:j + 1].astype(np.float64) * y[pk[ok, j]]
        ref[ok] += term
        mag[ok] += np.abs(term)
    # one bfloat16 rounding of the output (2^-9 relative) plus k fp32 roundings of the running sum
    assert (np.abs(out - ref) <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -18 * mag).all()


# ------------------------------------------------------------------------------------------ whole layer

CASES = [
    # name, dtype, T, H, F, E, k, routing kwargs
    ("tiny_f32_full_shape", "f32", 64, 128, 256, 4, 2, {}),
    ("f32_ragged", "f32", 75, 96, 160, 5, 2, {}),
    ("bf16_mixtral_like", "bf16", 384, 256, 448, 8, 2, {}),
    ("bf16_ragged_tail", "bf16", 333, 384, 192, 6, 2, {}),
    ("bf16_finegrained_like", "bf16", 256, 256, 128, 32, 8,
     {"routing": "zipf_gumbel", "zipf_s": 1.1, "n_zero": 4}),
    # large-tile path (H % 256 == 0, F % 128 == 0): several K steps, column tiles and ragged tiles
    ("bf16_large_tiles_ragged", "bf16", 700, 512, 384, 6, 2, {}),
    ("bf16_large_tiles_deep_k", "bf16", 300, 1024, 640, 3, 2, {}),
    # the most experts the routing takes: most experts empty or with one row, every tile partial
    ("bf16_many_experts", "bf16", 128, 256, 256, 1023, 8, {}),
]


@pytest.mark.parametrize("name,dtype,T,H,F,E,k,kw", CASES, ids=[c[0] for c in CASES])
def test_forward_matches_oracle(name, dtype, T, H, F, E, k, kw):
    inp = synth.make_layer(T=T, H=H, F=F, E=E, k=k, dtype=dtype, **kw)
    ref, *_ = oracle.forward(inp)
    d = dv.layer(inp)
    out = dv.host(dv.forward(mel, d))
    err = oracle.inf_norm_rel(out, ref)
    row_err = oracle.row_inf_norm_rel(out, ref)
    print(f"{name}: inf-norm rel err {err:.3e}, worst token {row_err:.3e}")
    assert err <= TOL[dtype]
    assert row_err <= TOL[dtype]       # per token, against that token's own largest output
    # determinism: a second call gives the same bits
    out2 = dv.host(dv.forward(mel, d))
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("head", [256, 512])
@pytest.mark.parametrize("T,H,F", [(700, 128, 192), (1100, 256, 256)], ids=["small_tiles", "large_tiles"])
def test_chunked_equals_unchunked(dtype, head, T, H, F):
    if dtype == "f32" and H > 128:
        pytest.skip("tile shapes are a bf16 matter")
    inp = synth.make_layer(T=T, H=H, F=F, E=5, k=2, dtype=dtype, seed=3)
    code = mel.F32 if dtype == "f32" else mel.BF16
    d = dv.layer(inp)
    base = dv.host(dv.forward(mel, d, 0))
    ws = torch.empty(mel.workspace_size(mel.problem(T, H, F, 5, 2, code, head)),
                     dtype=torch.uint8, device="cuda")
    out = dv.host(dv.forward(mel, d, head, workspace=ws))
    assert np.array_equal(out, base)
    done, expected = mel.chunk_counters(ws, 2 * T, H, F, head, code)
    torch.cuda.synchronize()
    assert done.shape[0] == -(-2 * T // head)
    assert np.array_equal(dv.host(done), dv.host(expected)) and dv.host(expected).min() > 0


def _layer_with_counts(counts, H, F, seed=11):
    """A bfloat16 k = 1 layer whose experts receive exactly `counts` tokens (seeded token order and
    routing weights; x and weights from the common generator)."""
    T, E = int(sum(counts)), len(counts)
    inp = synth.make_layer(T=T, H=H, F=F, E=E, k=1, dtype="bf16", seed=seed)
    rng = np.random.default_rng(seed)
    ids = rng.permutation(np.repeat(np.arange(E, dtype=np.int32), counts)).reshape(T, 1)
    probs = rng.uniform(0.5, 1.0, size=(T, 1)).astype(np.float32)
    return dataclasses.replace(inp, expert_ids=ids.astype(np.int32), probs=probs)


@pytest.mark.parametrize("counts", [[257, 300, 320, 321, 0, 64], [769, 812, 832, 833, 0, 64]],
                         ids=["small_groups", "large_groups"])
def test_short_partial_tiles_half_width_tasks(counts):
    """Last row tiles of 1, 44 and 64 rows and an expert with one 64-row tile beside a 65-row one and
    an empty expert.  With groups averaging at most two 256-row tiles (small_groups) both projections
    run every group's tiles in one run; with larger groups the down projection keeps the tails last
    and runs the short ones (at most 64 rows) as two half-width tasks each.  Either way the output
    matches the oracle, is bitwise the chunked one (chunked tables never split), and the backward that
    recomputes g and u (same kernel) is bitwise the one that takes the forward's saved values."""
    inp = _layer_with_counts(counts, H=512, F=256)
    ref, *_ = oracle.forward(inp)
    d = dv.layer(inp)
    out = dv.host(dv.forward(mel, d, 0))
    err = oracle.inf_norm_rel(out, ref)
    print(f"short tails: inf-norm rel err {err:.3e}")
    assert err <= TOL["bf16"]
    assert np.array_equal(dv.host(dv.forward(mel, d, 512)), out)
    dout = dv.tensor(synth.make_dout(inp))
    _, saved = mel.expert_forward_train(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs)
    a = mel.expert_backward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs, dout)
    b = mel.expert_backward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs, dout,
                            saved_gu=saved)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_invariances_bitwise():
    inp = synth.make_layer(T=200, H=128, F=128, E=6, k=2, dtype="bf16", seed=8)
    d = dv.layer(inp)
    base = dv.host(dv.forward(mel, d))
    rng = np.random.default_rng(1)
    tp = rng.permutation(200)
    tpi = torch.from_numpy(tp).cuda()
    d2 = dv.layer(inp)
    d2.x, d2.expert_ids, d2.probs = (d.x[tpi].contiguous(), d.expert_ids[tpi].contiguous(),
                                     d.probs[tpi].contiguous())
    assert np.array_equal(dv.host(dv.forward(mel, d2)), base[tp])
    rel = rng.permutation(6)
    inv = torch.from_numpy(np.argsort(rel)).cuda()
    d3 = dv.layer(inp)
    d3.w_gate, d3.w_up, d3.w_down = d.w_gate[inv].contiguous(), d.w_up[inv].contiguous(), d.w_down[inv].contiguous()
    d3.expert_ids = torch.from_numpy(rel.astype(np.int32)).cuda()[d.expert_ids.long()].contiguous()
    assert np.array_equal(dv.host(dv.forward(mel, d3)), base)
    d4 = dv.layer(inp)
    d4.probs = d.probs * 2
    out4 = dv.host(dv.forward(mel, d4))
    # bf16 output: doubling is exact unless the doubled value leaves bf16's range (it cannot here)
    assert np.array_equal(out4, 2 * base)


def test_empty_and_degenerate():
    # T = 0: nothing to do, call succeeds
    inp = synth.make_layer(T=0, H=128, F=64, E=4, k=2, dtype="bf16")
    d = dv.layer(inp)
    out = dv.forward(mel, d)
    assert out.shape == (0, 128)
    # every token to one expert (the other experts empty), k = 1, E = 1
    for E, k in ((3, 1), (1, 1)):
        inp = synth.make_layer(T=130, H=128, F=64, E=E, k=k, dtype="bf16", seed=2)
        inp.expert_ids[:] = E - 1
        ref, *_ = oracle.forward(inp)
        out = dv.host(dv.forward(mel, dv.layer(inp)))
        assert oracle.inf_norm_rel(out, ref) <= TOL["bf16"]


@pytest.mark.parametrize("dtype,T,H,F", [("bf16", 700, 512, 384), ("bf16", 333, 256, 192),
                                         ("mxfp8", 500, 1024, 1024), ("mxfp8", 300, 512, 512)],
                         ids=["bf16_large", "bf16_small", "mx_large", "mx_small"])
def test_permute_fused_into_fc1_is_bitwise_the_separate_kernel(dtype, T, H, F):
    """The default forward reads fc1's rows from x through the slot list (large tiles); the
    separate-permute flag runs the permute kernel first.  Same bits, unchunked and chunked; the
    small-tile sizes take the separate kernel either way."""
    inp = synth.make_layer(T=T, H=H, F=F, E=6, k=3, dtype=dtype, seed=21)
    d = dv.layer(inp)
    for head in (0, 512):
        fused = dv.host(dv.forward(mel, d, head))
        separate = dv.host(dv.forward(mel, d, head, separate_permute=True))
        assert np.array_equal(fused, separate)
    ref, *_ = oracle.forward(inp)
    assert oracle.inf_norm_rel(fused, ref) <= TOL[dtype]


def test_forward_out_of_range_ids_flagged():
    inp = synth.make_layer(T=100, H=128, F=64, E=4, k=2, dtype="bf16")
    inp.expert_ids[5, 1] = 9
    d = dv.layer(inp)
    ws = torch.empty(mel.workspace_size(mel.problem(100, 128, 64, 4, 2, mel.BF16)),
                     dtype=torch.uint8, device="cuda")
    out = dv.host(dv.forward(mel, d, workspace=ws))
    assert mel.device_status(ws) == 4
    # the dropped slot contributes nothing: token 5 gets only its first expert's share
    good = inp.expert_ids.copy()
    good[5, 1] = 0
    inp2 = synth.make_layer(T=100, H=128, F=64, E=4, k=2, dtype="bf16")
    inp2.expert_ids = good
    inp2.probs = inp.probs.copy()
    inp2.probs[5, 1] = 0.0
    ref, *_ = oracle.forward(inp2)
    assert oracle.inf_norm_rel(out, ref) <= TOL["bf16"]


def test_grouped_ffn_matches_oracle():
    g = synth.make_grouped(rows=900, H=256, F=192, E_local=2, sources=8, zipf_s=1.2, seed=2)
    ref = oracle.grouped_ffn(g)
    y = mel.grouped_ffn(dv.tensor(g.rows), dv.tensor(g.group_offsets), dv.tensor(g.group_expert),
                        dv.tensor(g.w_gate), dv.tensor(g.w_up), dv.tensor(g.w_down))
    assert oracle.inf_norm_rel(dv.host(y), ref) <= TOL["bf16"]
    assert oracle.row_inf_norm_rel(dv.host(y), ref) <= TOL["bf16"]
    y2 = mel.grouped_ffn(dv.tensor(g.rows), dv.tensor(g.group_offsets), dv.tensor(g.group_expert),
                         dv.tensor(g.w_gate), dv.tensor(g.w_up), dv.tensor(g.w_down),
                         head_m_size=256)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("sizes", [[257, 44, 64, 0, 65, 300], [1281, 44, 64, 0, 65, 1836]],
                         ids=["small_groups", "large_groups"])
def test_grouped_ffn_short_groups_large_tiles(sizes):
    """Source-major groups with partial tiles of 1, 44, 64 and 65 rows at large-tile sizes.  Groups
    averaging at most two 256-row tiles run their tiles as one run in both projections; larger ones
    (large_groups) run the down projection's short tails (at most 64 rows) as half-width tasks, the
    65-row one whole.  The output matches the oracle and is bitwise the chunked one."""
    g = synth.make_grouped(rows=sum(sizes), H=512, F=256, E_local=2, sources=3, seed=5)
    g = dataclasses.replace(g, group_offsets=np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32),
                            recv_counts=np.asarray(sizes, np.int64).reshape(3, 2))
    ref = oracle.grouped_ffn(g)
    args = (dv.tensor(g.rows), dv.tensor(g.group_offsets), dv.tensor(g.group_expert),
            dv.tensor(g.w_gate), dv.tensor(g.w_up), dv.tensor(g.w_down))
    y = mel.grouped_ffn(*args)
    err = oracle.inf_norm_rel(dv.host(y), ref)
    print(f"short groups: inf-norm rel err {err:.3e}")
    assert err <= TOL["bf16"]
    assert torch.equal(y, mel.grouped_ffn(*args, head_m_size=256))


@pytest.mark.parametrize("sizes", [[1, 31, 32, 33, 255, 256, 257, 0, 511, 512, 513, 1025],
                                   [767, 768, 769, 1023, 1024, 1026, 2, 0, 480, 544, 96, 160]],
                         ids=["tile_edges", "block_edges"])
def test_grouped_ffn_balanced_tile_edges(sizes):
    """Groups whose row counts sit at the edges of 32-row blocks and 256-row tiles, at large-tile
    sizes.  Unchunked, fc1 cuts every group into ceil(rows / 256) tiles of near-equal height (a
    group of 1025 rows: five tiles of 7, 7, 7, 6 and 6 blocks); fc2 does the same for the first set
    (groups averaging at most two tiles) and runs full tiles first with short tails split in two for
    the second.  Chunked tables cut each group's piece of a chunk the same way.  Every row matches
    the oracle, and the chunked results (512 and 256 rows) are bitwise the unchunked ones."""
    g = synth.make_grouped(rows=sum(sizes), H=256, F=256, E_local=3, sources=4, seed=7)
    g = dataclasses.replace(g, group_offsets=np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32),
                            recv_counts=np.asarray(sizes, np.int64).reshape(4, 3))
    ref = oracle.grouped_ffn(g)
    args = (dv.tensor(g.rows), dv.tensor(g.group_offsets), dv.tensor(g.group_expert),
            dv.tensor(g.w_gate), dv.tensor(g.w_up), dv.tensor(g.w_down))
    y = mel.grouped_ffn(*args)
    err, row_err = oracle.inf_norm_rel(dv.host(y), ref), oracle.row_inf_norm_rel(dv.host(y), ref)
    print(f"tile edges: inf-norm rel err {err:.3e}, worst row {row_err:.3e}")
    assert err <= TOL["bf16"] and row_err <= TOL["bf16"]
    for head in (512, 256):
        assert torch.equal(y, mel.grouped_ffn(*args, head_m_size=head))


def test_grouped_ffn_bad_group_expert_flagged():
    g = synth.make_grouped(rows=300, H=128, F=64, E_local=2, sources=8, seed=3)
    ge = g.group_expert.copy()
    ge[3] = 7
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    mel.grouped_ffn(dv.tensor(g.rows), dv.tensor(g.group_offsets), dv.tensor(ge),
                    dv.tensor(g.w_gate), dv.tensor(g.w_up), dv.tensor(g.w_down), workspace=ws)
    assert mel.device_status(ws) == 4


def test_mx_quantize_bit_exact():
    rng = np.random.default_rng(12)
    v = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-30, 30, (64, 1)))).astype(np.float32)
    v[0] = 0.0
    v[1, :32] = 1e-41                                   # float32 subnormals
    vals = np.array([oracle.e4m3_value(c) for c in range(127)])
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    v[2, :126] = np.resize(mids, 126)                    # ties, with a 448 anchor per block
    v[2, ::32] = 448.0
    v[3, :4] = [460.0, 464.0, 465.0, -0.0]
    v[3, 4] = 448.0
    codes, scales = mel.mx_quantize(dv.tensor(v))
    q, s = oracle.mx_quantize(v.astype(np.float64))
    assert np.array_equal(dv.host(scales), s)
    assert np.array_equal(dv.host(codes), q)


def _encoder_cases(rows, cols, seed):
    """float32 values that exercise the OCP-MX encoder: magnitudes spread over 60 binades per row,
    an all-zero row, subnormal blocks, E4M3 rounding midpoints (ties to even) with a 448 anchor per
    block, values just past the saturation point, negative zeros and a negative block."""
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-30, 30, (rows, 1)))).astype(np.float32)
    v[0] = 0.0
    v[1, :32] = 1e-41
    vals = np.array([oracle.e4m3_value(c) for c in range(127)])
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    n_mid = -(-mids.size // cols)                       # rows holding the 126 midpoints
    flat = v[2:2 + n_mid].reshape(-1)
    flat[:mids.size] = mids
    flat[::32] = 448.0                                  # the anchor that fixes each block's scale
    r = 2 + n_mid
    v[r, :4] = [460.0, 464.0, 465.0, -0.0]
    v[r, 4] = 448.0
    v[r + 1] = -np.abs(v[r + 1])
    v[r + 2, :32] = -0.0
    return v


def _broad_encoder_input():
    """[rows, 256] float32 blocks of 32 that pin the shared exponent to k (each block's first value is
    448 * 2^k, every other value at most that in magnitude): every finite bfloat16 value of magnitude
    at most 448, every E4M3 rounding midpoint and its float32 neighbours one ulp away on both sides,
    and 100000 uniform values in (-448, 448), each set at k = -100, -20, 0, 37 and 100 (so the
    encoder sees v * 2^k and must code v)."""
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    bf = bits.view(np.float32)
    bf = bf[np.isfinite(bf) & (np.abs(bf) <= 448.0)]
    vals = np.array([oracle.e4m3_value(c) for c in range(127)], np.float64)
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    mids = np.concatenate([mids, -mids])
    near = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))])
    near = near[np.abs(near) <= 448.0]
    rnd = np.random.default_rng(9).uniform(-448, 448, 100000).astype(np.float32)
    body = np.concatenate([bf, near, rnd]).astype(np.float32)
    body = np.resize(body, -(-body.size // 31) * 31).reshape(-1, 31)
    blocks = np.concatenate([np.full((body.shape[0], 1), 448.0, np.float32), body], axis=1)
    flat = np.concatenate([np.ldexp(blocks, k).astype(np.float32) for k in (-100, -20, 0, 37, 100)])
    flat = flat.reshape(-1)
    return np.resize(flat, -(-flat.size // 256) * 256).reshape(-1, 256)


def test_mx_encoders_bit_exact_on_every_bf16_value_and_rounding_midpoint():
    """The library's E4M3 encoding (hardware conversion of v / 2^e, clamped to the E4M3 range) on a
    broad input: the standalone encoder and both fc1 epilogues code every value as the oracle does."""
    v = _broad_encoder_input()
    q, sc = oracle.mx_quantize(v.astype(np.float64))
    vd = dv.tensor(v)
    codes, scales = mel.mx_quantize(vd)
    assert np.array_equal(dv.host(scales), sc) and np.array_equal(dv.host(codes), q)
    for large in (True, False):
        rows = min(v.shape[0], (1 << 28) // v.shape[1])
        c2, s2 = mel.mx_fc1_epilogue_encode(vd[:rows].contiguous(), large_tiles=large)
        assert np.array_equal(dv.host(s2), sc[:rows]) and np.array_equal(dv.host(c2), q[:rows])


@pytest.mark.parametrize("large,rows,cols", [(True, 300, 384), (True, 256, 128), (True, 37, 256),
                                             (False, 300, 192), (False, 128, 64), (False, 37, 128)],
                         ids=["large_ragged", "large_one_tile", "large_short", "small_ragged",
                              "small_one_tile", "small_short"])
def test_mx_fc1_epilogue_encoder_bit_exact(large, rows, cols):
    """fc1's MX epilogue (the GEMM kernels' own device code: accumulator registers -> LDS staging ->
    block maximum across lanes -> integer encoder -> stores) fed float32 values the host knows
    exactly, in place of the SwiGLU output: every code and every block scale equals the oracle's
    encoding of the same values, including ragged row tiles."""
    v = _encoder_cases(rows, cols, seed=rows + cols)
    codes, scales = mel.mx_fc1_epilogue_encode(dv.tensor(v), large_tiles=large)
    q, sc = oracle.mx_quantize(v.astype(np.float64))
    assert np.array_equal(dv.host(scales), sc)
    assert np.array_equal(dv.host(codes), q)


# ------------------------------------------------------------------------------------------ MX-FP8

def _dec_mx(codes, scales, axis):
    v = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()
    return v * np.repeat(np.exp2(np.asarray(scales, np.float64) - 127), 32, axis=axis)


def _mx_weights64(src):
    return (_dec_mx(src.w_gate, src.wg_scale, 1), _dec_mx(src.w_up, src.wu_scale, 1),
            _dec_mx(src.w_down, src.wd_scale, 1))


@pytest.mark.parametrize("T,H,F,E,k", [(200, 256, 256, 6, 4), (333, 384, 128, 5, 2),
                                       (96, 128, 384, 32, 4),
                                       (300, 512, 512, 5, 2),
                                       # large tiles (H, F multiples of 1024): ragged tails, K loops
                                       # of one and of several 16-step units
                                       (300, 1024, 2048, 5, 2), (700, 2048, 1024, 3, 2)])
def test_mx_forward_matches_oracle(T, H, F, E, k):
    inp = synth.make_layer(T=T, H=H, F=F, E=E, k=k, dtype="mxfp8", seed=T)
    ref, *_ = oracle.forward(inp)
    d = dv.layer(inp)
    out = dv.host(dv.forward(mel, d))
    err = oracle.inf_norm_rel(out, ref)
    row_err = oracle.row_inf_norm_rel(out, ref)
    print(f"mx T={T} H={H} F={F}: inf-norm rel err {err:.3e}, worst token {row_err:.3e}")
    assert err <= TOL["mxfp8"]
    assert row_err <= TOL["mxfp8"]
    assert np.array_equal(out, dv.host(dv.forward(mel, d)))


def _e4m3_codes(v):
    """E4M3 codes of float64 values already divided by their block scale (round to nearest even,
    saturated to +-448), through torch's float8_e4m3fn conversion; used only to classify which
    codes the GPU's accumulation error can move, never as the expected codes themselves."""
    t = torch.from_numpy(np.clip(v, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("T,H,F,E,k", [(200, 256, 384, 4, 2), (300, 1024, 1024, 3, 2)],
                         ids=["small_tiles", "large_tiles"])
def test_mx_h_encoding_agrees_with_oracle(T, H, F, E, k):
    """fc1's MX-encoded SwiGLU output, read back from the workspace, against the oracle's encoding
    of the exact h.  The GPU's g and u carry the scaled fp8 MFMA's accumulation error (measured: at
    most 1.5e-5 of the sum of |terms|; 6e-5 is assumed here) and the SwiGLU its hardware exp2 and
    reciprocal (2e-6 relative assumed), which bounds how far the GPU's h can sit from the exact one.
    Every block whose scale no h within that bound can change must carry the oracle's scale, and in
    such blocks every code that no h within the bound can change must be the oracle's code; the
    codes and scales left undecided must stay a small fraction (the encoder itself is checked
    bit-exactly on exact inputs by test_mx_fc1_epilogue_encoder_bit_exact)."""
    inp = synth.make_layer(T=T, H=H, F=F, E=E, k=k, dtype="mxfp8", seed=11)
    counts, offs, perm, _ = oracle.route(inp.expert_ids, E)
    xp, xps = oracle.permute(inp.x, perm, k), oracle.permute(inp.x_scale, perm, k)
    M = T * k
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    mel.grouped_ffn_mx(dv.tensor(xp), dv.tensor(xps), dv.tensor(offs),
                       dv.tensor(np.arange(E, dtype=np.int32)), dv.tensor(inp.w_gate),
                       dv.tensor(inp.wg_scale), dv.tensor(inp.w_up), dv.tensor(inp.wu_scale),
                       dv.tensor(inp.w_down), dv.tensor(inp.wd_scale), workspace=ws)
    hq_d, hs_d = mel.intermediate_h(ws, M, E, H, F, E, mel.MXFP8)
    hq, hs = dv.host(hq_d), dv.host(hs_d)
    X = _dec_mx(xp, xps, 1)
    Wg, Wu, _ = _mx_weights64(inp)
    row_e = np.repeat(np.arange(E), counts)
    h64 = np.empty((M, F))
    bound = np.empty((M, F))
    for e in range(E):
        rows = row_e == e
        g, u = X[rows] @ Wg[e], X[rows] @ Wu[e]
        sg, su = np.abs(X[rows]) @ np.abs(Wg[e]), np.abs(X[rows]) @ np.abs(Wu[e])
        sig = 1.0 / (1.0 + np.exp(-g))
        h64[rows] = g * sig * u
        dh_dg = np.abs(sig * (1.0 + g * (1.0 - sig)) * u)
        dh_du = np.abs(g * sig)
        bound[rows] = 6e-5 * (dh_dg * sg + dh_du * su) + 2e-6 * np.abs(h64[rows])
    q64, s64 = oracle.mx_quantize(h64)

    blocks = lambda a: a.reshape(M, F // 32, 32)
    lo = np.maximum(np.abs(h64) - bound, 0.0)
    hi = np.abs(h64) + bound
    # the scale exponent floor(log2 amax) - 8 of any h within the bound lies between these two
    e_lo = np.floor(np.log2(np.maximum(blocks(lo).max(axis=2), 1e-300)))
    e_hi = np.floor(np.log2(np.maximum(blocks(hi).max(axis=2), 1e-300)))
    nz = blocks(lo).max(axis=2) > 0
    scale_decided = (e_lo == e_hi) & nz & (e_hi - 8 >= -127) & (e_hi - 8 <= 127)
    assert np.array_equal(hs[scale_decided], s64[scale_decided])
    # codes in blocks with a decided scale: decided when both ends of the bound encode alike
    sc = np.repeat(np.exp2(s64.astype(np.float64) - 127), 32, axis=1)
    c_lo, c_hi = _e4m3_codes((h64 - bound) / sc), _e4m3_codes((h64 + bound) / sc)
    code_decided = np.repeat(scale_decided, 32, axis=1) & (c_lo == c_hi) & (c_lo == q64)
    assert np.array_equal(hq[code_decided], q64[code_decided])
    und_s = 1.0 - scale_decided[nz].mean()
    und_c = 1.0 - code_decided.mean()
    mis_s, mis_c = (hs != s64).mean(), (hq != q64).mean()
    print(f"h encoding: undecided scales {und_s:.2e}, undecided codes {und_c:.2e}; mismatches: "
          f"scales {mis_s:.2e}, codes {mis_c:.2e}")
    # the bound leaves 0.2-0.6% of the scales and 12-20% of the codes undecided at these shapes
    # (computed from the oracle's h alone); more would make the exact comparison above vacuous
    assert und_s < 1e-2 and und_c < 0.3
    # measured: no scale and 0.17% of the codes differ (all of them undecided ones)
    assert mis_s < 1e-3 and mis_c < 5e-3
    # value check: each decoded element is within the worst-case E4M3 rounding of its block (half a
    # top-binade step is 1/16 of amax, saturation at 448 loses up to 1/8) of the exact h
    amax = np.repeat(np.abs(h64).reshape(M, F // 32, 32).max(axis=2), 32, axis=1)
    err = np.abs(_dec_mx(hq, hs, 1) - h64) / np.maximum(amax, 1e-30)
    assert err.max() <= 0.125 + 1e-6


@pytest.mark.parametrize("T,H,F", [(600, 256, 256), (1100, 1024, 1024)], ids=["small_tiles", "large_tiles"])
def test_mx_chunked_equals_unchunked(T, H, F):
    inp = synth.make_layer(T=T, H=H, F=F, E=7, k=2, dtype="mxfp8", seed=5)
    d = dv.layer(inp)
    base = dv.host(dv.forward(mel, d, 0))
    assert np.array_equal(dv.host(dv.forward(mel, d, 256)), base)
    assert np.array_equal(dv.host(dv.forward(mel, d, 512)), base)


@pytest.mark.parametrize("H,F", [(256, 256), (1024, 1024)], ids=["small_tiles", "large_tiles"])
def test_mx_grouped_ffn_matches_oracle(H, F):
    g = synth.make_grouped(rows=700, H=H, F=F, E_local=2, sources=8, dtype="mxfp8", seed=4)
    ref = oracle.grouped_ffn(g)
    y = mel.grouped_ffn_mx(dv.tensor(g.rows), dv.tensor(g.rows_scale), dv.tensor(g.group_offsets),
                           dv.tensor(g.group_expert), dv.tensor(g.w_gate), dv.tensor(g.wg_scale),
                           dv.tensor(g.w_up), dv.tensor(g.wu_scale), dv.tensor(g.w_down),
                           dv.tensor(g.wd_scale))
    assert oracle.inf_norm_rel(dv.host(y), ref) <= TOL["mxfp8"]
    assert oracle.row_inf_norm_rel(dv.host(y), ref) <= TOL["mxfp8"]
