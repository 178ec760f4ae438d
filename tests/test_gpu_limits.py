"""Parity at the edge of the supported sizes: a bfloat16 grouped FFN on the 128-row-tile kernels
(H % 256 != 0) whose activation matrix holds more than 2^32 elements.  The kernels address a row
tile's rows by 32-bit offsets from the tile's first row, so rows past element 2^32 must come out as
right as the first ones; they are checked against the oracle on sampled rows on both sides of that
point and at the very end."""
import numpy as np
import pytest
import torch

import moe_expert_layer_amd as mel
import oracle
import synth

pytestmark = pytest.mark.gpu


def test_small_tiles_beyond_2_32_elements():
    H, F, E = 384, 64, 2
    boundary = -(-(1 << 32) // H)                     # first row whose first element lies past 2^32
    M = boundary + 3000
    sizes = [M // 3, 5, M - M // 3 - 5]
    experts = [1, 0, 1]
    print(f"[limits] M={M} H={H} F={F}: {M * H} elements of bf16 rows", flush=True)
    w = synth.make_layer(T=1, H=H, F=F, E=E, k=1, dtype="bf16", seed=17)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(17)
    rows = torch.randn((M, H), generator=gen, device="cuda", dtype=torch.bfloat16)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    y = mel.grouped_ffn(rows, torch.from_numpy(offs).cuda(),
                        torch.tensor(experts, dtype=torch.int32, device="cuda"),
                        *(torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
                          for a in (w.w_gate, w.w_up, w.w_down)))
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    idx = np.unique(np.concatenate([
        [0, 1, boundary - 1, boundary, boundary + 1, M - 1], offs[1:-1] - 1, offs[1:-1],
        rng.integers(boundary, M, 24), rng.integers(0, boundary, 8)]))
    idx_d = torch.from_numpy(idx).cuda()
    got = y[idx_d].float().cpu().numpy()
    sample = rows[idx_d].view(torch.int16).cpu().numpy().view(np.uint16)
    row_expert = np.repeat(np.asarray(experts, np.int32), sizes)[idx]
    ref = oracle.ffn_rows("bf16", sample, row_expert, w.w_gate, w.w_up, w.w_down)
    err, row_err = oracle.inf_norm_rel(got, ref), oracle.row_inf_norm_rel(got, ref)
    print(f"[limits] {len(idx)} sampled rows: inf-norm rel err {err:.3e}, worst row {row_err:.3e}",
          flush=True)
    assert np.isfinite(got).all()
    assert err <= 2e-2 and row_err <= 2e-2
