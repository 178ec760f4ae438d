"""The allocation-free routing entry point, moe_route_noalloc, called through the C ABI: its counts,
offsets, perm and pos equal moe_route's (which uses a caller workspace) bit for bit, on two calls
in a row whose second input is smaller than the first, so that the static scratch still holds the
first call's block counts and status when the second call runs."""
import ctypes

import numpy as np
import pytest

import oracle
from synth import device as dv

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mel = pytest.importorskip("moe_expert_layer_amd")

@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    return mel.library()


def _ids(T, k, E, seed, n_bad):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    bad = rng.choice(T * k, n_bad, replace=False)
    ids.ravel()[bad[: n_bad // 2]] = E + 5
    ids.ravel()[bad[n_bad // 2:]] = -2
    return ids


def _route_noalloc(lib, ids_d, E):
    T, k = ids_d.shape
    i32 = dict(dtype=torch.int32, device=ids_d.device)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    perm, pos = torch.empty(T * k, **i32), torch.empty(T * k, **i32)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.moe_route_noalloc(ctypes.c_void_p(ids_d.data_ptr()), T, k, E,
                               ctypes.c_void_p(counts.data_ptr()), ctypes.c_void_p(offsets.data_ptr()),
                               ctypes.c_void_p(perm.data_ptr()), ctypes.c_void_p(pos.data_ptr()), stream)
    assert st == 0, lib.moe_last_error()
    return counts, offsets, perm, pos


@pytest.mark.parametrize("first,second", [((6000, 8, 300, 11, 40), (700, 2, 8, 12, 6)),
                                          ((4096, 2, 8, 13, 0), (1, 1, 1, 14, 0))],
                         ids=["bad_ids_then_small", "mixtral_then_one_slot"])
def test_route_noalloc_equals_route_on_two_calls(lib, first, second):
    for T, k, E, seed, n_bad in (first, second):
        print(f"[no-alloc] T={T} k={k} E={E} seed={seed} bad={n_bad}", flush=True)
        ids = _ids(T, k, E, seed, n_bad)
        ids_d = dv.tensor(ids)
        got = _route_noalloc(lib, ids_d, E)
        ref = mel.route(ids_d, E)
        wrapped = mel.route_noalloc(ids_d, E)
        torch.cuda.synchronize()
        for a, b in zip(wrapped, ref[:4]):
            assert torch.equal(a, b)
        for a, b in zip(got, ref[:4]):
            assert torch.equal(a, b)
        if n_bad == 0:
            oc, oo, op, opos = oracle.route(ids, E)
            for a, b in zip(got, (oc, oo, op, opos)):
                assert np.array_equal(dv.host(a), b)
        else:
            assert int(dv.host(got[1])[E]) == T * k - n_bad      # offsets[E] tells of dropped slots


def test_route_noalloc_rejects_sizes_beyond_its_scratch(lib):
    # 1026 routing blocks of 2048 slots x 1024 counts exceed the 4 MiB of block counts
    st = lib.moe_route_noalloc(None, 2048 * 1025 + 1, 1, 1023, None, None, None, None, None)
    assert st == 2 and b"scratch" in lib.moe_last_error()
