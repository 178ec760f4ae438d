"""CPU-only checks of the C ABI: the shared library loads, exports every function the public header
declares, and rejects bad arguments on the host before enqueueing anything (no GPU needed: these
paths return before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_expert_layer.h")


@pytest.fixture(scope="module")
def mel():
    import moe_expert_layer_amd as m
    if not os.path.exists(m.lib_path):
        from moe_expert_layer_amd.build import build
        build(verbose=False)
    m.library()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("moe_expert_forward", "moe_expert_forward_mx", "moe_route", "moe_permute",
                     "moe_unpermute", "moe_grouped_ffn", "moe_grouped_ffn_mx", "moe_workspace_size",
                     "moe_query_device_status", "moe_mx_quantize"):
        assert required in names


def test_library_exports_every_declared_symbol(mel):
    lib = ctypes.CDLL(mel.lib_path)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def _status(mel, prob):
    n = ctypes.c_size_t()
    return mel.library().moe_workspace_size(ctypes.byref(prob), ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw,expected", [
    (dict(T=64, H=128, F=256, E=4, k=2, dtype=0), 0),
    (dict(T=64, H=128, F=256, E=4, k=5, dtype=0), 1),          # k > E
    (dict(T=-1, H=128, F=256, E=4, k=2, dtype=0), 1),
    (dict(T=64, H=0, F=256, E=4, k=2, dtype=0), 1),
    (dict(T=64, H=128, F=256, E=4, k=2, dtype=7), 2),          # unknown dtype
    (dict(T=64, H=128, F=256, E=1023, k=2, dtype=0), 0),
    (dict(T=64, H=128, F=256, E=1024, k=2, dtype=0), 2),       # more experts than supported
    (dict(T=64, H=100, F=256, E=4, k=2, dtype=1), 2),          # bf16 tile divisibility
    (dict(T=64, H=128, F=96, E=4, k=2, dtype=1), 2),
    (dict(T=64, H=4096, F=14336, E=8, k=2, dtype=1), 0),
    (dict(T=64, H=7168, F=2048, E=32, k=4, dtype=2), 0),
    (dict(T=64, H=7168, F=2000, E=32, k=4, dtype=2), 2),       # MX: multiples of 128
    (dict(T=64, H=128, F=256, E=4, k=2, dtype=1, head_m_size=300), 1),
    (dict(T=64, H=128, F=256, E=4, k=2, dtype=1, head_m_size=512), 0),
    (dict(T=64, H=128, F=256, E=4, k=2, dtype=0, flags=1), 0),      # MOE_FLAG_SEPARATE_PERMUTE
    (dict(T=64, H=128, F=256, E=4, k=2, dtype=0, flags=2), 1),      # unknown flag bit
    # H and F at most 2^22: the GEMMs' 32-bit offsets from a row tile's first row
    (dict(T=64, H=1 << 22, F=256, E=4, k=2, dtype=1), 0),
    (dict(T=64, H=(1 << 22) + 128, F=256, E=4, k=2, dtype=1), 2),
    (dict(T=64, H=128, F=(1 << 22) + 64, E=4, k=2, dtype=1), 2),
    (dict(T=64, H=(1 << 22) + 128, F=256, E=4, k=2, dtype=2), 2),
])
def test_problem_validation(mel, kw, expected):
    kw = dict(kw)
    flags = kw.pop("flags", 0)
    head = kw.pop("head_m_size", 0)
    prob = mel.problem(**kw, head_m_size=head)
    prob.flags = flags
    st, n = _status(mel, prob)
    assert st == expected, mel.library().moe_last_error()
    if st == 0:
        M = kw["T"] * kw["k"]
        esz = {0: 4, 1: 2, 2: 1}[kw["dtype"]]
        ysz = 4 if kw["dtype"] == 0 else 2
        assert n >= M * kw["H"] * esz + M * kw["F"] * esz + M * kw["H"] * ysz


def test_forward_rejects_before_enqueue(mel):
    lib = mel.library()
    prob = mel.problem(64, 128, 256, 4, 2, mel.BF16)
    need = mel.workspace_size(prob)
    # workspace too small / missing
    st = lib.moe_expert_forward(ctypes.byref(prob), None, None, None, None, None, None, None, None,
                                0, None)
    assert st == 3 and b"workspace" in lib.moe_last_error()
    # null data pointers with a (fake, never dereferenced) workspace of the right size
    st = lib.moe_expert_forward(ctypes.byref(prob), None, None, None, None, None, None, None,
                                ctypes.c_void_p(0x1000), need, None)
    assert st == 1
    # MX entry with a non-MX problem and vice versa
    st = lib.moe_expert_forward_mx(ctypes.byref(prob), *([None] * 12), 0, None)
    assert st == 1
    mx = mel.problem(64, 128, 256, 4, 2, mel.MXFP8)
    st = lib.moe_expert_forward(ctypes.byref(mx), *([None] * 8), 0, None)
    assert st == 1


def test_route_and_grouped_sizes(mel):
    lib = mel.library()
    n = ctypes.c_size_t()
    assert lib.moe_route_workspace_size(4096, 2, 8, ctypes.byref(n)) == 0 and n.value > 0
    assert lib.moe_route_workspace_size(4096, 9, 8, ctypes.byref(n)) == 1
    assert lib.moe_route_workspace_size(16, 1, 5000, ctypes.byref(n)) == 2
    prob = mel.problem(0, 4096, 14336, 2, 1, mel.BF16)
    assert lib.moe_grouped_ffn_workspace_size(ctypes.byref(prob), 16384, 16, ctypes.byref(n)) == 0
    assert n.value >= 16384 * 14336 * 2
    assert lib.moe_grouped_ffn_workspace_size(ctypes.byref(prob), -1, 16, ctypes.byref(n)) == 1
    st = lib.moe_mx_quantize(None, 4, 33, None, None, None)
    assert st == 1


def test_status_strings(mel):
    lib = mel.library()
    names = [lib.moe_status_string(i).decode() for i in range(6)]
    assert names == ["MOE_OK", "MOE_ERR_INVALID_ARGUMENT", "MOE_ERR_UNSUPPORTED",
                     "MOE_ERR_WORKSPACE_TOO_SMALL", "MOE_ERR_EXPERT_ID_OUT_OF_RANGE", "MOE_ERR_HIP"]


@pytest.mark.parametrize("kw,expected", [
    (dict(T=64, H=128, F=256, E=4, k=2, dtype=1), 0),
    (dict(T=0, H=128, F=256, E=4, k=2, dtype=1), 0),
    (dict(T=64, H=128, F=256, E=4, k=2, dtype=0), 2),          # the backward is bf16 only
    (dict(T=64, H=128, F=256, E=4, k=2, dtype=2), 2),
    (dict(T=64, H=128, F=192, E=4, k=2, dtype=1), 2),          # F % 128
    (dict(T=64, H=4096, F=14336, E=8, k=2, dtype=1), 0),
    (dict(T=64, H=128, F=256, E=4, k=2, dtype=1, head_m_size=256), 2),   # unchunked only
])
def test_backward_validation(mel, kw, expected):
    prob = mel.problem(**kw)
    n = ctypes.c_size_t()
    assert mel.library().moe_backward_workspace_size(ctypes.byref(prob), ctypes.byref(n)) == expected
    if expected == 0:
        assert n.value > 0


def test_backward_rejects_before_enqueue(mel):
    lib = mel.library()
    prob = mel.problem(64, 128, 256, 4, 2, mel.BF16)
    n = ctypes.c_size_t()
    assert lib.moe_backward_workspace_size(ctypes.byref(prob), ctypes.byref(n)) == 0
    st = lib.moe_expert_backward(ctypes.byref(prob), *([None] * 14), 0, None)
    assert st == 3 and b"workspace" in lib.moe_last_error()
    st = lib.moe_expert_backward(ctypes.byref(prob), *([None] * 13), ctypes.c_void_p(0x1000),
                                 n.value, None)
    assert st == 1
    # saving g and u: bf16 only, and saved_gu must be given
    need = mel.workspace_size(prob)
    st = lib.moe_expert_forward_train(ctypes.byref(prob), *([None] * 8), ctypes.c_void_p(0x1000),
                                      need, None)
    assert st == 1 and b"saved_gu" in lib.moe_last_error()
    f32 = mel.problem(64, 128, 256, 4, 2, mel.F32)
    st = lib.moe_expert_forward_train(ctypes.byref(f32), *([None] * 9), 0, None)
    assert st == 2


def test_route_noalloc_rejects_before_touching_the_gpu(mel):
    """The allocation-free route checks sizes against its static scratch (4 MiB of block counts)
    and its arguments on the host, before any HIP call."""
    lib = mel.library()
    # 1026 routing blocks x 1024 counts: beyond the scratch
    assert lib.moe_route_noalloc(None, 2048 * 1025 + 1, 1, 1023, None, None, None, None, None) == 2
    assert b"scratch" in lib.moe_last_error()
    assert lib.moe_route_noalloc(None, 16, 3, 2, None, None, None, None, None) == 1     # k > E
    assert lib.moe_route_noalloc(None, 16, 2, 8, None, None, None, None, None) == 1     # null outputs


def test_quantize_x_flag(mel):
    """MOE_FLAG_QUANTIZE_X is an MX-only flag; its workspace adds the token-order encoded x
    (T*H codes + T*H/32 scales), and the offsets query needs the flag."""
    lib = mel.library()
    n0, n1 = ctypes.c_size_t(), ctypes.c_size_t()
    bf = mel.problem(64, 128, 128, 4, 2, mel.BF16, 0, mel.FLAG_QUANTIZE_X)
    assert lib.moe_workspace_size(ctypes.byref(bf), ctypes.byref(n0)) == 1
    T, H = 300, 1024
    mx = mel.problem(T, H, 1024, 5, 2, mel.MXFP8, 0, 0)
    mxq = mel.problem(T, H, 1024, 5, 2, mel.MXFP8, 0, mel.FLAG_QUANTIZE_X)
    assert lib.moe_workspace_size(ctypes.byref(mx), ctypes.byref(n0)) == 0
    assert lib.moe_workspace_size(ctypes.byref(mxq), ctypes.byref(n1)) == 0
    assert n1.value >= n0.value + T * H + T * H // 32
    co, so, pm = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int32()
    assert lib.moe_quantized_x_offsets(ctypes.byref(mx), ctypes.byref(co), ctypes.byref(so),
                                       ctypes.byref(pm)) == 1
    assert lib.moe_quantized_x_offsets(ctypes.byref(mxq), ctypes.byref(co), ctypes.byref(so),
                                       ctypes.byref(pm)) == 0
    assert pm.value == 0 and so.value >= co.value + T * H and so.value + T * H // 32 <= n1.value
    # a bfloat16 x with a scale pointer is refused before anything is enqueued
    st = lib.moe_expert_forward_mx(ctypes.byref(mxq), ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1000),
                                   *([ctypes.c_void_p(0x1000)] * 9), ctypes.c_void_p(0x1000), n1.value,
                                   None)
    assert st == 1 and b"x_scale" in lib.moe_last_error()


def test_probe_entry_only_in_the_probe_library(mel):
    """moe_probe_phases (include/moe_expert_layer_probe.h) is exported by the probe build alone."""
    from moe_expert_layer_amd.build import PROBE_LIB_PATH
    probe_header = os.path.join(os.path.dirname(HEADER), "moe_expert_layer_probe.h")
    text = re.sub(r"/\*.*?\*/", "", open(probe_header).read(), flags=re.S)
    assert re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text) == ["moe_probe_phases"]
    assert not hasattr(ctypes.CDLL(mel.lib_path), "moe_probe_phases")
    if not os.path.exists(PROBE_LIB_PATH):
        pytest.skip("probe library not built")
    assert hasattr(ctypes.CDLL(PROBE_LIB_PATH), "moe_probe_phases")
