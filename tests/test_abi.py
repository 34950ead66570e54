"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, plans launches on the host, and rejects bad arguments before
touching a device."""

import ctypes
import math
import os
import re

import pytest

from quantized_decode_gemv_q8_amd import binding
from quantized_decode_gemv_q8_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8_gemv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB_PATH), reason="libq8gemv.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q8_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert header_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(5):
        s = binding.q8_status_string(code)
        assert s.startswith("Q8_")
    assert binding.q8_status_string(99) == "unknown q8_status"
    assert binding.q8_last_hip_error() == 0


# ------------------------------------------------------------------ plan (host logic)

def plan(M, K, N, w_align=256, s_align=256, cus=256):
    return binding.q8_matvec_choose_plan(M, K, N, w_align, s_align, cus)


@pytest.mark.parametrize("M,K,N", [(1, 256, 128), (1, 4096, 4096), (1, 8192, 28672), (1, 28672, 8192),
                                   (4, 4100, 5000), (3, 33, 7), (9, 1000, 17), (16, 64, 64), (1, 1, 1)])
def test_plan_is_valid_and_normalised(M, K, N):
    p = plan(M, K, N)
    KB = math.ceil(K / 32)
    if p["kind"] == binding.PLAN_MATRIX:
        # matrix cores: 2..64 rows, N a multiple of 4, 512-column tiles x K splits, 8 waves
        assert 2 <= M <= 64 and N % 4 == 0 and p["vec"] == 0 and p["m_tile"] == 0 and p["waves"] == 8
        tiles = math.ceil(N / 512)
        assert p["workgroups"] % tiles == 0
        splits = p["workgroups"] // tiles
        assert 1 <= splits <= KB and math.ceil(KB / math.ceil(KB / splits)) == splits
        return
    assert p["kind"] == binding.PLAN_STREAM
    assert p["vec"] in (16, 8, 4, 2, 1) and N % p["vec"] == 0
    assert p["m_tile"] in (1, 2, 4, 8) and p["m_tile"] * p["vec"] <= 32
    assert p["waves"] == 4
    units = math.ceil(N / (64 * p["vec"])) * math.ceil(KB / 4)  # (column tile, 4-block group) units
    assert 1 <= p["workgroups"] <= units        # every workgroup holds at least one unit
    count_max = math.ceil(units / p["workgroups"])
    assert p["m_tile"] * count_max * 32 <= 64 * 8  # a wave's activations fit its staging registers


def test_plan_vec_follows_shape_and_alignment():
    assert plan(1, 8192, 28672)["vec"] == 8     # automatic plans use at most 8-byte lanes
    assert plan(1, 4096, 4096)["vec"] == 4      # under 2 units per CU at vec 8: 4-byte lanes
    assert plan(1, 4096, 4096, cus=64)["vec"] == 8
    assert plan(4, 4100, 5000)["vec"] == 4      # 4 rows on the stream (K*N < 2^25): vec * m_tile <= 16
    assert plan(2, 12288, 8200)["vec"] == 8     # 2 rows on the stream (K*N < 2^27): 2 * 8 <= 16
    assert plan(1, 64, 4100)["vec"] == 4
    assert plan(1, 64, 4096, w_align=4)["vec"] == 4
    assert plan(1, 64, 4096, s_align=8)["vec"] == 2
    assert plan(1, 64, 7)["vec"] == 1
    assert plan(8, 64, 4100)["vec"] == 2        # 8 rows on the stream (a small W): 8 * vec <= 16
    assert plan(2, 64, 4104)["m_tile"] == 2


def test_plan_kind_follows_rows_and_layout():
    assert plan(1, 8192, 28672)["kind"] == binding.PLAN_STREAM
    assert plan(1, 64, 4096)["kind"] == binding.PLAN_STREAM        # one row: the matvec
    assert plan(2, 8192, 28672)["kind"] == binding.PLAN_MATRIX
    assert plan(32, 8192, 28672)["kind"] == binding.PLAN_MATRIX
    assert plan(33, 8192, 28672)["kind"] == binding.PLAN_MATRIX    # the 64-row instance
    assert plan(64, 8192, 28672)["kind"] == binding.PLAN_MATRIX
    assert plan(65, 8192, 28672)["kind"] == binding.PLAN_STREAM    # above it
    # ragged N: the matrix cores read W in 8- or 4-byte pieces, as long as
    # W rows are 4-byte aligned and S rows 16-byte aligned
    assert plan(16, 8192, 5000)["kind"] == binding.PLAN_MATRIX     # N % 8 == 0
    assert plan(16, 8192, 5004)["kind"] == binding.PLAN_MATRIX     # N % 4 == 0
    assert plan(16, 8192, 4096, w_align=4)["kind"] == binding.PLAN_MATRIX
    assert plan(16, 8192, 5002)["kind"] == binding.PLAN_STREAM     # N % 4 != 0
    assert plan(16, 8192, 4096, w_align=2)["kind"] == binding.PLAN_STREAM
    assert plan(16, 8192, 4096, s_align=8)["kind"] == binding.PLAN_STREAM
    # at 2 rows the matrix cores pay only with 16-byte W loads
    assert plan(2, 8192, 28672)["kind"] == binding.PLAN_MATRIX
    assert plan(2, 8192, 28680)["kind"] == binding.PLAN_STREAM     # N % 16 == 8
    assert plan(2, 8192, 28672, w_align=8)["kind"] == binding.PLAN_STREAM
    assert plan(3, 8192, 12296)["kind"] == binding.PLAN_MATRIX     # from 3 rows 8-byte loads still pay
    # up to 4 rows of a small W stay on the stream; 5 rows or a large W go to the matrix cores
    assert plan(4, 4096, 4096)["kind"] == binding.PLAN_STREAM
    assert plan(2, 4096, 4096)["kind"] == binding.PLAN_STREAM
    assert plan(5, 4096, 4096)["kind"] == binding.PLAN_MATRIX
    assert plan(3, 8192, 28672)["kind"] == binding.PLAN_MATRIX
    assert plan(4, 4096, 14336)["kind"] == binding.PLAN_MATRIX    # 3-4 rows: K*N >= 2^25, 224 workgroups
    assert plan(4, 14336, 4096)["kind"] == binding.PLAN_MATRIX    # a narrow W takes more splits: 8 x 32
    assert plan(8, 14336, 4096)["workgroups"] == 8 * 32            # one workgroup per CU
    assert plan(8, 4096, 4096)["workgroups"] == 8 * 16             # splits of at least 8 blocks
    assert plan(16, 4096, 1024)["kind"] == binding.PLAN_STREAM     # too narrow to fill half the device
    assert plan(64, 4096, 1024)["kind"] == binding.PLAN_MATRIX     # above 16 rows the stream needs many passes
    assert plan(2, 8192, 8192)["kind"] == binding.PLAN_STREAM     # 2 rows need K*N >= 2^27
    assert plan(5, 14336, 4096)["kind"] == binding.PLAN_MATRIX
    assert plan(16, 8192, 28672)["workgroups"] == 56 * 8          # two workgroups per CU up to 16 rows
    assert plan(32, 8192, 28672)["workgroups"] == 56 * 4          # one above
    assert plan(64, 8192, 28672)["workgroups"] == 56 * 4          # one workgroup per CU
    assert plan(16, 28672, 28672)["workgroups"] == 56 * 14       # at most 64 blocks per split
    # the matrix kernel addresses A with 32-bit byte offsets: 4*M*K must stay below 2^31
    assert plan(64, (1 << 23) - 32, 16)["kind"] == binding.PLAN_MATRIX
    assert plan(64, 1 << 23, 16)["kind"] == binding.PLAN_STREAM
    assert plan(8, (1 << 26) - 32, 16)["kind"] == binding.PLAN_MATRIX
    assert plan(8, 1 << 26, 16)["kind"] == binding.PLAN_STREAM


def test_plan_workgroups_fill_the_device():
    for M, K, N in [(1, 8192, 28672), (1, 28672, 8192)]:
        p = plan(M, K, N)
        assert 224 <= p["workgroups"] <= 256        # at most one workgroup per CU, most CUs busy
        G = math.ceil(math.ceil(K / 32) / 4)
        units = math.ceil(N / (64 * p["vec"])) * G
        assert units % p["workgroups"] == 0         # equal work for every workgroup at these shapes
        assert G % (units // p["workgroups"]) == 0  # and runs aligned with the tiles
    assert plan(1, 4096, 4096)["workgroups"] == 256  # all 512 units at vec 4, two each
    small = plan(1, 8192, 28672, cus=8)
    assert small["workgroups"] == 16 * 2 or math.ceil(3584 / small["workgroups"]) <= 16


def test_plan_rejects_bad_arguments():
    L = binding.load()
    out = binding.Q8Plan()
    assert L.q8_matvec_choose_plan(-1, 4, 4, 256, 256, 256, ctypes.byref(out)) == binding.Q8_ERR_INVALID
    assert L.q8_matvec_choose_plan(1, 4, 4, 256, 256, 0, ctypes.byref(out)) == binding.Q8_ERR_INVALID
    assert L.q8_matvec_choose_plan(1, 4, 4, 256, 256, 256, None) == binding.Q8_ERR_INVALID
    assert L.q8_matvec_choose_plan(1, 1 << 16, 1 << 15, 256, 256, 256, ctypes.byref(out)) == binding.Q8_ERR_TOO_LARGE


# ------------------------------------------------------------------ argument validation
# Every call below is rejected (or is a no-op) before the library touches HIP.

def test_matvec_rejects_bad_extents_and_pointers():
    L = binding.load()
    fake = ctypes.c_void_p(0x1000)
    null = None
    assert L.q8_matvec(fake, fake, fake, fake, -1, 4, 4, null) == binding.Q8_ERR_INVALID
    assert L.q8_matvec(fake, fake, fake, fake, 1, -4, 4, null) == binding.Q8_ERR_INVALID
    assert L.q8_matvec(null, fake, fake, fake, 1, 4, 4, null) == binding.Q8_ERR_INVALID
    assert L.q8_matvec(fake, null, fake, fake, 1, 4, 4, null) == binding.Q8_ERR_INVALID
    assert L.q8_matvec(fake, fake, null, fake, 1, 4, 4, null) == binding.Q8_ERR_INVALID
    assert L.q8_matvec(fake, fake, fake, null, 1, 4, 4, null) == binding.Q8_ERR_INVALID
    assert L.q8_matvec(fake, fake, fake, fake, 1, 1 << 16, 1 << 15, null) == binding.Q8_ERR_TOO_LARGE
    # empty outputs are a no-op: nothing is read, nothing is launched
    assert L.q8_matvec(null, null, null, null, 0, 4, 4, null) == binding.Q8_OK
    assert L.q8_matvec(null, null, null, null, 3, 4, 0, null) == binding.Q8_OK
    assert L.q8_matvec_with_plan(fake, fake, fake, fake, 1, 4, 4, None, null) == binding.Q8_ERR_INVALID


def test_dot_t_rejects_bad_extents_and_pointers():
    L = binding.load()
    fake = ctypes.c_void_p(0x1000)
    null = None
    assert L.q8_dot_t(fake, fake, fake, 1, -1, 4, null) == binding.Q8_ERR_INVALID
    assert L.q8_dot_t(null, fake, fake, 1, 4, 4, null) == binding.Q8_ERR_INVALID
    assert L.q8_dot_t(fake, null, fake, 1, 4, 4, null) == binding.Q8_ERR_INVALID
    assert L.q8_dot_t(fake, fake, null, 1, 4, 4, null) == binding.Q8_ERR_INVALID
    assert L.q8_dot_t(fake, fake, fake, 1 << 16, 1 << 16, 4, null) == binding.Q8_ERR_TOO_LARGE
    assert L.q8_dot_t(null, null, null, 0, 4, 4, null) == binding.Q8_OK


def test_dense_rejects_bad_extents_and_pointers():
    L = binding.load()
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1002)  # 2-byte aligned: not an f32 array
    ep = binding.Q8Epilogue(1.0, None)
    for fn in (L.q8_dot_f32, L.q8_dot_t_f32):
        assert fn(fake, fake, fake, -1, 4, 4, ctypes.byref(ep), None) == binding.Q8_ERR_INVALID
        assert fn(fake, fake, fake, 4, -1, 4, None, None) == binding.Q8_ERR_INVALID
        assert fn(None, fake, fake, 4, 4, 4, None, None) == binding.Q8_ERR_INVALID
        assert fn(fake, None, fake, 4, 4, 4, None, None) == binding.Q8_ERR_INVALID
        assert fn(fake, fake, None, 4, 4, 4, None, None) == binding.Q8_ERR_INVALID
        assert fn(odd, fake, fake, 4, 4, 4, None, None) == binding.Q8_ERR_INVALID
        bad_corr = binding.Q8Epilogue(1.0, 0x1001)
        assert fn(fake, fake, fake, 4, 4, 4, ctypes.byref(bad_corr), None) == binding.Q8_ERR_INVALID
        # (M + 128) * (K + 32) must stay below 2^30 (32-bit byte offsets with one tile of overhang)
        assert fn(fake, fake, fake, 1 << 20, 1 << 10, 4, None, None) == binding.Q8_ERR_TOO_LARGE
        assert fn(fake, fake, fake, 4, 1 << 10, 1 << 20, None, None) == binding.Q8_ERR_TOO_LARGE
        # empty outputs are a no-op
        assert fn(None, None, None, 0, 7, 5, None, None) == binding.Q8_OK
        assert fn(None, None, None, 3, 7, 0, None, None) == binding.Q8_OK


def test_release_without_work_is_safe():
    binding.q8_release()


def test_binding_refuses_overlapping_outputs():
    # host logic of the binding: byte ranges that share anything are refused
    import torch

    buf = torch.zeros(64, dtype=torch.float32)
    a, b, c = buf[:16], buf[16:32], buf[8:24]
    binding._check_disjoint("out", a, (("A", b), ("none", None), ("empty", buf[:0])))
    for other in (c, buf, a):
        with pytest.raises(ValueError, match="overlaps"):
            binding._check_disjoint("out", a, (("A", other),))
    # the last byte of one range and the first of the next do not overlap
    raw = torch.zeros(32, dtype=torch.uint8)
    binding._check_disjoint("out", raw[:16].view(torch.float32), (("W", raw[16:]),))
    with pytest.raises(ValueError, match="overlaps"):
        binding._check_disjoint("out", raw[:16].view(torch.float32), (("W", raw[15:]),))


def test_binding_checks_types_and_ranks_before_the_device():
    import torch

    with pytest.raises(TypeError):
        binding.q8_matvec([[1.0]], torch.zeros((1, 1), dtype=torch.int8), torch.zeros((1, 1)))
    with pytest.raises(ValueError, match="rank 2"):
        binding.q8_matvec(torch.zeros(4), torch.zeros((4, 1), dtype=torch.int8), torch.zeros((1, 1)))
    with pytest.raises(ValueError, match="rank 2"):
        binding.q8_dot_t_f32(torch.zeros((2, 2)), torch.zeros(2))


_NO_DEVICE_SCRIPT = r"""
import ctypes, sys
L = ctypes.CDLL(sys.argv[1])
p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
for name, args in (
        ("q8_matvec", [p, p, p, p, i64, i64, i64, p]),
        ("q8_matvec_noalloc", [p, p, p, p, i64, i64, i64, p]),
        ("q8_dot_t", [p, p, p, i64, i64, i64, p]),
        ("q8_dot_f32", [p, p, p, i64, i64, i64, p, p]),
        ("q8_dot_t_f32", [p, p, p, i64, i64, i64, p, p])):
    getattr(L, name).argtypes = args
    getattr(L, name).restype = ctypes.c_int
L.q8_last_hip_error.restype = ctypes.c_int
fake = [0x10000, 0x20000, 0x30000, 0x40000]
out = [L.q8_matvec(*fake, 1, 256, 128, None), L.q8_matvec_noalloc(*fake, 4, 4100, 5000, None),
       L.q8_dot_t(*fake[:3], 16, 4096, 4096, None), L.q8_dot_f32(*fake[:3], 130, 64, 200, None, None),
       L.q8_dot_t_f32(*fake[:3], 130, 64, 200, None, None)]
print(" ".join(str(x) for x in out), L.q8_last_hip_error())
"""


def test_valid_calls_without_a_device_return_an_error(tmp_path):
    """With no GPU, valid calls (non-null pointers, in-range sizes) return an
    error status from the first device query, before anything could touch the
    pointers, and the process survives.  Run in a child process with every GPU
    hidden, so that a crash cannot take the test runner down."""
    import subprocess
    import sys

    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: the fake pointers would be dereferenced")
    script = tmp_path / "no_device.py"
    script.write_text(_NO_DEVICE_SCRIPT)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    res = subprocess.run([sys.executable, str(script), binding.LIB_PATH], capture_output=True, text=True,
                         timeout=120, env=env)
    assert res.returncode == 0, res.stderr
    *statuses, hip_err = [int(x) for x in res.stdout.split()]
    assert all(s in (binding.Q8_ERR_HIP, binding.Q8_ERR_UNSUPPORTED_DEVICE) for s in statuses), statuses
    assert hip_err != 0
