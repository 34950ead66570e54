"""The plan log (Q8_LOG=debug): every call names the kernel path and plan it
took on stderr and, when it fell back from the matrix cores or from wider
loads, the reason ("dot and tensor cores", "When tensor cores apply", where
the pages' compiler log names each dot that fell back and why).  Without the
variable nothing is printed."""

import numpy as np
import pytest
import torch

from quantized_decode_gemv_q8_amd import binding, workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def test_plan_log_names_paths_and_fallbacks(monkeypatch, capfd):
    A4, W4, S4 = (to_dev(x) for x in workloads.q8_inputs(4, 4100, 5000, (91, 1)))
    A16, W16, S16 = (to_dev(x) for x in workloads.q8_inputs(16, 4096, 8192, (91, 2)))
    Ai, Wi = (to_dev(x) for x in workloads.dot_t_inputs(4, 256, 64, (91, 3)))
    Ad, Bd = (to_dev(x) for x in workloads.dense_inputs(33, 30, 40, (91, 4), transposed=True))

    def calls():
        binding.q8_matvec(A4, W4, S4)
        binding.q8_matvec(A16, W16, S16)
        binding.q8_dot_t(Ai, Wi)
        binding.q8_dot_t_f32(Ad, Bd)
        torch.cuda.synchronize()

    monkeypatch.delenv("Q8_LOG", raising=False)
    calls()
    assert "q8:" not in capfd.readouterr().err
    monkeypatch.setenv("Q8_LOG", "debug")
    calls()
    err = capfd.readouterr().err
    print(err)
    lines = [ln for ln in err.splitlines() if ln.startswith("q8: ")]
    # The 16-row product's 16 tiles keep their split-K partials in one XCD's
    # L2 each, which gets a line of its own after the plan's.
    xcd = [ln for ln in lines if "kept in the XCD L2" in ln]
    lines = [ln for ln in lines if ln not in xcd]
    assert len(xcd) == 1 and "16 tiles" in xcd[0], xcd
    assert len(lines) == 4, lines
    assert "matvec M=4 K=4100 N=5000" in lines[0] and "stream" in lines[0]
    assert "not on the matrix cores: too few rows or too small a W" in lines[0]
    assert "matvec M=16 K=4096 N=8192" in lines[1] and "matrix cores" in lines[1]
    assert "dot_t M=4 K=256 N=64: sdot4" in lines[2] and "M < 16" in lines[2]
    assert "dot_t_f32 M=33 K=30 N=40" in lines[3] and "4-byte loads: K % 4 != 0" in lines[3]
