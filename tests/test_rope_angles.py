"""CPU check of the kernels' RoPE angle routine (csrc/dah_rope.h), compiled
as host C++ with g++: cos and sin of pos * theta^(-2i/128) must match
NumPy's float64 evaluation to float32 accuracy over the whole shape domain
(pos up to 40,959; "At a glance" on the Qwen3-0.6B Model Spec page), for the
Qwen3-0.6B base (1e6) and the family's 5e6."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_head_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "native", "rope_angles_driver.cpp")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("rope") / "rope_angles")
    subprocess.run([gxx, "-O2", "-std=c++17", f"-I{CSRC}", DRIVER, "-o", exe], check=True)
    return exe


def _run(exe, rows):
    text = "\n".join(f"{t!r} {p} {i}" for t, p, i in rows) + "\n"
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    return np.array([[float(x) for x in ln.split()] for ln in out.strip().splitlines()])


@pytest.mark.parametrize("theta", [1e6, 5e6, 1e4])
def test_rope_angles_match_float64(driver, theta):
    rng = np.random.default_rng(3)
    pos = np.concatenate([[0, 1, 2, 15, 16, 2047, 4095, 16383, 32767, 40958, 40959],
                          rng.integers(0, 40960, 60)])
    rows = [(theta, int(p), i) for p in pos for i in range(64)]
    got = _run(driver, rows)
    phi = np.array([p * theta ** (-2.0 * i / 128) for _, p, i in rows])
    err_c = np.abs(got[:, 0] - np.cos(phi))
    err_s = np.abs(got[:, 1] - np.sin(phi))
    # float32 holds cos/sin to ~6e-8; the routine's own error is below 1e-7
    assert err_c.max() < 2.5e-7 and err_s.max() < 2.5e-7, (err_c.max(), err_s.max())


def test_rope_angle_zero_and_quadrants(driver):
    # pos 0 gives exactly (1, 0); angles near multiples of pi/2 keep their signs
    got = _run(driver, [(1e6, 0, i) for i in range(64)])
    assert np.all(got[:, 0] == 1.0) and np.all(got[:, 1] == 0.0)
    rows = [(1e6, p, 0) for p in (1, 2, 3, 4, 5, 6, 7, 100, 355, 40000)]
    got = _run(driver, rows)
    phi = np.array([p for _, p, _ in rows], dtype=float)
    np.testing.assert_allclose(got[:, 0], np.cos(phi), atol=2e-7)
    np.testing.assert_allclose(got[:, 1], np.sin(phi), atol=2e-7)
