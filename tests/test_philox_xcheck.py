"""S5 pin: the oracle's Philox4x32-10 against two independent open-source implementations
(rocRAND's and ATen's engines, compiled here as small host programs)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "philox_xcheck")


def _build(tmp_path_factory, name, cmd):
    out = str(tmp_path_factory.mktemp("philox") / name)
    r = subprocess.run(cmd + ["-o", out], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"cannot build {name}: {r.stderr[-400:]}")
    return out


@pytest.fixture(scope="module")
def cases():
    rng = np.random.default_rng(2024)
    n = 256
    c = rng.integers(0, 2 ** 32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    c[:, 0] &= np.uint32(0x0FFFFFFF)  # rocRAND positions by a 64-bit draw offset = 4 * block
    c[:, 1] = 0
    c[:64, 0] = np.arange(64)  # the counters the sampler uses: small words 0-1
    k = rng.integers(0, 2 ** 32, size=(n, 2), dtype=np.uint64).astype(np.uint32)
    return c, k


def _run(exe, c, k):
    text = "\n".join(" ".join(f"{int(x):x}" for x in list(ci) + list(ki)) for ci, ki in zip(c, k))
    r = subprocess.run([exe], input=text + "\n", capture_output=True, text=True, check=True)
    return np.array([[int(w, 16) for w in line.split()] for line in r.stdout.strip().splitlines()],
                    dtype=np.uint64).astype(np.uint32)


def test_philox_vs_aten(tmp_path_factory, cases):
    import torch
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    exe = _build(tmp_path_factory, "aten_philox",
                 [gxx, "-O1", "-std=c++17", "-I" + inc, os.path.join(HERE, "aten_philox.cpp")])
    c, k = cases
    np.testing.assert_array_equal(_run(exe, c, k), O.philox4x32_10(c, k))


def test_philox_vs_rocrand(tmp_path_factory, cases):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("no hipcc")
    exe = _build(tmp_path_factory, "rocrand_philox",
                 [hipcc, "-O1", os.path.join(HERE, "rocrand_philox.cpp")])
    c, k = cases
    np.testing.assert_array_equal(_run(exe, c, k), O.philox4x32_10(c, k))
