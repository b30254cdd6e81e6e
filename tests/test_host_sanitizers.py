"""Host sanitizer runs, on the CPU only.

  - The oracle's C (oracle/oracle.c) built with gcc's AddressSanitizer and UndefinedBehaviorSanitizer
    and driven through the whole step -- preprocess, binning and sort, ranges, the forward with and
    without decision records, the brute-force render, the L1 and L1 + D-SSIM losses, the backward,
    the preprocess backward, Adam and density control -- on small seeded scenes, including an
    empty one, ragged image sizes and every SH degree.
  - The host half of the C-ABI library (csrc/*.hip, device code untouched) built with clang's
    AddressSanitizer (-Xarch_host) and driven through every entry point's host-side checks and
    workspace queries, which run without a GPU.

Each runs in a subprocess with the sanitizer runtime preloaded; any report fails the test."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gaussian_splatting_differentiable_preprocess_amd")

ORACLE_DRIVER = r"""
import numpy as np
import oracle
from gaussian_splatting_differentiable_preprocess_amd import inputs
oracle.set_num_threads(2)
rng = np.random.default_rng(0)
for seed, n, deg, W, H in [(1, 300, 3, 64, 48), (2, 150, 0, 17, 33), (3, 0, 1, 32, 32), (4, 400, 2, 100, 70),
                           (5, 60, 1, 11, 11)]:
    R = oracle.rows_for_degree(deg)
    params = (inputs.small_scene(seed, n, deg, logscale_mean=-2.5, logscale_std=0.5) if n
              else np.zeros((R, 0), np.float32))
    cam = inputs.lookat_camera((3.0, 0.3, 0.2), W, H).flat()
    target = rng.uniform(0, 1, (H, W, 3))
    m, v = np.zeros(params.shape), np.zeros(params.shape)
    r = oracle.train_step_reference(params, deg, cam, W, H, target=target, m=m, v=v, t=2)
    r2 = oracle.train_step_reference(params, deg, cam, W, H, target=target, dssim_lambda=0.2)
    proj, radii, vals, rg = r["proj"], r["radii"], r["vals"], r["ranges"]
    rec = oracle.render_forward(proj, vals, rg, W, H, (0.1, 0.2, 0.3), record_decisions=True, walk=True,
                                margins=(1e-5, 3e-5, 1e-6))
    oracle.render_forward(proj, vals, rg, W, H, (0.1, 0.2, 0.3), decisions=rec["decisions"])
    oracle.render_backward(proj, vals, rg, W, H, r["dLdI"], (0.1, 0.2, 0.3), decisions=rec["decisions"])
    oracle.render_bruteforce(proj, radii, W, H)
    oracle.preprocess_margins(params, deg, cam, W, H)
    oracle.tile_rects(proj, radii, W, H)
    if n:
        oracle.debug_gaussian(params[:, 0], deg, cam, W, H)
        acc = rng.uniform(0, 4e-4, n).astype(np.float32)
        cnt = rng.integers(0, 3, n).astype(np.float32)
        z = rng.standard_normal((2, 3, n))
        oracle.densify(params, m, v, acc, cnt, z)
print("sanitized oracle run complete")
"""

ABI_DRIVER = r"""
import ctypes, sys
sys.path.insert(0, %(tests)r)
import test_abi
names = [k for k in dir(test_abi) if k.startswith("test_")]
for k in names:
    getattr(test_abi, k)()
print("sanitized host checks complete:", len(names))
"""


def _run(code, env, timeout):
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for bad in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert bad not in out, out[-4000:]
    return out


def _base_env():
    env = dict(os.environ)
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "2"
    return env


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    lib = str(tmp_path / "liboracle_sanitized.so")
    subprocess.check_call([gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           "-D_GNU_SOURCE", "-ffp-contract=off", "-fno-fast-math",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    runtime = subprocess.check_output([gcc, "-print-file-name=libasan.so"], text=True).strip()
    if not os.path.isfile(runtime):
        pytest.skip("gcc's AddressSanitizer runtime not found")
    env = _base_env()
    env["LD_PRELOAD"] = runtime
    env["ORACLE_LIBRARY"] = lib
    out = _run(ORACLE_DRIVER, env, timeout=900)
    assert "sanitized oracle run complete" in out


def test_library_host_half_under_address_sanitizer(tmp_path):
    sys.path.insert(0, PKG)
    import build as pkg_build
    hipcc = pkg_build.HIPCC
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    runtimes = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not runtimes:
        pytest.skip("clang's AddressSanitizer runtime not found")
    objs = []
    for src in pkg_build.sources():
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.check_call([hipcc, *pkg_build.FLAGS, "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                               "-fno-omit-frame-pointer", "-c", src, "-o", obj])
        objs.append(obj)
    lib = str(tmp_path / "libgsmi_hostasan.so")
    subprocess.check_call([hipcc, f"--offload-arch={pkg_build.ARCH}", "-shared", "-fPIC", "-Xarch_host",
                           "-fsanitize=address", *objs, "-o", lib])
    env = _base_env()
    env["LD_PRELOAD"] = runtimes[-1]
    env["GSMI_LIBRARY"] = lib
    out = _run(ABI_DRIVER % {"tests": os.path.join(ROOT, "tests")}, env, timeout=600)
    assert "sanitized host checks complete" in out
