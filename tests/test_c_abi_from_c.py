"""The C ABI from C: tests/c_abi_check.c compiled with gcc as C99 (pedantic,
warnings as errors) against include/*.h, linked to the built library and run
on the host (no GPU call)."""
import os
import shutil
import subprocess

import pytest

import conv2d_backward_implicit_amd as c2b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_headers_compile_as_c99_and_host_calls_answer(tmp_path):
    c2b.load_library()                         # the built library (raises if missing)
    libdir = os.path.dirname(os.path.abspath(c2b._LIB_PATH))
    exe = str(tmp_path / "c_abi_check")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_check.c"),
           "-L", libdir, "-l:" + os.path.basename(c2b._LIB_PATH), "-Wl,-rpath," + libdir,
           "-Wl,-rpath-link,/opt/rocm/lib", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = "/opt/rocm/lib:" + env.get("LD_LIBRARY_PATH", "")
    out = subprocess.run([exe], check=True, capture_output=True, text=True, env=env,
                         timeout=120).stdout
    lines = dict(l.split(" ", 1) for l in out.strip().splitlines())
    codes = {name: code for code, name in c2b.STATUS_NAMES.items()}
    assert lines["check"] == "0 %d" % codes["CONV2D_ERR_BAD_SHAPE"]
    assert lines["status"].startswith("bad shape")
    assert int(lines["variants"]) == c2b.num_variants()
    # the strided layer's plan: its useful products and its four classes
    assert lines["plan"] == "0 7398752256 4"
    for key in ("replay", "replay_fwd", "replay_gw", "replay_rms", "replay_mha"):
        assert lines[key] == "0", (key, out)
    assert lines["null"] == str(codes["CONV2D_ERR_NULL_PTR"])


@pytest.mark.gpu
@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_caller_on_the_gpu_matches_the_oracle(tmp_path):
    """tests/c_abi_gpu_check.c: hipMalloc'd buffers, conv2d_grad_input and
    conv2d_forward on a stream of its own, no Python or torch in the process,
    each compared with the oracle (linked in from oracle/oracle.c)."""
    c2b.load_library()
    libdir = os.path.dirname(os.path.abspath(c2b._LIB_PATH))
    exe = str(tmp_path / "c_abi_gpu_check")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-fopenmp",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_gpu_check.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           "-L", libdir, "-l:" + os.path.basename(c2b._LIB_PATH), "-L", "/opt/rocm/lib",
           "-lamdhip64", "-lm", "-Wl,-rpath," + libdir, "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    print("case c caller", flush=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(run.stdout, flush=True)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    lines = dict(l.split(" ", 1) for l in run.stdout.strip().splitlines())
    for key in ("grad_input", "forward"):
        rc, err = lines[key].split()
        assert rc == "0" and float(err) <= 1e-4, (key, lines[key])
