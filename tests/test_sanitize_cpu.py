"""The C-ABI's host layer (argument validation, size arithmetic and dispatch
in moe_api.cpp) built with AddressSanitizer and UndefinedBehaviorSanitizer
and driven through every entry point on the CPU: the rejection cases of
test_abi_cpu, sizes at the edges of 64-bit arithmetic, and well-formed calls
that reach the launch layer.  The kernels' launchers are replaced by stubs
that return success (generated from internal.h), so no GPU is involved; a
sanitizer report anywhere fails the test."""
import os
import re
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "routing_grouped_gemm_router_amd", "csrc")
ROCM = "/opt/rocm"


def _stubs():
    """Definitions of every function internal.h declares: launchers return
    hipSuccess, workspace sizes 2^40 bytes (so the size checks still
    reject), the scratch lookup an error."""
    src = open(os.path.join(CSRC, "internal.h")).read()
    src = re.sub(r"//[^\n]*", "", src)
    out = ['#include "internal.h"', "namespace moe {"]
    for ret, name, params in re.findall(r"\b(hipError_t|size_t)\s+(\w+)\s*\(([^;{]*)\)\s*;", src):
        if name == "route_noalloc_scratch_bytes":
            body = "return size_t(4) << 20;"
        elif name == "route_scratch_ptr":
            body = "return hipErrorNoDevice;"
        else:
            body = "return hipSuccess;" if ret == "hipError_t" else "return size_t(1) << 40;"
        out.append(f"{ret} {name}({params}) {{ {body} }}")
    out.append("}  // namespace moe")
    return "\n".join(out) + "\n"


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the ROCm headers")
    d = tmp_path_factory.mktemp("san")
    stub = d / "stub_launchers.cpp"
    stub.write_text(_stubs())
    lib = d / "libmoe_san.so"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "moe_api.cpp"), str(stub), "-o", str(lib),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return str(lib), asan


DRIVER = textwrap.dedent('''
    import ctypes, sys
    sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
    from routing_grouped_gemm_router_amd import abi
    import test_abi_cpu as t
    lib = ctypes.CDLL({lib!r})
    for name, (res, args) in abi.SIGNATURES.items():
        f = getattr(lib, name); f.restype = res; f.argtypes = args
    fake = t._fake
    n = 0
    for (name, args), expect in t.VALIDATION_CASES:
        st = getattr(lib, name)(*args)
        assert st == expect, (name, args, st, lib.moe_last_error())
        n += 1
    big = 1 << 62
    # sizes at the edge of 64-bit arithmetic: rejected, never overflowed
    edge = [
        ("moe_permute", (fake(), 1, fake(), big, big, 2, big, fake(), None)),
        ("moe_permute", (fake(), 1, fake(), big, 64, 64, big, fake(), None)),
        ("moe_route_topk", (fake(), big, 256, 8, 0, 1, fake(), fake(), fake(), fake(), fake(),
                            fake(), fake(), 1 << 40, None)),
        ("moe_route_topk_noalloc", (fake(), big, 256, 8, 0, 1, fake(), fake(), fake(), fake(),
                                    fake(), fake(), None)),
        ("moe_grouped_gemm_fwd", (fake(), fake(), fake(), 4, big, big, big, 1, 0, fake(), None,
                                  None)),
        ("moe_grouped_gemm_wgrad", (fake(), fake(), fake(), 4, big, 128, big, 1, 1, 0, fake(),
                                    None)),
        ("moe_grouped_gemm_fp8_wgrad", (fake(), fake(), fake(), fake(), fake(), 4, big, big, big,
                                        0, 0, fake(), None)),
        ("moe_grouped_gemm_mxfp8_wgrad", (fake(), fake(), fake(), fake(), fake(), 4, big, 128,
                                          big, 0, 0, fake(), None)),
        ("moe_quant_fp8_token_tiles", (fake(), fake(), fake(), 4, big, 128, big, fake(), fake(),
                                       None)),
        ("moe_unpermute_combine", (fake(), 1, fake(), fake(), None, big, big, 8, big, fake(),
                                   None)),
        ("moe_router_logits", (fake(), 1, fake(), None, big, big, 256, fake(), None)),
        ("moe_aux_loss", (fake(), fake(), big, 256, 8, 0, 0.01, fake(), None, fake(), 1 << 40,
                          None)),
        ("moe_pad_to_max", (fake(), fake(), fake(), fake(), fake(), big, 256, 8, big, fake(),
                            fake(), fake(), fake(), None)),
        ("moe_check_finite", (fake(), big, fake(), None)),
        ("moe_padded_offsets", (fake(), 4, big, 128, fake(), None)),
    ]
    for name, args in edge:
        st = getattr(lib, name)(*args)
        assert st in (0, -1, -2, -3, -4, -5, -6), (name, st)
        n += 1
    assert lib.moe_padded_rows_bound(big, 1000, 128) != 12345   # reached, whatever it returns
    # well-formed calls reach the (stub) launchers and return OK
    ws = abi.SIGNATURES  # noqa
    ok = [
        ("moe_permute", (fake(), 1, fake(), 100, 64, 2, 200, fake(), None)),
        ("moe_unpermute_combine", (fake(), 1, fake(), fake(), None, 100, 64, 2, 200, fake(),
                                   None)),
        ("moe_grouped_gemm_fwd", (fake(), fake(), fake(), 4, 100, 128, 256, 1, 0, fake(), None,
                                  None)),
        ("moe_router_logits", (fake(), 1, fake(), None, 100, 64, 8, fake(), None)),
        ("moe_check_finite", (fake(), 100, fake(), None)),
    ]
    for name, args in ok:
        st = getattr(lib, name)(*args)
        assert st == 0, (name, st, lib.moe_last_error())
        n += 1
    print("calls", n)
''')


def test_host_layer_under_asan_and_ubsan(sanitized_lib):
    lib, asan = sanitized_lib
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["LD_LIBRARY_PATH"] = os.path.join(ROCM, "lib") + ":" + env.get("LD_LIBRARY_PATH", "")
    code = DRIVER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=300)
    report = r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert "calls" in r.stdout
