"""The C-ABI library loads, exports every function include/moe.h declares,
and rejects invalid arguments on the host (no GPU needed: validation runs
before any HIP call)."""
import ctypes
import os
import re

import pytest

from routing_grouped_gemm_router_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(abi.library_path()):
        from routing_grouped_gemm_router_amd import build
        build.build()
    return abi.lib()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), n
    # the binding covers exactly the declared functions
    assert set(names) == set(abi.SIGNATURES)


def test_status_strings(lib):
    assert abi.moe_abi_version() == 2
    for code in range(-6, 1):
        assert abi.moe_status_string(code)
    assert abi.moe_status_string(-99) == "unknown status"


def _fake(n=1 << 20):
    # a host address: validation must reject the call before using it
    return ctypes.c_void_p(n)


# (function, args) -> status: calls that validation must reject before any HIP call
VALIDATION_CASES = [
    (("moe_check_finite", (None, 16, None, None)), -1),
    (("moe_router_logits_bwd_topk", (None, 1, None, None, None, None, None, 10, 64, 300, 8, _fake(),
                                     None, None)), -4),
    (("moe_router_logits_bwd_topk", (None, 1, None, None, None, None, None, 10, 60, 16, 8, _fake(),
                                     None, None)), -4),
    (("moe_router_logits_bwd_topk", (None, 1, None, None, None, None, None, 10, 64, 16, 8, _fake(),
                                     None, None)), -1),
    (("moe_router_logits_bwd_topk", (None, 1, None, None, None, None, None, 10, 64, 128, 65,
                                     _fake(), None, None)), -4),
    (("moe_check_dispatch", (None, None, None, None, None, 10, 8, 2, 20, None, None)), -1),
    (("moe_check_dispatch", (_fake(), _fake(), _fake(), _fake(), _fake(), 10, 2000, 2, 20, _fake(),
                             None)), -4),
    (("moe_check_dispatch", (_fake(), _fake(), _fake(), _fake(), _fake(), -1, 8, 2, 20, _fake(),
                             None)), -2),
    (("moe_route_topk_noalloc", (_fake(), 1 << 20, 1024, 1, 0, 1, _fake(), _fake(), _fake(),
                                 _fake(), _fake(), _fake(), None)), -4),
    (("moe_route_topk_noalloc", (_fake(), 10, 2000, 2, 0, 1, _fake(), _fake(), _fake(), _fake(),
                                 _fake(), _fake(), None)), -4),
    (("moe_route_topk_noalloc", (None, 10, 8, 2, 0, 1, None, None, _fake(), _fake(), None, None,
                                 None)), -1),
    (("moe_check_finite", (_fake(), -1, _fake(), None)), -2),
    (("moe_check_finite", (_fake((1 << 20) + 4), 16, _fake(), None)), -4),
    (("moe_permute", (None, 1, None, 10, 64, 2, 20, None, None)), -1),
    (("moe_permute", (None, 7, None, 10, 64, 2, 20, None, None)), -3),
    (("moe_permute", (None, 1, None, -1, 64, 2, 20, None, None)), -2),
    (("moe_permute", (_fake(), 1, _fake(), 10, 60, 2, 20, _fake(), None)), -4),
    (("moe_route_topk", (None, 10, 4, 5, 0, 1, None, None, None, None, None, None, None, 0, None)), -2),
    (("moe_route_topk", (None, 10, 2000, 5, 0, 1, None, None, None, None, None, None, None, 0, None)), -4),
    (("moe_route_topk", (None, 10, 256, 80, 0, 1, None, None, None, None, None, None, None, 0, None)), -4),
    (("moe_route_topk", (None, 10, 8, 2, 5, 1, None, None, None, None, None, None, None, 0, None)), -2),
    (("moe_route_topk", (_fake(), 10, 8, 2, 0, 1, _fake(), _fake(), _fake(), _fake(), _fake(), _fake(),
                         _fake(), 16, None)), -5),
    (("moe_route_topk_bwd", (None, None, None, None, 10, 8, 2, 0, 1, None, None)), -1),
    (("moe_grouped_gemm_fwd", (_fake(), _fake(), _fake(), 4, 100, 96, 128, 1, 0, _fake(), None, None)), -4),
    (("moe_grouped_gemm_fwd", (_fake(), _fake(), _fake(), 4, 100, 128, 100, 1, 0, _fake(), None, None)), -4),
    (("moe_grouped_gemm_fwd", (_fake(), _fake(), _fake(), 4, 100, 128, 256, 1, 1, _fake(), None, None)), -1),
    (("moe_grouped_gemm_fwd", (_fake(), _fake(), _fake(), 4, 100, 128, 256, 1, 2, _fake(), None, None)), -2),
    (("moe_grouped_gemm_fwd", (_fake(), _fake(), _fake(), 2000, 100, 128, 256, 1, 0, _fake(), None, None)), -4),
    (("moe_grouped_gemm_fwd", (None, _fake(), _fake(), 4, 100, 128, 256, 1, 0, _fake(), None, None)), -1),
    # one expert's bf16 weights at 4 GiB or more (32-bit offsets inside the kernels)
    (("moe_grouped_gemm_fwd", (_fake(), _fake(), _fake(), 4, 100, 65536, 32768, 1, 0, _fake(), None, None)), -4),
    (("moe_grouped_gemm_dgrad", (_fake(), _fake(), _fake(), 4, 100, 65536, 32768, 1, 0, None, _fake(), None)), -4),
    (("moe_grouped_gemm_wgrad", (_fake(), _fake(), _fake(), 4, 1 << 20, 4096, 128, 1, 1, 0, _fake(), None)), -4),
    (("moe_grouped_gemm_fp8_fwd", (_fake(), _fake(), _fake(), _fake(), _fake(), 4, 100, 65536, 65536, 0,
                                   _fake(), None, None)), -4),
    (("moe_grouped_gemm_dgrad", (_fake(), _fake(), _fake(), 4, 100, 96, 128, 1, 0, None, _fake(), None)), -4),
    (("moe_grouped_gemm_dgrad", (_fake(), _fake(), _fake(), 4, 100, 128, 128, 1, 2, None, _fake(), None)), -1),
    (("moe_grouped_gemm_wgrad", (_fake(), _fake(), _fake(), 4, 100, 128, 96, 1, 1, 0, _fake(), None)), -4),
    (("moe_grouped_gemm_wgrad", (_fake(), _fake(), _fake(), 4, 100, 128, 128, 0, 1, 0, _fake(), None)), -3),
    (("moe_swiglu", (None, 1, 10, 12, None, None)), -4),
    (("moe_swiglu_bwd", (None, None, 1, 10, 16, None, None)), -1),
    (("moe_unpermute_combine", (None, 1, None, None, None, 10, 64, 2, 20, None, None)), -1),
    (("moe_permute", (None, 1, None, 10, 64, 2, -1, None, None)), -2),
    (("moe_pad_to_max", (None, None, None, None, None, 10, 8, 2, 0, None, None, None, None, None)),
     -2),
    (("moe_pad_to_max", (None, None, None, None, None, 10, 8, 2, 4, None, None, None, None, None)),
     -1),
    (("moe_zero_unmapped_rows", (None, 1, None, 10, 60, None)), -4),
    (("moe_zero_unmapped_rows", (None, 5, None, 10, 64, None)), -3),
    (("moe_route_topk_expert_bias", (None, None, 10, 8, 9, 1, None, None, None, None, None, None,
                                     None, 0, None)), -2),
    (("moe_expert_bias_update", (None, 2000, 0.001, None, None)), -4),
    (("moe_quant_mxfp8_rows", (None, 10, 100, None, None, None)), -4),
    (("moe_permute_quant_mxfp8", (None, 10, 128, None, None, 4, 40, None, None, None)), -1),
    (("moe_scatter_quant_mxfp8", (None, 10, 128, None, 2, None, 4, 40, None, None, None)), -1),
    (("moe_scatter_quant_mxfp8", (None, 10, 100, None, 2, None, 4, 40, None, None, None)), -4),
    (("moe_scatter_quant_mxfp8", (None, 10, 128, None, 0, None, 4, 40, None, None, None)), -2),
    (("moe_quant_mxfp8_token_tiles", (None, 10, None, None, None, 4, 20, 128, 128, None, None,
                                      None)), -2),
    (("moe_grouped_gemm_mxfp8_fwd", (None, None, None, None, None, 4, 10, 100, 128, 0, None, None,
                                     None)), -4),
    (("moe_unpermute_combine_bwd", (None, None, 1, None, None, 10, 64, 65, 650, None, None,
                                    None)), -4),
    (("moe_router_logits", (None, 1, None, None, 10, 64, 2000, None, None)), -4),
    (("moe_router_logits", (None, 1, None, None, 10, 64, 8, None, None)), -1),
    (("moe_router_logits_bwd", (None, 1, None, None, 10, 64, 8, _fake(), None, None)), -1),
]


@pytest.mark.parametrize("case,expect", VALIDATION_CASES)
def test_validation_rejects_before_launch(lib, case, expect):
    name, args = case
    st = getattr(lib, name)(*args)
    assert st == expect, (name, st, abi.moe_last_error())
    assert abi.moe_last_error()


def test_zero_sized_calls_are_noops(lib):
    assert lib.moe_permute(None, 1, None, 0, 64, 2, 0, None, None) == 0
    assert lib.moe_check_finite(None, 0, None, None) == 0
    assert lib.moe_unpermute_combine(None, 1, None, None, None, 0, 64, 2, 0, None, None) == 0
    assert lib.moe_swiglu(None, 1, 0, 64, None, None) == 0
    assert lib.moe_router_logits(None, 1, None, None, 0, 64, 8, None, None) == 0
    assert lib.moe_route_topk_bwd(None, None, None, None, 0, 8, 2, 0, 1, None, None) == 0
    assert lib.moe_scatter_quant_mxfp8(None, 0, 128, None, 8, None, 4, 40, None, None, None) == 0
    assert lib.moe_scatter_quant_mxfp8(None, 10, 128, None, 8, None, 4, 0, None, None, None) == 0
    assert lib.moe_permute_quant_mxfp8(None, 10, 128, None, None, 4, 0, None, None, None) == 0


def test_workspace_size_grows_with_tokens(lib):
    a = abi.moe_route_topk_workspace_bytes(64, 256, 8)
    b = abi.moe_route_topk_workspace_bytes(8192, 256, 8)
    assert 0 < a < b
    assert b >= (8192 // 64) * 256 * 12
