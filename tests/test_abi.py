"""CPU-side checks of the C ABI: the library loads, exports exactly what
include/w4a16.h declares, and its host-side argument checks return the
documented status without enqueueing anything (no GPU is touched)."""
import ctypes
import os
import re
import subprocess

import pytest

import int4_w4a16_group_g32_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")


def _header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"W4A16_API\s+[\w\s\*]+?\b(w4a16_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libw4a16.so is not built: run python -m int4_w4a16_group_g32_amd.build")
    return L.load_library()


def test_header_and_binding_agree():
    assert _header_functions() == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = sorted(set(re.findall(r"\sT\s(w4a16_\w+)$", out, flags=re.M)))
    assert exported == sorted(L.EXPORTS)
    for name in L.EXPORTS:
        assert hasattr(lib, name)


def test_status_strings(lib):
    for st in range(5):
        s = L.status_string(st)
        assert s and s != "unknown status"
    assert L.status_string(99) == "unknown status"


def _desc(K=64, N=64, group=32, E=1, layout=L.LAYOUT_GROUPED, qw=0x1000, sc=0x2000):
    return L.WeightDesc(qw, sc, K, N, group, E, layout)


def test_workspace_queries_are_host_only(lib):
    d = _desc(K=7168, N=18432)
    n = lib.w4a16_gemm_workspace_bytes(4, ctypes.byref(d), L.F32)
    assert n > 0 and n % 256 == 0
    assert lib.w4a16_gemm_workspace_bytes(0, ctypes.byref(d), L.F32) == 0
    for g in (16, 96, 256):  # 32, 64 and 128 are the supported group sizes
        bad = _desc(group=g)
        assert lib.w4a16_gemm_workspace_bytes(4, ctypes.byref(bad), L.F32) == 0
    assert lib.w4a16_gemm_workspace_bytes(4, ctypes.byref(_desc(K=7168, N=18432, group=128)), L.F32) > 0
    g, u, dn = _desc(7168, 18432), _desc(7168, 18432), _desc(18432, 7168)
    assert lib.w4a16_swiglu_mlp_workspace_bytes(4, L.F32, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn)) > 0
    mismatched = _desc(18432, 4096)
    assert lib.w4a16_swiglu_mlp_workspace_bytes(4, L.F32, ctypes.byref(g), ctypes.byref(u),
                                                ctypes.byref(mismatched)) == 0
    eg, eu, ed = _desc(7168, 2048, E=384), _desc(7168, 2048, E=384), _desc(2048, 7168, E=384)
    assert lib.w4a16_moe_workspace_bytes(64, 8, L.BF16, ctypes.byref(eg), ctypes.byref(eu), ctypes.byref(ed)) > 0


@pytest.mark.parametrize("field,value,status", [
    ("group_size", 96, L.ERR_UNSUPPORTED),
    ("group_size", 16, L.ERR_UNSUPPORTED),
    ("K", 48, L.ERR_UNSUPPORTED),
    ("N", 96, L.ERR_UNSUPPORTED),
    ("layout", L.LAYOUT_CANONICAL, L.ERR_UNSUPPORTED),
    ("num_experts", 2, L.ERR_UNSUPPORTED),
    ("K", -32, L.ERR_INVALID_ARG),
    ("qw", 0, L.ERR_INVALID_ARG),
    ("qw", 0x1004, L.ERR_INVALID_ARG),
])
def test_gemm_rejects_bad_weight_before_launch(lib, field, value, status):
    d = _desc()
    setattr(d, field, value)
    st = lib.w4a16_gemm(ctypes.c_void_p(0x3000), L.F32, 4, ctypes.byref(d), ctypes.c_void_p(0x4000),
                        ctypes.c_void_p(0x5000), 1 << 20, None)
    assert st == status


def test_gemm_argument_checks(lib):
    d = _desc()
    ws = lib.w4a16_gemm_workspace_bytes(4, ctypes.byref(d), L.F32)
    call = lambda x, xt, M, y, w, n: lib.w4a16_gemm(ctypes.c_void_p(x), xt, M, ctypes.byref(d),
                                                    ctypes.c_void_p(y), ctypes.c_void_p(w), n, None)
    assert call(0x3000, L.F32, 0, 0x4000, 0x5000, ws) == L.OK            # M == 0: no-op
    assert call(0x3000, L.F32, -1, 0x4000, 0x5000, ws) == L.ERR_INVALID_ARG
    assert call(0x3000, 7, 4, 0x4000, 0x5000, ws) == L.ERR_INVALID_ARG   # unknown dtype
    assert call(0, L.F32, 4, 0x4000, 0x5000, ws) == L.ERR_INVALID_ARG
    assert call(0x3008, L.F32, 4, 0x4000, 0x5000, ws) == L.ERR_INVALID_ARG  # misaligned
    assert call(0x3000, L.F32, 4, 0x3000, 0x5000, ws) == L.ERR_INVALID_ARG  # y aliases x
    assert call(0x3000, L.F32, 4, 0x4000, 0x5000, ws - 1) == L.ERR_WORKSPACE


def test_moe_argument_checks(lib):
    g, u, dn = _desc(64, 128, E=4), _desc(64, 128, E=4), _desc(128, 64, E=4)
    n = lib.w4a16_moe_workspace_bytes(8, 2, L.BF16, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn))
    call = lambda k, ws: lib.w4a16_moe_grouped(ctypes.c_void_p(0x3000), L.BF16, 8, ctypes.c_void_p(0x6000),
                                               ctypes.c_void_p(0x7000), k, ctypes.byref(g), ctypes.byref(u),
                                               ctypes.byref(dn), ctypes.c_void_p(0x4000), ctypes.c_void_p(0x5000),
                                               ws, None)
    assert call(5, n) == L.ERR_INVALID_ARG   # top_k > E
    assert call(0, n) == L.ERR_INVALID_ARG
    assert call(2, n - 1) == L.ERR_WORKSPACE
    dn_bad = _desc(128, 64, E=3)
    assert lib.w4a16_moe_grouped(ctypes.c_void_p(0x3000), L.BF16, 8, ctypes.c_void_p(0x6000),
                                 ctypes.c_void_p(0x7000), 2, ctypes.byref(g), ctypes.byref(u),
                                 ctypes.byref(dn_bad), ctypes.c_void_p(0x4000), ctypes.c_void_p(0x5000),
                                 n, None) == L.ERR_UNSUPPORTED
    assert lib.w4a16_moe_route(ctypes.c_void_p(0x6000), 8, 9, 8, ctypes.c_void_p(0x1000),
                               ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000),
                               None) == L.ERR_INVALID_ARG


def test_topk_argument_checks(lib):
    """Every rejection happens on the host, before anything is launched."""
    call = lambda M, E, k, logits=0x1000, ids=0x2000, w=0x3000: lib.w4a16_moe_topk(
        ctypes.c_void_p(logits), M, E, k, ctypes.c_void_p(ids), ctypes.c_void_p(w), None)
    assert call(-1, 8, 2) == L.ERR_INVALID_ARG
    assert call(4, 0, 1) == L.ERR_INVALID_ARG
    assert call(4, 8, 0) == L.ERR_INVALID_ARG
    assert call(4, 8, 9) == L.ERR_INVALID_ARG      # top_k > E
    assert call(4, 1025, 8) == L.ERR_UNSUPPORTED   # more experts than one wave holds
    assert call(4, 64, 33) == L.ERR_UNSUPPORTED
    assert call(4, 64, 8, logits=0) == L.ERR_INVALID_ARG
    assert call(4, 64, 8, ids=0x2004) == L.ERR_INVALID_ARG  # misaligned
    assert call(0, 64, 8, logits=0, ids=0, w=0) == L.OK     # M == 0: nothing to do


def test_quantize_and_prepack_checks(lib):
    big = 1 << 30
    assert lib.w4a16_quantize(ctypes.c_void_p(0x1000), 48, 64, 1, ctypes.c_void_p(0x2000), big,
                              ctypes.c_void_p(0x3000), big, None) == L.ERR_UNSUPPORTED
    assert lib.w4a16_quantize(None, 64, 64, 1, ctypes.c_void_p(0x2000), big, ctypes.c_void_p(0x3000), big,
                              None) == L.ERR_INVALID_ARG
    src = _desc(layout=L.LAYOUT_GROUPED)
    out = L.WeightDesc()
    assert lib.w4a16_prepack(ctypes.byref(src), ctypes.c_void_p(0x8000), big, ctypes.byref(out),
                             None) == L.ERR_UNSUPPORTED
    src = _desc(layout=L.LAYOUT_CANONICAL, qw=0x1000)
    assert lib.w4a16_prepack(ctypes.byref(src), ctypes.c_void_p(0x1100), big, ctypes.byref(out),
                             None) == L.ERR_INVALID_ARG  # overlapping destination


def test_output_sizes_are_checked_before_launch(lib):
    """Every format entry point takes the size of its output buffer and returns
    INVALID_ARG, with nothing enqueued (these pointers are not device memory),
    when the buffer is one byte short."""
    K, N, E = 256, 128, 3
    qw_bytes, sc_bytes = E * K // 8 * N * 4, E * K // 32 * N * 4
    q = lambda qb, sb: lib.w4a16_quantize(ctypes.c_void_p(0x1000), K, N, E, ctypes.c_void_p(0x2000), qb,
                                          ctypes.c_void_p(0x3000), sb, None)
    assert q(qw_bytes - 1, sc_bytes) == L.ERR_INVALID_ARG
    assert q(qw_bytes, sc_bytes - 1) == L.ERR_INVALID_ARG
    sc64 = E * K // 64 * N * 4
    qg = lambda sb: lib.w4a16_quantize_group(ctypes.c_void_p(0x1000), K, N, E, 64, ctypes.c_void_p(0x2000),
                                             qw_bytes, ctypes.c_void_p(0x3000), sb, None)
    assert qg(sc64 - 1) == L.ERR_INVALID_ARG
    src = _desc(K=K, N=N, E=E, layout=L.LAYOUT_CANONICAL, qw=0x10000)
    assert lib.w4a16_prepacked_bytes(ctypes.byref(src)) == qw_bytes
    out = L.WeightDesc()
    assert lib.w4a16_prepack(ctypes.byref(src), ctypes.c_void_p(0x100000), qw_bytes - 1, ctypes.byref(out),
                             None) == L.ERR_INVALID_ARG
    deq_bytes = E * K * N * 4
    assert lib.w4a16_dequantize(ctypes.byref(src), ctypes.c_void_p(0x100000), deq_bytes - 1,
                                None) == L.ERR_INVALID_ARG
    # the query rejects what prepack rejects
    assert lib.w4a16_prepacked_bytes(ctypes.byref(_desc(group=96))) == 0
    assert lib.w4a16_prepacked_bytes(ctypes.byref(_desc(N=96))) == 0
    assert lib.w4a16_prepacked_bytes(None) == 0


def test_static_mlp_size_check_is_host_only(lib):
    """w4a16_swiglu_mlp_static rejects a call that needs more than its static
    scratch before touching any device (these pointers are not device memory)."""
    g, u, dn = _desc(7168, 18432), _desc(7168, 18432), _desc(18432, 7168)
    need = lib.w4a16_swiglu_mlp_workspace_bytes(512, L.F32, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn))
    assert need > 64 << 20
    st = lib.w4a16_swiglu_mlp_static(ctypes.c_void_p(0x100000), L.F32, 512, ctypes.byref(g), ctypes.byref(u),
                                     ctypes.byref(dn), ctypes.c_void_p(0x200000), None)
    assert st == L.ERR_WORKSPACE
    assert lib.w4a16_swiglu_mlp_static(None, L.F32, 0, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), None,
                                       None) == L.OK  # M == 0: nothing to do
    assert lib.w4a16_swiglu_mlp_static(None, 7, 4, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), None,
                                       None) == L.ERR_INVALID_ARG


def test_static_scratch_limits_match_the_header(lib):
    """The header's stated reach of w4a16_swiglu_mlp_static for the hidden
    7168 / intermediate 18432 MLP: every M up to 64 (float32) and up to 192
    (bf16) needs at most W4A16_STATIC_SCRATCH_BYTES of workspace, and the
    next row count needs more."""
    text = open(HEADER).read()
    assert "up to M = 64 with float32 x" in text and "up to M = 192 with bf16 x" in text
    limit = 64 << 20
    assert re.search(r"#define W4A16_STATIC_SCRATCH_BYTES \(\(size_t\)64 << 20\)", text)
    g, u, dn = _desc(7168, 18432), _desc(7168, 18432), _desc(18432, 7168)

    def need(M, xt):
        return lib.w4a16_swiglu_mlp_workspace_bytes(M, xt, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn))

    for xt, last in ((L.F32, 64), (L.BF16, 192)):
        assert all(0 < need(M, xt) <= limit for M in range(1, last + 1))
        assert need(last + 1, xt) > limit
