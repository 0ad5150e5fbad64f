"""The C ABI on the host: the library loads, exports what include/moe.h declares, sizes
workspaces, and refuses bad arguments before touching the GPU (no kernels run here)."""
import ctypes
import os
import re
import subprocess

import pytest

from grouped_expert_ffn_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(abi.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return abi.lib()


def test_library_exports_every_declared_function(L):
    decl = declared_functions()
    assert decl == set(abi.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", abi.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (moe_[a-z_]+)$", out, flags=re.M))
    assert decl <= exported
    for name in decl:
        assert hasattr(L, name)


def test_header_compiles_as_c():
    res = subprocess.run(["gcc", "-x", "c", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-"],
                         input=f'#include "{HEADER}"\nint main(void){{return 0;}}\n', text=True,
                         capture_output=True)
    assert res.returncode == 0, res.stderr


def desc(**kw):
    base = dict(d_model=2048, n_experts=64, top_k=8, d_ff=1024)
    base.update(kw)
    return abi.make_desc(**base)


def test_status_strings(L):
    assert abi.status_str(0) == "MOE_OK"
    assert abi.status_str(-3) == "MOE_ERR_WORKSPACE"
    assert L.moe_version() >= 100


def test_workspace_sizes(L):
    d = desc()
    T = 64
    ffn = abi.moe_workspace_bytes(d, T, abi.MOE_WS_GROUPED_FFN)
    assert ffn >= T * 8 * 1024 * 2  # h: R x I bf16
    fwd = abi.moe_workspace_bytes(d, T, abi.MOE_WS_FORWARD)
    assert fwd > ffn + T * 8 * 2048 * 2  # plus rows
    assert abi.moe_workspace_bytes(d, T, abi.MOE_WS_PERMUTE) > 0
    # pre_norm adds the normalised input
    assert abi.moe_workspace_bytes(desc(pre_norm=True), T, abi.MOE_WS_FORWARD) >= fwd + T * 2048 * 2
    # monotone in T
    assert abi.moe_workspace_bytes(d, 2 * T, abi.MOE_WS_FORWARD) > fwd
    # invalid descriptor -> 0
    assert abi.moe_workspace_bytes(desc(top_k=65), T, abi.MOE_WS_FORWARD) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=0), abi.MOE_ERR_INVALID),
    (dict(top_k=65), abi.MOE_ERR_INVALID),
    (dict(n_experts=0), abi.MOE_ERR_INVALID),
    (dict(d_model=-8), abi.MOE_ERR_INVALID),
    (dict(n_shared=-1), abi.MOE_ERR_INVALID),
    (dict(capacity_factor=-1.0), abi.MOE_ERR_INVALID),
    (dict(capacity_factor=float("nan")), abi.MOE_ERR_INVALID),
    (dict(capacity_factor=float("inf")), abi.MOE_ERR_INVALID),
    (dict(n_experts=512), abi.MOE_ERR_UNSUPPORTED),
    (dict(top_k=17, n_experts=64), abi.MOE_ERR_UNSUPPORTED),
    (dict(d_model=2040), abi.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=abi.MOE_F32, w_dtype=abi.MOE_I8), abi.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=abi.MOE_I8), abi.MOE_ERR_UNSUPPORTED),
])
def test_bad_descriptor_is_refused_before_any_launch(L, kw, status):
    with pytest.raises(abi.MoeError) as ei:
        abi.moe_route(desc(**kw), 4, 0x1000, 0x1000, None, None, 0x1000, 0x1000, 0x1000, stream=0)
    assert ei.value.status == status
    assert abi.last_error()


def test_null_and_misaligned_pointers_are_refused(L):
    d = desc()
    with pytest.raises(abi.MoeError) as ei:
        abi.moe_route(d, 4, None, 0x1000, None, None, 0x1000, 0x1000, 0x1000, stream=0)
    assert ei.value.status == abi.MOE_ERR_INVALID and "x" in str(ei.value)
    with pytest.raises(abi.MoeError) as ei:
        abi.moe_combine(d, 4, 0x1000, 0x1008, 0x1000, None, 0x1000, stream=0)
    assert ei.value.status == abi.MOE_ERR_INVALID and "aligned" in str(ei.value)
    with pytest.raises(abi.MoeError) as ei:
        abi.moe_route(d, -1, 0x1000, 0x1000, None, None, 0x1000, 0x1000, 0x1000, stream=0)
    assert ei.value.status == abi.MOE_ERR_INVALID


def test_small_workspace_is_refused(L):
    d = desc()
    need = abi.moe_workspace_bytes(d, 8, abi.MOE_WS_FORWARD)
    w = abi.make_weights(0x1000, 0x1000, 0x1000)
    with pytest.raises(abi.MoeError) as ei:
        abi.moe_forward(d, 8, 0x1000, 0x1000, None, w, None, 0x1000, None, None, 0x1000, need - 1,
                        stream=0)
    assert ei.value.status == abi.MOE_ERR_WORKSPACE
    plan = abi.moe_workspace_bytes(d, 8, abi.MOE_WS_PERMUTE)
    with pytest.raises(abi.MoeError) as ei:
        abi.moe_permute(d, 8, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, plan - 1, stream=0)
    assert ei.value.status == abi.MOE_ERR_WORKSPACE


def test_int8_requires_scales(L):
    d = desc(w_dtype=abi.MOE_I8)
    w = abi.make_weights(0x1000, 0x1000, 0x1000)
    with pytest.raises(abi.MoeError) as ei:
        abi.moe_grouped_ffn(d, 8, 0x1000, w, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1 << 30,
                            stream=0)
    assert ei.value.status == abi.MOE_ERR_INVALID and "s_gate" in str(ei.value)


def test_zero_tokens_is_a_no_op(L):
    d = desc()
    w = abi.make_weights(0x1000, 0x1000, 0x1000)
    # nothing is enqueued for T == 0, so fake addresses are never dereferenced
    abi.moe_route(d, 0, 0x1000, 0x1000, None, None, 0x1000, 0x1000, 0x1000, stream=0)
    abi.moe_permute(d, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1 << 20, stream=0)
    abi.moe_grouped_ffn(d, 0, 0x1000, w, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1 << 20, stream=0)
    abi.moe_combine(d, 0, 0x1000, 0x1000, 0x1000, None, 0x1000, stream=0)
    abi.moe_forward(d, 0, 0x1000, 0x1000, None, w, None, 0x1000, None, None, 0x1000, 1 << 20,
                    stream=0)
    assert abi.last_error() == ""


def test_timing_hook_refusals(L):
    # host-only argument checks of moe_time_next_launch (no events are touched)
    fake = ctypes.c_void_p(0x1000)
    assert L.moe_time_next_launch(-1, None, None) == abi.MOE_ERR_INVALID
    assert L.moe_time_next_launch(abi.MOE_KERNEL_COMBINE + 1, None, None) == abi.MOE_ERR_INVALID
    assert L.moe_time_next_launch(abi.MOE_KERNEL_GATE_UP, fake, None) == abi.MOE_ERR_INVALID
    assert L.moe_time_next_launch(abi.MOE_KERNEL_GATE_UP, None, fake) == abi.MOE_ERR_INVALID
    # both NULL disarms, which is always valid
    assert L.moe_time_next_launch(abi.MOE_KERNEL_GATE_UP, None, None) == abi.MOE_OK


# The kernel family per layer and T: the regime edges of the dispatch rule, host-only.
#   OLMoE shapes (E=64, k=8, routed only): VALU GEMV up to 3 mean rows per group (T <= 24;
#   int8 2 rows, T <= 16), matrix-core GEMV up to 8 (T <= 64; int8 6 rows, T <= 48);
#   DeepSeek shapes (one or more shared experts): T <= 7 / 8-16 / beyond;
#   fp32 layers always the VALU GEMV; d not a multiple of 64: no matrix-core GEMV.
G, GM, MM = abi.MOE_FFN_GEMV, abi.MOE_FFN_GEMV_MFMA, abi.MOE_FFN_GEMM
FFN_CASES = [
    (dict(), [(1, G), (24, G), (25, GM), (64, GM), (65, MM), (2048, MM)]),
    (dict(w_dtype=abi.MOE_I8), [(16, G), (17, GM), (48, GM), (49, MM)]),
    (dict(top_k=6, d_ff=1408, n_shared=2), [(7, G), (8, GM), (16, GM), (17, MM)]),
    (dict(top_k=6, d_ff=1408, n_shared=2, w_dtype=abi.MOE_I8), [(7, G), (8, GM), (16, GM), (17, MM)]),
    (dict(act_dtype=abi.MOE_F32, w_dtype=abi.MOE_F32), [(1, G), (2048, G)]),
    (dict(d_model=272, d_ff=208, n_experts=8, top_k=2, n_shared=1), [(8, G), (9, MM)]),
    (dict(d_model=272, d_ff=208, n_experts=8, top_k=2), [(32, G), (33, MM)]),
]


@pytest.mark.parametrize("kw,points", FFN_CASES, ids=[str(c[0]) for c in FFN_CASES])
def test_ffn_kernel_regimes(L, kw, points):
    d = desc(**kw)
    assert [(T, abi.moe_ffn_kernel(d, T)) for T, _ in points] == points


def test_ffn_kernel_refusals(L):
    with pytest.raises(abi.MoeError):
        abi.moe_ffn_kernel(desc(), 0)
    with pytest.raises(abi.MoeError):
        abi.moe_ffn_kernel(desc(top_k=65), 8)


def test_pre_norm_is_refused_by_the_calls_that_take_x(L):
    # the RMSNorm prologue belongs to moe_forward; the step calls take x as given, so a
    # descriptor asking for it (with or without logits_in) is refused rather than ignored
    d = desc(pre_norm=True)
    w = abi.make_weights(0x1000, 0x1000, 0x1000)
    for logits_in in (None, 0x1000):
        with pytest.raises(abi.MoeError) as ei:
            abi.moe_route(d, 4, 0x1000, 0x1000, None, logits_in, 0x1000, 0x1000, 0x1000, stream=0)
        assert ei.value.status == abi.MOE_ERR_UNSUPPORTED and "pre_norm" in str(ei.value)
    with pytest.raises(abi.MoeError) as ei:
        abi.moe_grouped_ffn(d, 8, 0x1000, w, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1 << 30,
                            stream=0)
    assert ei.value.status == abi.MOE_ERR_UNSUPPORTED and "pre_norm" in str(ei.value)


def test_noalloc_refuses_a_layer_beyond_its_scratch_and_takes_zero_tokens(L):
    # both decided on the host: no GPU is touched
    d = desc()
    w = abi.make_weights(0x1000, 0x1000, 0x1000)
    assert abi.moe_workspace_bytes(d, 4096, abi.MOE_WS_FORWARD) > 128 << 20
    with pytest.raises(abi.MoeError) as ei:
        abi.moe_forward_noalloc(d, 4096, 0x1000, 0x1000, None, w, None, 0x1000, None, None, stream=0)
    assert ei.value.status == abi.MOE_ERR_WORKSPACE and "scratch" in str(ei.value)
    abi.moe_forward_noalloc(d, 0, 0x1000, 0x1000, None, w, None, 0x1000, None, None, stream=0)
    with pytest.raises(abi.MoeError) as ei:
        abi.moe_forward_noalloc(d, 4, None, 0x1000, None, w, None, 0x1000, None, None, stream=0)
    assert ei.value.status == abi.MOE_ERR_INVALID


def test_last_error_is_per_thread(L):
    # each thread sees the message of its own last refusal, whatever the other threads did
    import ctypes
    import threading
    results = {}
    barrier = threading.Barrier(2)

    def refuse(name, T, top_k):
        d = desc(top_k=top_k)
        barrier.wait(timeout=30)
        for _ in range(200):
            st = L.moe_ffn_kernel(ctypes.byref(d), T)
            msg = L.moe_last_error().decode()
        results[name] = (st, msg)

    a = threading.Thread(target=refuse, args=("tokens", 0, 8))
    b = threading.Thread(target=refuse, args=("top_k", 8, 65))
    a.start(); b.start(); a.join(timeout=60); b.join(timeout=60)
    assert results["tokens"][0] == abi.MOE_ERR_INVALID and "T = 0" in results["tokens"][1]
    assert results["top_k"][0] < 0 and "T = 0" not in results["top_k"][1]
    assert "top_k" in results["top_k"][1] or "k =" in results["top_k"][1], results["top_k"][1]
