"""Host-side checks of the C-ABI library (no GPU needed): it builds, loads, and
exports every entry point include/moe.h declares; host-only calls validate
their arguments."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def B():
    from mixture_experts_layer_19_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from mixture_experts_layer_19_amd import build
        build.build()
    binding.lib()
    return binding


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer_forward"):
        assert n in names


def test_library_exports_every_declared_symbol(B):
    lib = B.lib()
    for n in _declared():
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTS) == _declared()


def test_exports_are_c_symbols(B):
    out = os.popen("nm -D --defined-only %s" % B.LIB_PATH).read()
    syms = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for n in _declared():
        assert n in syms, n


def test_status_strings(B):
    for s in range(5):
        assert B.moe_status_string(s)
    assert B.moe_status_string(99) == "unknown status"


def _desc(B, **kw):
    d = dict(hidden=4096, num_experts=192, top_k=8, inter=1536, shared_inter=1536,
             router_scaling_factor=2.826, route_norm=1, act_dtype=B.MOE_BF16,
             expert_dtype=B.MOE_BF16, out_dtype=B.MOE_BF16)
    d.update(kw)
    return B.MoeDesc(**d)


def test_workspace_and_packed_sizes(B):
    d = _desc(B)
    assert B.moe_packed_bytes(d, 0, B.MOE_PACK_GATE_UP) == 192 * 2 * 1536 * 4096 * 2
    assert B.moe_packed_bytes(d, 0, B.MOE_PACK_DOWN) == 192 * 4096 * 1536 * 2
    assert B.moe_packed_bytes(d, 1, B.MOE_PACK_GATE_UP) == 2 * 1536 * 4096 * 2
    assert B.moe_packed_bytes(d, 0, B.MOE_PACK_GATE_UP_SCALE) == 0
    mx = _desc(B, expert_dtype=B.MOE_MXFP8)
    assert B.moe_packed_bytes(mx, 0, B.MOE_PACK_GATE_UP) == 192 * 2 * 1536 * 4096
    assert B.moe_packed_bytes(mx, 0, B.MOE_PACK_DOWN_SCALE) == 192 * 4096 * 1536 // 32
    ws = B.moe_workspace_bytes(d, 64, B.MOE_WS_LAYER)
    # holds at least y [T*k, H] bf16 and the shared output [T, H]
    assert ws >= 64 * 8 * 4096 * 2 + 64 * 4096 * 2
    assert B.moe_workspace_bytes(d, 0, B.MOE_WS_LAYER) >= 0
    assert B.moe_workspace_bytes(d, -1, B.MOE_WS_LAYER) == 0
    assert B.moe_workspace_bytes(d, 64, 17) == 0
    i0, w0 = B.moe_layer_ws_topk(d, 64)
    assert i0 != w0


def test_token_pairs_beyond_int32_are_rejected(B):
    # (token, slot) pairs are int32 indices: T * k must stay below 2^31
    d = _desc(B)                                   # k = 8
    T_ok = (2 ** 31 - 1) // 8
    assert B.moe_workspace_bytes(d, T_ok, B.MOE_WS_PERMUTE) > 0
    assert B.moe_workspace_bytes(d, T_ok + 1, B.MOE_WS_PERMUTE) == 0
    with pytest.raises(B.MoeError) as ei:
        B.moe_layer_ws_topk(d, T_ok + 1)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("bad", [dict(top_k=0), dict(top_k=17), dict(num_experts=2000),
                                 dict(top_k=9, num_experts=8), dict(hidden=100),
                                 dict(inter=100), dict(route_norm=3), dict(act_dtype=7)])
def test_bad_descriptors_are_rejected(B, bad):
    d = _desc(B, **bad)
    assert B.moe_workspace_bytes(d, 64, B.MOE_WS_LAYER) == 0
    assert B.moe_packed_bytes(d, 0, B.MOE_PACK_GATE_UP) == 0


def test_unsupported_dtype_combination(B):
    d = _desc(B, act_dtype=B.MOE_F32)            # fp32 x with bf16 experts
    with pytest.raises(B.MoeError) as ei:
        B.moe_pack_experts(d, 0, B.MOE_BF16, 1, 1, 1, 1, 1)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED


def test_mx_quantize_argument_checks(B):
    with pytest.raises(B.MoeError) as ei:
        B.moe_mx_quantize(1, B.MOE_F32, 4, 33, 1, 1)       # cols not a multiple of 32
    assert ei.value.status == B.MOE_ERR_INVALID_ARG
    with pytest.raises(B.MoeError):
        B.moe_mx_quantize(None, B.MOE_F32, 4, 32, 1, 1)
    B.moe_mx_quantize(None, B.MOE_F32, 0, 32, None, None)   # zero rows: no-op


def test_null_context_is_rejected(B):
    d = _desc(B)
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(None, d, 1, 4, 1, None, 1, 1, 1, 1 << 30)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG
    with pytest.raises(B.MoeError) as ei:
        B.moe_layer_forward_noalloc(None, d, B.MoeWeights(), 1, 4, 1)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG


def test_noalloc_scratch_size_matches_header(B):
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    assert "#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in hdr
    assert B.MOE_NOALLOC_SCRATCH_BYTES == 64 << 20


def test_w4a8_and_fp8_packed_sizes(B):
    w4 = _desc(B, expert_dtype=B.MOE_MXFP4)
    E, I, H = 192, 1536, 4096
    assert B.moe_packed_bytes(w4, 0, B.MOE_PACK_GATE_UP) == E * 2 * I * H // 2   # E2M1: 2 per byte
    assert B.moe_packed_bytes(w4, 0, B.MOE_PACK_DOWN) == E * H * I // 2
    assert B.moe_packed_bytes(w4, 0, B.MOE_PACK_GATE_UP_SCALE) == E * 2 * I * H // 32
    # the shared expert of a W4A8 layer stays MX-fp8
    assert B.moe_packed_bytes(w4, 1, B.MOE_PACK_GATE_UP) == 2 * I * H
    assert B.moe_packed_bytes(w4, 1, B.MOE_PACK_DOWN_SCALE) == H * I // 32
    f8 = _desc(B, expert_dtype=B.MOE_FP8, fp8_x_scale=2.0 ** -5, fp8_h_scale=0.125,
               fp8_sh_h_scale=0.125)
    assert B.moe_packed_bytes(f8, 0, B.MOE_PACK_GATE_UP) == E * 2 * I * H
    assert B.moe_packed_bytes(f8, 0, B.MOE_PACK_GATE_UP_SCALE) == E * 2 * 4   # fp32 per tensor
    assert B.moe_packed_bytes(f8, 0, B.MOE_PACK_DOWN_SCALE) == E * 4
    assert B.moe_packed_bytes(f8, 1, B.MOE_PACK_GATE_UP_SCALE) == 2 * 4
    # 8-bit activations: the workspace holds 1-byte x and h instead of bf16
    d16 = _desc(B)
    assert B.moe_workspace_bytes(f8, 4096, B.MOE_WS_LAYER) < B.moe_workspace_bytes(d16, 4096,
                                                                                   B.MOE_WS_LAYER)


@pytest.mark.parametrize("bad", [dict(fp8_x_scale=0.0), dict(fp8_h_scale=-1.0),
                                 dict(fp8_sh_h_scale=float("nan")),
                                 dict(fp8_x_scale=float("inf")), dict(inter=128)])
def test_fp8_descriptor_checks(B, bad):
    kw = dict(expert_dtype=B.MOE_FP8, fp8_x_scale=2.0 ** -5, fp8_h_scale=0.125,
              fp8_sh_h_scale=0.125)
    kw.update(bad)
    d = _desc(B, **kw)
    assert B.moe_packed_bytes(d, 0, B.MOE_PACK_GATE_UP) == 0


def test_low_precision_dtype_combinations(B):
    # MXFP4 and FP8 are expert formats only: not for activations or outputs
    for kw in (dict(act_dtype=B.MOE_MXFP4, expert_dtype=B.MOE_MXFP4),
               dict(out_dtype=B.MOE_FP8, expert_dtype=B.MOE_FP8, fp8_x_scale=1.0, fp8_h_scale=1.0,
                    fp8_sh_h_scale=1.0),
               dict(act_dtype=B.MOE_F32, expert_dtype=B.MOE_MXFP4)):
        d = _desc(B, **kw)
        with pytest.raises(B.MoeError) as ei:
            B.moe_pack_experts(d, 0, B.MOE_F32, 1, 1, 1, 1, 1, 1, 1)
        assert ei.value.status == B.MOE_ERR_UNSUPPORTED
    assert B.moe_packed_bytes(_desc(B, expert_dtype=5), 0, B.MOE_PACK_GATE_UP) == 0


def test_fp8_quantize_argument_checks(B):
    for args in ((1, B.MOE_F32, 12, 1.0, 1),          # n not a multiple of 8
                 (1, B.MOE_F32, 16, 0.0, 1),          # scale must be > 0
                 (None, B.MOE_F32, 16, 1.0, 1),
                 (1, B.MOE_FP8, 16, 1.0, 1)):          # source dtype
        with pytest.raises(B.MoeError) as ei:
            B.moe_fp8_quantize(*args)
        assert ei.value.status == B.MOE_ERR_INVALID_ARG
    B.moe_fp8_quantize(None, B.MOE_F32, 0, 1.0, None)   # n = 0: no-op
