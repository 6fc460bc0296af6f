"""The C ABI without a GPU: the library loads, exports every function the
header declares, the Python structs match the C layout, and every
host-side validation path returns its documented status (no kernel is
launched on any of these paths)."""
import ctypes
import math
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

moe = pytest.importorskip("mixture_experts_layer_steered_amd")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 19, names
    lib = moe.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe.EXPORTED)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_struct_layout_matches_header(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "moe.h"\n'
        "int main(void){\n"
        'printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(moe_params), offsetof(moe_params, norm_eps),'
        " offsetof(moe_params, scmoe), offsetof(moe_params, w4), sizeof(moe_weights), sizeof(moe_probes),"
        " offsetof(moe_probes, events), sizeof(moe_finish), offsetof(moe_finish, post_norm));\n"
        "return 0;}\n")
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", str(prog), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("HIP headers unusable from gcc: " + r.stderr[:200])
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    want = [ctypes.sizeof(moe.moe_params), moe.moe_params.norm_eps.offset,
            moe.moe_params.scmoe.offset, moe.moe_params.w4.offset, ctypes.sizeof(moe.moe_weights),
            ctypes.sizeof(moe.moe_probes), moe.moe_probes.events.offset,
            ctypes.sizeof(moe.moe_finish), moe.moe_finish.post_norm.offset]
    assert got == want


def P(**kw):
    base = dict(T=64, H=128, E=8, k=2, I=256, I_shared=256, routed_scaling_factor=1.0,
                swiglu_limit=7.0, scmoe=False, norm_eps=1e-6, w4=False)
    base.update(kw)
    return moe.make_params(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(k=17, E=32), moe.MOE_ERR_INVALID_ARG),
    (dict(k=9, E=8), moe.MOE_ERR_INVALID_ARG),
    (dict(E=0), moe.MOE_ERR_INVALID_ARG),
    (dict(H=0), moe.MOE_ERR_INVALID_ARG),
    (dict(I=0), moe.MOE_ERR_INVALID_ARG),
    (dict(I_shared=-8), moe.MOE_ERR_INVALID_ARG),
    (dict(T=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(swiglu_limit=0.0), moe.MOE_ERR_INVALID_ARG),
    (dict(swiglu_limit=-1.0), moe.MOE_ERR_INVALID_ARG),
    (dict(swiglu_limit=math.nan), moe.MOE_ERR_INVALID_ARG),
    (dict(swiglu_limit=math.inf), moe.MOE_ERR_INVALID_ARG),
    (dict(routed_scaling_factor=math.inf), moe.MOE_ERR_INVALID_ARG),
    (dict(scmoe=True, norm_eps=0.0), moe.MOE_ERR_INVALID_ARG),
    (dict(H=100), moe.MOE_ERR_UNSUPPORTED),
    (dict(I=260), moe.MOE_ERR_UNSUPPORTED),
    (dict(I_shared=12), moe.MOE_ERR_UNSUPPORTED),
    (dict(E=1025, k=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=2 ** 28, k=8), moe.MOE_ERR_UNSUPPORTED),
    (dict(scmoe=True, H=8200), moe.MOE_ERR_UNSUPPORTED),
    (dict(w4=True, I=192), moe.MOE_ERR_UNSUPPORTED),       # W4A16: H, I multiples of 128
    (dict(w4=True, H=136), moe.MOE_ERR_UNSUPPORTED),
])
def test_param_validation(kw, status):
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_workspace_size(P(**kw))
    assert ei.value.status == status
    assert moe.lib().moe_last_error().decode() != ""


def test_workspace_size_is_pure_and_grows():
    a = moe.moe_workspace_size(P())
    assert a == moe.moe_workspace_size(P()) and a > 0
    assert moe.moe_workspace_size(P(T=128)) > a
    assert moe.moe_workspace_size(P(T=0)) >= 0


def test_entry_points_reject_before_launch():
    """Null / misaligned pointers and short workspaces fail on the host."""
    p = P()
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_router_topk(p, None, 16, None, 16, 16, 16, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_router_topk(p, 18, 16, None, 16, 16, 16, stream=0)   # misaligned x
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    # workspace of 0 bytes (an int pointer carries no size)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_router_topk(p, 16, 16, None, 16, 16, 16, stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    with pytest.raises(moe.MoeError) as ei:   # a gather target without rows to gather
        moe.moe_permute(p, 16, 16, 16, 16, 16, x=None, x_perm=16, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:   # misaligned gather source
        moe.moe_permute(p, 16, 16, 16, 16, 16, x=18, x_perm=16, stream=0)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_grouped_swiglu_gemm(4, 100, 128, 256, float("nan"), 16, None, 16, 16, 16, 16, 16,
                                    16, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_grouped_swiglu_gemm(0, 100, 128, 256, 7.0, 16, None, 16, 16, 16, 16, 16, 16,
                                    stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    w = moe.make_weights(16, None, 16, 16, 16, 16)
    with pytest.raises(moe.MoeError) as ei:   # ScMoE without the shared input
        moe.moe_forward(P(scmoe=True), 16, None, w, 16, None, 16, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:   # shared expert weights missing
        moe.moe_forward(P(), 16, None, moe.make_weights(16, None, 16, 16), 16, None, 16, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:   # workspace too small
        moe.moe_forward(P(), 16, None, w, 16, None, 16, stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    # W4A16 routed experts: all four arrays, K multiples of 128, decode-sized batches
    w4 = dict(w_gate_up_q=16, w_gate_up_scale=16, w_down_q=16, w_down_scale=16)
    with pytest.raises(moe.MoeError) as ei:   # a scale array missing
        moe.moe_forward(P(w4=True), 16, None, moe.make_weights(16, None, None, None, 16, 16,
                                                                **dict(w4, w_down_scale=None)),
                        16, None, 16, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:   # misaligned tensor scales
        moe.moe_forward(P(w4=True), 16, None,
                        moe.make_weights(16, None, None, None, 16, 16, **w4, w_down_tscale=20),
                        16, None, 16, stream=0)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError) as ei:   # W4A16 arrays but params.w4 = 0: bf16 expected
        moe.moe_forward(P(), 16, None, moe.make_weights(16, None, None, None, 16, 16, **w4),
                        16, None, 16, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:   # I not a multiple of 128
        moe.moe_forward(P(I=192, w4=True), 16, None,
                        moe.make_weights(16, None, None, None, 16, 16, **w4), 16, None, 16, stream=0)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    for T in (64, 4096):   # decode-sized and prefill-sized: both reach the workspace check
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_forward(P(T=T, w4=True), 16, None,
                            moe.make_weights(16, None, None, None, 16, 16, **w4), 16, None, 16,
                            stream=0)
        assert ei.value.status == moe.MOE_ERR_WORKSPACE
    # mid-sized W4A16 batches (the 128-row tiles) read the experts dequantised
    # in the workspace (E * 3 * I * H bf16); prefill-sized ones (the
    # ping-pong tile, K >= 256 in both projections) and decode-sized ones
    # unpack the codes in the kernel
    extra = moe.moe_workspace_size(P(T=1024, w4=True)) - moe.moe_workspace_size(P(T=1024))
    assert extra >= 8 * 3 * 256 * 128 * 2
    assert moe.moe_workspace_size(P(T=64, w4=True)) == moe.moe_workspace_size(P(T=64))
    assert (moe.moe_workspace_size(P(T=4096, H=256, w4=True))
            == moe.moe_workspace_size(P(T=4096, H=256)))
    # prefill-sized with H = 128 < 256: dequantised as well
    extra = moe.moe_workspace_size(P(T=4096, w4=True)) - moe.moe_workspace_size(P(T=4096))
    assert extra >= 8 * 3 * 256 * 128 * 2


def test_packed_experts_validation():
    """The tile-blocked expert copies: sizes (E * ceil(I/128) * 256 * H for
    gate_up, E * ceil(H/256) * 256 * I for down), H and I multiples of 32,
    and the forward's host checks of the *_packed fields."""
    assert moe.moe_packed_experts_size(P(H=4096, E=64, I=1536)) == (
        64 * 12 * 256 * 4096, 64 * 16 * 256 * 1536)
    # ragged: I = 160 -> two gate_up tiles; H = 288 -> two down tiles
    assert moe.moe_packed_experts_size(P(H=288, E=3, I=160)) == (
        3 * 2 * 256 * 288, 3 * 2 * 256 * 160)
    for kw in (dict(H=136), dict(I=200)):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_packed_experts_size(P(**kw))
        assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError) as ei:   # a NULL source
        moe.moe_pack_experts(P(), 16, None, 16, 16, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:   # misaligned output
        moe.moe_pack_experts(P(), 16, 16, 16, 24, stream=0)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    base = dict(w_router=16, corr_bias=None, w_gate_up=16, w_down=16, ws_gate_up=16, ws_down=16)
    full = dict(w_gate_up_packed=16, w_down_packed=16, ws_gate_up_packed=16, ws_down_packed=16)
    w4 = dict(w_gate_up_q=16, w_gate_up_scale=16, w_down_q=16, w_down_scale=16)
    cases = [
        (P(), dict(full, w_down_packed=None), moe.MOE_ERR_INVALID_ARG),    # routed pair split
        (P(), dict(full, ws_down_packed=None), moe.MOE_ERR_INVALID_ARG),   # shared pair split
        (P(), dict(full, ws_gate_up_packed=24), moe.MOE_ERR_UNSUPPORTED),  # misaligned
        (P(I_shared=0), dict(w_gate_up_packed=16, w_down_packed=16), moe.MOE_ERR_WORKSPACE),
        (P(I_shared=136), full, moe.MOE_ERR_UNSUPPORTED),                  # not 32-multiple
        (P(w4=True), dict(full, **w4), moe.MOE_ERR_INVALID_ARG),           # W4A16 + packed
        (P(), dict(ws_gate_up_packed=16, ws_down_packed=16), moe.MOE_ERR_INVALID_ARG),
        (P(w4=True), dict(ws_gate_up_packed=16, ws_down_packed=16, **w4),  # shared alone
         moe.MOE_ERR_WORKSPACE),
        (P(), full, moe.MOE_ERR_WORKSPACE),                                # valid
    ]
    for p, extra, status in cases:
        w = moe.make_weights(**dict(base, **extra))
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_forward(p, 16, None, w, 16, None, 16, stream=0)
        assert ei.value.status == status, (extra, status)


def test_finish_validation():
    """moe_forward_finish / moe_combine_finish: the finish is checked on the
    host like every other argument."""
    w = moe.make_weights(16, None, 16, 16, 16, 16)
    cases = [
        (None, P(), moe.MOE_ERR_INVALID_ARG),                                   # no finish
        (moe.make_finish(None), P(), moe.MOE_ERR_INVALID_ARG),                  # no residual
        (moe.make_finish(18), P(), moe.MOE_ERR_UNSUPPORTED),                    # misaligned
        (moe.make_finish(16, out_scale=math.inf), P(), moe.MOE_ERR_INVALID_ARG),
        (moe.make_finish(16, residual_scale=math.nan), P(), moe.MOE_ERR_INVALID_ARG),
        (moe.moe_finish(16, 1.0, 1.0, 2), P(), moe.MOE_ERR_INVALID_ARG),        # flag not 0/1
        (moe.make_finish(16, post_norm=True), P(norm_eps=0.0), moe.MOE_ERR_INVALID_ARG),
        (moe.make_finish(16, post_norm=True), P(H=8200), moe.MOE_ERR_UNSUPPORTED),
        (moe.make_finish(16, 0.6, 0.8, True), P(), moe.MOE_ERR_WORKSPACE),      # valid
        (moe.make_finish(16), P(scmoe=True, H=8192), moe.MOE_ERR_INVALID_ARG),  # no x_shared
    ]
    for fin, p, status in cases:
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_forward_finish(p, 16, None, w, fin, 16, None, 16, stream=0)
        assert ei.value.status == status, (fin, status)
    for fin, p, status in cases[:8]:
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_combine_finish(p, 16, 16, 16, None, None, fin, 16, stream=0)
        assert ei.value.status == status, (fin, status)
    # an empty batch needs no buffers, also with a finish
    moe.moe_forward_finish(P(T=0), None, None, moe.make_weights(None, None, None, None),
                           moe.make_finish(None), None, None, None, stream=0)
    moe.moe_combine_finish(P(T=0), None, None, None, None, None, moe.make_finish(None), None,
                           stream=0)


def test_router_backward_validation():
    p = P(T=300, H=512, E=24)
    need = moe.moe_router_backward_workspace_size(p)
    assert need == moe.moe_router_backward_workspace_size(p) and need > 0
    cases = [
        (dict(strides=(-1, 1)), moe.MOE_ERR_INVALID_ARG),                  # negative stride
        (dict(grad_logits=None), moe.MOE_ERR_INVALID_ARG),
        (dict(grad_logits=18), moe.MOE_ERR_UNSUPPORTED),                   # misaligned dL
        (dict(grad_x=16, w_router=None), moe.MOE_ERR_INVALID_ARG),         # grad_x needs W_r
        (dict(grad_w=16, x=None), moe.MOE_ERR_INVALID_ARG),                # grad_w needs x
        (dict(grad_w=16), moe.MOE_ERR_INVALID_ARG),                        # no workspace
        (dict(grad_w=16, ws=16), moe.MOE_ERR_WORKSPACE),                   # 0 bytes of it
        (dict(grad_x=24), moe.MOE_ERR_UNSUPPORTED),                        # misaligned output
    ]
    for kw, status in cases:
        args = dict(grad_logits=16, x=16, w_router=16, strides=(24, 1))
        args.update(kw)
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_router_backward(p, **args, stream=0)
        assert ei.value.status == status, (kw, status)
    # nothing asked for: nothing to do, also without buffers
    moe.moe_router_backward(p, 16, 16, 16, strides=(24, 1), stream=0)
    moe.moe_router_backward(P(T=0), None, None, None, stream=0)


def test_w4_dequantize_validation():
    cases = [
        (dict(rows=-1), moe.MOE_ERR_INVALID_ARG),
        (dict(K=200), moe.MOE_ERR_UNSUPPORTED),                  # not a multiple of 128
        (dict(n_groups=1 << 16, rows=1 << 15), moe.MOE_ERR_UNSUPPORTED),  # 2^31 rows
        (dict(q=None), moe.MOE_ERR_INVALID_ARG),
        (dict(scale=8), moe.MOE_ERR_UNSUPPORTED),                # misaligned
        (dict(tscale=18), moe.MOE_ERR_UNSUPPORTED),              # tensor scales misaligned
        (dict(out=None), moe.MOE_ERR_INVALID_ARG),
    ]
    for kw, status in cases:
        args = dict(q=16, scale=16, out=16, n_groups=2, rows=64, K=256)
        args.update(kw)
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_w4_dequantize(**args, stream=0)
        assert ei.value.status == status, (kw, status)
    # empty: nothing to do, also without buffers
    moe.moe_w4_dequantize(None, None, None, 0, 64, 256, stream=0)
    moe.moe_w4_dequantize(None, None, None, 2, 64, 0, stream=0)


def test_empty_batch_is_a_noop_without_pointers():
    p = P(T=0)
    moe.moe_forward(p, None, None, moe.make_weights(None, None, None, None), None, None, None,
                    stream=0)
    moe.moe_router_topk(p, None, None, None, None, None, None, stream=0)
    moe.moe_combine(p, None, None, None, None, None, None, stream=0)
    moe.moe_grouped_swiglu_gemm(3, 0, 128, 256, 7.0, None, None, None, None, None, None, None,
                                None, stream=0)


def test_status_strings():
    for s, name in [(0, "MOE_OK"), (1, "MOE_ERR_INVALID_ARG"), (2, "MOE_ERR_UNSUPPORTED"),
                    (3, "MOE_ERR_WORKSPACE"), (4, "MOE_ERR_DEVICE")]:
        assert moe.lib().moe_status_string(s).decode() == name
