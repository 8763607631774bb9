"""libmoe4.so loads, exports what include/moe4.h declares, and rejects bad calls
before touching the GPU (CPU only: every call here fails its argument checks)."""
import ctypes
import os
import re

import pytest

from bit_moe_expert_amd import _lib
from bit_moe_expert_amd._lib import Shape, W4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe4.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libmoe4.so not built (python -m bit_moe_expert_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe4_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ["moe4_route", "moe4_permute", "moe4_expert_ffn", "moe4_combine_norm", "moe4_layer"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_abi_version():
    assert _lib.load().moe4_abi_version() == 2
    m = re.search(r"#define MOE4_ABI_VERSION (\d+)", open(HEADER).read())
    assert int(m.group(1)) == 2


def shape(**kw):
    d = dict(T=8, H=2048, E=128, k=8, I=768, n_shared=0, eps=1e-6)
    d.update(kw)
    return Shape(d["T"], d["H"], d["E"], d["k"], d["I"], d["n_shared"], d["eps"])


def test_workspace_sizes():
    lib = _lib.load()
    s = shape()
    n = lib.moe4_layer_workspace_bytes(s)
    pairs, rows = 64, 64
    assert n >= rows * (768 + 2048) * 2 + 3 * pairs * 4
    assert lib.moe4_permute_workspace_bytes(s) == 0  # one workgroup for small plans
    big = shape(T=8192, H=4096, E=128, I=1536)
    assert lib.moe4_permute_workspace_bytes(big) == (65536 // 4096) * 128 * 4
    assert lib.moe4_layer_workspace_bytes(shape(H=100)) == 0
    assert lib.moe4_layer_workspace_bytes(None) == 0
    sh = shape(T=8192, H=6144, E=160, I=2048, n_shared=1)
    assert lib.moe4_layer_workspace_bytes(sh) >= (65536 + 8192) * (2048 + 6144) * 2


FAKE = 0x10000  # aligned, never dereferenced: every call below fails its checks first


@pytest.mark.parametrize("kw,status", [
    (dict(H=100), _lib.MOE4_ERR_UNSUPPORTED),
    (dict(H=64), _lib.MOE4_ERR_UNSUPPORTED),
    (dict(I=96), _lib.MOE4_ERR_UNSUPPORTED),
    (dict(E=300, k=8), _lib.MOE4_ERR_UNSUPPORTED),
    (dict(k=17, E=64), _lib.MOE4_ERR_UNSUPPORTED),
    (dict(k=9, E=8), _lib.MOE4_ERR_UNSUPPORTED),
    (dict(n_shared=2), _lib.MOE4_ERR_UNSUPPORTED),
    (dict(T=-1), _lib.MOE4_ERR_INVALID_ARG),
    (dict(k=0), _lib.MOE4_ERR_INVALID_ARG),
    (dict(eps=0.0), _lib.MOE4_ERR_INVALID_ARG),
])
def test_route_rejects_bad_shapes(kw, status):
    lib = _lib.load()
    st = lib.moe4_route(shape(**kw), None, None, FAKE, FAKE, FAKE, None)
    assert st == status
    assert lib.moe4_last_error()


def test_null_and_misaligned_pointers():
    lib = _lib.load()
    s = shape()
    assert lib.moe4_route(s, None, None, None, FAKE, FAKE, None) == _lib.MOE4_ERR_INVALID_ARG
    assert b"logits" in lib.moe4_last_error()
    assert lib.moe4_route(s, FAKE, None, FAKE, FAKE, FAKE, None) == _lib.MOE4_ERR_INVALID_ARG
    assert lib.moe4_route(s, FAKE + 2, FAKE, FAKE, FAKE, FAKE, None) == _lib.MOE4_ERR_INVALID_ARG
    assert b"aligned" in lib.moe4_last_error()
    assert lib.moe4_permute(s, FAKE, None, FAKE, FAKE, None, 0, None) == _lib.MOE4_ERR_INVALID_ARG
    w = W4(FAKE, FAKE, FAKE, _lib.MOE4_W4_TILED)
    nul = W4(FAKE, None, FAKE, _lib.MOE4_W4_TILED)
    assert lib.moe4_expert_ffn(s, FAKE, FAKE, None, w, w, FAKE, FAKE, None) == _lib.MOE4_ERR_INVALID_ARG
    assert lib.moe4_expert_ffn(s, FAKE, FAKE, FAKE, w, nul, FAKE, FAKE, None) == _lib.MOE4_ERR_INVALID_ARG
    assert b"w2.scales" in lib.moe4_last_error()
    odd = W4(FAKE, FAKE + 2, FAKE, _lib.MOE4_W4_TILED)  # scales are read a dword at a time
    assert lib.moe4_expert_ffn(s, FAKE, FAKE, FAKE, odd, w, FAKE, FAKE, None) == _lib.MOE4_ERR_INVALID_ARG
    assert b"w13.scales is not 4-byte aligned" in lib.moe4_last_error()
    assert lib.moe4_combine_norm(s, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, None) == _lib.MOE4_ERR_INVALID_ARG
    assert b"gamma" in lib.moe4_last_error()


def test_permute_workspace_too_small():
    lib = _lib.load()
    big = shape(T=8192, H=4096, E=128, I=1536)
    assert lib.moe4_permute(big, FAKE, FAKE, FAKE, FAKE, None, 0, None) == _lib.MOE4_ERR_WORKSPACE
    assert lib.moe4_permute(big, FAKE, FAKE, FAKE, FAKE, FAKE, 100, None) == _lib.MOE4_ERR_WORKSPACE


def test_layer_workspace_and_shared_checks():
    lib = _lib.load()
    s = shape()
    w = W4(FAKE, FAKE, FAKE, _lib.MOE4_W4_TILED)
    need = lib.moe4_layer_workspace_bytes(s)
    st = lib.moe4_layer(s, FAKE, None, FAKE, w, w, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, need - 1, None)
    assert st == _lib.MOE4_ERR_WORKSPACE
    sh = shape(n_shared=1)
    st = lib.moe4_layer(sh, FAKE, None, FAKE, w, w, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, 1 << 40, None)
    assert st == _lib.MOE4_ERR_INVALID_ARG and b"shared13" in lib.moe4_last_error()


def test_layer_side_needs_events():
    """A distinct side stream with a shared expert needs both events; the check comes
    before anything is enqueued (the stream handles are never used)."""
    lib = _lib.load()
    sh = shape(n_shared=1)
    w = W4(FAKE, FAKE, FAKE, _lib.MOE4_W4_TILED)
    side = ctypes.c_void_p(0x2000)
    st = lib.moe4_layer_side(sh, FAKE, None, FAKE, w, w, w, w, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, 1 << 40, None, side, None, FAKE)
    assert st == _lib.MOE4_ERR_INVALID_ARG and b"fork_event" in lib.moe4_last_error()
    # without a shared expert the side stream is not used, and the other checks still apply
    s = shape()
    st = lib.moe4_layer_side(s, FAKE, None, FAKE, w, w, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, 16, None, side, None, None)
    assert st == _lib.MOE4_ERR_WORKSPACE


def test_prepack_checks():
    lib = _lib.load()
    assert lib.moe4_prepack_w4(1, 48, 256, FAKE, FAKE, FAKE, FAKE, None) == _lib.MOE4_ERR_UNSUPPORTED
    assert lib.moe4_prepack_w4(1, 64, 200, FAKE, FAKE, FAKE, FAKE, None) == _lib.MOE4_ERR_UNSUPPORTED
    assert lib.moe4_prepack_w4(-1, 64, 256, FAKE, FAKE, FAKE, FAKE, None) == _lib.MOE4_ERR_INVALID_ARG
    assert lib.moe4_prepack_w4(1, 64, 256, None, FAKE, FAKE, FAKE, None) == _lib.MOE4_ERR_INVALID_ARG
    assert lib.moe4_prepack_w4(0, 64, 256, None, None, None, None, None) == _lib.MOE4_OK


def test_rmsnorm_glue_checks():
    """add_rmsnorm / group_rmsnorm reject bad sizes and pointers before any launch."""
    lib = _lib.load()
    E_ARG, E_UNS, OK = _lib.MOE4_ERR_INVALID_ARG, _lib.MOE4_ERR_UNSUPPORTED, _lib.MOE4_OK
    out2 = ctypes.c_void_p(0x3000)
    # sizes
    assert lib.moe4_add_rmsnorm(-1, 64, FAKE, FAKE, FAKE, 1e-6, FAKE, out2, None) == E_ARG
    assert lib.moe4_add_rmsnorm(4, 60, FAKE, FAKE, FAKE, 1e-6, FAKE, out2, None) == E_UNS
    assert lib.moe4_add_rmsnorm(4, 16392, FAKE, FAKE, FAKE, 1e-6, FAKE, out2, None) == E_UNS
    assert lib.moe4_add_rmsnorm(4, 64, FAKE, FAKE, FAKE, 0.0, FAKE, out2, None) == E_ARG
    assert lib.moe4_group_rmsnorm(4, 64, 12, FAKE, FAKE, 1e-6, FAKE, None) == E_UNS   # not a multiple of 8
    assert lib.moe4_group_rmsnorm(4, 64, 48, FAKE, FAKE, 1e-6, FAKE, None) == E_UNS   # does not divide H
    assert lib.moe4_group_rmsnorm(4, 64, 0, FAKE, FAKE, 1e-6, FAKE, None) == E_ARG
    # pointers
    assert lib.moe4_add_rmsnorm(4, 64, None, FAKE, FAKE, 1e-6, FAKE, out2, None) == E_ARG
    assert lib.moe4_add_rmsnorm(4, 64, FAKE, None, FAKE, 1e-6, FAKE, out2, None) == E_ARG
    assert lib.moe4_add_rmsnorm(4, 64, FAKE, FAKE, FAKE, 1e-6, None, out2, None) == E_ARG
    assert lib.moe4_add_rmsnorm(4, 64, FAKE, FAKE, ctypes.c_void_p(0x1008), 1e-6, FAKE, out2, None) == E_ARG
    assert b"gamma" in lib.moe4_last_error()
    assert lib.moe4_add_rmsnorm(4, 64, FAKE, FAKE, FAKE, 1e-6, out2, out2, None) == E_ARG
    assert b"same buffer" in lib.moe4_last_error()
    assert lib.moe4_group_rmsnorm(4, 64, 16, FAKE, out2, 1e-6, out2, None) == E_ARG
    assert b"gamma aliases" in lib.moe4_last_error()
    # T == 0 does nothing, NULL buffers included
    assert lib.moe4_add_rmsnorm(0, 64, None, None, None, 1e-6, None, None, None) == OK
    assert lib.moe4_group_rmsnorm(0, 64, 16, None, None, 1e-6, None, None) == OK


@pytest.mark.parametrize("layout", [0, 3, -1, 0x7FFFFFFF])
def test_weight_layout_tag_is_required(layout):
    """A weight descriptor must name its layout (canonical or tiled): an untagged
    (zero-initialised) or unknown tag is rejected before anything is enqueued, in
    every entry point that reads weights."""
    lib = _lib.load()
    s = shape()
    good = W4(FAKE, FAKE, FAKE, _lib.MOE4_W4_TILED)
    bad = W4(FAKE, FAKE, FAKE, layout)
    E_ARG = _lib.MOE4_ERR_INVALID_ARG
    assert lib.moe4_expert_ffn(s, FAKE, FAKE, FAKE, bad, good, FAKE, FAKE, None) == E_ARG
    assert b"w13.layout" in lib.moe4_last_error()
    assert lib.moe4_expert_ffn(s, FAKE, FAKE, FAKE, good, bad, FAKE, FAKE, None) == E_ARG
    assert b"w2.layout" in lib.moe4_last_error()
    assert lib.moe4_expert_up(s, FAKE, FAKE, FAKE, bad, FAKE, None) == E_ARG
    assert lib.moe4_expert_down(s, FAKE, FAKE, bad, FAKE, None) == E_ARG
    st = lib.moe4_layer(s, FAKE, None, FAKE, good, bad, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, 1 << 40, None)
    assert st == E_ARG and b"w2.layout" in lib.moe4_last_error()
    sh = shape(n_shared=1)
    st = lib.moe4_layer(sh, FAKE, None, FAKE, good, good, bad, good, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, 1 << 40, None)
    assert st == E_ARG and b"shared13.layout" in lib.moe4_last_error()
    # both named layouts pass the descriptor check (the call then fails on the workspace)
    for lay in (_lib.MOE4_W4_CANONICAL, _lib.MOE4_W4_TILED):
        w = W4(FAKE, FAKE, FAKE, lay)
        st = lib.moe4_layer(s, FAKE, None, FAKE, w, w, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, 16, None)
        assert st == _lib.MOE4_ERR_WORKSPACE


def test_noalloc_layer_checks():
    """moe4_layer_noalloc checks its arguments like moe4_layer, and rejects shapes whose
    workspace exceeds its static scratch, all before any GPU call."""
    lib = _lib.load()
    w = W4(FAKE, FAKE, FAKE, _lib.MOE4_W4_TILED)
    big = shape(T=8192, H=4096, E=128, I=1536)
    assert lib.moe4_layer_workspace_bytes(big) > _lib.MOE4_NOALLOC_SCRATCH_BYTES
    st = lib.moe4_layer_noalloc(big, FAKE, None, FAKE, w, w, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == _lib.MOE4_ERR_UNSUPPORTED and b"scratch" in lib.moe4_last_error()
    s = shape()
    st = lib.moe4_layer_noalloc(s, FAKE, None, None, w, w, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == _lib.MOE4_ERR_INVALID_ARG and b"logits" in lib.moe4_last_error()
    bad = W4(FAKE, FAKE, FAKE, 0)
    st = lib.moe4_layer_noalloc(s, FAKE, None, FAKE, w, bad, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == _lib.MOE4_ERR_INVALID_ARG and b"w2.layout" in lib.moe4_last_error()
    assert lib.moe4_layer_noalloc(shape(T=0), None, None, None, None, None, None, None, None, None, None, None,
                                  None, None, None) == _lib.MOE4_OK
    # the header's scratch size is the one the binding knows
    m = re.search(r"#define MOE4_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert int(m.group(1)) << int(m.group(2)) == _lib.MOE4_NOALLOC_SCRATCH_BYTES


def test_w4a8_checks():
    """The FP8 (W4A8) entry points: shape limits, workspace size, pointer and descriptor
    checks, all before any GPU call."""
    lib = _lib.load()
    E_ARG, E_UNS, E_WS, OK = (_lib.MOE4_ERR_INVALID_ARG, _lib.MOE4_ERR_UNSUPPORTED,
                              _lib.MOE4_ERR_WORKSPACE, _lib.MOE4_OK)
    w = W4(FAKE, FAKE, FAKE, _lib.MOE4_W4_TILED)
    # the quantiser
    assert lib.moe4_quant_mxfp8(4, 48, FAKE, FAKE, FAKE, None) == E_UNS
    assert lib.moe4_quant_mxfp8(-1, 64, FAKE, FAKE, FAKE, None) == E_ARG
    assert lib.moe4_quant_mxfp8(4, 0, FAKE, FAKE, FAKE, None) == E_ARG
    assert lib.moe4_quant_mxfp8(4, 64, FAKE, None, FAKE, None) == E_ARG
    assert lib.moe4_quant_mxfp8(4, 64, FAKE + 8, FAKE, FAKE, None) == E_ARG
    assert lib.moe4_quant_mxfp8(0, 64, None, None, None, None) == OK
    assert lib.moe4_quant_mxfp8(1 << 40, 64, FAKE, FAKE, FAKE, None) == E_UNS
    # workspace: x8 + scales, h8 + scales and y over the routed and shared rows
    s = shape(n_shared=1)
    need = lib.moe4_w4a8_workspace_bytes(s)
    rows = 8 * 8 + 8
    assert need >= 8 * 2048 * (1 + 1 / 32) + rows * (768 * (1 + 1 / 32) + 2048 * 2)
    assert lib.moe4_w4a8_workspace_bytes(shape(H=2048 + 128)) == 0   # H % 256
    assert lib.moe4_w4a8_workspace_bytes(shape(I=768 + 64)) == 0     # I % 128
    assert lib.moe4_w4a8_workspace_bytes(None) == 0
    # FFN
    assert lib.moe4_expert_ffn_w4a8(shape(I=832), FAKE, FAKE, FAKE, w, w, None, FAKE, FAKE, 1 << 40,
                                    None) == E_UNS
    st = lib.moe4_expert_ffn_w4a8(shape(), FAKE, FAKE, FAKE, w, w, None, FAKE, FAKE, 16, None)
    assert st == E_WS
    st = lib.moe4_expert_ffn_w4a8(shape(), FAKE, FAKE, None, w, w, None, FAKE, FAKE, 1 << 40, None)
    assert st == E_ARG
    bad = W4(FAKE, FAKE, FAKE, 0)
    st = lib.moe4_expert_ffn_w4a8(shape(), FAKE, FAKE, FAKE, w, bad, None, FAKE, FAKE, 1 << 40, None)
    assert st == E_ARG and b"w2.layout" in lib.moe4_last_error()
    st = lib.moe4_expert_ffn_w4a8(shape(), FAKE, FAKE, FAKE, w, w, None, FAKE, FAKE + 8, 1 << 40, None)
    assert st == E_ARG and b"ws" in lib.moe4_last_error()
    # layer
    st = lib.moe4_layer_w4a8(s, FAKE, None, FAKE, w, w, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, 1 << 40, None)
    assert st == E_ARG and b"shared13" in lib.moe4_last_error()
    st = lib.moe4_layer_w4a8(s, FAKE, None, FAKE, w, w, w, w, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, need - 1, None)
    assert st == E_WS
    assert lib.moe4_layer_w4a8(shape(T=0), None, None, None, None, None, None, None, None, None, None, None,
                               None, None, None, 0, None) == OK


def test_f16_activation_checks():
    """The FP16-activation pre-pass and up GEMM: shape limits, pointer and descriptor
    checks, and the layer's workspace growing by x16 and xexp where its up projections
    run on the GEMM, all before any GPU call."""
    lib = _lib.load()
    E_ARG, E_UNS, OK = _lib.MOE4_ERR_INVALID_ARG, _lib.MOE4_ERR_UNSUPPORTED, _lib.MOE4_OK
    w = W4(FAKE, FAKE, FAKE, _lib.MOE4_W4_TILED)
    # the pre-pass
    assert lib.moe4_act_f16(4, 20, FAKE, FAKE, FAKE, None) == E_UNS           # K % 8
    assert lib.moe4_act_f16(4, 16384 + 8, FAKE, FAKE, FAKE, None) == E_UNS    # K > 16384
    assert lib.moe4_act_f16(-1, 64, FAKE, FAKE, FAKE, None) == E_ARG
    assert lib.moe4_act_f16(4, 64, FAKE, FAKE, None, None) == E_ARG
    assert lib.moe4_act_f16(4, 64, FAKE, FAKE, FAKE + 2, None) == E_ARG       # xexp alignment
    assert lib.moe4_act_f16(4, 64, FAKE, FAKE + 8, FAKE, None) == E_ARG       # x16 alignment
    assert lib.moe4_act_f16(1 << 31, 64, FAKE, FAKE, FAKE, None) == E_UNS
    assert lib.moe4_act_f16(0, 64, None, None, None, None) == OK
    # the GEMM
    s = shape(T=8192, H=4096, E=128, I=1536)
    assert lib.moe4_expert_up_f16(shape(H=2048 + 128), FAKE, FAKE, FAKE, FAKE, w, FAKE, None) == E_UNS
    assert lib.moe4_expert_up_f16(s, FAKE, FAKE, FAKE, None, w, FAKE, None) == E_ARG
    assert lib.moe4_expert_up_f16(s, FAKE, None, FAKE, FAKE, w, FAKE, None) == E_ARG
    assert lib.moe4_expert_up_f16(s, FAKE, FAKE, FAKE, FAKE, W4(FAKE, FAKE, FAKE, 0), FAKE, None) == E_ARG
    assert lib.moe4_expert_up_f16(s, FAKE, FAKE, FAKE, FAKE, w, None, None) == E_ARG
    assert lib.moe4_expert_up_f16(shape(T=0), None, None, None, None, None, None, None) == OK
    # the layer's workspace: x16 [T][H] and xexp [T] on top of the BF16 form's needs
    # where the up projection runs on the GEMM (40 routed rows per expert on average)
    pre = shape(T=8192, H=4096, E=128, I=1536)
    pairs, T, H, I, E = 8192 * 8, 8192, 4096, 1536, 128
    need = lib.moe4_layer_workspace_bytes(pre)
    assert need >= (E + 1) * 4 + 2 * pairs * 4 + pairs * (I + H) * 2 + T * H * 2 + T * 4
    dec = shape()  # decode: no GEMM, no FP16 copy
    assert lib.moe4_layer_workspace_bytes(dec) < 8 * 2048 * 2 + 64 * (768 + 2048) * 2 + (1 << 20)
