"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/moe.h declares, validates configurations, and sizes its
row buffers and workspace as the capacity rule says."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "mixture_experts_layer_13_amd", "libmoe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoe.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    names = declared_functions()
    assert {"moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    lib.moe_abi_version.restype = ctypes.c_int32
    assert lib.moe_abi_version() == 3


@pytest.fixture(scope="module")
def B():
    from mixture_experts_layer_13_amd import binding
    return binding


def test_validation_errors(B):
    ok = B.make_cfg(64, 128, 8, 2, 256, act="f32", expert="f32")
    assert B.validate(ok) == B.MOE_OK
    bad = [
        dict(T=-1), dict(E=0), dict(E=257), dict(k=0), dict(k=9), dict(d=100), dict(ffn=64),
        dict(n_shared=1, ffn_shared=0), dict(act_dtype=7), dict(expert_dtype=2), dict(score=3), dict(renorm=2),
        dict(cap_num=1, cap_den=0), dict(cap_num=-1, cap_den=1), dict(gate_scale=float("nan")),
        dict(weight_layout=2), dict(weight_layout=-1),
    ]
    for change in bad:
        c = B.MoeCfg.from_buffer_copy(ok)
        for f, v in change.items():
            setattr(c, f, v)
        st = B.validate(c)
        assert st in (B.MOE_ERR_INVALID_ARG, B.MOE_ERR_UNSUPPORTED), change
        assert B.lib.moe_last_error().decode()
        assert B.workspace_bytes(c) == 0 and B.rows(c) < 0
    c = B.MoeCfg.from_buffer_copy(ok)
    c.k = 3
    c.E = 2
    assert B.validate(c) == B.MOE_ERR_UNSUPPORTED   # k > E
    assert B.validate(B.make_cfg(32, 2048, 128, 8, 768, expert="int4")) == B.MOE_OK
    assert B.validate(B.make_cfg(32, 2048, 128, 8, 768, act="f32", expert="int4")) == B.MOE_ERR_UNSUPPORTED
    assert B.validate(B.make_cfg(32, 2048, 128, 8, 768, layout="tiled")) == B.MOE_OK
    # an expert matrix must stay under 2 GiB (32-bit offsets inside one matrix)
    assert B.validate(B.make_cfg(4, 32768, 8, 2, 32768)) == B.MOE_ERR_UNSUPPORTED
    assert B.validate(B.make_cfg(4, 32768, 8, 2, 16384)) == B.MOE_OK               # 1 GiB
    assert B.validate(B.make_cfg(4, 32768, 8, 2, 16384, act="f32", expert="f32")) == B.MOE_ERR_UNSUPPORTED
    assert B.validate(B.make_cfg(4, 1024, 8, 2, 512, 1, 1 << 20)) != B.MOE_OK
    # FP8 experts: bf16 activations, decode sizes (T <= 64), no shared experts
    assert B.validate(B.make_cfg(64, 2048, 64, 8, 1024, expert="fp8")) == B.MOE_OK
    assert B.validate(B.make_cfg(65, 2048, 64, 8, 1024, expert="fp8")) == B.MOE_ERR_UNSUPPORTED
    assert B.validate(B.make_cfg(8, 2048, 64, 8, 1024, act="f32", expert="fp8")) == B.MOE_ERR_UNSUPPORTED
    assert B.validate(B.make_cfg(8, 2048, 64, 8, 1024, 1, 1024, expert="fp8")) == B.MOE_ERR_UNSUPPORTED
    # group-limited selection: G divides E, G <= 64, 1 <= M <= G, k <= M * E / G; 0 / 0 = none
    g = lambda grp, E=256, k=8: B.validate(B.make_cfg(16, 1024, E, k, 512, score="sigmoid", groups=grp))
    assert g((8, 4)) == B.MOE_OK and g((8, 8)) == B.MOE_OK and g((0, 0)) == B.MOE_OK
    assert g((64, 8), E=64) == B.MOE_OK and g((8, 1), E=64) == B.MOE_OK
    assert g((8, 1), E=64, k=8) == B.MOE_OK          # k = 8 fills the one group of 8
    assert g((16, 1), E=64, k=8) == B.MOE_ERR_INVALID_ARG  # 4 experts left for k = 8
    assert g((7, 4)) == B.MOE_ERR_UNSUPPORTED        # 7 does not divide 256
    assert g((128, 8)) == B.MOE_ERR_UNSUPPORTED      # more than 64 groups
    assert g((8, 9)) == B.MOE_ERR_INVALID_ARG and g((8, 0)) == B.MOE_ERR_INVALID_ARG
    assert g((0, 4)) == B.MOE_ERR_UNSUPPORTED


def test_rows_capacity_and_workspace(B):
    c = B.make_cfg(8192, 2048, 64, 6, 1408, 2, 1408, capacity=(5, 4))
    assert B.capacity(c) == 960 and B.rows(c) == min(8192 * 6, 64 * 960)
    h = B.make_cfg(8192, 2048, 64, 6, 1408, 2, 1408, capacity=(1, 2))
    assert B.capacity(h) == 384 and B.rows(h) == 64 * 384
    d = B.make_cfg(8192, 2048, 64, 6, 1408, 2, 1408)
    assert B.capacity(d) == -1 and B.rows(d) == 8192 * 6
    # exact-integer capacity: ceil(5/4 * 8 * 2 / 4) = 5 exactly
    e = B.make_cfg(8, 128, 4, 2, 128, capacity=(5, 4))
    assert B.capacity(e) == 5
    # workspace grows with T and holds at least the intermediate activations
    w1 = B.workspace_bytes(B.make_cfg(64, 2048, 64, 8, 1024))
    w2 = B.workspace_bytes(B.make_cfg(4096, 2048, 64, 8, 1024))
    assert w2 > w1 > 0
    assert w2 >= 4096 * 8 * (1024 + 2048) * 2
    assert B.workspace_bytes(B.make_cfg(0, 2048, 64, 8, 1024)) > 0
    assert B.forward_launches(B.make_cfg(64, 2048, 64, 8, 1024)) == 5
    assert B.forward_launches(B.make_cfg(16384, 7168, 256, 8, 2048, 1, 2048)) == 5


def test_entry_points_reject_bad_arguments_before_launch(B):
    """Argument errors come back from the host before anything touches a device."""
    c = B.make_cfg(64, 128, 8, 2, 256, act="f32", expert="f32")
    P = ctypes.c_void_p
    fake = P(0x10000)   # never dereferenced: every call below fails validation first
    st = B.lib.moe_route(ctypes.byref(c), fake, fake, None, None, fake, fake, None, None, 0, None)
    assert st == B.MOE_ERR_WORKSPACE
    st = B.lib.moe_route(ctypes.byref(c), None, fake, None, None, fake, fake, None, fake, 1 << 30, None)
    assert st == B.MOE_ERR_INVALID_ARG
    st = B.lib.moe_route(ctypes.byref(c), P(0x10004), fake, None, None, fake, fake, None, fake, 1 << 30, None)
    assert st == B.MOE_ERR_INVALID_ARG          # misaligned x
    w = B.MoeExperts()
    st = B.lib.moe_forward(ctypes.byref(c), fake, fake, None, None, ctypes.byref(w), fake, fake, fake, fake, fake,
                           1 << 30, None)
    assert st == B.MOE_ERR_INVALID_ARG          # null expert weights
    st = B.lib.moe_combine(ctypes.byref(c), fake, fake, fake, fake, fake, None)
    assert st == B.MOE_ERR_INVALID_ARG          # y_shared given without shared experts
    st = B.lib.moe_permute(ctypes.byref(c), fake, fake, fake, fake, fake, fake, fake, 16, None)
    assert st == B.MOE_ERR_WORKSPACE
    st = B.lib.moe_forward_with_routes(ctypes.byref(c), fake, fake, fake, ctypes.byref(w), fake, fake, fake,
                                       1 << 30, None)
    assert st == B.MOE_ERR_INVALID_ARG          # null expert weights
    ew = B.MoeExperts()
    ew.w_gate = ew.w_up = ew.w_down = 0x10000
    st = B.lib.moe_forward_with_routes(ctypes.byref(c), fake, None, fake, ctypes.byref(ew), fake, fake, fake,
                                       1 << 30, None)
    assert st == B.MOE_ERR_INVALID_ARG          # null topk_idx
    st = B.lib.moe_forward_with_routes(ctypes.byref(c), fake, fake, fake, ctypes.byref(ew), fake, fake, fake, 16,
                                       None)
    assert st == B.MOE_ERR_WORKSPACE
    assert B.lib.moe_status_str(B.MOE_ERR_HIP) == b"HIP error"


def test_pack_rejects_bad_arguments_before_launch(B):
    P = ctypes.c_void_p
    src, dst = P(0x100000), P(0x200000)   # never dereferenced: every call below fails validation first
    pack = B.lib.moe_pack_weights
    assert pack(B.MOE_BF16, src, dst, 0, 64, None) == B.MOE_OK            # nothing to do
    assert pack(7, src, dst, 16, 64, None) == B.MOE_ERR_INVALID_ARG       # dtype
    assert pack(B.MOE_BF16, src, dst, 8, 64, None) == B.MOE_ERR_INVALID_ARG      # rows not a multiple of 16
    assert pack(B.MOE_BF16, src, dst, -16, 64, None) == B.MOE_ERR_INVALID_ARG
    assert pack(B.MOE_BF16, src, dst, 16, 16, None) == B.MOE_ERR_INVALID_ARG     # 32-byte rows
    assert pack(B.MOE_INT4_G128, src, dst, 16, 64, None) == B.MOE_ERR_INVALID_ARG  # K not a multiple of 128
    assert pack(B.MOE_F32, src, dst, 16, 8, None) == B.MOE_ERR_INVALID_ARG
    assert pack(B.MOE_BF16, None, dst, 16, 64, None) == B.MOE_ERR_INVALID_ARG
    assert pack(B.MOE_BF16, P(0x100008), dst, 16, 64, None) == B.MOE_ERR_INVALID_ARG  # misaligned
    assert pack(B.MOE_BF16, src, P(0x100400), 16, 64, None) == B.MOE_ERR_INVALID_ARG  # overlapping
    assert pack(B.MOE_BF16, src, src, 16, 64, None) == B.MOE_ERR_INVALID_ARG
