"""C-ABI contract tests that need no GPU: the library loads, exports every
symbol the header declares, and rejects invalid arguments before any HIP call
(on a machine without a GPU, a valid call returns KVPOP_EHIP)."""
import ctypes
import os
import re

import pytest
import torch

import attention_target_amd as kv
from tests.conftest import gpu_available

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kvpop.h")
FAKE = 1 << 20  # never dereferenced: validation fails before any access


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvpop_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = kv.load()
    decl = declared_functions()
    assert set(decl) == set(kv.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "kvpop.h"\nint main(void){ return kvpop_status_str(0) == 0; }\n')
    import subprocess
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-c", str(src),
                        "-o", str(tmp_path / "t.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def shape(B=1, S=64, Hq=4, Hkv=2, D=64, dtype=kv.BF16, cu=None):
    sh = kv.Shape()
    sh.batch, sh.seqlen, sh.n_q_heads, sh.n_kv_heads, sh.head_dim, sh.dtype = B, S, Hq, Hkv, D, dtype
    sh.softmax_scale = 0.0
    keep = None
    if cu is not None:
        keep = torch.tensor(cu, dtype=torch.int32)
        sh.cu_seqlens = FAKE
        sh.cu_seqlens_host = keep.data_ptr()
        sh.n_docs = len(cu) - 1
    return sh, keep


def fwd(sh):
    return kv.load().kvpop_attn_fwd_lse(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, None)


def tgt(sh, window=4, agg=0, eps=0.0, ws=FAKE, ws_bytes=1 << 40):
    return kv.load().kvpop_future_target(ctypes.byref(sh), FAKE, FAKE, FAKE, window, agg, 0, eps, FAKE, ws,
                                         ws_bytes, None)


def bud(sh, s=4, w=8, k=16, ws_bytes=1 << 40):
    return kv.load().kvpop_budget_mask_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, s, w, k, FAKE, FAKE, None,
                                           None, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=3, Hkv=2), kv.EINVAL),
    (dict(S=0), kv.EINVAL),
    (dict(B=0), kv.EINVAL),
    (dict(D=96), kv.EUNSUPPORTED),
    (dict(dtype=7), kv.EUNSUPPORTED),
    (dict(cu=[0, 10, 10, 64]), kv.EINVAL),
    (dict(cu=[0, 10, 60]), kv.EINVAL),
    (dict(cu=[1, 10, 64]), kv.EINVAL),
    (dict(B=2, cu=[0, 10, 64]), kv.EINVAL),
    (dict(dtype=kv.F32, D=128), kv.EUNSUPPORTED),
])
def test_forward_validation(kw, status):
    sh, _keep = shape(**kw)
    assert fwd(sh) == status
    assert kv.last_error() != ""


def test_null_pointers_and_shape():
    lib = kv.load()
    assert lib.kvpop_attn_fwd_lse(None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == kv.EINVAL
    sh, _ = shape()
    assert lib.kvpop_attn_fwd_lse(ctypes.byref(sh), None, FAKE, FAKE, FAKE, FAKE, None) == kv.EINVAL
    assert lib.kvpop_attn_fwd_lse(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, None, None) == kv.EINVAL
    sh.cu_seqlens = FAKE  # device offsets without host copy
    assert fwd(sh) == kv.EINVAL


def test_target_validation():
    sh, _ = shape()
    assert tgt(sh, window=-1) == kv.EINVAL
    assert tgt(sh, agg=5) == kv.EINVAL
    assert tgt(sh, eps=-1.0) == kv.EINVAL
    assert tgt(sh, eps=float("nan")) == kv.EINVAL
    need = kv.load().kvpop_workspace_size(kv.CALL_FUTURE_TARGET, ctypes.byref(sh), 0, 4, 0)
    assert need > 0
    assert tgt(sh, ws_bytes=need - 1) == kv.EWORKSPACE
    assert tgt(sh, ws=None) == kv.EWORKSPACE


def test_budget_validation():
    sh, _ = shape()
    assert bud(sh, s=-1) == kv.EINVAL
    assert bud(sh, w=-1) == kv.EINVAL
    assert bud(sh, k=-2) == kv.EINVAL
    shp, _keep = shape(cu=[0, 30, 64])
    assert bud(shp, s=-1) == kv.EINVAL
    if not gpu_available():  # packed documents pass validation (never launched on fake pointers)
        assert bud(shp) == kv.EHIP
    need = kv.load().kvpop_workspace_size(kv.CALL_BUDGET_MASK_FWD, ctypes.byref(sh), 4, 8, 16)
    assert bud(sh, ws_bytes=need - 1) == kv.EWORKSPACE


def test_workspace_sizes():
    lib = kv.load()
    sh, _ = shape(S=4096, Hq=32, Hkv=8, D=128)
    assert lib.kvpop_workspace_size(kv.CALL_FWD_LSE, ctypes.byref(sh), 0, 0, 0) == 0
    t = lib.kvpop_workspace_size(kv.CALL_FUTURE_TARGET, ctypes.byref(sh), 0, 64, 0)
    assert t >= 4 * 32 * 4096
    b1 = lib.kvpop_workspace_size(kv.CALL_BUDGET_MASK_FWD, ctypes.byref(sh), 4, 128, 100)
    b2 = lib.kvpop_workspace_size(kv.CALL_BUDGET_MASK_FWD, ctypes.byref(sh), 4, 128, 1900)
    assert 0 < b1 < b2
    assert lib.kvpop_workspace_size(kv.CALL_BUDGET_MASK_FWD, ctypes.byref(sh), -1, 128, 100) == 0
    bad, _ = shape(Hq=3, Hkv=2)
    assert lib.kvpop_workspace_size(kv.CALL_FUTURE_TARGET, ctypes.byref(bad), 0, 0, 0) == 0


def test_status_strings():
    assert kv.status_str(kv.OK) == "ok"
    assert "workspace" in kv.status_str(kv.EWORKSPACE)
    assert kv.status_str(99) == "unknown status"


@pytest.mark.skipif(gpu_available(), reason="checks the no-device path")
def test_valid_call_without_device_reports_ehip():
    sh, _ = shape()
    assert fwd(sh) == kv.EHIP
    assert "device" in kv.last_error()


def test_binding_refuses_cpu_tensors():
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kv.attn_fwd_lse(q, q[:, :1], q[:, :1])


def test_teacher_and_loss_validation():
    lib = kv.load()
    P = ctypes.c_void_p
    dummy = ctypes.c_void_p(16)
    # bad sizes, null pointers, negative parameters, decay step, tau
    assert lib.kvpop_teacher_labels(0, 1, 10, dummy, None, 1, 0, 0, 1, dummy, dummy, None, None, dummy, 1 << 20,
                                    None) == kv.EINVAL
    assert lib.kvpop_teacher_labels(1, 1, 10, None, None, 1, 0, 0, 1, dummy, dummy, None, None, dummy, 1 << 20,
                                    None) == kv.EINVAL
    assert lib.kvpop_teacher_labels(1, 1, 10, dummy, None, 0, 0, 0, 1, dummy, dummy, None, None, dummy, 1 << 20,
                                    None) == kv.EINVAL
    assert lib.kvpop_teacher_labels(1, 1, 10, dummy, None, 1, -1, 0, 1, dummy, dummy, None, None, dummy, 1 << 20,
                                    None) == kv.EINVAL
    assert lib.kvpop_teacher_labels(1, 1, 10, dummy, None, 1, 0, 0, 1, dummy, dummy, None, None, dummy, 1,
                                    None) == kv.EWORKSPACE
    assert lib.kvpop_boundary_loss(1, 1, 10, dummy, dummy, dummy, 0, 0, 1, 0.0, None, dummy, dummy, dummy, 1 << 20,
                                   None) == kv.EINVAL
    assert lib.kvpop_boundary_loss(1, 1, 10, dummy, None, dummy, 0, 0, 1, 1.0, None, dummy, dummy, dummy, 1 << 20,
                                   None) == kv.EINVAL
    assert lib.kvpop_boundary_loss(1, 1, 10, dummy, dummy, dummy, 0, 0, 1, 1.0, None, dummy, dummy, dummy, 1,
                                   None) == kv.EWORKSPACE
    assert lib.kvpop_teacher_workspace_size(1, 2, 1000) > 0
    assert lib.kvpop_teacher_workspace_size(0, 2, 1000) == 0
    assert lib.kvpop_boundary_loss_workspace_size(2, 2, 1000) >= 3 * 2 * 2 * 1000 * 4


def decode_shape(B=1, Hq=4, Hkv=1, D=128, dtype=kv.BF16, s=4, w=16, k=32):
    sh = kv.DecodeShape()
    sh.batch, sh.n_q_heads, sh.n_kv_heads, sh.head_dim, sh.dtype = B, Hq, Hkv, D, dtype
    sh.softmax_scale = 0.0
    sh.sinks, sh.window, sh.topk = s, w, k
    return sh


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=12, Hkv=1), kv.EUNSUPPORTED),        # more than 8 query heads per KV head
    (dict(Hq=6, Hkv=4), kv.EINVAL),               # not a multiple
    (dict(D=96), kv.EUNSUPPORTED),
    (dict(dtype=7), kv.EUNSUPPORTED),
    (dict(s=0, w=0, k=0), kv.EINVAL),             # no slot at all
    (dict(s=-1), kv.EINVAL),
    (dict(k=(1 << 20) + 1), kv.EUNSUPPORTED),     # more than 2^20 slots
    (dict(B=0), kv.EINVAL),
])
def test_decode_validation(kw, status):
    lib = kv.load()
    sh = decode_shape(**kw)
    assert lib.kvpop_decode_state_size(ctypes.byref(sh)) == 0
    assert lib.kvpop_decode_init(ctypes.byref(sh), FAKE, 1 << 40, None) == status


def test_decode_state_size_and_step_errors():
    lib = kv.load()
    sh = decode_shape()
    n = lib.kvpop_decode_state_size(ctypes.byref(sh))
    # at least the K and V slots: s + (w + 1) + k slots of D bf16 values, per KV head
    assert n >= 2 * (4 + 17 + 32) * 128 * 2
    assert lib.kvpop_decode_init(ctypes.byref(sh), FAKE, n - 1, None) == kv.EWORKSPACE
    assert lib.kvpop_decode_init(ctypes.byref(sh), None, n, None) == kv.EWORKSPACE
    step = lambda pos, state_bytes, q=FAKE: lib.kvpop_decode_step(ctypes.byref(sh), FAKE, state_bytes, pos, q, FAKE,
                                                                  FAKE, FAKE, FAKE, FAKE, None)
    assert step(-1, n) == kv.EINVAL
    assert step(0, n, q=None) == kv.EINVAL
    assert step(0, n - 1) == kv.EWORKSPACE
    if not gpu_available():  # valid arguments reach the device check (never launched on fake pointers)
        assert step(0, n) == kv.EHIP


def test_misaligned_pointers_are_rejected():
    """Tensors the kernels move in 16-byte vectors (Q, K, V, O, workspaces, the
    decode state) must be 16-byte aligned and fp32/int32 arrays 4-byte
    aligned; a violation is EINVAL before any device access."""
    lib = kv.load()
    sh, _ = shape()
    odd, half = FAKE + 4, FAKE + 2  # 4-byte aligned but not 16; 2-byte aligned
    fwd_call = lambda q=FAKE, o=FAKE, lse=FAKE: lib.kvpop_attn_fwd_lse(ctypes.byref(sh), q, FAKE, FAKE, o, lse, None)
    assert fwd_call(q=odd) == kv.EINVAL
    assert "aligned" in kv.last_error()
    assert fwd_call(o=odd) == kv.EINVAL
    assert fwd_call(lse=half) == kv.EINVAL
    assert tgt(sh, ws=odd) == kv.EINVAL
    assert lib.kvpop_future_target(ctypes.byref(sh), FAKE, FAKE, FAKE, 4, 0, 0, 0.0, half, FAKE, 1 << 40,
                                   None) == kv.EINVAL
    assert lib.kvpop_budget_mask_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, half, 4, 8, 16, FAKE, FAKE, None, None,
                                     FAKE, 1 << 40, None) == kv.EINVAL
    assert lib.kvpop_budget_mask_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, 4, 8, 16, FAKE, FAKE, half, None,
                                     FAKE, 1 << 40, None) == kv.EINVAL
    dummy = ctypes.c_void_p(16)
    assert lib.kvpop_teacher_labels(1, 1, 10, dummy, None, 1, 0, 0, 1, ctypes.c_void_p(18), dummy, None, None,
                                    dummy, 1 << 20, None) == kv.EINVAL
    assert lib.kvpop_boundary_loss(1, 1, 10, dummy, dummy, dummy, 0, 0, 1, 1.0, None, dummy, ctypes.c_void_p(18),
                                   dummy, 1 << 20, None) == kv.EINVAL
    dsh = decode_shape()
    n = lib.kvpop_decode_state_size(ctypes.byref(dsh))
    assert lib.kvpop_decode_init(ctypes.byref(dsh), odd, n, None) == kv.EINVAL
    assert lib.kvpop_decode_step(ctypes.byref(dsh), FAKE, n, 0, odd, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 None) == kv.EINVAL
    if not gpu_available():  # 4-byte alignment is enough for fp32 arrays (never launched on fake pointers)
        assert fwd_call(lse=odd) == kv.EHIP


def test_grids_beyond_int_range_are_rejected():
    """Shapes the validation accepts but whose workgroup count would not fit a
    32-bit grid return EUNSUPPORTED (counted in 64 bits) instead of launching
    a wrapped-around grid."""
    lib = kv.load()
    # forward: 2^24 / 32 query blocks x 4096 KV heads > 2^31 workgroups
    sh, _ = shape(S=1 << 24, Hq=16384, Hkv=4096, D=64)
    assert fwd(sh) == kv.EUNSUPPORTED
    assert "workgroups" in kv.last_error()
    # target: one 2^24-token document has ~5.4e8 (key tile, query chunk) blocks per KV head
    sh, _ = shape(S=1 << 24, Hq=32, Hkv=8, D=128)
    assert tgt(sh, window=4) == kv.EUNSUPPORTED
    assert "workgroups" in kv.last_error()
    if not gpu_available():  # one KV head fits (never launched on fake pointers)
        sh, _ = shape(S=1 << 24, Hq=4, Hkv=1, D=128)
        assert tgt(sh, window=4, ws_bytes=1 << 50) == kv.EHIP
