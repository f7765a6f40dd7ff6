"""The C-ABI library: it loads, exports every function include/qkrope.h declares, and its
host-side argument checks answer without a GPU (no compute call is made here)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qkrope.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qkrope_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import qk_rmsnorm_rope_amd as qr
    if not os.path.exists(qr.LIB_PATH):
        pytest.fail(f"{qr.LIB_PATH} is not built (run __graft_entry__.build())")
    return qr.lib()


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("qkrope_create", "qkrope_run_table", "qkrope_run_3d", "qkrope_destroy"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} missing from libqkrope.so"


def test_status_strings_and_null_handle(lib):
    assert lib.qkrope_status_str(0) == b"ok"
    assert lib.qkrope_status_str(1) == b"invalid argument"
    assert lib.qkrope_status_str(99) == b"unknown status"
    assert lib.qkrope_destroy(None) == 0
    # NULL handle: rejected before any HIP call
    rc = lib.qkrope_run_3d(None, None, None, None, 0, 1, 1, 1, 0, 0, 64, 1, 1, 1, 64, 1e-6,
                           1e4, 1, 1.0, 0.0, 0.0, 1.0, 1, 0, 1.0, 1.0, None, None, None, None)
    assert rc == 1
    assert b"handle" in lib.qkrope_last_error()
    rc = lib.qkrope_run_table(None, None, None, None, None, None, 0, 1e-6, 0, 1, 1, 64, 64, 1, 1,
                              64, 64, 64, None, None, 64, 64, None)
    assert rc == 1
    assert lib.qkrope_create(0, None) == 1          # out pointer NULL


def test_library_links_torchs_hip_runtime(lib):
    import qk_rmsnorm_rope_amd as qr
    runtimes = qr._hip_runtimes_loaded()
    assert len(runtimes) == 1 and "torch" in next(iter(runtimes)), runtimes


def test_new_entry_points_reject_null_handle(lib):
    rc = lib.qkrope_run_table_ex(None, None, None, None, None, None, None, 0, 0, 0, 1.0, 1e-6, 0,
                                 1, 1, 64, 64, 1, 1, 64, 64, 32, 32, None, None, 64, 64, None)
    assert rc == 1 and b"handle" in lib.qkrope_last_error()
    assert lib.qkrope_sumsq_3d(None, None, 4, 1, 1, 1, 64, None, None) == 1
    rc = lib.qkrope_run_3d_sharded(None, None, None, None, 0, 0, None, 0, 0, 1, 1, 1, 0, 0, 64,
                                   1, 1, 1, 64, 1e-6, 1e4, 1, 1.0, 0.0, 0.0, 1.0, 1, 0, 1.0, 1.0,
                                   None, None, None, None)
    assert rc == 1 and b"handle" in lib.qkrope_last_error()
    rc = lib.qkrope_cam_prep(None, None, None, None, 0, None, None, None, None, 1.0, 1, 1, 1, 64,
                             64, 64, 64, None, None, None, 1, None, None)
    assert rc == 1 and b"handle" in lib.qkrope_last_error()


# --- the fused-vs-eager threshold (vLLM-Omni fused_qk_norm_rope_min_tokens rules) -------------

@pytest.mark.parametrize("env,default,expect", [
    (None, 2048, 2048), ("", 2048, 2048), ("   ", 512, 512), ("0", 2048, 0),
    ("4096", 2048, 4096), (" 17 ", 5, 17), ("0007", 1, 7)])
def test_min_tokens_resolution(monkeypatch, env, default, expect):
    import qk_rmsnorm_rope_amd as qr
    if env is None:
        monkeypatch.delenv("QKROPE_FUSED_MIN_TOKENS", raising=False)
    else:
        monkeypatch.setenv("QKROPE_FUSED_MIN_TOKENS", env)
    assert qr.fused_qk_norm_rope_min_tokens(default) == expect


@pytest.mark.parametrize("env", ["-1", "abc", "1.5", "12x", "+3", "1e3", "99999999999999999999"])
def test_min_tokens_rejects_non_integers(monkeypatch, env):
    import qk_rmsnorm_rope_amd as qr
    monkeypatch.setenv("QKROPE_FUSED_MIN_TOKENS", env)
    with pytest.raises(ValueError, match="QKROPE_FUSED_MIN_TOKENS"):
        qr.qkrope_min_tokens(2048)


def test_min_tokens_resolved_at_call_time(monkeypatch):
    import qk_rmsnorm_rope_amd as qr
    monkeypatch.setenv("QKROPE_FUSED_MIN_TOKENS", "100")
    assert qr.qkrope_min_tokens(2048) == 100
    monkeypatch.setenv("QKROPE_FUSED_MIN_TOKENS", "0")
    assert qr.qkrope_min_tokens(2048) == 0
    monkeypatch.delenv("QKROPE_FUSED_MIN_TOKENS")
    assert qr.qkrope_min_tokens(2048) == 2048
    with pytest.raises(ValueError):
        qr.qkrope_min_tokens(-1)


def test_binding_refuses_host_tensors_before_any_call():
    """The library dereferences raw device pointers, so the binding must refuse host tensors."""
    import torch
    import qk_rmsnorm_rope_amd as qr
    x = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    P = torch.zeros(1, 8, 4, 4)
    t = torch.zeros(8, 32)
    o = [torch.zeros(1, 2, 64, 8, dtype=torch.bfloat16) for _ in range(3)]
    with pytest.raises(ValueError, match="GPU"):
        qr.qkrope_cam_prep(x, x, x, P, P, t, t, 1.0, q_out=o[0], k_out=o[1], v_out=o[2])


def test_binding_weight_checks():
    """The C ABI takes weights as bare pointers, so the binding checks their length and dtype;
    a region without heads reads no weight and may pass None."""
    import torch
    import qk_rmsnorm_rope_amd as qr
    qr._check_weight(None, 0, torch.bfloat16, "k_weight")
    qr._check_weight(torch.ones(128, dtype=torch.bfloat16), 128, torch.bfloat16, "q_weight")
    for w, need, dt in ((None, 1, torch.bfloat16),
                        (torch.ones(127, dtype=torch.bfloat16), 128, torch.bfloat16),
                        (torch.ones(128, dtype=torch.float32), 128, torch.bfloat16),
                        (torch.ones(256, dtype=torch.bfloat16)[::2], 128, torch.bfloat16)):
        with pytest.raises(ValueError, match="q_weight"):
            qr._check_weight(w, need, dt, "q_weight")
    assert qr._weight_elems("none", 8, 128) == 0
    assert qr._weight_elems("per_head", 0, 128) == 0
    assert qr._weight_elems("per_head", 8, 128) == 128
    assert qr._weight_elems("across_heads", 8, 128) == 1024


# --- the binding's shape rules, checked before any device is touched ----------------------------

def test_3d_binding_requires_seq_len_of_the_grid():
    """A [batch, seq_len, row] qkv must have seq_len == ppf*pph*ppw (FlashInfer's parameter
    list: seq_len = ppf * pph * ppw); a 2D [tokens, row] qkv only needs whole sequences, which
    the library checks."""
    import torch
    import qk_rmsnorm_rope_amd as qr
    H, D = 2, 64
    kw = dict(ppf=2, pph=3, ppw=4, num_frame_channels=16, num_height_channels=24,
              num_width_channels=24, num_heads_q=H, num_heads_k=H, num_heads_v=H, head_dim=D)
    qkv = torch.zeros((1, 48, 3 * H * D), dtype=torch.bfloat16)    # two sequences in one row
    with pytest.raises(ValueError, match="seq_len == ppf\\*pph\\*ppw = 24"):
        qr.fused_qk_rmsnorm_rope(qkv, None, None, **kw)
    with pytest.raises(ValueError, match="seq_len"):
        qr.qkrope_run_3d(qkv, None, None, q_out=None, k_out=None, v_out=None, **kw)


def test_native_marshaller_loads_and_checks_arguments_on_the_host():
    """The page signatures go through the C++ marshaller (_qkrope_native), linked to the same
    libqkrope.so; its argument checks raise ValueError before any device is touched."""
    import torch
    import qk_rmsnorm_rope_amd as qr
    n = qr.native()
    assert hasattr(n, "table") and hasattr(n, "rope3d")
    maps = open("/proc/self/maps").read()
    assert qr.LIB_PATH in maps and "_qkrope_native" in maps
    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16)
    tab = torch.zeros((4, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        qr.fused_qk_norm_rope(q, q, None, None, tab, 1e-6)
    with pytest.raises(ValueError, match="bfloat16 or both float16"):
        qr.fused_qk_norm_rope(q.float(), q.float(), None, None, tab, 1e-6)
    with pytest.raises(ValueError, match="qkv must be"):
        qr.fused_qk_rmsnorm_rope(torch.zeros((4, 100), dtype=torch.bfloat16), None, None, ppf=1,
                                 pph=1, ppw=4, num_frame_channels=0, num_height_channels=0,
                                 num_width_channels=64, num_heads_q=1, num_heads_k=1,
                                 num_heads_v=1, head_dim=64)


def test_binding_refuses_ints_past_the_c_int():
    """The C ABI takes counts and sizes as 32-bit `int`; ctypes and a C++ cast would pass only
    the low 32 bits of a larger Python int (2**32 + 2 as 2), so every such argument is checked
    first, in the Python functions and in the C++ marshaller of the page signatures."""
    import torch
    import qk_rmsnorm_rope_amd as qr
    H, D = 2, 64
    kw = dict(ppf=2, pph=3, ppw=4, num_frame_channels=16, num_height_channels=24,
              num_width_channels=24, num_heads_q=H, num_heads_k=H, num_heads_v=H, head_dim=D)
    qkv = torch.zeros((24, 3 * H * D), dtype=torch.bfloat16)
    for name, bad in (("ppf", (1 << 32) + 2), ("pph", (1 << 32) + 3), ("ppw", -(1 << 32) + 4),
                      ("num_frame_channels", (1 << 32) + 16), ("num_heads_v", (1 << 31))):
        args = {**kw, name: bad}
        with pytest.raises(ValueError, match=f"{name} = {bad} does not fit"):
            qr.fused_qk_rmsnorm_rope(qkv, None, None, **args)
        with pytest.raises(ValueError, match=f"{name} = {bad} does not fit"):
            qr.qkrope_run_3d(qkv, None, None, q_out=None, k_out=None, v_out=None, **args)
        with pytest.raises(ValueError, match=f"{name} = {bad} does not fit"):
            qr.qkrope_run_3d_sharded(qkv, None, None, q_out=None, k_out=None, v_out=None, **args)
    # 32-bit values whose products pass int64: refused by the shape rules, no overflow
    big = (1 << 31) - 1
    with pytest.raises(ValueError, match="qkv must be"):
        qr.fused_qk_rmsnorm_rope(qkv, None, None, **{**kw, "num_heads_q": big, "num_heads_k": big,
                                                     "num_heads_v": big, "head_dim": big})
    with pytest.raises(ValueError, match="seq_len == ppf\\*pph\\*ppw"):
        qr.fused_qk_rmsnorm_rope(qkv.view(1, 24, -1), None, None,
                                 **{**kw, "ppf": big, "pph": big, "ppw": big})
    # table form: head_dim and rotary_dim
    q = torch.zeros((4, H, D), dtype=torch.bfloat16)
    tab = torch.zeros((4, D), dtype=torch.float32)
    with pytest.raises(ValueError, match="rotary_dim = 4294967360 does not fit"):
        qr.fused_qk_norm_rope(q, q, None, None, tab, 1e-6, rotary_dim=(1 << 32) + 64)
    with pytest.raises(ValueError, match="head_dim = -4294967232 does not fit"):
        qr.fused_qk_norm_rope(q, q, None, None, tab, 1e-6, head_dim=-(1 << 32) + 64)
    # camera prologue: head_dim from the tensor's shape (a zero-stride view, no storage)
    x = torch.zeros(1, dtype=torch.bfloat16).as_strided((1, 1, 1, (1 << 31) + 64), (0, 0, 0, 0))
    with pytest.raises(ValueError, match="head_dim = 2147483712 does not fit"):
        qr.qkrope_cam_prep(x, x, x, proj_q=None, proj_kv=None, rope_cos=None, rope_sin=None,
                           k_scale=1.0, q_out=None, k_out=None, v_out=None)
