"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and validates arguments before touching the GPU.  CPU only:
none of these calls reaches a kernel launch."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from block_diffusion_drafting_pass_amd import binding as B
from block_diffusion_drafting_pass_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libdflash.so not built (run __graft_entry__.build())")
    return B.lib()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "dflash.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", src)))


def test_header_declares_the_three_calls():
    names = _declared_functions()
    for n in ("dflash_fuse_ctx", "dflash_draft_block", "dflash_accept_len"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    names = _declared_functions()
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def _cfg(name="tiny", **kw):
    c = B.Config.from_spec(I.spec(name))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _err(rc):
    return B.STATUS[rc]


def test_status_strings():
    L = _lib()
    for code in B.STATUS:
        assert L.dflash_status_str(code)
    assert L.dflash_status_str(12345) == b"unknown status"


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 96, "DFLASH_EUNSUPPORTED"),
    ("n_kv_heads", 3, "DFLASH_ESHAPE"),
    ("hidden", 200, "DFLASH_EUNSUPPORTED"),
    ("hidden", 16640, "DFLASH_EUNSUPPORTED"),
    ("vocab", 4104, "DFLASH_EUNSUPPORTED"),
    ("max_block", 33, "DFLASH_EUNSUPPORTED"),
    ("max_block", 1, "DFLASH_EUNSUPPORTED"),
    ("mask_token_id", 4096, "DFLASH_EINVAL"),
    ("n_layers", 0, "DFLASH_EINVAL"),
    ("rms_eps", 0.0, "DFLASH_EINVAL"),
])
def test_model_create_rejects_bad_configs(field, value, code):
    L = _lib()
    cfg = _cfg(**{field: value})
    n = max(3, 3 + 9 * max(cfg.n_layers, 0))
    ptrs = (ctypes.c_void_p * n)(*([0x10000] * n))
    h = ctypes.c_void_p()
    rc = L.dflash_model_create(ctypes.byref(cfg), ptrs, ctypes.byref(h))
    assert _err(rc) == code
    assert not h.value
    assert L.dflash_last_error()


def test_model_create_checks_pointers():
    L = _lib()
    cfg = _cfg()
    n = L.dflash_weight_count(ctypes.byref(cfg))
    assert n == 3 + 9 * cfg.n_layers
    h = ctypes.c_void_p()
    ptrs = (ctypes.c_void_p * n)(*([0x10000] * n))
    ptrs[4] = None
    assert _err(L.dflash_model_create(ctypes.byref(cfg), ptrs, ctypes.byref(h))) == "DFLASH_EINVAL"
    ptrs[4] = 0x10008
    assert _err(L.dflash_model_create(ctypes.byref(cfg), ptrs, ctypes.byref(h))) == "DFLASH_EALIGN"
    ptrs[4] = 0x10010
    assert L.dflash_model_create(ctypes.byref(cfg), ptrs, ctypes.byref(h)) == 0
    assert h.value
    L.dflash_model_destroy(h)


def _fake_model(name="tiny"):
    L = _lib()
    cfg = _cfg(name)
    n = L.dflash_weight_count(ctypes.byref(cfg))
    ptrs = (ctypes.c_void_p * n)(*([0x100000] * n))
    h = ctypes.c_void_p()
    assert L.dflash_model_create(ctypes.byref(cfg), ptrs, ctypes.byref(h)) == 0
    return cfg, h


def test_ctx_bytes_layout():
    L = _lib()
    cfg = _cfg("q8b_ctx1024")
    cap = (ctypes.c_int64 * 1)(1024)
    nbytes = L.dflash_ctx_bytes(ctypes.byref(cfg), 1, cap)
    slots = (1024 + cfg.max_block + 63) // 64 * 64
    kv = 5 * 2 * (2 * 8 * slots * 128 * 2)
    rope = 2 * slots * 64 * 4
    assert kv <= nbytes <= kv + rope + 12 * 256
    # K/V planes cost 8 bytes per (token, kv head, dim) — the same as fp32 K and V
    assert kv == 5 * slots * 8 * 128 * 8
    bad = (ctypes.c_int64 * 1)(-1)
    assert L.dflash_ctx_bytes(ctypes.byref(cfg), 1, bad) == 0
    assert L.dflash_ctx_bytes(ctypes.byref(cfg), 0, cap) == 0
    assert L.dflash_ctx_bytes(ctypes.byref(cfg), 129, (ctypes.c_int64 * 129)(*[1] * 129)) == 0


def test_ctx_create_validates_before_any_device_call():
    L = _lib()
    cfg, m = _fake_model()
    cap = (ctypes.c_int64 * 1)(128)
    h = ctypes.c_void_p()
    assert _err(L.dflash_ctx_create(m, None, 1 << 20, 1, cap, None, ctypes.byref(h))) == "DFLASH_EINVAL"
    assert _err(L.dflash_ctx_create(m, 0x1000 + 16, 1 << 20, 1, cap, None, ctypes.byref(h))) == "DFLASH_EALIGN"
    assert _err(L.dflash_ctx_create(m, 0x1000, 16, 1, cap, None, ctypes.byref(h))) == "DFLASH_ECAPACITY"
    assert _err(L.dflash_ctx_create(m, 0x1000, 1 << 20, 0, cap, None, ctypes.byref(h))) == "DFLASH_EUNSUPPORTED"
    assert not h.value
    L.dflash_model_destroy(m)


def test_workspace_bytes():
    L = _lib()
    cfg, m = _fake_model("q8b_ctx1024")
    a = L.dflash_workspace_bytes(m, 1, 16, 0)
    b = L.dflash_workspace_bytes(m, 32, 16, 0)
    c = L.dflash_workspace_bytes(m, 1, 16, 65536)
    assert 0 < a < b and a <= c
    assert L.dflash_workspace_bytes(m, 1, 1, 0) == 0
    assert L.dflash_workspace_bytes(m, 1, cfg.max_block + 1, 0) == 0
    assert L.dflash_workspace_bytes(m, 0, 16, 0) == 0
    L.dflash_model_destroy(m)


def test_model_pack_size_and_validation():
    L = _lib()
    cfg, m = _fake_model("q8b_ctx1024")
    H, I_, V = cfg.hidden, cfg.intermediate, cfg.vocab
    qkv = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim
    per_layer = (qkv * H + H * cfg.n_q_heads * cfg.head_dim + 2 * I_ * H + H * I_) * 2
    expect = H * cfg.n_target_layers * H * 2 + V * H * 2 + cfg.n_layers * per_layer
    assert L.dflash_model_pack_bytes(m) == expect  # every matrix a multiple of 256 bytes here
    assert L.dflash_model_pack_bytes(None) == 0
    assert _err(L.dflash_model_pack(None, 0x1000, 1 << 40, None)) == "DFLASH_EINVAL"
    assert _err(L.dflash_model_pack(m, 0x1000 + 16, 1 << 40, None)) == "DFLASH_EALIGN"
    assert _err(L.dflash_model_pack(m, 0x1000, expect - 1, None)) == "DFLASH_EWORKSPACE"
    assert L.dflash_model_pack(m, None, 0, None) == 0  # back to the row-major weights: no launch
    L.dflash_model_destroy(m)


def test_accept_len_validation():
    L = _lib()
    assert _err(L.dflash_accept_len(None, None, -1, 16, None, None, None)) == "DFLASH_EINVAL"
    assert _err(L.dflash_accept_len(None, None, 1, 1, None, None, None)) == "DFLASH_EINVAL"
    assert _err(L.dflash_accept_len(None, 0x1000, 1, 16, 0x1000, None, None)) == "DFLASH_EINVAL"
    assert _err(L.dflash_accept_len(0x1002, 0x1000, 1, 16, 0x1000, None, None)) == "DFLASH_EALIGN"
    # nothing to do is not an error
    assert L.dflash_accept_len(None, None, 0, 16, None, None, None) == 0


def test_draft_and_fuse_validation_without_context():
    L = _lib()
    cfg, m = _fake_model()
    assert _err(L.dflash_draft_block(m, None, 0x1000, 16, 0x1000, None, 0x1000, 1 << 20, None)) == "DFLASH_EINVAL"
    n_new = (ctypes.c_int32 * 1)(1)
    assert _err(L.dflash_fuse_ctx(m, None, 0x1000, n_new, 0x1000, 1 << 20, None)) == "DFLASH_EINVAL"
    assert _err(L.dflash_ctx_truncate(None, 0, 0)) == "DFLASH_EINVAL"
    assert L.dflash_ctx_length(None, 0) == -1
    L.dflash_model_destroy(m)


def test_probe_validation_and_empty_read():
    L = _lib()
    cfg, m = _fake_model()
    assert _err(L.dflash_probe_arm(None, 1, 4)) == "DFLASH_EINVAL"
    assert _err(L.dflash_probe_arm(m, 0, 4)) == "DFLASH_EINVAL"
    assert _err(L.dflash_probe_arm(m, len(B.STAGES) + 1, 4)) == "DFLASH_EINVAL"
    assert _err(L.dflash_probe_arm(m, B.STAGES["lm_head"], 0)) == "DFLASH_EINVAL"
    ms, n, missed = ctypes.c_double(-1.0), ctypes.c_int32(-1), ctypes.c_int32(-1)
    # a probe that was never armed reads as nothing timed, without any device call
    assert L.dflash_probe_read(m, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(missed)) == 0
    assert (ms.value, n.value, missed.value) == (0.0, 0, 0)
    assert _err(L.dflash_probe_read(m, None, ctypes.byref(n), None)) == "DFLASH_EINVAL"
    L.dflash_model_destroy(m)


def test_model_create_rejects_wide_gqa_groups():
    L = _lib()
    cfg = _cfg("q8b_ctx1024", n_kv_heads=2)  # 16 query heads per kv head
    n = L.dflash_weight_count(ctypes.byref(cfg))
    ptrs = (ctypes.c_void_p * n)(*([0x10000] * n))
    h = ctypes.c_void_p()
    assert _err(L.dflash_model_create(ctypes.byref(cfg), ptrs, ctypes.byref(h))) == "DFLASH_EUNSUPPORTED"


def test_verify_sample_validation_without_device_calls():
    L = _lib()
    sp = B.Sampling(0.8, 42)
    assert L.dflash_verify_workspace_bytes(4, 16, 4096) >= 4 * 16 * 32
    assert L.dflash_verify_workspace_bytes(4, 1, 4096) == 0
    assert L.dflash_verify_workspace_bytes(4, 16, 0) == 0
    assert L.dflash_verify_workspace_bytes(4, 16, 262145) == 0
    fake = ctypes.c_void_p(0x100000)
    acc = ctypes.c_void_p(0x200000)
    big = B.Sampling(1.0, 1)
    assert _err(L.dflash_verify_sample(fake, fake, fake, 1, 16, 262145, ctypes.byref(big), acc, acc, fake, 1 << 30,
                                       None)) == "DFLASH_EINVAL"
    # zero sequences: nothing to do, no device call
    assert L.dflash_verify_sample(None, None, None, 0, 16, 4096, ctypes.byref(sp), None, None, None, 0, None) == 0
    for bad_t in (0.0, -1.0, float("inf"), float("nan"), 2e6):
        bad = B.Sampling(bad_t, 1)
        assert _err(L.dflash_verify_sample(fake, fake, fake, 1, 16, 4096, ctypes.byref(bad), acc, acc, fake, 1 << 20,
                                           None)) == "DFLASH_EINVAL", bad_t
    assert _err(L.dflash_verify_sample(fake, fake, fake, 1, 16, 4096, None, acc, acc, fake, 1 << 20,
                                       None)) == "DFLASH_EINVAL"
    assert _err(L.dflash_verify_sample(fake, None, fake, 1, 16, 4096, ctypes.byref(sp), acc, acc, fake, 1 << 20,
                                       None)) == "DFLASH_EINVAL"
    assert _err(L.dflash_verify_sample(fake, fake, fake, 1, 1, 4096, ctypes.byref(sp), acc, acc, fake, 1 << 20,
                                       None)) == "DFLASH_EINVAL"
    assert _err(L.dflash_verify_sample(fake, fake, fake, 2, 16, 4096, ctypes.byref(sp), acc, acc, fake, 64,
                                       None)) == "DFLASH_EWORKSPACE"
    assert _err(L.dflash_verify_sample(ctypes.c_void_p(0x100002), fake, fake, 1, 16, 4096, ctypes.byref(sp), acc,
                                       acc, fake, 1 << 20, None)) == "DFLASH_EALIGN"


def test_sampled_draft_validation_without_context():
    L = _lib()
    cfg, m = _fake_model()
    sp = B.Sampling(1.0, 0)
    fake = ctypes.c_void_p(0x100000)
    assert _err(L.dflash_draft_sample(m, None, fake, 16, ctypes.byref(sp), fake, None, fake, 1 << 30,
                                      None)) == "DFLASH_EINVAL"
    assert _err(L.dflash_step_sample(m, None, None, None, fake, 16, None, fake, None, fake, 1 << 30,
                                     None)) == "DFLASH_EINVAL"
    L.dflash_model_destroy(m)
