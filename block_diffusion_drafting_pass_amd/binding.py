"""Thin ctypes binding over ``libdflash.so`` (the C ABI in ``include/dflash.h``).

Argument marshalling only: torch tensors supply device memory
(``data_ptr()``) and the current HIP stream; every step of the draft pass
runs in the library's kernels.  There is no fallback: if the library is
missing, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdflash.so")

DFLASH_OK = 0
STATUS = {0: "DFLASH_OK", -1: "DFLASH_EINVAL", -2: "DFLASH_ESHAPE", -3: "DFLASH_ECAPACITY",
          -4: "DFLASH_EWORKSPACE", -5: "DFLASH_EALIGN", -6: "DFLASH_EHIP", -7: "DFLASH_EUNSUPPORTED"}

# Every symbol include/dflash.h declares.
EXPORTS = ("dflash_weight_count", "dflash_model_create", "dflash_model_destroy", "dflash_model_pack_bytes",
           "dflash_model_pack", "dflash_ctx_bytes",
           "dflash_ctx_create", "dflash_ctx_destroy", "dflash_ctx_length", "dflash_ctx_truncate",
           "dflash_workspace_bytes", "dflash_fuse_ctx", "dflash_draft_block", "dflash_draft_refine", "dflash_draft_anchored", "dflash_draft_sample",
    "dflash_verify_workspace_bytes", "dflash_verify_sample", "dflash_step", "dflash_step_noalloc",
           "dflash_step_sample", "dflash_accept_len",
           "dflash_probe_arm", "dflash_probe_read", "dflash_status_str", "dflash_last_error")

# Stages a measurement probe can bracket (dflash_stage in include/dflash.h).
STAGES = {"lm_head": 1, "gate_up": 2, "down": 3, "qkv": 4, "oproj": 5, "attention": 6, "fusion": 7,
          "kv_proj": 8}


class DFlashError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code
        self.name = STATUS.get(code, str(code))


class Config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("n_target_layers", ctypes.c_int32), ("mask_token_id", ctypes.c_int32),
                ("max_block", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_double)]

    @classmethod
    def from_spec(cls, s, max_block: Optional[int] = None) -> "Config":
        return cls(s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.intermediate, s.vocab,
                   s.n_target_layers, s.mask_token_id, max_block or max(s.block, 2), s.rms_eps, s.rope_theta)


_lib = None


def lib():
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_diffusion_drafting_pass_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.dflash_weight_count.argtypes = [ctypes.POINTER(Config)]
        L.dflash_weight_count.restype = i32
        L.dflash_model_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(vp), ctypes.POINTER(vp)]
        L.dflash_model_create.restype = ctypes.c_int
        L.dflash_model_destroy.argtypes = [vp]
        L.dflash_model_pack_bytes.restype = sz
        L.dflash_model_pack_bytes.argtypes = [vp]
        L.dflash_model_pack.restype = ctypes.c_int
        L.dflash_model_pack.argtypes = [vp, vp, sz, vp]
        L.dflash_model_destroy.restype = None
        L.dflash_ctx_bytes.argtypes = [ctypes.POINTER(Config), i32, ctypes.POINTER(i64)]
        L.dflash_ctx_bytes.restype = sz
        L.dflash_ctx_create.argtypes = [vp, vp, sz, i32, ctypes.POINTER(i64), vp, ctypes.POINTER(vp)]
        L.dflash_ctx_create.restype = ctypes.c_int
        L.dflash_ctx_destroy.argtypes = [vp]
        L.dflash_ctx_destroy.restype = None
        L.dflash_ctx_length.argtypes = [vp, i32]
        L.dflash_ctx_length.restype = i64
        L.dflash_ctx_truncate.argtypes = [vp, i32, i64]
        L.dflash_ctx_truncate.restype = ctypes.c_int
        L.dflash_workspace_bytes.argtypes = [vp, i32, i32, i64]
        L.dflash_workspace_bytes.restype = sz
        L.dflash_fuse_ctx.argtypes = [vp, vp, vp, ctypes.POINTER(i32), vp, sz, vp]
        L.dflash_fuse_ctx.restype = ctypes.c_int
        L.dflash_draft_block.argtypes = [vp, vp, vp, i32, vp, vp, vp, sz, vp]
        L.dflash_draft_block.restype = ctypes.c_int
        L.dflash_draft_refine.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, sz, vp]
        L.dflash_draft_refine.restype = ctypes.c_int
        L.dflash_draft_anchored.argtypes = [vp, vp, i32, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_int64), vp, vp,
                                            i32, vp, vp, vp, sz, vp]
        L.dflash_draft_anchored.restype = ctypes.c_int
        sp = ctypes.POINTER(Sampling)
        L.dflash_draft_sample.argtypes = [vp, vp, vp, i32, sp, vp, vp, vp, sz, vp]
        L.dflash_draft_sample.restype = ctypes.c_int
        L.dflash_step_sample.argtypes = [vp, vp, vp, ctypes.POINTER(i32), vp, i32, sp, vp, vp, vp, sz, vp]
        L.dflash_step_sample.restype = ctypes.c_int
        L.dflash_verify_workspace_bytes.argtypes = [i32, i32, i32]
        L.dflash_verify_workspace_bytes.restype = sz
        L.dflash_verify_sample.argtypes = [vp, vp, vp, i32, i32, i32, sp, vp, vp, vp, sz, vp]
        L.dflash_verify_sample.restype = ctypes.c_int
        L.dflash_step.argtypes = [vp, vp, vp, ctypes.POINTER(i32), vp, i32, vp, vp, vp, sz, vp]
        L.dflash_step.restype = ctypes.c_int
        L.dflash_step_noalloc.argtypes = [vp, vp, vp, ctypes.POINTER(i32), vp, i32, vp, vp, vp]
        L.dflash_step_noalloc.restype = ctypes.c_int
        L.dflash_accept_len.argtypes = [vp, vp, i32, i32, vp, vp, vp]
        L.dflash_accept_len.restype = ctypes.c_int
        L.dflash_probe_arm.argtypes = [vp, ctypes.c_int, i32]
        L.dflash_probe_arm.restype = ctypes.c_int
        L.dflash_probe_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.dflash_probe_read.restype = ctypes.c_int
        L.dflash_status_str.argtypes = [ctypes.c_int]
        L.dflash_status_str.restype = ctypes.c_char_p
        L.dflash_last_error.argtypes = []
        L.dflash_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def check(rc: int) -> None:
    if rc != DFLASH_OK:
        raise DFlashError(rc, lib().dflash_last_error().decode(errors="replace"))


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class Model:
    """A drafter whose weights live in torch bf16 device tensors (kept alive here)."""

    def __init__(self, cfg: Config, weights: Sequence):
        self.cfg = cfg
        self._weights = list(weights)
        n = lib().dflash_weight_count(ctypes.byref(cfg))
        if n != len(self._weights):
            raise DFlashError(-2, f"expected {n} weight tensors, got {len(self._weights)}")
        arr = (ctypes.c_void_p * n)(*[_ptr(w) for w in self._weights])
        h = ctypes.c_void_p()
        check(lib().dflash_model_create(ctypes.byref(cfg), arr, ctypes.byref(h)))
        self.handle = h

    def pack_bytes(self) -> int:
        return int(lib().dflash_model_pack_bytes(self.handle))

    def pack(self, device="cuda", stream=None) -> None:
        """Write the packed weight copy (dflash_model_pack) into a buffer kept here."""
        import torch
        n = self.pack_bytes()
        old = getattr(self, "_packed", None)
        if old is not None:
            torch.cuda.synchronize()  # passes already queued may still read the old copy
        self._packed = torch.empty(n, dtype=torch.uint8, device=device)
        check(lib().dflash_model_pack(self.handle, _ptr(self._packed), n, _stream(stream)))

    def unpack(self) -> None:
        """Go back to the original (row-major) weights."""
        import torch
        check(lib().dflash_model_pack(self.handle, None, 0, _stream(None)))
        if getattr(self, "_packed", None) is not None:
            # queued passes (on any stream) may still read the packed copy:
            # wait for them before its memory returns to the allocator
            torch.cuda.synchronize()
        self._packed = None

    def close(self) -> None:
        if getattr(self, "handle", None):
            lib().dflash_model_destroy(self.handle)
            self.handle = None

    __del__ = close


class Context:
    """Injected-context KV cache over a torch uint8 device buffer."""

    def __init__(self, model: Model, capacity: Sequence[int], device="cuda", stream=None):
        import torch
        self.model = model
        n = len(capacity)
        self._cap = (ctypes.c_int64 * n)(*[int(c) for c in capacity])
        nbytes = lib().dflash_ctx_bytes(ctypes.byref(model.cfg), n, self._cap)
        if nbytes == 0:
            raise DFlashError(-1, "invalid context arguments: " + lib().dflash_last_error().decode())
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        check(lib().dflash_ctx_create(model.handle, _ptr(self.buffer), nbytes, n, self._cap,
                                      _stream(stream), ctypes.byref(h)))
        self.handle = h
        self.n_seqs = n

    def length(self, seq: int) -> int:
        return int(lib().dflash_ctx_length(self.handle, seq))

    def lengths(self) -> List[int]:
        return [self.length(b) for b in range(self.n_seqs)]

    def truncate(self, seq: int, new_len: int) -> None:
        check(lib().dflash_ctx_truncate(self.handle, seq, int(new_len)))

    def close(self) -> None:
        if getattr(self, "handle", None):
            lib().dflash_ctx_destroy(self.handle)
            self.handle = None

    __del__ = close


def probe_arm(model: Model, stage: str, max_launches: int) -> None:
    """Bracket every later launch of ``stage`` with HIP events (measurement only)."""
    check(lib().dflash_probe_arm(model.handle, STAGES[stage], int(max_launches)))


def probe_read(model: Model):
    """Wait for the probe's events; return (total_ms, timed_launches, missed) and disarm it."""
    ms, n, missed = ctypes.c_double(), ctypes.c_int32(), ctypes.c_int32()
    check(lib().dflash_probe_read(model.handle, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(missed)))
    return ms.value, n.value, missed.value


def workspace_bytes(model: Model, n_seqs: int, block: int, max_new_tokens: int = 0) -> int:
    return int(lib().dflash_workspace_bytes(model.handle, n_seqs, block, max_new_tokens))


def workspace(model: Model, n_seqs: int, block: int, max_new_tokens: int = 0, device="cuda"):
    import torch
    n = workspace_bytes(model, n_seqs, block, max_new_tokens)
    if n == 0:
        raise DFlashError(-1, "invalid workspace arguments")
    return torch.empty(n, dtype=torch.uint8, device=device)


def fuse_ctx(model: Model, ctx: Context, features, n_new: Sequence[int], ws, stream=None) -> None:
    arr = (ctypes.c_int32 * ctx.n_seqs)(*[int(v) for v in n_new])
    check(lib().dflash_fuse_ctx(model.handle, ctx.handle, _ptr(features), arr, _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)))


def draft_block(model: Model, ctx: Context, anchors, block: int, ws, draft=None, logits=None, stream=None):
    import torch
    if draft is None:
        draft = torch.empty((ctx.n_seqs, block - 1), dtype=torch.int32, device=anchors.device)
    check(lib().dflash_draft_block(model.handle, ctx.handle, _ptr(anchors), block, _ptr(draft), _ptr(logits),
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return draft


def draft_refine(model: Model, ctx: Context, anchors, block: int, n_steps: int, ws, init_tokens=None, draft=None,
                 logits=None, stream=None):
    """n_steps denoising passes; each later pass feeds the previous pass's drafts."""
    import torch
    if draft is None:
        draft = torch.empty((ctx.n_seqs, block - 1), dtype=torch.int32, device=anchors.device)
    check(lib().dflash_draft_refine(model.handle, ctx.handle, _ptr(anchors), _ptr(init_tokens), block, n_steps,
                                    _ptr(draft), _ptr(logits), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)))
    return draft


def draft_anchored(model: Model, ctx: Context, block_seq: Sequence[int], anchor_pos: Sequence[int], anchors,
                   block: int, ws, block_tokens=None, draft=None, logits=None, stream=None):
    """Blocks anchored at given positions of shared contexts (each sees its
    sequence's context before its anchor, and itself)."""
    import torch
    n = len(block_seq)
    if len(anchor_pos) != n:
        raise ValueError("block_seq and anchor_pos differ in length")
    if draft is None:
        draft = torch.empty((n, block - 1), dtype=torch.int32, device=anchors.device)
    seq_arr = (ctypes.c_int32 * n)(*[int(v) for v in block_seq])
    pos_arr = (ctypes.c_int64 * n)(*[int(v) for v in anchor_pos])
    check(lib().dflash_draft_anchored(model.handle, ctx.handle, n, seq_arr, pos_arr, _ptr(anchors),
                                      _ptr(block_tokens), block, _ptr(draft), _ptr(logits), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)))
    return draft


class Sampling(ctypes.Structure):
    """dflash_sampling: temperature (> 0) and the seed of the random numbers."""
    _fields_ = [("temperature", ctypes.c_double), ("seed", ctypes.c_uint64)]


def draft_sample(model: Model, ctx: Context, anchors, block: int, temperature: float, seed: int, ws, draft=None,
                 logits=None, stream=None):
    """Sampled drafts (softmax(logits / temperature) by the Gumbel-max rule)."""
    import torch
    if draft is None:
        draft = torch.empty((ctx.n_seqs, block - 1), dtype=torch.int32, device=anchors.device)
    sp = Sampling(float(temperature), int(seed) & ((1 << 64) - 1))
    check(lib().dflash_draft_sample(model.handle, ctx.handle, _ptr(anchors), block, ctypes.byref(sp), _ptr(draft),
                                    _ptr(logits), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return draft


def verify_sample(draft, draft_logits, target_logits, block: int, temperature: float, seed: int, ws=None,
                  accept=None, next_token=None, stream=None):
    """Lossless verification of sampled blocks; returns (accept, next_token)."""
    import torch
    n = draft.shape[0]
    vocab = target_logits.shape[-1]
    dev = draft.device
    if accept is None:
        accept = torch.empty(n, dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty(n, dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.empty(max(1, int(lib().dflash_verify_workspace_bytes(n, block, vocab))), dtype=torch.uint8,
                         device=dev)
    sp = Sampling(float(temperature), int(seed) & ((1 << 64) - 1))
    check(lib().dflash_verify_sample(_ptr(draft), _ptr(draft_logits), _ptr(target_logits), n, block, vocab,
                                     ctypes.byref(sp), _ptr(accept), _ptr(next_token), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)))
    return accept, next_token


def step(model: Model, ctx: Context, features, n_new: Sequence[int], anchors, block: int, ws, draft=None,
         logits=None, stream=None):
    """Append n_new verified positions per sequence and draft a block at the new lengths."""
    import torch
    if draft is None:
        draft = torch.empty((ctx.n_seqs, block - 1), dtype=torch.int32, device=anchors.device)
    arr = (ctypes.c_int32 * ctx.n_seqs)(*[int(v) for v in n_new])
    check(lib().dflash_step(model.handle, ctx.handle, _ptr(features), arr, _ptr(anchors), block, _ptr(draft),
                            _ptr(logits), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return draft


def step_noalloc(model: Model, ctx: Context, features, n_new: Sequence[int], anchors, block: int, draft=None,
                 logits=None, stream=None):
    """dflash_step without a workspace argument: the library's static device scratch."""
    import torch
    if draft is None:
        draft = torch.empty((ctx.n_seqs, block - 1), dtype=torch.int32, device=anchors.device)
    arr = (ctypes.c_int32 * ctx.n_seqs)(*[int(v) for v in n_new])
    check(lib().dflash_step_noalloc(model.handle, ctx.handle, _ptr(features), arr, _ptr(anchors), block,
                                    _ptr(draft), _ptr(logits), _stream(stream)))
    return draft


def step_sample(model: Model, ctx: Context, features, n_new: Sequence[int], anchors, block: int, temperature: float,
                seed: int, ws, draft=None, logits=None, stream=None):
    """dflash_step with sampled drafts."""
    import torch
    if draft is None:
        draft = torch.empty((ctx.n_seqs, block - 1), dtype=torch.int32, device=anchors.device)
    arr = (ctypes.c_int32 * ctx.n_seqs)(*[int(v) for v in n_new])
    sp = Sampling(float(temperature), int(seed) & ((1 << 64) - 1))
    check(lib().dflash_step_sample(model.handle, ctx.handle, _ptr(features), arr, _ptr(anchors), block,
                                   ctypes.byref(sp), _ptr(draft), _ptr(logits), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)))
    return draft


def accept_len(draft, target, block: int, accept=None, next_anchor=None, stream=None):
    import torch
    n = draft.shape[0]
    if accept is None:
        accept = torch.empty(n, dtype=torch.int32, device=draft.device)
    if next_anchor is None:
        next_anchor = torch.empty(n, dtype=torch.int32, device=draft.device)
    check(lib().dflash_accept_len(_ptr(draft), _ptr(target), n, block, _ptr(accept), _ptr(next_anchor),
                                  _stream(stream)))
    return accept, next_anchor


def upload_weights(spec, weights: Dict, device="cuda") -> List:
    """bf16 bit arrays (numpy uint16) -> torch bf16 device tensors in ABI order."""
    import numpy as np
    import torch
    from .inputs import weight_names
    out = []
    for name in weight_names(spec):
        a = np.ascontiguousarray(weights[name])
        out.append(torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16))
    return out
