"""GPU checks that hold at any size, without the oracle:

* argmax ties: with two bitwise-equal rows of the shared embedding / LM head
  the GPU logits of the two vocabulary entries are bitwise equal and the draft
  is the lower index (the contract's lowest-index tie-break), while every
  other logit is unchanged bit for bit;
* guard bands: bytes just before and after the context buffer, the workspace,
  the drafts and the logits keep their fill pattern through ingest, a fused
  step, a step that falls back to append-then-draft, a draft pass and the
  accept scan (an out-of-range write by any kernel would change them)."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from block_diffusion_drafting_pass_amd import binding as B
from block_diffusion_drafting_pass_amd import inputs as I
from tests.gpu_harness import say, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    B.lib()
    return torch


# ----------------------------------------------------------------------------
# lowest-index tie-break on exactly equal logits
# ----------------------------------------------------------------------------

def _draft(torch, model, ctx, anchors, block, ws, vocab):
    n = ctx.n_seqs
    lg = torch.empty((n, block - 1, vocab), dtype=torch.float32, device="cuda")
    d = B.draft_block(model, ctx, anchors, block, ws, logits=lg)
    torch.cuda.synchronize()
    return d.cpu().numpy(), lg.cpu().numpy()


def _free_index(start, step, vocab, avoid):
    u = start
    while 0 <= u < vocab and u in avoid:
        u += step
    return u if 0 <= u < vocab else None


def _tie_case(torch, spec, w, lens, packed, label):
    dev = B.upload_weights(spec, w)
    cfg = B.Config.from_spec(spec, max_block=32)
    model = B.Model(cfg, dev)
    if packed:
        model.pack()
    ctx = B.Context(model, [c + 64 for c in lens])
    ws = B.workspace(model, len(lens), spec.block, sum(lens))
    feats = [I.gen_features(spec, 1, b, c) for b, c in enumerate(lens)]
    B.fuse_ctx(model, ctx, to_dev_bf16(np.concatenate(feats, 0)), lens, ws)
    anchors_np = I.gen_anchors(spec.with_(ctx_lens=tuple(lens)), 2)
    anchors = torch.from_numpy(anchors_np).cuda()
    d0, l0 = _draft(torch, model, ctx, anchors, spec.block, ws, spec.vocab)
    # the row whose top token leads its runner-up by the most (GPU logits)
    srt = np.sort(l0, axis=-1)
    gap = srt[..., -1] - srt[..., -2]
    gap[d0 == 0] = -1.0  # a lower index must exist
    b, i = np.unravel_index(int(np.argmax(gap)), gap.shape)
    assert gap[b, i] > 0.05, f"{label}: no clearly decided row"
    v = int(d0[b, i])
    avoid = set(int(a) for a in anchors_np) | {spec.mask_token_id, v}
    variants = [("lower", _free_index(v - 1, -1, spec.vocab, avoid), True),
                ("higher", _free_index(v + 1, 1, spec.vocab, avoid), False)]
    for name, u, wins in variants:
        if u is None:
            continue
        dev2 = list(dev)
        emb = dev[1].clone()
        emb[u] = emb[v]  # row u of the embedding / LM head becomes a copy of row v
        dev2[1] = emb
        m2 = B.Model(cfg, dev2)
        if packed:
            m2.pack()
        d1, l1 = _draft(torch, m2, ctx, anchors, spec.block, ws, spec.vocab)
        assert l1[b, i, u].view(np.uint32) == l1[b, i, v].view(np.uint32), f"{label}: tied logits differ"
        assert int(d1[b, i]) == (u if wins else v), f"{label} ({name}): draft {d1[b, i]}, tie of {u} and {v}"
        keep = np.ones(spec.vocab, bool)
        keep[u] = False
        assert np.array_equal(l1[..., keep].view(np.uint32), l0[..., keep].view(np.uint32)), \
            f"{label}: logits other than column {u} changed"
        say(f"{label}: row ({b}, {i}) top {v}; copy at {u} ({name}) -> draft {int(d1[b, i])}")
        m2.close()


def test_tie_break_tiny(torch_cuda):
    spec = I.spec("tiny")
    w = I.gen_weights(spec, seed=4, std=0.05)
    _tie_case(torch_cuda, spec, w, [100, 37], packed=False, label="tiny two seqs")


def test_tie_break_tiny_many_rows(torch_cuda):
    spec = I.spec("tiny")
    w = I.gen_weights(spec, seed=5, std=0.05)
    _tie_case(torch_cuda, spec, w, [30, 64, 9], packed=False, label="tiny three seqs (many-row LM head)")


def test_tie_break_q8_packed(torch_cuda):
    spec = I.spec("q8b_ctx1024")
    say("generating 5-layer weights")
    w = I.gen_weights(spec, seed=0)
    _tie_case(torch_cuda, spec, w, [1024], packed=True, label="5-layer packed ctx 1024")


# ----------------------------------------------------------------------------
# guard bands around every buffer a call writes
# ----------------------------------------------------------------------------

GUARD = 4096  # bytes; a multiple of 256 keeps the interior 256-byte aligned
FILL = 0xA5


class _Guarded:
    """A uint8 device buffer with GUARD fill bytes on both sides of `nbytes`."""

    def __init__(self, torch, nbytes):
        self.t = torch.full((nbytes + 2 * GUARD,), FILL, dtype=torch.uint8, device="cuda")
        self.nbytes = nbytes
        self.inner = self.t[GUARD:GUARD + nbytes]
        assert self.inner.data_ptr() % 256 == 0

    def intact(self):
        host = self.t.cpu().numpy()
        return bool(np.all(host[:GUARD] == FILL) and np.all(host[GUARD + self.nbytes:] == FILL))


class _Ctx:
    """dflash_ctx over a guarded buffer (the binding's Context allocates its own)."""

    def __init__(self, model, caps, buf):
        n = len(caps)
        self._cap = (ctypes.c_int64 * n)(*caps)
        h = ctypes.c_void_p()
        B.check(B.lib().dflash_ctx_create(model.handle, buf.inner.data_ptr(), buf.nbytes, n, self._cap,
                                          B._stream(None), ctypes.byref(h)))
        self.handle = h
        self.n_seqs = n

    def lengths(self):
        return [int(B.lib().dflash_ctx_length(self.handle, b)) for b in range(self.n_seqs)]

    def truncate(self, b, n):
        B.check(B.lib().dflash_ctx_truncate(self.handle, b, n))

    def close(self):
        B.lib().dflash_ctx_destroy(self.handle)


def _guard_case(torch, spec, w, lens, block, appends, packed, label):
    dev = B.upload_weights(spec, w)
    cfg = B.Config.from_spec(spec, max_block=32)
    model = B.Model(cfg, dev)
    if packed:
        model.pack()
    n = len(lens)
    caps = [c + sum(a[b] for a in appends) + 8 for b, c in enumerate(lens)]
    cbytes = B.lib().dflash_ctx_bytes(ctypes.byref(cfg), n, (ctypes.c_int64 * n)(*caps))
    cbuf = _Guarded(torch, cbytes)
    ctx = _Ctx(model, caps, cbuf)
    max_new = max(sum(lens), max(sum(a) for a in appends))
    wbuf = _Guarded(torch, B.workspace_bytes(model, n, block, max_new))
    wsz = wbuf.nbytes
    ws = wbuf.inner
    nd = n * (block - 1)
    dbuf = torch.full((nd + 2 * GUARD // 4,), -0x5A5A5A5B, dtype=torch.int32, device="cuda")
    draft = dbuf[GUARD // 4:GUARD // 4 + nd].view(n, block - 1)
    nl = nd * spec.vocab
    lbuf = torch.full((nl + 2 * GUARD // 4,), float("nan"), dtype=torch.float32, device="cuda")
    logits = lbuf[GUARD // 4:GUARD // 4 + nl].view(n, block - 1, spec.vocab)
    anchors = torch.from_numpy(I.gen_anchors(spec.with_(ctx_lens=tuple(lens)), 3)).cuda()

    def check(what):
        torch.cuda.synchronize()
        d = dbuf.cpu().numpy()
        lg = lbuf.cpu().numpy().view(np.uint32)
        nan = np.float32(np.nan).view(np.uint32)
        assert cbuf.intact(), f"{label}: context guard changed after {what}"
        assert wbuf.intact(), f"{label}: workspace guard changed after {what}"
        g = GUARD // 4
        assert np.all(d[:g] == -0x5A5A5A5B) and np.all(d[g + nd:] == -0x5A5A5A5B), f"{label}: draft guard ({what})"
        assert np.all(lg[:g] == nan) and np.all(lg[g + nl:] == nan), f"{label}: logits guard ({what})"

    feats = [I.gen_features(spec, 1, b, c) for b, c in enumerate(lens)]
    nz = [f for f in feats if f.shape[0]]
    B.check(B.lib().dflash_fuse_ctx(model.handle, ctx.handle, to_dev_bf16(np.concatenate(nz, 0)).data_ptr(),
                                    (ctypes.c_int32 * n)(*lens), ws.data_ptr(), wsz, B._stream(None)))
    check("ingest")
    for k, app in enumerate(appends):
        f = [I.gen_features(spec, 10 + k, b, a) for b, a in enumerate(app)]
        nz = [x for x in f if x.shape[0]]
        fd = to_dev_bf16(np.concatenate(nz, 0)) if nz else None
        B.check(B.lib().dflash_step(model.handle, ctx.handle, None if fd is None else fd.data_ptr(),
                                    (ctypes.c_int32 * n)(*app), anchors.data_ptr(), block, draft.data_ptr(),
                                    logits.data_ptr(), ws.data_ptr(), wsz, B._stream(None)))
        check(f"step {app}")
    B.check(B.lib().dflash_draft_block(model.handle, ctx.handle, anchors.data_ptr(), block, draft.data_ptr(),
                                       logits.data_ptr(), ws.data_ptr(), wsz, B._stream(None)))
    check("draft")
    assert np.all(np.isfinite(logits.cpu().numpy())), f"{label}: a logit was left unwritten"
    target = torch.randint(0, spec.vocab, (n, block), dtype=torch.int32, device="cuda")
    acc, nxt = B.accept_len(draft, target, block)
    check("accept")
    say(f"{label}: guard bands intact; lengths {ctx.lengths()}")
    ctx.close()


def test_guard_bands_tiny_few_rows(torch_cuda):
    spec = I.spec("tiny")
    w = I.gen_weights(spec, seed=6, std=0.05)
    _guard_case(torch_cuda, spec, w, [70, 13], 16, [(9, 7), (20, 30)], packed=False, label="tiny 2 seqs B16")


def test_guard_bands_tiny_many_rows(torch_cuda):
    spec = I.spec("tiny")
    w = I.gen_weights(spec, seed=7, std=0.05)
    _guard_case(torch_cuda, spec, w, [5, 200, 64, 0, 31], 32, [(1, 2, 3, 4, 5), (0, 0, 0, 0, 0)], packed=False,
                label="tiny 5 seqs B32 (many-row kernels)")


def test_guard_bands_q8_packed(torch_cuda):
    spec = I.spec("q8b_ctx1024")
    say("generating 5-layer weights")
    w = I.gen_weights(spec, seed=0)
    _guard_case(torch_cuda, spec, w, [1000], 16, [(16,), (3,)], packed=True, label="5-layer packed 1 seq")
