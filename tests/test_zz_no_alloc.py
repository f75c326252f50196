"""The allocation-free step (dflash_step_noalloc) against dflash_step.

Two contexts receive the same ingest; one then steps through dflash_step with
a workspace, the other through dflash_step_noalloc (the library's static
device scratch).  Drafts, logits and every cache byte must be bitwise equal,
on two calls in a row, the second one smaller than the first (so the second
call runs over scratch the first left behind).  Oversized steps are rejected
before any work is enqueued."""
from __future__ import annotations

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


def _pair(torch, spec, w, lens, extra, packed=False):
    dev = B.upload_weights(spec, w)
    cfg = B.Config.from_spec(spec, max_block=32)
    model = B.Model(cfg, dev)
    if packed:
        model.pack()
    caps = [c + extra for c in lens]
    ctxs = [B.Context(model, caps), B.Context(model, caps)]
    ws = B.workspace(model, len(lens), 32, sum(lens))
    feats = [I.gen_features(spec, 5, b, c) for b, c in enumerate(lens)]
    packed_feats = to_dev_bf16(np.concatenate([f for f in feats if f.shape[0]], axis=0))
    for ctx in ctxs:
        B.fuse_ctx(model, ctx, packed_feats, lens, ws)
    torch.cuda.synchronize()
    return model, ctxs, ws, dev


def _step_both(torch, spec, model, ctxs, ws, n_new, block, seed, label):
    n = len(n_new)
    feats = [I.gen_features(spec, seed, b, k) for b, k in enumerate(n_new)]
    nz = [f for f in feats if f.shape[0]]
    fdev = to_dev_bf16(np.concatenate(nz, axis=0)) if nz else None
    anchors = torch.from_numpy(I.gen_anchors(spec.with_(ctx_lens=(0,) * n), seed).astype(np.int32)).cuda()
    outs = []
    for k, ctx in enumerate(ctxs):
        logits = torch.full((n, block - 1, spec.vocab), float("nan"), dtype=torch.float32, device="cuda")
        if k == 0:
            d = B.step(model, ctx, fdev, n_new, anchors, block, ws, logits=logits)
        else:
            d = B.step_noalloc(model, ctx, fdev, n_new, anchors, block, logits=logits)
        torch.cuda.synchronize()
        outs.append((d.cpu().numpy(), logits.cpu().numpy()))
    (d0, l0), (d1, l1) = outs
    np.testing.assert_array_equal(d1, d0)
    assert np.array_equal(l1.view(np.uint32), l0.view(np.uint32)), f"{label}: logits differ"
    assert ctxs[0].lengths() == ctxs[1].lengths()
    assert torch.equal(ctxs[0].buffer, ctxs[1].buffer), f"{label}: cache bytes differ"
    say(f"{label}: drafts, logits and cache equal; lengths {ctxs[1].lengths()}")


def test_noalloc_step_tiny_two_calls(torch_cuda):
    torch = torch_cuda
    spec = I.spec("tiny")
    w = I.gen_weights(spec, seed=3, gain_jitter=0.1, std=0.05)
    lens = [90, 41]
    model, ctxs, ws, _ = _pair(torch, spec, w, lens, extra=64)
    # fused sweep (8 + 8 block rows, 7 + 9 appended)
    _step_both(torch, spec, model, ctxs, ws, [7, 9], 8, 11, "tiny 2 seqs B8 + 16 appended")
    # smaller: block 4 and 3 + 0 appended rows
    _step_both(torch, spec, model, ctxs, ws, [3, 0], 4, 12, "tiny 2 seqs B4 + 3 appended")
    # larger than one sweep (falls back to append, then draft), then small again
    _step_both(torch, spec, model, ctxs, ws, [20, 19], 16, 13, "tiny 2 seqs B16 + 39 appended (two calls)")
    _step_both(torch, spec, model, ctxs, ws, [1, 1], 2, 14, "tiny 2 seqs B2 + 2 appended")


def test_noalloc_step_5layer_packed(torch_cuda):
    torch = torch_cuda
    spec = I.spec("q8b_ctx1024")
    say("generating 5-layer weights")
    w = I.gen_weights(spec, seed=0)
    model, ctxs, ws, _ = _pair(torch, spec, w, [1008], extra=64, packed=True)
    _step_both(torch, spec, model, ctxs, ws, [16], 16, 21, "5-layer ctx 1008 + 16, B16")
    _step_both(torch, spec, model, ctxs, ws, [4], 8, 22, "5-layer ctx 1024 + 4, B8")


def test_noalloc_step_rejects_oversized(torch_cuda):
    torch = torch_cuda
    spec = I.spec("q8b_ctx1024")
    cfg = B.Config.from_spec(spec, max_block=32)
    # weights are never read: the size check runs before any launch
    dummy = torch.zeros(256, dtype=torch.bfloat16, device="cuda")
    n = B.lib().dflash_weight_count(cfg)
    model = B.Model(cfg, [dummy] * n)
    ctx = B.Context(model, [64, 64, 64])
    need = B.workspace_bytes(model, 3, 32, 0)
    assert need > (48 << 20)
    anchors = torch.zeros(3, dtype=torch.int32, device="cuda")
    with pytest.raises(B.DFlashError) as ei:
        B.step_noalloc(model, ctx, None, [0, 0, 0], anchors, 32)
    assert ei.value.name == "DFLASH_EWORKSPACE"
    assert ctx.lengths() == [0, 0, 0]
