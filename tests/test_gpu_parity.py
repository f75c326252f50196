"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
on identical seeded inputs.  Covers the five workload shapes (tiny drafter;
Qwen3-8B-shaped drafter at context 1024, 8192, concurrency 32, and a ragged
3-layer block-32 batch) plus edge cases: empty context, ragged lengths, block
sizes 2/4/32, the tiled (many-row) GEMM path, incremental appends with a
truncation, determinism, and the accepted-prefix scan."""
from __future__ import annotations

import os

import numpy as np
import pytest

from block_diffusion_drafting_pass_amd import binding as B
from block_diffusion_drafting_pass_amd import inputs as I
from oracle import dflash_oracle as O
from tests.gpu_harness import LOGIT_TOL, GpuRun, accept_check, assert_parity, oracle_run, say, to_dev_bf16

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="session")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    B.lib()  # fails loudly when the library is missing
    return torch


@pytest.fixture(scope="session")
def q8(torch_cuda):
    """Qwen3-8B-shaped drafter weights (5 layers), host bits and device tensors."""
    spec = I.spec("q8b_ctx1024")
    say("generating 5-layer Qwen3-8B-shaped weights")
    w = I.gen_weights(spec, seed=0)
    dev = B.upload_weights(spec, w)
    torch_cuda.cuda.synchronize()
    return spec, w, dev


def _feats(spec, seed, lens):
    return [I.gen_features(spec, seed, b, c) for b, c in enumerate(lens)]


# ----------------------------------------------------------------------------
# accepted-prefix scan
# ----------------------------------------------------------------------------

def test_accept_len_golden_cases(torch_cuda):
    torch = torch_cuda
    path = os.path.join(HERE, "golden", "accept_cases.txt")
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        blk, dr, tg, res = (p.split() for p in line.split("|"))
        Bk = int(blk[0])
        d = torch.tensor([[int(v) for v in dr]], dtype=torch.int32, device="cuda")
        t = torch.tensor([[int(v) for v in tg]], dtype=torch.int32, device="cuda")
        acc, nxt = B.accept_len(d, t, Bk)
        assert (int(acc.item()), int(nxt.item())) == (int(res[0]), int(res[1])), line


@pytest.mark.parametrize("block,n", [(16, 1000), (32, 777), (2, 5), (16, 1)])
def test_accept_len_constructed(torch_cuda, block, n):
    torch = torch_cuda
    spec = I.spec("q8b_conc32").with_(block=block, ctx_lens=(0,) * n)
    rng = np.random.default_rng(block * 1000 + n)
    draft = rng.integers(0, spec.vocab, size=(n, block - 1)).astype(np.int32)
    K, r, bonus = I.gen_accept_construction(spec, seed=block)
    target = I.make_targets(draft, K, r, bonus, spec.vocab)
    acc_ref, nxt_ref = O.accept_len(draft, target)
    acc, nxt = B.accept_len(torch.from_numpy(draft).cuda(), torch.from_numpy(target).cuda(), block)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
    np.testing.assert_array_equal(nxt.cpu().numpy(), nxt_ref)
    np.testing.assert_array_equal(acc_ref, np.minimum(K, block - 1))


def test_accept_len_empty_batch(torch_cuda):
    torch = torch_cuda
    d = torch.empty((0, 15), dtype=torch.int32, device="cuda")
    t = torch.empty((0, 16), dtype=torch.int32, device="cuda")
    acc, _ = B.accept_len(d, t, 16)
    assert acc.numel() == 0


# ----------------------------------------------------------------------------
# tiny drafter: full configuration and edge cases
# ----------------------------------------------------------------------------

def _tiny_case(spec, lens, block, wseed=0, jitter=0.0, std=0.02, label=""):
    say(f"tiny case {label}: lens={lens} block={block}")
    spec = spec.with_(ctx_lens=tuple(lens), block=block)
    w = I.gen_weights(spec, seed=wseed, gain_jitter=jitter, std=std)
    run = GpuRun(spec, B.upload_weights(spec, w), capacity=[c + 8 for c in lens], max_new=sum(lens))
    feats = _feats(spec, 1, lens)
    run.ingest(feats)
    anchors = I.gen_anchors(spec, 2)
    drafts, logits = run.draft(anchors, block)
    ref = oracle_run(spec, w, feats, anchors, block)
    assert_parity(logits, drafts, ref, label)
    accept_check(drafts, ref, spec, 3, label)
    return run, drafts, logits


def test_tiny_config(torch_cuda):
    _tiny_case(I.spec("tiny"), (128,), 16, label="tiny ctx128 B16")


@pytest.mark.parametrize("lens,block,jitter,std,label", [
    # the benchmark's 0.02 weights leave every row of the tiny drafter's
    # context-free pass within 0.04 of its runner-up, so nothing would be decided
    ((0,), 16, 0.0, 0.05, "empty context"),
    ((37, 5, 0), 4, 0.0, 0.05, "ragged 3 seqs B4"),
    ((10, 20), 16, 0.0, 0.05, "two seqs M32 skinny"),
    ((100, 64, 33), 16, 0.0, 0.05, "three seqs M48 tiled"),
    ((64, 200), 32, 0.1, 0.05, "B32 two seqs tiled"),
    ((50,), 2, 0.1, 0.05, "block 2"),
    ((128,), 16, 0.1, 0.05, "gain jitter"),
    ((300,) * 5, 32, 0.0, 0.03, "five seqs B32 M160"),
    ((20, 5, 0, 33, 64, 7, 100, 12), 16, 0.0, 0.05, "eight seqs M128 big tiles"),
    (tuple(range(3, 3 + 16 * 13, 13)), 16, 0.1, 0.05, "sixteen seqs M256 big tiles"),
    ((130, 64, 200, 9), 32, 0.0, 0.05, "four seqs B32 M128 big tiles"),
])
def test_tiny_variants(torch_cuda, lens, block, jitter, std, label):
    _tiny_case(I.spec("tiny"), lens, block, jitter=jitter, std=std, label=label)


# One sequence of the tiny drafter (two kv heads) at contexts whose key tiles
# give 3, 7, 15, 20, 30, 45 and 60 attention splits of one tile, and 126
# tiles in 63 splits of two: every size of the split merge.
@pytest.mark.parametrize("ctx", [172, 428, 940, 1260, 1900, 2860, 3820, 8044])
def test_tiny_attention_splits(torch_cuda, ctx):
    _tiny_case(I.spec("tiny"), (ctx,), 16, std=0.05, label=f"ctx {ctx} splits")


# Long contexts whose splits hold several tiles, so that each query unit
# runs as two waves over the two halves of every tile (blocks of 4, 16 and
# 32; the last tile holds 44, 48, 64 and 28 keys: at context 12300 its second
# half has no valid key).
@pytest.mark.parametrize("ctx,block", [(9000, 4), (20000, 16), (20000, 32), (12300, 16)])
def test_tiny_attention_halves(torch_cuda, ctx, block):
    _tiny_case(I.spec("tiny"), (ctx,), block, std=0.05, label=f"ctx {ctx} B{block} halves")


# The splits above hold at most eight tiles, which the double-buffered
# attention kernel takes; eight sequences of 135-141 tiles give splits of
# nine tiles, which take the single-buffer sixteen-wave one (as 32 x 2048 does).
def test_tiny_attention_long_splits(torch_cuda):
    lens = (8900, 8700, 9000, 8950, 8800, 8999, 8600, 8912)
    _tiny_case(I.spec("tiny"), lens, 16, std=0.05, label="8 seqs ~8900 long splits")


def test_tiny_incremental_append_and_truncate(torch_cuda):
    spec = I.spec("tiny").with_(ctx_lens=(0, 0))
    w = I.gen_weights(spec, seed=4, std=0.05)
    run = GpuRun(spec, B.upload_weights(spec, w), capacity=[300, 300], max_new=200)
    model = O.OracleModel.from_spec(spec, w)
    octx = O.OracleContext(model, 2)
    anchors = I.gen_anchors(spec, 5)
    steps = [([100, 7], 0), ([40, 0], 1), ([1, 33], 2)]
    for n_new, fseed in steps:
        feats = [I.gen_features(spec, 10 + fseed, b, n) for b, n in enumerate(n_new)]
        run.ingest(feats)
        for b in range(2):
            O.fuse_ctx(model, octx, b, feats[b])
        assert run.ctx.lengths() == [octx.length(0), octx.length(1)]
        drafts, logits = run.draft(anchors, 16)
        assert_parity(logits, drafts, O.draft_block(model, octx, anchors, 16), f"append {n_new}")
    # roll sequence 0 back and append different positions there
    run.ctx.truncate(0, 90)
    O.truncate_ctx(octx, 0, 90)
    feats = [I.gen_features(spec, 99, 0, 12), I.gen_features(spec, 99, 1, 0)]
    run.ingest(feats)
    O.fuse_ctx(model, octx, 0, feats[0])
    drafts, logits = run.draft(anchors, 16)
    assert_parity(logits, drafts, O.draft_block(model, octx, anchors, 16), "after truncate")


def test_capacity_error_leaves_lengths(torch_cuda):
    spec = I.spec("tiny").with_(ctx_lens=(10,))
    w = I.gen_weights(spec, seed=0)
    run = GpuRun(spec, B.upload_weights(spec, w), capacity=[20], max_new=40)
    run.ingest(_feats(spec, 1, [10]))
    with pytest.raises(B.DFlashError) as e:
        run.ingest(_feats(spec, 1, [11]))
    assert e.value.name == "DFLASH_ECAPACITY"
    assert run.ctx.lengths() == [10]


def test_draft_is_deterministic(torch_cuda):
    run, d1, l1 = _tiny_case(I.spec("tiny"), (128, 3), 16, std=0.05, label="determinism")
    anchors = I.gen_anchors(run.spec, 2)
    for _ in range(3):
        d2, l2 = run.draft(anchors, 16)
        assert np.array_equal(d1, d2)
        assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


# ----------------------------------------------------------------------------
# Qwen3-8B-shaped drafter at the workload sizes
# ----------------------------------------------------------------------------

def _q8_case(q8, name, seqs=None, n_layers=None, label="", ctx_lens=None):
    spec5, w, dev = q8
    spec = I.spec(name)
    if ctx_lens is not None:
        spec = spec.with_(ctx_lens=tuple(ctx_lens))
    nl = spec.n_layers
    dev_w = dev[: 3 + 9 * nl]
    lens = spec.ctx_lens
    say(f"{label}: {name} lens[:4]={lens[:4]} n_seqs={len(lens)} block={spec.block} layers={nl}")
    run = GpuRun(spec, dev_w, capacity=[c + 64 for c in lens], max_new=sum(lens))
    feats = _feats(spec, 1, lens)
    run.ingest(feats)
    anchors = I.gen_anchors(spec, 2)
    drafts, logits = run.draft(anchors, spec.block)
    say(f"{label}: GPU pass done; running the oracle on sequences {seqs if seqs else 'all'}")
    ref = oracle_run(spec, w, feats, anchors, spec.block, seqs=seqs)
    sel = list(range(len(lens))) if seqs is None else seqs
    assert_parity(logits[sel], drafts[sel], ref, label)
    accept_check(drafts[sel], ref, spec, 3, label)
    return run, drafts, logits


def test_q8_ctx1024(q8):
    _q8_case(q8, "q8b_ctx1024", label="5-layer ctx1024")


def test_q8_two_seqs_m32(q8):
    # 32 block rows on the weight-streaming kernel: the SwiGLU projection
    # with two row groups over six column tiles per workgroup
    _q8_case(q8, "q8b_ctx1024", label="5-layer two seqs M32", ctx_lens=(512, 1000))


def test_q8_ctx8192(q8):
    _q8_case(q8, "q8b_ctx8192", label="5-layer ctx8192")


def test_q8_conc32(q8):
    _q8_case(q8, "q8b_conc32", seqs=[0, 13, 31], label="5-layer conc32")


def test_q8_ragged_b32(q8):
    lens = I.spec("q8b_l3_b32_ragged").ctx_lens
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 3})
    _q8_case(q8, "q8b_l3_b32_ragged", seqs=seqs, label="3-layer ragged B32")


def _short_ragged(seed, n, lo=64, hi=300):
    rng = np.random.default_rng(seed)
    return tuple(int(v) for v in rng.integers(lo, hi + 1, size=n))


def test_q8_conc32_every_sequence(q8):
    # the 32-sequence shape (512 block rows on the many-row kernels) over
    # short ragged contexts, so that the oracle runs every sequence
    _q8_case(q8, "q8b_conc32", label="5-layer 32 seqs short ctx, all compared", ctx_lens=_short_ragged(77, 32))


def test_q8_l3_b32_every_sequence(q8):
    # the 3-layer block-32 batch of eight sequences, every sequence compared
    _q8_case(q8, "q8b_l3_b32_ragged", label="3-layer B32 8 seqs short ctx, all compared",
             ctx_lens=_short_ragged(78, 8))


# ----------------------------------------------------------------------------
# dflash_step: append + draft in one call (fused weight sweep when <= 32 rows)
# ----------------------------------------------------------------------------

def _step_case(spec, w, dev_w, base_lens, n_new, block, label, two_call_check=True):
    """Ingest base_lens, then dflash_step(n_new) vs the oracle (fuse then draft) and
    vs the two-call GPU path on a second context."""
    import torch
    spec = spec.with_(ctx_lens=tuple(base_lens), block=block)
    cap = [b + k + 8 for b, k in zip(base_lens, n_new)]
    run = GpuRun(spec, dev_w, capacity=cap, max_new=sum(base_lens) + sum(n_new), max_block=32)
    run2 = GpuRun(spec, dev_w, capacity=cap, max_new=sum(base_lens) + sum(n_new), max_block=32)
    feats = [I.gen_features(spec, 1, b, c + k) for b, (c, k) in enumerate(zip(base_lens, n_new))]
    run.ingest([f[:c] for f, c in zip(feats, base_lens)])
    run2.ingest([f[:c] for f, c in zip(feats, base_lens)])
    newrows = [f[c:] for f, c in zip(feats, base_lens)]
    nonempty = [r for r in newrows if r.shape[0]]
    dev_new = (torch.from_numpy(np.ascontiguousarray(np.concatenate(nonempty, 0)).view(np.int16)).cuda()
               .view(torch.bfloat16) if nonempty else None)
    anchors = I.gen_anchors(spec, 2)
    a = torch.from_numpy(anchors).cuda()
    n = len(base_lens)
    lg = torch.empty((n, block - 1, spec.vocab), dtype=torch.float32, device="cuda")
    d = B.step(run.model, run.ctx, dev_new, n_new, a, block, run.ws, logits=lg)
    torch.cuda.synchronize()
    assert run.ctx.lengths() == [c + k for c, k in zip(base_lens, n_new)]
    model = O.OracleModel.from_spec(spec, w)
    octx = O.OracleContext(model, n)
    for b in range(n):
        O.fuse_ctx(model, octx, b, feats[b])
    ref = O.draft_block(model, octx, anchors, block)
    gl, gd = lg.cpu().numpy(), d.cpu().numpy()
    assert_parity(gl, gd, ref, label)
    if two_call_check:
        B.fuse_ctx(run2.model, run2.ctx, dev_new, n_new, run2.ws)
        lg2 = torch.empty_like(lg)
        B.draft_block(run2.model, run2.ctx, a, block, run2.ws, logits=lg2)
        torch.cuda.synchronize()
        diff = float(np.max(np.abs(lg2.cpu().numpy() - gl)))
        say(f"{label}: step vs fuse+draft max-abs logit diff {diff:.2e}")
        assert diff <= 1e-3, f"{label}: fused step differs from the two-call path by {diff}"
    return run


@pytest.mark.parametrize("base,new,block,label", [
    ((112,), (16,), 16, "one seq, 16+16 rows fused"),
    ((40, 9), (3, 5), 4, "two seqs ragged, fused"),
    ((30, 0, 17), (0, 7, 1), 8, "three seqs with empty appends, fused"),
    ((64,), (1,), 16, "single appended row"),
    ((64, 10), (20, 5), 16, "57 rows: append then draft"),
])
def test_step_tiny(torch_cuda, base, new, block, label):
    spec = I.spec("tiny")
    w = I.gen_weights(spec, seed=7, std=0.05)
    _step_case(spec, w, B.upload_weights(spec, w), base, new, block, label)


def test_step_capacity_error_leaves_lengths(torch_cuda):
    spec = I.spec("tiny").with_(ctx_lens=(10,))
    w = I.gen_weights(spec, seed=0)
    run = GpuRun(spec, B.upload_weights(spec, w), capacity=[12], max_new=40)
    run.ingest(_feats(spec, 1, [10]))
    feats = torch_cuda.zeros((3, spec.fused_width), dtype=torch_cuda.bfloat16, device="cuda")
    a = torch_cuda.zeros(1, dtype=torch_cuda.int32, device="cuda")
    with pytest.raises(B.DFlashError) as e:
        B.step(run.model, run.ctx, feats, [3], a, 16, run.ws)
    assert e.value.name == "DFLASH_ECAPACITY"
    assert run.ctx.lengths() == [10]


def test_step_q8_ctx1024(q8):
    spec5, w, dev = q8
    _step_case(spec5, w, dev, (1008,), (16,), 16, "5-layer step ctx 1008+16")


# ----------------------------------------------------------------------------
# packed weights (dflash_model_pack): a layout change only, so every output is
# bitwise equal to the row-major run's (which the tests above hold to the
# oracle)
# ----------------------------------------------------------------------------

def _packed_case(spec, dev_w, base_lens, n_new, block, label):
    import torch
    spec = spec.with_(ctx_lens=tuple(base_lens), block=block)
    cap = [b + 2 * k + 8 for b, k in zip(base_lens, n_new)]
    runs = [GpuRun(spec, dev_w, capacity=cap, max_new=sum(base_lens) + 2 * sum(n_new), max_block=32)
            for _ in range(2)]
    feats = [I.gen_features(spec, 1, b, c + 2 * k) for b, (c, k) in enumerate(zip(base_lens, n_new))]
    for r in runs:
        r.ingest([f[:c] for f, c in zip(feats, base_lens)])
    runs[1].model.pack()
    torch.cuda.synchronize()
    say(f"{label}: packed {runs[1].model.pack_bytes() / 1e6:.1f} MB")
    n = len(base_lens)
    rows1 = to_dev_bf16(np.concatenate([f[c:c + k] for f, c, k in zip(feats, base_lens, n_new)], 0))
    rows2 = to_dev_bf16(np.concatenate([f[c + k:c + 2 * k] for f, c, k in zip(feats, base_lens, n_new)], 0))
    a = torch.from_numpy(I.gen_anchors(spec, 2)).cuda()
    outs = []
    for r in runs:
        o = []
        lg = torch.empty((n, block - 1, spec.vocab), dtype=torch.float32, device="cuda")
        d = B.step(r.model, r.ctx, rows1, n_new, a, block, r.ws, logits=lg)  # fused: every packed GEMM
        torch.cuda.synchronize()
        o += [d.cpu().numpy(), lg.cpu().numpy().view(np.uint32)]
        lg2 = torch.empty_like(lg)
        d2 = B.draft_sample(r.model, r.ctx, a, block, 0.7, 11, r.ws, logits=lg2)
        torch.cuda.synchronize()
        o += [d2.cpu().numpy(), lg2.cpu().numpy().view(np.uint32)]
        B.fuse_ctx(r.model, r.ctx, rows2, n_new, r.ws)  # the two-call path
        d3, l3 = r.draft(I.gen_anchors(spec, 3), block)
        o += [d3, l3.view(np.uint32)]
        outs.append(o)
    for i, (x, y) in enumerate(zip(outs[0], outs[1])):
        assert np.array_equal(x, y), f"{label}: output {i} differs with packed weights"
    runs[1].model.unpack()
    d4, l4 = runs[1].draft(I.gen_anchors(spec, 4), block)
    d5, l5 = runs[0].draft(I.gen_anchors(spec, 4), block)
    assert np.array_equal(d4, d5) and np.array_equal(l4.view(np.uint32), l5.view(np.uint32))


@pytest.mark.parametrize("base,new,block,label", [
    ((112,), (16,), 16, "one seq, fused 16 + 16 rows"),
    ((40, 9), (3, 5), 8, "two seqs ragged"),
    ((30, 41, 7, 64, 19, 33, 50, 12, 25), (20, 3, 17, 9, 31, 1, 12, 8, 24), 16,
     "nine seqs: many-row GEMMs over the packed copy"),
])
def test_packed_weights_tiny(torch_cuda, base, new, block, label):
    spec = I.spec("tiny")
    w = I.gen_weights(spec, seed=7, std=0.05)
    _packed_case(spec, B.upload_weights(spec, w), base, new, block, label)


def test_packed_weights_q8_ctx1024(q8):
    spec5, w, dev = q8
    _packed_case(spec5, dev, (1008,), (16,), 16, "5-layer ctx 1008 + 16 + 16, packed")


def test_packed_weights_q8_many_rows(q8):
    # 64 block rows and 64 appended rows: every GEMM takes the many-row kernel,
    # which copies its weight tiles from the packed blocks
    spec5, w, dev = q8
    _packed_case(spec5, dev, (200, 300, 150, 250), (16, 16, 16, 16), 16, "5-layer 4 seqs, many-row packed")


# ----------------------------------------------------------------------------
# several denoising passes over one block (block tokens fed back)
# ----------------------------------------------------------------------------

def _refine_case(spec, w, dev_w, lens, block, label, steps=2):
    """refine(1, tokens) vs the oracle pass over the same tokens; refine(steps) vs
    chained single passes (bitwise) and vs the oracle pass over the GPU's
    previous drafts."""
    import torch
    spec = spec.with_(ctx_lens=tuple(lens), block=block)
    say(f"refine {label}: lens={lens} block={block} steps={steps}")
    run = GpuRun(spec, dev_w, capacity=[c + 8 for c in lens], max_new=sum(lens))
    feats = _feats(spec, 1, lens)
    run.ingest(feats)
    n = len(lens)
    anchors = I.gen_anchors(spec, 2)
    a = torch.from_numpy(anchors).cuda()
    rng = np.random.default_rng(block * 7 + n)
    init = rng.integers(0, spec.vocab, size=(n, block - 1)).astype(np.int32)
    init[:, ::3] = spec.mask_token_id  # some positions stay masked
    model = O.OracleModel.from_spec(spec, w)
    octx = O.OracleContext(model, n)
    for b in range(n):
        O.fuse_ctx(model, octx, b, feats[b])

    def gpu(n_steps, tokens):
        lg = torch.empty((n, block - 1, spec.vocab), dtype=torch.float32, device="cuda")
        t = None if tokens is None else torch.from_numpy(np.ascontiguousarray(tokens, np.int32)).cuda()
        d = B.draft_refine(run.model, run.ctx, a, block, n_steps, run.ws, init_tokens=t, logits=lg)
        torch.cuda.synchronize()
        return d.cpu().numpy(), lg.cpu().numpy()

    d1, l1 = gpu(1, init)
    assert_parity(l1, d1, O.draft_block(model, octx, anchors, block, block_tokens=init), f"{label} pass 1")
    d2, l2 = gpu(2, init)
    d2c, l2c = gpu(1, d1)
    assert np.array_equal(d2, d2c), f"{label}: two passes differ from chained single passes"
    assert np.array_equal(l2.view(np.uint32), l2c.view(np.uint32)), f"{label}: logits not bitwise equal"
    assert_parity(l2, d2, O.draft_block(model, octx, anchors, block, block_tokens=d1), f"{label} pass 2")
    if steps > 2:
        ds, ls = gpu(steps, None)
        prev = None
        for _ in range(steps - 1):
            prev, _ = gpu(1, prev)
        assert_parity(ls, ds, O.draft_block(model, octx, anchors, block, block_tokens=prev), f"{label} pass {steps}")
    # masked start, one pass: identical to dflash_draft_block
    dm, lm = gpu(1, None)
    db, lb = run.draft(anchors, block)
    assert np.array_equal(dm, db) and np.array_equal(lm.view(np.uint32), lb.view(np.uint32))


@pytest.mark.parametrize("lens,block,steps,label", [
    ((128,), 16, 3, "tiny B16 three passes"),
    ((37, 5, 0), 8, 2, "ragged three seqs B8"),
    ((64, 200), 32, 2, "B32 two seqs tiled"),
    ((20, 5, 0, 33, 64, 7, 100, 12), 4, 2, "eight seqs B4"),
])
def test_refine_tiny(torch_cuda, lens, block, steps, label):
    spec = I.spec("tiny")
    w = I.gen_weights(spec, seed=3, std=0.05)
    _refine_case(spec, w, B.upload_weights(spec, w), lens, block, label, steps=steps)


def test_refine_rejects_bad_step_counts(torch_cuda):
    spec = I.spec("tiny").with_(ctx_lens=(4,))
    w = I.gen_weights(spec, seed=0)
    run = GpuRun(spec, B.upload_weights(spec, w), capacity=[8], max_new=8)
    a = torch_cuda.zeros(1, dtype=torch_cuda.int32, device="cuda")
    for bad in (0, -1, 65):
        with pytest.raises(B.DFlashError) as e:
            B.draft_refine(run.model, run.ctx, a, 16, bad, run.ws)
        assert e.value.name == "DFLASH_EINVAL"


def test_refine_q8_ctx1024_b8(q8):
    spec5, w, dev = q8
    _refine_case(spec5, w, dev, (1024,), 8, "5-layer ctx1024 B8")


# ----------------------------------------------------------------------------
# anchored blocks over shared contexts (training-attention forward)
# ----------------------------------------------------------------------------

def _anchored_case(spec, w, dev_w, lens, bseq, apos, block, label, tokens=False, check_blocks=None):
    import torch
    spec = spec.with_(ctx_lens=tuple(lens), block=block)
    n = len(bseq)
    say(f"anchored {label}: lens={lens} blocks={n} block={block}")
    run = GpuRun(spec, dev_w, capacity=[c + 8 for c in lens], max_new=sum(lens))
    feats = _feats(spec, 1, lens)
    run.ingest(feats)
    ws = B.workspace(run.model, n, block, 0)
    rng = np.random.default_rng(n * 31 + block)
    anchors = rng.integers(0, spec.vocab - 1, size=n).astype(np.int32)
    toks = None
    if tokens:
        toks = rng.integers(0, spec.vocab, size=(n, block - 1)).astype(np.int32)
        toks[:, 1::2] = spec.mask_token_id
    lg = torch.empty((n, block - 1, spec.vocab), dtype=torch.float32, device="cuda")
    d = B.draft_anchored(run.model, run.ctx, bseq, apos, torch.from_numpy(anchors).cuda(), block, ws,
                         block_tokens=None if toks is None else torch.from_numpy(toks).cuda(), logits=lg)
    torch.cuda.synchronize()
    assert run.ctx.lengths() == list(lens)
    sel = list(range(n)) if check_blocks is None else check_blocks
    model = O.OracleModel.from_spec(spec, w)
    octx = O.OracleContext(model, len(lens))
    for b in sorted({bseq[j] for j in sel}):
        O.fuse_ctx(model, octx, b, feats[b])
    ref = O.draft_anchored(model, octx, [bseq[j] for j in sel], [apos[j] for j in sel], anchors[sel], block,
                           block_tokens=None if toks is None else toks[sel])
    assert_parity(lg.cpu().numpy()[sel], d.cpu().numpy()[sel], ref, label)
    return run, d


@pytest.mark.parametrize("lens,bseq,apos,block,tokens,label", [
    ((100, 40), [0, 0, 1, 0, 1, 0, 0, 1], [0, 37, 40, 100, 0, 64, 63, 17], 16, False, "eight blocks M128"),
    ((50,), [0, 0, 0], [10, 12, 50], 4, True, "overlapping B4 with tokens"),
    ((130, 3, 70), [2, 0, 1, 0], [70, 129, 3, 65], 8, False, "three seqs B8 skinny"),
    ((300,), [0] * 16, list(range(0, 300, 19)), 32, False, "sixteen blocks B32 M512"),
    ((0, 5), [0, 1], [0, 5], 16, False, "empty context"),
])
def test_anchored_tiny(torch_cuda, lens, bseq, apos, block, tokens, label):
    spec = I.spec("tiny")
    w = I.gen_weights(spec, seed=9, std=0.05)
    _anchored_case(spec, w, B.upload_weights(spec, w), lens, bseq, apos, block, label, tokens=tokens)


def test_anchored_leaves_the_context_unchanged(torch_cuda):
    """Anchored blocks only read the cache: a later draft_block is bitwise unchanged."""
    import torch
    spec = I.spec("tiny").with_(ctx_lens=(90,))
    w = I.gen_weights(spec, seed=2, std=0.05)
    run = GpuRun(spec, B.upload_weights(spec, w), capacity=[100], max_new=90)
    run.ingest(_feats(spec, 1, [90]))
    anchors = I.gen_anchors(spec, 2)
    d0, l0 = run.draft(anchors, 16)
    ws = B.workspace(run.model, 4, 16, 0)
    a = torch.zeros(4, dtype=torch.int32, device="cuda")
    B.draft_anchored(run.model, run.ctx, [0, 0, 0, 0], [0, 30, 60, 90], a, 16, ws)
    torch.cuda.synchronize()
    d1, l1 = run.draft(anchors, 16)
    assert np.array_equal(d0, d1) and np.array_equal(l0.view(np.uint32), l1.view(np.uint32))


def test_anchored_rejects_bad_blocks(torch_cuda):
    import torch
    spec = I.spec("tiny").with_(ctx_lens=(10, 4))
    w = I.gen_weights(spec, seed=0)
    run = GpuRun(spec, B.upload_weights(spec, w), capacity=[16, 16], max_new=14)
    run.ingest(_feats(spec, 1, [10, 4]))
    ws = B.workspace(run.model, 2, 16, 0)
    a = torch.zeros(2, dtype=torch.int32, device="cuda")
    for bseq, apos in (([0, 2], [1, 1]), ([0, 1], [1, 5]), ([0, -1], [0, 0]), ([0, 1], [-1, 0])):
        with pytest.raises(B.DFlashError) as e:
            B.draft_anchored(run.model, run.ctx, bseq, apos, a, 16, ws)
        assert e.value.name == "DFLASH_EINVAL", (bseq, apos)
    small = B.workspace(run.model, 1, 16, 0)
    with pytest.raises(B.DFlashError) as e:
        B.draft_anchored(run.model, run.ctx, [0, 1], [1, 1], a, 16, small)
    assert e.value.name == "DFLASH_EWORKSPACE"


def test_anchored_q8_ctx1024(q8):
    """The 5-layer drafter over one 1024-position context with 16 blocks of 16
    (M = 256): the training-attention forward at the bench shapes."""
    spec5, w, dev = q8
    apos = [int(v) for v in I.gen_train_anchors(1024, 16, 16, seed=3)]
    _anchored_case(spec5, w, dev, (1024,), [0] * 16, apos, 16, "5-layer ctx1024 16 blocks",
                   check_blocks=[0, 7, 15])


# ----------------------------------------------------------------------------
# sampled drafts (temperature > 0) and lossless verification
# ----------------------------------------------------------------------------

def _check_sampled(gpu_logits, gpu_drafts, ref_logits, T, seed, label, n_check=None):
    """GPU sampled drafts vs the oracle's Gumbel-max samples of the oracle's
    logits (equal wherever the top-2 perturbed-score gap > GAP / T), and vs
    the same rule applied to the GPU's own logits (its pick must be the
    largest score up to float32 rounding of that score)."""
    from oracle import sampling as S
    n, bm1, V = ref_logits.shape
    sure = checked = 0
    for b in range(n if n_check is None else n_check):
        for i in range(1, bm1 + 1):
            ref_sc = S.sample_scores(ref_logits[b, i - 1], T, seed, b, i)
            top2 = np.sort(ref_sc)[-2:]
            if top2[1] - top2[0] > 0.05 / T:
                sure += 1
                assert gpu_drafts[b, i - 1] == int(np.argmax(ref_sc)), f"{label}: seq {b} pos {i} differs"
            own = S.sample_scores(gpu_logits[b, i - 1].astype(np.float64), T, seed, b, i)
            x = int(gpu_drafts[b, i - 1])
            assert own[x] >= own.max() - 1e-5 * max(1.0, abs(own.max())), f"{label}: seq {b} pos {i} not the max"
            checked += 1
    say(f"{label}: sampled drafts checked on {checked} positions ({sure} decided by the oracle)")


@pytest.mark.parametrize("lens,block,T,seed,label", [
    ((128,), 16, 1.0, 1, "tiny T1"),
    ((128,), 16, 0.6, 77, "tiny T0.6"),
    ((37, 5, 0), 4, 1.4, 5, "ragged B4 T1.4"),
    ((20, 5, 0, 33, 64, 7, 100, 12), 16, 0.8, 9, "eight seqs M128 T0.8"),
])
def test_sampled_draft_tiny(torch_cuda, lens, block, T, seed, label):
    import torch
    spec = I.spec("tiny").with_(ctx_lens=tuple(lens), block=block)
    w = I.gen_weights(spec, seed=3, std=0.05)
    run = GpuRun(spec, B.upload_weights(spec, w), capacity=[c + 8 for c in lens], max_new=sum(lens))
    feats = _feats(spec, 1, lens)
    run.ingest(feats)
    anchors = I.gen_anchors(spec, 2)
    a = torch.from_numpy(anchors).cuda()
    n = len(lens)
    lg = torch.empty((n, block - 1, spec.vocab), dtype=torch.float32, device="cuda")
    d = B.draft_sample(run.model, run.ctx, a, block, T, seed, run.ws, logits=lg)
    torch.cuda.synchronize()
    gl, gd = lg.cpu().numpy(), d.cpu().numpy()
    ref = oracle_run(spec, w, feats, anchors, block)
    err = float(np.max(np.abs(gl - ref.logits)))
    assert err <= LOGIT_TOL, f"{label}: logits error {err}"
    _check_sampled(gl, gd, ref.logits, T, seed, label)
    # the same seed gives the same drafts; another seed other drafts
    d2 = B.draft_sample(run.model, run.ctx, a, block, T, seed, run.ws)
    d3 = B.draft_sample(run.model, run.ctx, a, block, T, seed + 1, run.ws)
    torch.cuda.synchronize()
    assert np.array_equal(d2.cpu().numpy(), gd)
    assert not np.array_equal(d3.cpu().numpy(), gd)


def test_sampled_step_matches_two_calls(torch_cuda):
    import torch
    spec = I.spec("tiny").with_(ctx_lens=(112,), block=16)
    w = I.gen_weights(spec, seed=7, std=0.05)
    dev_w = B.upload_weights(spec, w)
    feats = _feats(spec, 1, [128])[0]
    runs = [GpuRun(spec, dev_w, capacity=[140], max_new=128) for _ in range(2)]
    for r in runs:
        r.ingest([feats[:112]])
    new = torch.from_numpy(np.ascontiguousarray(feats[112:]).view(np.int16)).cuda().view(torch.bfloat16)
    a = torch.from_numpy(I.gen_anchors(spec, 2)).cuda()
    lg1 = torch.empty((1, 15, spec.vocab), dtype=torch.float32, device="cuda")
    lg2 = torch.empty_like(lg1)
    d1 = B.step_sample(runs[0].model, runs[0].ctx, new, [16], a, 16, 0.9, 123, runs[0].ws, logits=lg1)
    B.fuse_ctx(runs[1].model, runs[1].ctx, new, [16], runs[1].ws)
    d2 = B.draft_sample(runs[1].model, runs[1].ctx, a, 16, 0.9, 123, runs[1].ws, logits=lg2)
    torch.cuda.synchronize()
    model = O.OracleModel.from_spec(spec, w)
    octx = O.OracleContext(model, 1)
    O.fuse_ctx(model, octx, 0, feats)
    ref = O.draft_block(model, octx, I.gen_anchors(spec, 2), 16)
    _check_sampled(lg1.cpu().numpy(), d1.cpu().numpy(), ref.logits, 0.9, 123, "sampled step")
    _check_sampled(lg2.cpu().numpy(), d2.cpu().numpy(), ref.logits, 0.9, 123, "sampled two calls")
    assert runs[0].ctx.lengths() == [128]


def test_sampled_draft_q8_ctx1024(q8):
    import torch
    spec5, w, dev = q8
    lens = (1024,)
    spec = spec5.with_(ctx_lens=lens)
    run = GpuRun(spec, dev, capacity=[1100], max_new=1024)
    feats = _feats(spec, 1, lens)
    run.ingest(feats)
    anchors = I.gen_anchors(spec, 2)
    lg = torch.empty((1, 15, spec.vocab), dtype=torch.float32, device="cuda")
    d = B.draft_sample(run.model, run.ctx, torch.from_numpy(anchors).cuda(), 16, 0.7, 2026, run.ws, logits=lg)
    torch.cuda.synchronize()
    ref = oracle_run(spec, w, feats, anchors, 16)
    gl = lg.cpu().numpy()
    assert float(np.max(np.abs(gl - ref.logits))) <= LOGIT_TOL
    _check_sampled(gl, d.cpu().numpy(), ref.logits, 0.7, 2026, "5-layer sampled T0.7")


def test_sampled_draft_q8_many_rows(q8):
    # sixteen sequences of the 5-layer drafter: 256 block rows, so the sampled
    # LM head runs on the many-row kernel at the full vocabulary
    import torch
    spec5, w, dev = q8
    lens = _short_ragged(91, 16)
    spec = spec5.with_(ctx_lens=lens)
    run = GpuRun(spec, dev, capacity=[c + 8 for c in lens], max_new=sum(lens))
    feats = _feats(spec, 1, lens)
    run.ingest(feats)
    anchors = I.gen_anchors(spec, 2)
    lg = torch.empty((len(lens), 15, spec.vocab), dtype=torch.float32, device="cuda")
    d = B.draft_sample(run.model, run.ctx, torch.from_numpy(anchors).cuda(), 16, 0.8, 4049, run.ws, logits=lg)
    torch.cuda.synchronize()
    ref = oracle_run(spec, w, feats, anchors, 16)
    gl = lg.cpu().numpy()
    assert float(np.max(np.abs(gl - ref.logits))) <= LOGIT_TOL
    # logits of every sequence above; the samples of four (0.1 s of oracle per position)
    _check_sampled(gl, d.cpu().numpy(), ref.logits, 0.8, 4049, "5-layer 16 seqs sampled T0.8", n_check=4)


def _verify_case(n, block, V, T, seed, scale, label, qp_same=False):
    import torch
    from oracle import sampling as S
    rng = np.random.default_rng(seed)
    q = (rng.normal(size=(n, block - 1, V)) * scale).astype(np.float32)
    p = (rng.normal(size=(n, block, V)) * scale).astype(np.float32)
    if qp_same:
        p[:, : block - 1] = q
    # drafts: mostly the likely tokens under q, some arbitrary
    draft = np.argmax(q + rng.gumbel(size=q.shape) * T, axis=-1).astype(np.int32)
    draft[:, ::5] = rng.integers(0, V, size=draft[:, ::5].shape)
    acc_ref, nxt_ref = S.verify_sampled(draft, q, p, T, seed)
    margins = S.accept_margins(draft, q, p, T, seed)
    dq, dp, dd = (torch.from_numpy(x).cuda() for x in (q, p, draft))
    acc, nxt = B.verify_sample(dd, dq, dp, block, T, seed)
    torch.cuda.synchronize()
    acc, nxt = acc.cpu().numpy(), nxt.cpu().numpy()
    checked = 0
    for b in range(n):
        if np.min(margins[b, : acc_ref[b] + 1 if acc_ref[b] < block - 1 else block - 1]) < 1e-9:
            continue  # a decision within rounding of its threshold
        checked += 1
        assert (acc[b], nxt[b]) == (acc_ref[b], nxt_ref[b]), f"{label}: seq {b}: {(acc[b], nxt[b])} vs " \
                                                             f"{(acc_ref[b], nxt_ref[b])}"
    say(f"{label}: accept {acc.tolist()[:12]} ... ({checked}/{n} sequences compared)")
    assert checked >= n - 1
    return acc, nxt


@pytest.mark.parametrize("n,block,V,T,seed,scale,label", [
    (24, 16, 4096, 1.0, 1, 2.0, "V4096 T1"),
    (16, 4, 4096, 0.5, 2, 3.0, "B4 T0.5"),
    (8, 32, 1000, 1.5, 3, 1.0, "B32 V1000"),
    (2, 16, 151936, 0.8, 4, 3.0, "full vocab"),
])
def test_verify_sample_matches_oracle(torch_cuda, n, block, V, T, seed, scale, label):
    _verify_case(n, block, V, T, seed, scale, label)


def test_verify_sample_keeps_everything_when_draft_equals_target(torch_cuda):
    acc, _ = _verify_case(8, 16, 2048, 1.0, 5, 2.0, "q equals p", qp_same=True)
    assert np.all(acc == 15)


# ----------------------------------------------------------------------------
# the decode step captured once as a HIP graph and replayed
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("sampled,base,n_new", [
    (False, (112,), (16,)),       # fused: 16 block rows + 16 appended rows in one sweep
    (True, (112,), (16,)),
    (False, (100, 40), (8, 8)),   # 48 rows: append, then draft
    (True, (100, 40), (8, 8)),
])
def test_step_graph_replays_match_eager(torch_cuda, sampled, base, n_new):
    """dflash_step (greedy or sampled) + the accept scan captured in a graph:
    three replays, with eager work and synchronisation between them, each
    bitwise equal to the eager step.  The host rolls the context back before
    each replay, so every replay appends to the same slots."""
    torch = torch_cuda
    n = len(base)
    spec = I.spec("tiny").with_(ctx_lens=tuple(base), block=16)
    w = I.gen_weights(spec, seed=5, std=0.05)
    dev_w = B.upload_weights(spec, w)
    cap = [b + k + 16 for b, k in zip(base, n_new)]
    run = GpuRun(spec, dev_w, capacity=cap, max_new=sum(base) + sum(n_new), max_block=32)
    other = GpuRun(spec, dev_w, capacity=cap, max_new=sum(base) + sum(n_new), max_block=32)
    feats = _feats(spec, 1, [b + k for b, k in zip(base, n_new)])
    run.ingest([f[:b] for f, b in zip(feats, base)])
    other.ingest([f[:b] for f, b in zip(feats, base)])
    new = torch.from_numpy(np.ascontiguousarray(np.concatenate([f[b:] for f, b in zip(feats, base)])).view(np.int16)) \
        .cuda().view(torch.bfloat16)
    a = torch.from_numpy(I.gen_anchors(spec, 2)).cuda()
    draft = torch.empty((n, 15), dtype=torch.int32, device="cuda")
    logits = torch.empty((n, 15, spec.vocab), dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(3)
    target = torch.from_numpy(rng.integers(0, spec.vocab, size=(n, 16)).astype(np.int32)).cuda()
    acc = torch.empty(n, dtype=torch.int32, device="cuda")
    nxt = torch.empty(n, dtype=torch.int32, device="cuda")

    def step():
        if sampled:
            B.step_sample(run.model, run.ctx, new, list(n_new), a, 16, 0.8, 77, run.ws, draft=draft, logits=logits)
        else:
            B.step(run.model, run.ctx, new, list(n_new), a, 16, run.ws, draft=draft, logits=logits)
        B.accept_len(draft, target, 16, acc, nxt)

    def rollback():
        for b, c in enumerate(base):
            run.ctx.truncate(b, c)

    step()
    torch.cuda.synchronize()
    ref = (draft.cpu().numpy().copy(), logits.cpu().numpy().copy(), acc.cpu().numpy().copy(),
           nxt.cpu().numpy().copy())
    rollback()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        draft.fill_(-1)
        logits.zero_()
        rollback()
        g.replay()
        torch.cuda.synchronize()
        got = (draft.cpu().numpy(), logits.cpu().numpy(), acc.cpu().numpy(), nxt.cpu().numpy())
        for x, y in zip(got, ref):
            assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                                  y.view(np.uint32) if y.dtype == np.float32 else y), f"replay {rep} differs"
        # eager work on another context between replays
        B.draft_block(other.model, other.ctx, a, 16, other.ws)
        torch.cuda.synchronize()
    assert run.ctx.lengths() == list(base)
    say(f"graph replays equal the eager step (sampled={sampled}, base={base})")


# ----------------------------------------------------------------------------
# maximum sizes of one call
# ----------------------------------------------------------------------------

def test_max_sequences_per_call(torch_cuda):
    """128 sequences (the most one call takes) at block 16: 2048 block rows on
    the many-row path; the oracle checks a spread of sequences."""
    spec = I.spec("tiny")
    lens = tuple(int(v) for v in np.random.default_rng(11).integers(0, 200, size=128))
    spec = spec.with_(ctx_lens=lens, block=16)
    w = I.gen_weights(spec, seed=6, std=0.05)
    run = GpuRun(spec, B.upload_weights(spec, w), capacity=[c + 8 for c in lens], max_new=sum(lens))
    feats = _feats(spec, 1, lens)
    run.ingest(feats)
    anchors = I.gen_anchors(spec, 2)
    drafts, logits = run.draft(anchors, 16)
    seqs = [0, 1, 17, 63, 64, 100, 126, 127]
    ref = oracle_run(spec, w, feats, anchors, 16, seqs=seqs)
    assert_parity(logits[seqs], drafts[seqs], ref, "128 sequences")
    accept_check(drafts[seqs], ref, spec.with_(ctx_lens=tuple(lens[s] for s in seqs)), 3, "128 sequences")


def test_max_anchored_blocks_per_call(torch_cuda):
    """128 anchored blocks of 16 over two shared contexts (2048 rows)."""
    lens = (700, 300)
    bseq = [0] * 80 + [1] * 48
    rng = np.random.default_rng(12)
    apos = [int(v) for v in rng.integers(0, 701, size=80)] + [int(v) for v in rng.integers(0, 301, size=48)]
    spec = I.spec("tiny")
    w = I.gen_weights(spec, seed=8, std=0.05)
    _anchored_case(spec, w, B.upload_weights(spec, w), lens, bseq, apos, 16, "128 anchored blocks",
                   check_blocks=[0, 5, 79, 80, 100, 127])
