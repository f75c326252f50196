"""Pins of the CPU oracle against things other than itself: an independent
scalar-loop evaluation, a torch-library formulation, closed forms, invariants
and hand-derived verification cases.  CPU only."""
from __future__ import annotations

import dataclasses
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from block_diffusion_drafting_pass_amd import inputs as I
from oracle import brute
from oracle import dflash_oracle as O
from tests.torch_cpu_ref import torch_draft

HERE = os.path.dirname(os.path.abspath(__file__))

# A drafter small enough for the scalar-loop evaluation: 2 layers, 4/2 heads
# (GQA groups of two), d = 4, vocab 16, two target layers.
MICRO = I.DraftSpec("micro", n_layers=2, hidden=8, n_q_heads=4, n_kv_heads=2, head_dim=4,
                    intermediate=12, vocab=16, n_target_layers=2, block=4, ctx_lens=(3, 0))


def _model(spec, seed=0, jitter=0.1, std=0.3):
    # a larger weight scale than the benchmark's 0.02 keeps tiny models far from trivial
    w = I.gen_weights(spec, seed=seed, gain_jitter=jitter, std=std)
    return O.OracleModel.from_spec(spec, w), w


def _ingest(model, spec, seed, lens=None, pos_offset=0):
    lens = spec.ctx_lens if lens is None else lens
    ctx = O.OracleContext(model, len(lens), pos_offset=pos_offset)
    feats = []
    for b, c in enumerate(lens):
        f = I.gen_features(spec, seed, b, c)
        feats.append(f)
        O.fuse_ctx(model, ctx, b, f)
    return ctx, feats


# ----------------------------------------------------------------------------
# whole-pass pins
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1])
def test_oracle_matches_scalar_brute_force(seed):
    model, w = _model(MICRO, seed)
    ctx, feats = _ingest(model, MICRO, seed)
    anchors = I.gen_anchors(MICRO, seed)
    res = O.draft_block(model, ctx, anchors, MICRO.block)
    bl, bd = brute.brute_draft(MICRO, w, feats, anchors, MICRO.block)
    np.testing.assert_allclose(res.logits, np.array(bl), rtol=0, atol=1e-12)
    assert res.drafts.tolist() == bd


def test_oracle_matches_brute_force_without_rope():
    model, w = _model(MICRO, 5)
    ctx = O.OracleContext(model, 2)
    feats = []
    for b, c in enumerate(MICRO.ctx_lens):
        f = I.gen_features(MICRO, 5, b, c)
        feats.append(f)
        O.fuse_ctx(model, ctx, b, f, use_rope=False)
    anchors = I.gen_anchors(MICRO, 5)
    res = O.draft_block(model, ctx, anchors, MICRO.block, use_rope=False)
    bl, _ = brute.brute_draft(MICRO, w, feats, anchors, MICRO.block, use_rope=False)
    np.testing.assert_allclose(res.logits, np.array(bl), rtol=0, atol=1e-12)


@pytest.mark.parametrize("name,lens", [("tiny", (128,)), ("tiny", (0,)), ("tiny", (37, 5))])
def test_oracle_matches_torch_library_formulation(name, lens):
    spec = I.spec(name).with_(ctx_lens=lens)
    model, w = _model(spec, 3, jitter=0.1, std=0.02)
    ctx, feats = _ingest(model, spec, 3)
    anchors = I.gen_anchors(spec, 3)
    res = O.draft_block(model, ctx, anchors, spec.block)
    tl, td = torch_draft(spec, w, feats, anchors, spec.block)
    np.testing.assert_allclose(res.logits, tl, rtol=0, atol=1e-10)


def test_batched_equals_per_sequence():
    spec = I.spec("tiny").with_(ctx_lens=(40, 7, 0))
    model, _ = _model(spec, 2)
    ctx, _ = _ingest(model, spec, 2)
    anchors = I.gen_anchors(spec, 2)
    full = O.draft_block(model, ctx, anchors, spec.block)
    for b in range(spec.n_seqs):
        one = O.draft_block(model, ctx, anchors, spec.block, seqs=[b])
        np.testing.assert_array_equal(one.logits[0], full.logits[b])


def test_rope_shift_invariance_of_the_pass():
    """Moving every position (context and block) by the same amount leaves the
    attention scores, hence the logits, unchanged up to rounding."""
    spec = I.spec("tiny").with_(ctx_lens=(64,))
    model, _ = _model(spec, 4, std=0.02)
    a, _ = _ingest(model, spec, 4, pos_offset=0)
    b, _ = _ingest(model, spec, 4, pos_offset=7168)
    anchors = I.gen_anchors(spec, 4)
    la = O.draft_block(model, a, anchors, spec.block).logits
    lb = O.draft_block(model, b, anchors, spec.block).logits
    assert np.max(np.abs(la - lb)) < 1e-9
    # and a shift does change the individual keys (the test is not vacuous)
    assert np.max(np.abs(a.k[0][0] - b.k[0][0])) > 1e-3


def test_without_rope_all_mask_rows_agree():
    """Mask rows share token and (without RoPE) position, and attention is
    unmasked, so their outputs must be identical."""
    spec = I.spec("tiny").with_(ctx_lens=(20,))
    model, _ = _model(spec, 6)
    ctx = O.OracleContext(model, 1)
    O.fuse_ctx(model, ctx, 0, I.gen_features(spec, 6, 0, 20), use_rope=False)
    res = O.draft_block(model, ctx, I.gen_anchors(spec, 6), spec.block, use_rope=False)
    assert np.max(np.abs(res.logits[0] - res.logits[0][0][None])) < 1e-12
    res2 = O.draft_block(model, ctx, I.gen_anchors(spec, 6), spec.block, use_rope=True)
    assert np.max(np.abs(res2.logits[0] - res2.logits[0][0][None])) > 1e-6


# ----------------------------------------------------------------------------
# fusion and injection
# ----------------------------------------------------------------------------

def test_zero_features_give_zero_context_kv():
    spec = I.spec("tiny")
    model, _ = _model(spec, 1)
    ctx = O.OracleContext(model, 1)
    O.fuse_ctx(model, ctx, 0, np.zeros((50, spec.fused_width), np.uint16))
    for l in range(spec.n_layers):
        assert np.all(ctx.k[0][l] == 0.0) and np.all(ctx.v[0][l] == 0.0)


def test_zero_context_attention_closed_form():
    """With c zero-valued context keys and values, each context score is 0 and
    o = sum_j e^{s_j} v_j / (c + sum_j e^{s_j}) over the block keys only."""
    rng = np.random.default_rng(0)
    c, B, nq, nkv, d = 9, 5, 4, 2, 8
    q = rng.standard_normal((B, nq, d))
    kb = rng.standard_normal((B, nkv, d))
    vb = rng.standard_normal((B, nkv, d))
    keys = np.concatenate([np.zeros((c, nkv, d)), kb])
    vals = np.concatenate([np.zeros((c, nkv, d)), vb])
    o = O.attention(q, keys, vals)
    for h in range(nq):
        g = h // (nq // nkv)
        for i in range(B):
            e = np.array([np.exp(np.dot(q[i, h], kb[j, g]) / np.sqrt(d)) for j in range(B)])
            want = (e[:, None] * vb[:, g, :]).sum(0) / (c + e.sum())
            np.testing.assert_allclose(o[i, h], want, rtol=1e-13, atol=1e-14)


def test_identity_fusion_selects_first_target_layer():
    spec = I.spec("tiny")
    model, w = _model(spec, 1)
    H = spec.hidden
    eye = np.zeros((H, spec.fused_width), np.uint16)
    eye[np.arange(H), np.arange(H)] = 0x3F80  # bf16 1.0
    model.weights = dict(w, w_fc=eye)
    f = I.gen_features(spec, 9, 0, 11)
    np.testing.assert_array_equal(O.fuse_features(model, f), O.bf16_to_f64(f[:, :H]))


def test_injection_reaches_every_layer():
    """Changing one layer's injected context changes the drafts' logits."""
    spec = I.spec("tiny").with_(n_layers=2, ctx_lens=(30,))
    model, _ = _model(spec, 8)
    ctx, _ = _ingest(model, spec, 8)
    anchors = I.gen_anchors(spec, 8)
    base = O.draft_block(model, ctx, anchors, spec.block).logits
    for l in range(2):
        saved = ctx.v[0][l].copy()
        ctx.v[0][l] = ctx.v[0][l] * 1.5
        moved = O.draft_block(model, ctx, anchors, spec.block).logits
        ctx.v[0][l] = saved
        assert np.max(np.abs(moved - base)) > 1e-4


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((16, 4, 64)) * 3
    k = rng.standard_normal((100, 2, 64))
    v = rng.standard_normal((100, 2, 64))
    _, p = O.attention(q, k, v, return_probs=True)
    assert np.max(np.abs(p.sum(-1) - 1.0)) < 1e-12
    assert np.all(p > 0)


@pytest.mark.parametrize("chunk", [1, 7, 32, 1000])
def test_full_softmax_equals_chunked_online_softmax(chunk):
    """Flash-style evaluation with running (max, sum, output) per query row,
    written here from the definition of the online softmax."""
    rng = np.random.default_rng(2)
    R, S, nq, nkv, d = 16, 301, 4, 2, 32
    q = rng.standard_normal((R, nq, d)) * 2
    k = rng.standard_normal((S, nkv, d))
    v = rng.standard_normal((S, nkv, d))
    ref = O.attention(q, k, v)
    out = np.empty_like(ref)
    for h in range(nq):
        g = h * nkv // nq
        m = np.full(R, -np.inf)
        l = np.zeros(R)
        acc = np.zeros((R, d))
        for s0 in range(0, S, chunk):
            s = q[:, h] @ k[s0:s0 + chunk, g].T / np.sqrt(d)
            m_new = np.maximum(m, s.max(1))
            scale = np.exp(m - m_new)
            p = np.exp(s - m_new[:, None])
            l = l * scale + p.sum(1)
            acc = acc * scale[:, None] + p @ v[s0:s0 + chunk, g]
            m = m_new
        out[:, h] = acc / l[:, None]
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("nq,nkv", [(4, 4), (4, 2), (32, 8), (4, 1)])
def test_attention_matches_torch_sdpa(nq, nkv):
    rng = np.random.default_rng(nq * 10 + nkv)
    R, S, d = 16, 57, 16
    q = rng.standard_normal((R, nq, d))
    k = rng.standard_normal((S, nkv, d))
    v = rng.standard_normal((S, nkv, d))
    ours = O.attention(q, k, v)
    tq, tk, tv = (torch.from_numpy(a).permute(1, 0, 2)[None] for a in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, enable_gqa=(nq != nkv))[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-13)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((5, 2, 8))
    k = rng.standard_normal((1, 1, 8))
    v = rng.standard_normal((1, 1, 8))
    o = O.attention(q, k, v)
    np.testing.assert_allclose(o, np.broadcast_to(v[0, 0], o.shape), rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------
# RoPE, RMSNorm, argmax
# ----------------------------------------------------------------------------

def test_rope_position_zero_is_identity_and_preserves_norm():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 3, 128))
    np.testing.assert_array_equal(O.apply_rope(x, np.zeros(6), 1e6), x)
    y = O.apply_rope(x, np.array([1, 5, 100, 1000, 8191, 123456]), 1e6)
    d = 64
    n0 = x[..., :d] ** 2 + x[..., d:] ** 2
    n1 = y[..., :d] ** 2 + y[..., d:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-13)


def test_rope_relative_position_property():
    """<RoPE(q, p), RoPE(k, p')> depends on p - p' only."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    dots = [np.sum(O.apply_rope(q, np.array([p + 3]), 1e6) * O.apply_rope(k, np.array([p]), 1e6))
            for p in (0, 17, 4096, 9000)]
    assert np.ptp(dots) < 1e-10


def test_rope_matches_complex_rotation_at_theta_1e4():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 2, 16))
    pos = np.array([0, 3, 11])
    y = O.apply_rope(x, pos, 1e4)
    z = (x[..., :8] + 1j * x[..., 8:]) * np.exp(1j * pos[:, None, None] * 1e4 ** (-np.arange(8) / 8))
    np.testing.assert_allclose(y, np.concatenate([z.real, z.imag], -1), rtol=0, atol=1e-14)


def test_rmsnorm_unit_gain_has_unit_rms():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((10, 4096)) * 5
    y = O.rms_norm(x, np.ones(4096), 1e-6)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)), 1.0, rtol=1e-7)


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 256))
    g = rng.standard_normal(256)
    ref = F.rms_norm(torch.from_numpy(x), (256,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, g, 1e-6), ref, rtol=1e-14, atol=1e-14)


def test_argmax_ties_go_to_lowest_index():
    x = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [0.0, -1.0, 0.5, 0.5]])
    assert O.argmax_lowest(x).tolist() == [1, 0, 2]


def test_bf16_decode_known_values():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x3E80, 0x0000, 0x8000, 0x7F7F, 0x0001], np.uint16)
    vals = O.bf16_to_f64(bits)
    assert vals[:6].tolist() == [1.0, -1.0, 2.0, 0.25, 0.0, -0.0]
    assert vals[6] == pytest.approx(3.3895313892515355e38)
    assert vals[7] == 2.0 ** -133


# ----------------------------------------------------------------------------
# accepted-prefix scan
# ----------------------------------------------------------------------------

def _golden_accept_cases():
    cases = []
    with open(os.path.join(HERE, "golden", "accept_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            blk, dr, tg, res = (p.split() for p in line.split("|"))
            cases.append((int(blk[0]), [int(v) for v in dr], [int(v) for v in tg], int(res[0]), int(res[1])))
    return cases


@pytest.mark.parametrize("case", _golden_accept_cases())
def test_accept_len_golden(case):
    B, dr, tg, acc, nxt = case
    assert len(dr) == B - 1 and len(tg) == B
    a, n = O.accept_len(np.array([dr]), np.array([tg]))
    assert (int(a[0]), int(n[0])) == (acc, nxt)


@pytest.mark.parametrize("name", ["q8b_conc32", "q8b_l3_b32_ragged"])
def test_accept_len_closed_form_on_constructed_targets(name):
    spec = I.spec(name)
    rng = np.random.default_rng(11)
    n = 4000
    draft = rng.integers(0, spec.vocab, size=(n, spec.block - 1))
    K, r, bonus = I.gen_accept_construction(spec.with_(ctx_lens=(0,) * n), seed=3)
    t = I.make_targets(draft, K, r, bonus, spec.vocab)
    acc, nxt = O.accept_len(draft, t)
    want = np.minimum(K, spec.block - 1)
    np.testing.assert_array_equal(acc, want)
    np.testing.assert_array_equal(nxt, t[np.arange(n), want])
    # mean of min(K, B-1) for K ~ Geometric(0.15) from 0: sum_{k=1}^{B-1} 0.85^k
    mean = sum(0.85 ** k for k in range(1, spec.block))
    assert abs(acc.mean() - mean) < 0.25


# ----------------------------------------------------------------------------
# multi-step refinement (denoising steps > 1)
# ----------------------------------------------------------------------------

def test_block_tokens_pass_matches_brute_force():
    """A pass with given block tokens in place of the masks, against the
    independent scalar evaluation fed the same tokens."""
    model, w = _model(MICRO, 3)
    ctx, feats = _ingest(model, MICRO, 3)
    anchors = I.gen_anchors(MICRO, 3)
    rng = np.random.default_rng(11)
    toks = rng.integers(0, MICRO.vocab, size=(len(anchors), MICRO.block - 1))
    res = O.draft_block(model, ctx, anchors, MICRO.block, block_tokens=toks)
    bl, bd = brute.brute_draft(MICRO, w, feats, anchors, MICRO.block, block_tokens=toks.tolist())
    np.testing.assert_allclose(res.logits, np.array(bl), rtol=0, atol=1e-12)
    assert res.drafts.tolist() == bd


def test_refine_one_step_is_the_single_pass_and_chains_passes():
    model, w = _model(MICRO, 4)
    ctx, feats = _ingest(model, MICRO, 4)
    anchors = I.gen_anchors(MICRO, 4)
    single = O.draft_block(model, ctx, anchors, MICRO.block)
    passes = O.refine(model, ctx, anchors, MICRO.block, 3)
    np.testing.assert_array_equal(passes[0].logits, single.logits)
    # each later pass is the brute-force pass fed the previous pass's drafts
    for s in (1, 2):
        bl, bd = brute.brute_draft(MICRO, w, feats, anchors, MICRO.block,
                                   block_tokens=passes[s - 1].drafts.tolist())
        np.testing.assert_allclose(passes[s].logits, np.array(bl), rtol=0, atol=1e-12)
        assert passes[s].drafts.tolist() == bd


def test_block_tokens_equal_to_masks_reproduce_the_masked_pass():
    model, _ = _model(MICRO, 6)
    ctx, _ = _ingest(model, MICRO, 6)
    anchors = I.gen_anchors(MICRO, 6)
    masks = np.full((len(anchors), MICRO.block - 1), MICRO.mask_token_id)
    a = O.draft_block(model, ctx, anchors, MICRO.block)
    b = O.draft_block(model, ctx, anchors, MICRO.block, block_tokens=masks)
    np.testing.assert_array_equal(a.logits, b.logits)


# ----------------------------------------------------------------------------
# anchored blocks over shared contexts (the training attention of Fig. 4)
# ----------------------------------------------------------------------------

SMALL = I.DraftSpec("small", n_layers=2, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8,
                    intermediate=48, vocab=64, n_target_layers=2, block=4, ctx_lens=(23, 9))


def _anchored_case(spec, seed):
    model, w = _model(spec, seed)
    ctx, feats = _ingest(model, spec, seed)
    rng = np.random.default_rng(seed)
    lens = spec.ctx_lens
    # several blocks per sequence, anchors at 0, interior positions and the end
    block_seq = [0, 0, 0, 1, 1, 0, 1]
    anchor_pos = [0, 7, lens[0], 0, lens[1], 16, 4]
    anchors = rng.integers(0, spec.vocab - 1, size=len(block_seq))
    return model, w, ctx, feats, block_seq, anchor_pos, anchors


@pytest.mark.parametrize("seed", [0, 3])
def test_anchored_equals_inference_on_the_prefix(seed):
    """Each anchored block drafts exactly what inference drafts at that anchor:
    a fresh context holding only the first anchor_pos features."""
    spec = SMALL
    model, w, ctx, feats, bseq, apos, anchors = _anchored_case(spec, seed)
    res = O.draft_anchored(model, ctx, bseq, apos, anchors, spec.block)
    for j, (sq, a) in enumerate(zip(bseq, apos)):
        one = O.OracleContext(model, 1)
        O.fuse_ctx(model, one, 0, feats[sq][:a])
        ref = O.draft_block(model, one, np.array([anchors[j]]), spec.block)
        np.testing.assert_allclose(res.logits[j], ref.logits[0], rtol=0, atol=1e-12)


def test_anchored_matches_scalar_brute_force():
    spec = MICRO.with_(ctx_lens=(5, 3))
    model, w = _model(spec, 2)
    ctx, feats = _ingest(model, spec, 2)
    bseq, apos, anchors = [0, 0, 1, 0], [2, 5, 1, 0], np.array([3, 9, 14, 0])
    res = O.draft_anchored(model, ctx, bseq, apos, anchors, spec.block)
    for j, (sq, a) in enumerate(zip(bseq, apos)):
        bl, _ = brute.brute_draft(spec, w, [feats[sq][:a]], [anchors[j]], spec.block)
        np.testing.assert_allclose(res.logits[j], np.array(bl[0]), rtol=0, atol=1e-12)


def test_anchored_matches_packed_sdpa_formulation():
    from tests.torch_cpu_ref import torch_anchored
    spec = SMALL
    model, w, ctx, feats, bseq, apos, anchors = _anchored_case(spec, 1)
    res = O.draft_anchored(model, ctx, bseq, apos, anchors, spec.block)
    tl, td = torch_anchored(spec, w, feats, bseq, apos, anchors, spec.block)
    np.testing.assert_allclose(res.logits, tl, rtol=0, atol=1e-10)


def test_anchored_block_sees_only_its_prefix_and_itself():
    spec = SMALL
    model, w, ctx, feats, bseq, apos, anchors = _anchored_case(spec, 4)
    base = O.draft_anchored(model, ctx, bseq, apos, anchors, spec.block)
    # features at or after a block's anchor, and other blocks' tokens, change nothing for it
    j = 1  # sequence 0, anchor 7
    f2 = [f.copy() for f in feats]
    f2[0][apos[j]:] = I.gen_features(spec, 77, 0, len(feats[0]))[apos[j]:]
    ctx2 = O.OracleContext(model, 2)
    for b in range(2):
        O.fuse_ctx(model, ctx2, b, f2[b])
    toks = np.full((len(bseq), spec.block - 1), spec.mask_token_id)
    toks[0] = [1, 2, 3]
    toks[2] = [5, 6, 7]
    r2 = O.draft_anchored(model, ctx2, bseq, apos, anchors, spec.block, block_tokens=toks)
    np.testing.assert_allclose(r2.logits[j], base.logits[j], rtol=0, atol=1e-12)
    # ... while a feature before the anchor does
    f3 = [f.copy() for f in feats]
    f3[0][apos[j] - 1] = I.gen_features(spec, 78, 0, len(feats[0]))[apos[j] - 1]
    ctx3 = O.OracleContext(model, 2)
    for b in range(2):
        O.fuse_ctx(model, ctx3, b, f3[b])
    r3 = O.draft_anchored(model, ctx3, bseq, apos, anchors, spec.block)
    assert np.max(np.abs(r3.logits[j] - base.logits[j])) > 1e-6


def test_masked_attention_reduces_to_attention_on_the_allowed_keys():
    rng = np.random.default_rng(5)
    q, k, v = rng.normal(size=(6, 4, 8)), rng.normal(size=(11, 2, 8)), rng.normal(size=(11, 2, 8))
    np.testing.assert_allclose(O.masked_attention(q, k, v, np.ones((6, 11), bool)), O.attention(q, k, v),
                               rtol=0, atol=1e-14)
    keep = np.array([0, 3, 4, 9])
    allowed = np.zeros((6, 11), bool)
    allowed[:, keep] = True
    np.testing.assert_allclose(O.masked_attention(q, k, v, allowed), O.attention(q, k[keep], v[keep]),
                               rtol=0, atol=1e-14)


@pytest.mark.parametrize("seq_len,n,blk,prompt", [(1024, 16, 16, 0), (64, 4, 16, 0), (4096, 64, 16, 1024), (40, 3, 8, 10)])
def test_train_anchor_placement_is_valid(seq_len, n, blk, prompt):
    a = I.gen_train_anchors(seq_len, n, blk, seed=1, prompt_len=prompt)
    assert len(a) == n and a[0] >= prompt and a[-1] + blk <= seq_len
    assert np.all(np.diff(a) >= blk)


# ----------------------------------------------------------------------------
# the parity bar's helper (top-2 gap) and context truncation
# ----------------------------------------------------------------------------

def test_top2_gap_hand_cases():
    """Gap = largest minus second largest, never negative; a tie at the top
    gives 0 (so a tied row is never counted as decided)."""
    x = np.array([[3.0, 1.0, 2.0], [5.0, 5.0, 1.0], [1.0, 2.0, 3.0], [-4.0, -1.0, -2.5],
                  [0.0, 0.0, 0.0], [7.0, -7.0, 6.5]])
    assert O.top2_gap(x).tolist() == [1.0, 0.0, 1.0, 1.5, 0.0, 0.5]


def test_top2_gap_matches_sorting_on_random_rows():
    """Against Python's own sort of each row (no numpy partition), over shapes
    with leading batch axes as the parity checks use them."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((3, 5, 97)) * 2.0
    x[0, 1, 10] = x[0, 1, 20] = 50.0  # an exact tie at the top
    got = O.top2_gap(x)
    assert got.shape == (3, 5)
    for idx in np.ndindex(3, 5):
        s = sorted(x[idx].tolist())
        assert got[idx] == s[-1] - s[-2]
    assert got[0, 1] == 0.0 and np.all(got >= 0.0)


def test_truncate_then_reappend_equals_fresh_ingest():
    """Truncating a sequence to n positions and appending the same features
    again gives exactly the K/V a context that took the same appends without
    the detour holds, for every layer, K and V alike; the other sequence is
    untouched; and the drafts over both contexts are bitwise equal."""
    spec = I.spec("tiny").with_(ctx_lens=(40, 25))
    model, _ = _model(spec, 4, std=0.05)
    fa = I.gen_features(spec, 9, 0, 40)
    fb = I.gen_features(spec, 9, 1, 25)
    extra = I.gen_features(spec, 10, 0, 12)
    ctx = O.OracleContext(model, 2)
    O.fuse_ctx(model, ctx, 0, fa[:30])
    O.fuse_ctx(model, ctx, 0, fa[30:])
    O.fuse_ctx(model, ctx, 1, fb)
    O.fuse_ctx(model, ctx, 0, extra)          # 52 positions, then take the last 22 back
    k_before = [k.copy() for k in ctx.k[0]]
    O.truncate_ctx(ctx, 0, 30)
    assert ctx.length(0) == 30 and ctx.length(1) == 25
    for l in range(model.n_layers):
        assert ctx.k[0][l].shape[0] == 30 and ctx.v[0][l].shape[0] == 30
        np.testing.assert_array_equal(ctx.k[0][l], k_before[l][:30])
    O.fuse_ctx(model, ctx, 0, fa[30:])
    fresh = O.OracleContext(model, 2)
    O.fuse_ctx(model, fresh, 0, fa[:30])
    O.fuse_ctx(model, fresh, 0, fa[30:])
    O.fuse_ctx(model, fresh, 1, fb)
    for b in range(2):
        for l in range(model.n_layers):
            np.testing.assert_array_equal(ctx.k[b][l], fresh.k[b][l])
            np.testing.assert_array_equal(ctx.v[b][l], fresh.v[b][l])
    anchors = I.gen_anchors(spec, 9)
    r1 = O.draft_block(model, ctx, anchors, spec.block)
    r2 = O.draft_block(model, fresh, anchors, spec.block)
    np.testing.assert_array_equal(r1.logits, r2.logits)


def test_truncate_to_zero_and_to_full_length():
    spec = I.spec("tiny").with_(ctx_lens=(20,))
    model, _ = _model(spec, 5, std=0.05)
    f = I.gen_features(spec, 3, 0, 20)
    ctx = O.OracleContext(model, 1)
    O.fuse_ctx(model, ctx, 0, f)
    full = [(k.copy(), v.copy()) for k, v in zip(ctx.k[0], ctx.v[0])]
    O.truncate_ctx(ctx, 0, 20)  # no-op
    for l, (k, v) in enumerate(full):
        np.testing.assert_array_equal(ctx.k[0][l], k)
        np.testing.assert_array_equal(ctx.v[0][l], v)
    O.truncate_ctx(ctx, 0, 0)
    assert ctx.length(0) == 0
    assert all(k.shape[0] == 0 for k in ctx.k[0]) and all(v.shape[0] == 0 for v in ctx.v[0])
