"""Plain float64 CPU oracle of the DFlash block-diffusion draft pass.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

What is computed, and where it comes from
-----------------------------------------
DFlash (arXiv 2602.06036, "DFlash: Block Diffusion for Flash Speculative
Decoding") drafts a whole block of tokens with a small block-diffusion model in
one forward pass (paper Abstract; forum post "Parallel Diffusion Meets
Speculative Decoding", section 1 "Block Diffusion and Denoising Folding").
Hidden features taken from several layers of the frozen target model are fused
and injected as key/value entries into every draft layer's KV cache (paper
Fig. 2 "DFlash Inference Design"; atlas summary, "Approach").  The drafted
block is verified by the target in parallel and the matched prefix is accepted;
the reported metric is the average acceptance length tau at temperature 0
(atlas summary, "Key results" and "Experimental setup").

The pages do not spell out the layer internals.  This oracle takes the plainest
reading of a Qwen3-shaped drafter (pre-norm RMSNorm, rotate-half RoPE, GQA
attention, SwiGLU MLP, no biases, final norm before a shared LM head) and the
readings listed in the repository's design notes:

* fusion is one bias-free linear map h = W_fc F of the concatenated features;
* context K/V use each layer's own W_k / W_v on h, with RoPE on K at the
  context position; there is no norm on h;
* positions: context tokens 0..c-1, block positions c..c+B-1;
* the block is (anchor, mask, ..., mask); every block query sees all context
  keys and all block keys (no mask at all);
* block row i >= 1 predicts the token at its own position; its draft is the
  lowest index of the maximum logit;
* accept length n = length of the prefix on which draft and target agree,
  next anchor = target[n], tau = n + 1.

Everything is evaluated in float64 with no intermediate rounding; bf16 weights
and features are exact real numbers.  Library primitives used as steps: numpy
matmul, exp, sqrt, cos, sin, argmax.  Nothing is blocked or fused, except that
the LM-head product is evaluated over vocabulary slabs to bound host memory
(each logit is still one plain dot product).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

_LM_SLAB = 16384  # vocabulary rows per LM-head slab (host memory bound only)


# ----------------------------------------------------------------------------
# elementary pieces
# ----------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact float64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: gain * x / sqrt(mean(x^2) + eps)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return gain * x / np.sqrt(ms + eps)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def rope_angles(positions: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """Angles p * theta^(-2j/d) for j < d/2, shape [len(positions)][d/2]."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / head_dim)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]


def apply_rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE.  x: [P][heads][d]; positions: [P].

    For j < d/2 the pair (x_j, x_{j+d/2}) is rotated by the angle p*w_j:
    (x_j cos - x_{j+d/2} sin, x_{j+d/2} cos + x_j sin).
    """
    d = x.shape[-1]
    a = rope_angles(positions, d, theta)[:, None, :]  # [P][1][d/2]
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """exp(s) / sum(exp(s)) along the last axis (the row maximum is subtracted
    first, which leaves the value unchanged)."""
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, return_probs: bool = False):
    """Unmasked GQA attention of one sequence.

    q: [R][n_q][d] queries, k, v: [S][n_kv][d] keys/values.  Query head h reads
    key/value head floor(h * n_kv / n_q).  Scores are scaled by 1/sqrt(d); every
    query sees every key.  Returns o [R][n_q][d] (and probabilities
    [n_q][R][S] when asked).
    """
    R, n_q, d = q.shape
    n_kv = k.shape[1]
    o = np.empty_like(q)
    probs = np.empty((n_q, R, k.shape[0])) if return_probs else None
    for h in range(n_q):
        g = (h * n_kv) // n_q
        s = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(d)
        p = softmax_rows(s)
        o[:, h, :] = p @ v[:, g, :]
        if return_probs:
            probs[h] = p
    return (o, probs) if return_probs else o


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """GQA attention where query r sees key s only if allowed[r][s].

    Same as ``attention`` over the allowed keys of each row: scores of the
    other keys are left out of the softmax.  Every row must allow at least
    one key.  q: [R][n_q][d], k, v: [S][n_kv][d], allowed: [R][S] bool.
    """
    R, n_q, d = q.shape
    n_kv = k.shape[1]
    allowed = np.asarray(allowed, dtype=bool)
    assert allowed.shape == (R, k.shape[0]) and np.all(allowed.any(axis=1))
    o = np.empty_like(q)
    for h in range(n_q):
        g = (h * n_kv) // n_q
        s = np.where(allowed, (q[:, h, :] @ k[:, g, :].T) / np.sqrt(d), -np.inf)
        o[:, h, :] = softmax_rows(s) @ v[:, g, :]
    return o


def argmax_lowest(x: np.ndarray) -> np.ndarray:
    """Index of the maximum along the last axis; ties go to the lowest index."""
    return np.argmax(x, axis=-1)


# ----------------------------------------------------------------------------
# model and context state
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class OracleModel:
    """Drafter hyper-parameters plus its bf16 weights (bit arrays, decoded on use)."""
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    n_target_layers: int
    mask_token_id: int
    rms_eps: float
    rope_theta: float
    weights: Dict[str, np.ndarray]

    @classmethod
    def from_spec(cls, spec, weights: Dict[str, np.ndarray]) -> "OracleModel":
        return cls(spec.n_layers, spec.hidden, spec.n_q_heads, spec.n_kv_heads, spec.head_dim,
                   spec.intermediate, spec.vocab, spec.n_target_layers, spec.mask_token_id,
                   spec.rms_eps, spec.rope_theta, weights)

    def w(self, name: str) -> np.ndarray:
        return bf16_to_f64(self.weights[name])

    def lw(self, layer: int, name: str) -> np.ndarray:
        return self.w(f"layers.{layer}.{name}")


class OracleContext:
    """Per-sequence, per-layer injected context K/V (post-RoPE), float64.

    ``k[b][l]`` and ``v[b][l]`` are [c_b][n_kv][d].  ``pos_offset`` shifts every
    position (context and block) by a constant; it exists only to test the
    shift invariance of RoPE attention.
    """

    def __init__(self, model: OracleModel, n_seqs: int, pos_offset: int = 0):
        self.model = model
        self.pos_offset = int(pos_offset)
        shp = (0, model.n_kv_heads, model.head_dim)
        self.k: List[List[np.ndarray]] = [[np.zeros(shp) for _ in range(model.n_layers)] for _ in range(n_seqs)]
        self.v: List[List[np.ndarray]] = [[np.zeros(shp) for _ in range(model.n_layers)] for _ in range(n_seqs)]

    def length(self, b: int) -> int:
        return self.k[b][0].shape[0]


def fuse_features(model: OracleModel, features_bits: np.ndarray) -> np.ndarray:
    """h = W_fc F: one bias-free linear map of the concatenated target features
    (paper Fig. 2: target features are fused).  features: [T][L_t*H] bf16 bits."""
    return bf16_to_f64(features_bits) @ model.w("w_fc").T


def fuse_ctx(model: OracleModel, ctx: OracleContext, seq: int, features_bits: np.ndarray,
             use_rope: bool = True) -> None:
    """Append T verified positions to sequence ``seq``'s injected context.

    Fused features are projected by every layer's own W_k and W_v and written to
    that layer's KV cache (paper Fig. 2; atlas summary "Approach": injected as
    key/value entries into every draft layer).  K carries RoPE at the context
    position; V does not.
    """
    T = features_bits.shape[0]
    if T == 0:
        return
    h = fuse_features(model, features_bits)
    p0 = ctx.length(seq)
    pos = ctx.pos_offset + p0 + np.arange(T)
    kv, d = model.n_kv_heads, model.head_dim
    for l in range(model.n_layers):
        k = (h @ model.lw(l, "wk").T).reshape(T, kv, d)
        v = (h @ model.lw(l, "wv").T).reshape(T, kv, d)
        if use_rope:
            k = apply_rope(k, pos, model.rope_theta)
        ctx.k[seq][l] = np.concatenate([ctx.k[seq][l], k], axis=0)
        ctx.v[seq][l] = np.concatenate([ctx.v[seq][l], v], axis=0)


def truncate_ctx(ctx: OracleContext, seq: int, new_len: int) -> None:
    for l in range(len(ctx.k[seq])):
        ctx.k[seq][l] = ctx.k[seq][l][:new_len]
        ctx.v[seq][l] = ctx.v[seq][l][:new_len]


@dataclasses.dataclass
class DraftResult:
    logits: np.ndarray      # [n_seqs][B-1][V] float64
    drafts: np.ndarray      # [n_seqs][B-1] int64
    hidden: np.ndarray      # [n_seqs][B][H] final residual stream (before the final norm)


def draft_block(model: OracleModel, ctx: OracleContext, anchors: np.ndarray, block: int,
                use_rope: bool = True, seqs: Optional[List[int]] = None,
                block_tokens: Optional[np.ndarray] = None) -> DraftResult:
    """One block-diffusion draft pass over every sequence (or the listed ones).

    The block is the anchor token followed by B-1 mask tokens at positions
    c_b .. c_b+B-1; it runs through all draft layers in a single pass (forward
    post, section 1; atlas summary "Approach"), attending to [context K/V |
    block K/V] with no mask.  Rows 1..B-1 are the drafts.  block_tokens
    ([n_seqs][B-1], indexed like anchors) replaces the mask tokens of rows
    1..B-1 when given (a refinement pass, see ``refine``).
    """
    m = model
    seqs = list(range(len(anchors))) if seqs is None else list(seqs)
    n, B, H = len(seqs), int(block), m.hidden
    nq, nkv, d = m.n_q_heads, m.n_kv_heads, m.head_dim
    E = m.weights["embed"]
    toks = np.full((n, B), m.mask_token_id, dtype=np.int64)
    toks[:, 0] = np.asarray(anchors, dtype=np.int64)[seqs]
    if block_tokens is not None:
        toks[:, 1:] = np.asarray(block_tokens, dtype=np.int64)[seqs]
    x = bf16_to_f64(E[toks.reshape(-1)]).reshape(n, B, H)
    pos = [ctx.pos_offset + ctx.length(b) + np.arange(B) for b in seqs]

    for l in range(m.n_layers):
        u = rms_norm(x, m.lw(l, "attn_norm"), m.rms_eps)
        q = (u @ m.lw(l, "wq").T).reshape(n, B, nq, d)
        k = (u @ m.lw(l, "wk").T).reshape(n, B, nkv, d)
        v = (u @ m.lw(l, "wv").T).reshape(n, B, nkv, d)
        o = np.empty((n, B, nq, d))
        for i, b in enumerate(seqs):
            qi, ki = q[i], k[i]
            if use_rope:
                qi = apply_rope(qi, pos[i], m.rope_theta)
                ki = apply_rope(ki, pos[i], m.rope_theta)
            keys = np.concatenate([ctx.k[b][l], ki], axis=0)
            vals = np.concatenate([ctx.v[b][l], v[i]], axis=0)
            o[i] = attention(qi, keys, vals)
        x = x + o.reshape(n, B, nq * d) @ m.lw(l, "wo").T
        w = rms_norm(x, m.lw(l, "mlp_norm"), m.rms_eps)
        a = silu(w @ m.lw(l, "wgate").T) * (w @ m.lw(l, "wup").T)
        x = x + a @ m.lw(l, "wdown").T

    y = rms_norm(x[:, 1:, :], m.w("final_norm"), m.rms_eps).reshape(n * (B - 1), H)
    logits = np.empty((n * (B - 1), m.vocab))
    for v0 in range(0, m.vocab, _LM_SLAB):
        v1 = min(m.vocab, v0 + _LM_SLAB)
        logits[:, v0:v1] = y @ bf16_to_f64(E[v0:v1]).T
    logits = logits.reshape(n, B - 1, m.vocab)
    return DraftResult(logits=logits, drafts=argmax_lowest(logits), hidden=x)


def refine(model: OracleModel, ctx: OracleContext, anchors: np.ndarray, block: int, steps: int,
           init_tokens: Optional[np.ndarray] = None) -> List[DraftResult]:
    """Several denoising passes over one block (forum post, section 1: the
    efficiency of a draft is block size over diffusion steps times the
    acceptance rate; one step is DFlash's default).  The pages do not state
    how a later step re-masks; this takes the plainest reading: every pass
    after the first feeds the previous pass's drafts in place of the mask
    tokens.  Returns the result of every pass; the last one is the draft."""
    out: List[DraftResult] = []
    toks = init_tokens
    for _ in range(steps):
        r = draft_block(model, ctx, anchors, block, block_tokens=toks)
        out.append(r)
        toks = r.drafts
    return out


def draft_anchored(model: OracleModel, ctx: OracleContext, block_seq, anchor_pos, anchors: np.ndarray,
                   block: int, block_tokens: Optional[np.ndarray] = None) -> DraftResult:
    """Forward of the training attention (paper Fig. 4; atlas summary
    "Approach": random anchor-token block sampling).

    Each training sequence's target features are injected as context for
    all of its positions.  Block j starts at the clean anchor token at
    position anchor_pos[j] of sequence block_seq[j], followed by B-1 mask
    tokens (or block_tokens[j]), at positions anchor_pos[j] ..
    anchor_pos[j]+B-1.  All blocks of a sequence go through each layer
    together, in one attention over [the sequence's context keys | every
    block's keys] under a block-sparse mask: a query of block j sees the
    context keys at positions < anchor_pos[j] (what has been verified when
    that block is drafted at inference) and the keys of block j, and nothing
    else.  Rows 1..B-1 of each block are its drafts.
    """
    m = model
    block_seq = np.asarray(block_seq, dtype=np.int64)
    anchor_pos = np.asarray(anchor_pos, dtype=np.int64)
    n, B, H = len(block_seq), int(block), m.hidden
    nq, nkv, d = m.n_q_heads, m.n_kv_heads, m.head_dim
    E = m.weights["embed"]
    toks = np.full((n, B), m.mask_token_id, dtype=np.int64)
    toks[:, 0] = np.asarray(anchors, dtype=np.int64)
    if block_tokens is not None:
        toks[:, 1:] = np.asarray(block_tokens, dtype=np.int64)
    x = bf16_to_f64(E[toks.reshape(-1)]).reshape(n, B, H)
    pos = [ctx.pos_offset + int(anchor_pos[j]) + np.arange(B) for j in range(n)]

    for l in range(m.n_layers):
        u = rms_norm(x, m.lw(l, "attn_norm"), m.rms_eps)
        q = (u @ m.lw(l, "wq").T).reshape(n, B, nq, d)
        k = (u @ m.lw(l, "wk").T).reshape(n, B, nkv, d)
        v = (u @ m.lw(l, "wv").T).reshape(n, B, nkv, d)
        q = np.stack([apply_rope(q[j], pos[j], m.rope_theta) for j in range(n)])
        k = np.stack([apply_rope(k[j], pos[j], m.rope_theta) for j in range(n)])
        o = np.empty((n, B, nq, d))
        for sq in sorted(set(block_seq.tolist())):
            J = np.nonzero(block_seq == sq)[0]
            T = ctx.length(sq)
            keys = np.concatenate([ctx.k[sq][l]] + [k[j] for j in J], axis=0)
            vals = np.concatenate([ctx.v[sq][l]] + [v[j] for j in J], axis=0)
            allowed = np.zeros((len(J) * B, T + len(J) * B), dtype=bool)
            for jj, j in enumerate(J):
                rows = slice(jj * B, (jj + 1) * B)
                allowed[rows, : anchor_pos[j]] = True
                allowed[rows, T + jj * B: T + (jj + 1) * B] = True
            oj = masked_attention(np.concatenate([q[j] for j in J], axis=0), keys, vals, allowed)
            o[J] = oj.reshape(len(J), B, nq, d)
        x = x + o.reshape(n, B, nq * d) @ m.lw(l, "wo").T
        w = rms_norm(x, m.lw(l, "mlp_norm"), m.rms_eps)
        a = silu(w @ m.lw(l, "wgate").T) * (w @ m.lw(l, "wup").T)
        x = x + a @ m.lw(l, "wdown").T

    y = rms_norm(x[:, 1:, :], m.w("final_norm"), m.rms_eps).reshape(n * (B - 1), H)
    logits = np.empty((n * (B - 1), m.vocab))
    for v0 in range(0, m.vocab, _LM_SLAB):
        v1 = min(m.vocab, v0 + _LM_SLAB)
        logits[:, v0:v1] = y @ bf16_to_f64(E[v0:v1]).T
    logits = logits.reshape(n, B - 1, m.vocab)
    return DraftResult(logits=logits, drafts=argmax_lowest(logits), hidden=x)


def accept_len(draft: np.ndarray, target: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Greedy verification of a drafted block (atlas summary, "Key results":
    temperature 0; metric: acceptance length tau).

    draft: [n][B-1] tokens for block positions 1..B-1; target: [n][B] the
    target's tokens for positions 1..B (the last one is the bonus token).
    Returns (accept, next_anchor): accept[b] = number of leading positions on
    which draft and target agree (0..B-1), next_anchor[b] = target[b][accept[b]].
    tau = accept + 1.
    """
    draft = np.asarray(draft)
    target = np.asarray(target)
    n, bm1 = draft.shape
    acc = np.zeros(n, dtype=np.int64)
    nxt = np.zeros(n, dtype=np.int64)
    for b in range(n):
        k = 0
        while k < bm1 and draft[b, k] == target[b, k]:
            k += 1
        acc[b] = k
        nxt[b] = target[b, k]
    return acc, nxt


def top2_gap(logits: np.ndarray) -> np.ndarray:
    """max logit minus the second largest logit along the last axis."""
    part = np.partition(logits, -2, axis=-1)
    return part[..., -1] - part[..., -2]
