"""Seeded synthetic workloads for the DFlash draft pass.

This module only *generates inputs*: drafter shapes, random-init weights,
target-model features, anchors, ragged context lengths and constructed
target tokens.  It contains none of the method's arithmetic, so both the
GPU path and the CPU oracle may take their inputs from it.

All floating-point tensors are returned as bfloat16 bit patterns
(``numpy.uint16``), produced by rounding float32 normal samples to nearest
even.  Every tensor draws from its own counter-addressed PCG64 stream
(``SeedSequence(seed, spawn_key=(tensor_key, chunk))``), so a tensor, a
sequence's features, or a sub-range of chunks can be regenerated alone and
generation can run on several threads without changing a single value.

The workloads stand in for the pages' benchmark traffic (DFlash paper,
p2 "Experimental setup": math, code and chat suites), which this build does
not reproduce: shapes follow a Qwen3-8B-sized drafter, values are
N(0, 0.02) weights and N(0, 1) features.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "DraftSpec", "SPECS", "spec", "weight_names", "f32_to_bf16_bits",
    "gen_weights", "gen_features", "gen_anchors", "gen_accept_construction",
    "make_targets",
]

_CHUNK = 1 << 22  # elements per independently seeded chunk


@dataclasses.dataclass(frozen=True)
class DraftSpec:
    """Shape of one drafter and one synthetic decode-step workload."""
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    n_target_layers: int
    block: int
    ctx_lens: Tuple[int, ...]
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    geometric_p: float = 0.15
    # training-forward workloads: anchored blocks per sequence, placed in the
    # response part after prompt_len positions (0: a decode workload)
    train_blocks: int = 0
    prompt_len: int = 0

    @property
    def mask_token_id(self) -> int:
        return self.vocab - 1

    @property
    def n_seqs(self) -> int:
        return len(self.ctx_lens)

    @property
    def fused_width(self) -> int:
        return self.n_target_layers * self.hidden

    def with_(self, **kw) -> "DraftSpec":
        return dataclasses.replace(self, **kw)


def _ragged_lens(seed: int, n: int, lo: int, hi: int) -> Tuple[int, ...]:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(7,))))
    return tuple(int(v) for v in rng.integers(lo, hi + 1, size=n))


_Q8 = dict(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, intermediate=12288,
           vocab=151936, n_target_layers=5)

SPECS: Dict[str, DraftSpec] = {
    # 1-layer toy drafter, context 128, block 16, one sequence.
    "tiny": DraftSpec("tiny", n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                      intermediate=768, vocab=4096, n_target_layers=3, block=16,
                      ctx_lens=(128,)),
    # 5-layer Qwen3-8B-shaped drafter, context 1024, block 16, concurrency 1.
    "q8b_ctx1024": DraftSpec("q8b_ctx1024", n_layers=5, block=16, ctx_lens=(1024,), **_Q8),
    # The same widths and context with 1 and 3 layers: draft cost against
    # drafter depth (the paper's Fig. 3 compares 1-, 3- and 5-layer drafters).
    "q8b_l1_ctx1024": DraftSpec("q8b_l1_ctx1024", n_layers=1, block=16, ctx_lens=(1024,), **_Q8),
    "q8b_l3_ctx1024": DraftSpec("q8b_l3_ctx1024", n_layers=3, block=16, ctx_lens=(1024,), **_Q8),
    # Same drafter with 8192 injected context positions.
    "q8b_ctx8192": DraftSpec("q8b_ctx8192", n_layers=5, block=16, ctx_lens=(8192,), **_Q8),
    # Same drafter at concurrency 32, context 2048 each.
    "q8b_conc32": DraftSpec("q8b_conc32", n_layers=5, block=16, ctx_lens=(2048,) * 32, **_Q8),
    # 3-layer drafter, block 32, eight sequences with ragged contexts in [512, 4096].
    "q8b_l3_b32_ragged": DraftSpec("q8b_l3_b32_ragged", n_layers=3, block=32,
                                   ctx_lens=_ragged_lens(20260205, 8, 512, 4096), **_Q8),
    # Training-attention forward: 4 sequences of 4096 positions (1024 prompt,
    # 3072 response), 32 anchored blocks of 16 in each response.
    "q8b_train4x4096": DraftSpec("q8b_train4x4096", n_layers=5, block=16, ctx_lens=(4096,) * 4,
                                 train_blocks=32, prompt_len=1024, **_Q8),
}


def spec(name: str) -> DraftSpec:
    return SPECS[name]


def weight_names(s: DraftSpec) -> List[str]:
    """Weight tensors in the order the C ABI takes them."""
    names = ["w_fc", "embed", "final_norm"]
    for l in range(s.n_layers):
        names += [f"layers.{l}.{n}" for n in
                  ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "wgate", "wup", "wdown")]
    return names


def weight_shape(s: DraftSpec, name: str) -> Tuple[int, ...]:
    H, d = s.hidden, s.head_dim
    short = name.split(".")[-1]
    return {
        "w_fc": (H, s.fused_width), "embed": (s.vocab, H), "final_norm": (H,),
        "attn_norm": (H,), "mlp_norm": (H,),
        "wq": (s.n_q_heads * d, H), "wk": (s.n_kv_heads * d, H), "wv": (s.n_kv_heads * d, H),
        "wo": (H, s.n_q_heads * d), "wgate": (s.intermediate, H), "wup": (s.intermediate, H),
        "wdown": (H, s.intermediate),
    }[short]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 samples to bfloat16 (nearest, ties to even); returns the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_bf16(seed: int, key: Tuple[int, ...], lo: int, hi: int, std: float,
                 mean: float = 0.0) -> np.ndarray:
    """Elements [lo, hi) of an endless stream of N(mean, std^2) samples rounded to
    bf16.  Chunk j of the stream (elements [j*C, (j+1)*C)) is drawn from its own
    generator keyed by (seed, key, j); a shorter draw from a generator is a prefix
    of a longer one, so any range can be produced on its own."""
    out = np.empty(hi - lo, dtype=np.uint16)
    c0, c1 = lo // _CHUNK, (hi + _CHUNK - 1) // _CHUNK

    def fill(j: int) -> None:
        base = j * _CHUNK
        want = min(_CHUNK, hi - base)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key) + (j,))))
        x = rng.standard_normal(want, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        if mean != 0.0:
            x += np.float32(mean)
        skip = max(lo - base, 0)
        out[base + skip - lo: base + want - lo] = f32_to_bf16_bits(x[skip:])

    if c1 - c0 <= 1:
        for j in range(c0, c1):
            fill(j)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(c0, c1)))
    return out


def gen_weights(s: DraftSpec, seed: int = 0, gain_jitter: float = 0.0,
                std: float = 0.02) -> Dict[str, np.ndarray]:
    """Random-init drafter weights as bf16 bit arrays.

    Matrices are ``nn.Linear`` layout ``[out][in]`` drawn from N(0, std^2);
    the embedding (shared with the LM head) likewise.  Norm gains are exactly
    1.0, or 1 + N(0, gain_jitter^2) when ``gain_jitter`` > 0.
    """
    out: Dict[str, np.ndarray] = {}
    for key, name in enumerate(weight_names(s)):
        shape = weight_shape(s, name)
        n = int(np.prod(shape))
        if name.endswith("norm"):
            if gain_jitter > 0:
                w = _normal_bf16(seed, (1, key), 0, n, gain_jitter, 1.0)
            else:
                w = np.full(n, 0x3F80, dtype=np.uint16)
        else:
            w = _normal_bf16(seed, (1, key), 0, n, std)
        out[name] = w.reshape(shape)
    return out


def gen_features(s: DraftSpec, seed: int, seq: int, n_rows: int, first_row: int = 0) -> np.ndarray:
    """Target-model features for sequence ``seq``: rows [first_row, first_row+n_rows)
    of an N(0, 1) bf16 stream, each row the L_t selected target layers concatenated."""
    W = s.fused_width
    return _normal_bf16(seed, (2, seq), first_row * W, (first_row + n_rows) * W, 1.0).reshape(n_rows, W)


def gen_anchors(s: DraftSpec, seed: int) -> np.ndarray:
    """Anchor (last verified) token per sequence, uniform over the non-mask vocabulary."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(3,))))
    return rng.integers(0, s.vocab - 1, size=s.n_seqs).astype(np.int32)


def gen_accept_construction(s: DraftSpec, seed: int, n_seqs: Optional[int] = None):
    """Random draws for the constructed target tokens.

    Returns ``(K, r, bonus)``: K[b] ~ Geometric(p) counted from 0
    (P(K = k) = (1-p)^k p), r[b][j] uniform in {1..V-1}, bonus[b] uniform in
    {0..V-1}.  ``make_targets`` turns them into target tokens whose matched
    prefix with the drafts is exactly min(K, B-1).
    """
    n = s.n_seqs if n_seqs is None else n_seqs
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(4,))))
    K = (rng.geometric(s.geometric_p, size=n) - 1).astype(np.int64)
    r = rng.integers(1, s.vocab, size=(n, s.block - 1)).astype(np.int64)
    bonus = rng.integers(0, s.vocab, size=n).astype(np.int64)
    return K, r, bonus


def make_targets(draft: np.ndarray, K: np.ndarray, r: np.ndarray, bonus: np.ndarray,
                 vocab: int) -> np.ndarray:
    """Target tokens ``[n][B]`` for drafts ``[n][B-1]``: equal to the draft on the
    first min(K, B-1) positions, a uniformly random different token
    ((draft + r) mod V, r != 0) on the rest, and a random bonus token last."""
    draft = np.asarray(draft, dtype=np.int64)
    n, bm1 = draft.shape
    t = np.empty((n, bm1 + 1), dtype=np.int32)
    for b in range(n):
        k = int(min(K[b], bm1))
        t[b, :k] = draft[b, :k]
        t[b, k:bm1] = (draft[b, k:] + r[b, k:]) % vocab
        t[b, bm1] = bonus[b]
    return t


def gen_train_anchors(seq_len: int, n_blocks: int, block: int, seed: int, prompt_len: int = 0) -> np.ndarray:
    """Anchor positions of ``n_blocks`` non-overlapping blocks inside the
    response part [prompt_len, seq_len) of a training sequence, uniform over
    all such placements, sorted.  Each block [a, a + block) lies inside the
    sequence."""
    free = seq_len - prompt_len - n_blocks * block
    if free < 0:
        raise ValueError("blocks do not fit in the response")
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(5,))))
    c = np.sort(rng.choice(free + n_blocks, size=n_blocks, replace=False))
    return (prompt_len + c + np.arange(n_blocks) * (block - 1)).astype(np.int64)
