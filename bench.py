"""Throughput of the DFlash draft pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

One *step* is one steady-state decode iteration of the drafter, every part of
the hot path once, for every sequence of the workload:

  1. dflash_step        fuse the target features of the B newly verified
                         positions (the largest possible tau), append them as
                         injected K/V to every draft layer's cache, and run one
                         block-diffusion pass over (anchor, B-1 masks) ending in
                         the LM-head argmax (--two-call: the same work as
                         dflash_fuse_ctx followed by dflash_draft_block);
  2. dflash_accept_len   accepted-prefix scan against constructed target tokens.

A training-forward workload (e.g. --workload q8b_train4x4096) instead
times the forward of the training attention: one step ingests every
training sequence's target features as injected context (dflash_fuse_ctx)
and drafts all of its anchored blocks (dflash_draft_anchored), each block
seeing the context before its anchor and itself.

--phase draft times the draft pass alone over a resident context: every
position already ingested, one step = dflash_draft_block + dflash_accept_len
(no append), the pass as the method statement defines it.

--phase ingest times the other phase of the method instead: every
sequence's whole context ingested from its target features (the fusion map
and every layer's injected K/V, dflash_fuse_ctx), in ingested positions/s.

--temperature T > 0 samples the drafts instead (dflash_step_sample, which
also writes the drafter's logits) and verifies them losslessly against
resident synthetic target logits (dflash_verify_sample) in place of the
greedy scan.

--denoise-steps S > 1 adds S - 1 further passes over the block
(dflash_draft_refine, each fed the previous pass's drafts), the multi-step
alternative that the block size / steps efficiency trade-off compares against.

Before each step the host rolls every context back by B positions (metadata
only), so each step sees the same context length and does identical work.
Inputs are seeded synthetic tensors already resident in HBM.  The default
workload is the 5-layer Qwen3-8B-shaped drafter at context 1024, block 16,
one sequence.

Printed (stdout, one JSON line): draft tokens/s over the K timed steps (two
events around the K steps and nothing else recorded between them), the
per-step p10 / p50 / p90 from a second loop of K steps, the roofline fraction
of the dominant kernel (the LM head), timed live with HIP events that the
library records around that kernel's launches on the same stream in a third
loop, and the CPU oracle timed on the host cores on a bounded sample.  For the
decode workloads the line also carries the draft pass alone over the resident
context (phase_d: dflash_draft_block + dflash_accept_len, K more iterations)
with its fractions of HBM and bf16 matrix-core peak, the executed matrix-core
fraction and busy share when a rocprofv3 counter summary of the current
kernels is committed, and the pass-level aim with whether it is met
(pass_target).  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "draft tokens/sec at block 16, 5-layer, ctx 1024, conc 1; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, datasheet
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 matrix peak, datasheet (no sparsity)
# Pass-level aims of the draft pass alone over a resident context (phase D):
# the single-sequence workloads are weight-streaming (fraction of HBM peak),
# the 32-sequence one is matrix-core work (algorithmic bf16 fraction).
PASS_TARGETS = {"q8b_ctx1024": ("hbm", 0.60), "q8b_ctx8192": ("hbm", 0.60), "q8b_conc32": ("mfma", 0.40)}


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# algorithmic work (bytes and flops), counted from the shapes
# ----------------------------------------------------------------------------

def stage_work(spec, stage: str, rows: int, ctx_keys: int = 0):
    """(bytes, flops) of one launch of `stage` over `rows` activation rows.

    Bytes count every weight once (bf16), plus the injected context K/V read by
    attention as fp32 (4 bytes per element, the precision the path keeps it
    in), plus features read by the fusion.  Small activations are ignored.
    Flops count 2 per multiply-add."""
    H, I, V, d = spec.hidden, spec.intermediate, spec.vocab, spec.head_dim
    nq, nkv, fw = spec.n_q_heads, spec.n_kv_heads, spec.fused_width
    if stage == "lm_head":
        return V * H * 2, 2 * rows * H * V
    if stage == "gate_up":
        return 2 * I * H * 2, 2 * rows * H * 2 * I
    if stage == "down":
        return H * I * 2, 2 * rows * I * H
    if stage == "qkv":
        n = (nq + 2 * nkv) * d
        return n * H * 2, 2 * rows * H * n
    if stage == "oproj":
        return H * nq * d * 2, 2 * rows * nq * d * H
    if stage == "attention":
        # ctx_keys = sum over sequences of (context + block) keys
        return ctx_keys * nkv * d * 2 * 4, 4 * nq * d * spec.block * ctx_keys
    if stage == "fusion":
        return H * fw * 2 + rows * fw * 2, 2 * rows * fw * H
    if stage == "kv_proj":
        return 2 * nkv * d * H * 2, 2 * rows * H * 2 * nkv * d
    raise KeyError(stage)


def pass_work(spec):
    """Algorithmic (bytes, flops) of one further draft pass over the block
    (no appended rows): layers, attention over context + block, LM head."""
    B, n, L = spec.block, spec.n_seqs, spec.n_layers
    M = n * B
    keys = sum(c + B for c in spec.ctx_lens)
    by, fl = stage_work(spec, "lm_head", n * (B - 1))
    for st in ("qkv", "oproj", "gate_up", "down"):
        b, f = stage_work(spec, st, M)
        by, fl = by + L * b, fl + L * f
    b, f = stage_work(spec, "attention", M, keys)
    by, fl = by + L * b, fl + L * f
    by += L * 2 * spec.hidden * 2 + spec.hidden * 2
    return by, fl


def step_work(spec):
    """Algorithmic (bytes, flops) of one step (append B + draft + accept)."""
    B, n, L = spec.block, spec.n_seqs, spec.n_layers
    M = n * B
    keys = sum(c + B for c in spec.ctx_lens)
    by = fl = 0
    for st, r, times in (("fusion", M, 1), ("lm_head", n * (B - 1), 1)):
        b, f = stage_work(spec, st, r)
        by, fl = by + b * times, fl + f * times
    # context K/V projection of the appended rows: W_k/W_v are the same bytes
    # the block's q|k|v projection reads, so only its flops count here
    fl += L * stage_work(spec, "kv_proj", M)[1]
    for st in ("qkv", "oproj", "gate_up", "down"):
        b, f = stage_work(spec, st, M)
        by, fl = by + L * b, fl + L * f
    b, f = stage_work(spec, "attention", M, keys)
    by, fl = by + L * b, fl + L * f
    by += L * 2 * spec.hidden * 2 + spec.hidden * 2  # norm gains
    return by, fl


# ----------------------------------------------------------------------------
# GPU side
# ----------------------------------------------------------------------------

class Workload:
    def __init__(self, spec, weights, torch, B_, two_call=False, denoise_steps=1, temperature=0.0,
                 draft_only=False):
        self.spec, self.torch, self.B = spec, torch, B_
        self.two_call = two_call
        self.draft_only = draft_only
        self.denoise_steps = denoise_steps
        self.temperature = temperature
        I = _inputs()
        n, blk = spec.n_seqs, spec.block
        self.cfg = B_.Config.from_spec(spec, max_block=max(blk, 16))
        self.model = B_.Model(self.cfg, B_.upload_weights(spec, weights))
        self.ctx = B_.Context(self.model, list(spec.ctx_lens))
        self.ws = B_.workspace(self.model, n, blk, max(spec.ctx_lens) * n)
        # context: positions 0 .. c_b - B come from an initial ingest; the step
        # appends c_b - B .. c_b - 1 (the same rows every step).  Draft only:
        # every position is ingested up front and the step appends nothing.
        self.host_feats = [I.gen_features(spec, 1, b, c) for b, c in enumerate(spec.ctx_lens)]
        self.base = list(spec.ctx_lens) if draft_only else [c - blk for c in spec.ctx_lens]
        assert min(self.base) >= 0, "context shorter than a block"
        self._ingest([f[:c] for f, c in zip(self.host_feats, self.base)])
        step_rows = np.concatenate([f[c:] for f, c in zip(self.host_feats, self.base)], axis=0)
        self.step_feats = None if draft_only else self._dev_bf16(step_rows)
        self.anchors = torch.from_numpy(I.gen_anchors(spec, 2)).cuda()
        self.draft = torch.empty((n, blk - 1), dtype=torch.int32, device="cuda")
        self.accept = torch.empty(n, dtype=torch.int32, device="cuda")
        self.next_anchor = torch.empty(n, dtype=torch.int32, device="cuda")
        self.n_new = [blk] * n
        if temperature > 0:
            # the drafter's logits (q) and resident target logits (p): the
            # first pass's q plus N(0, 1/2) noise for the draft positions, and
            # N(0, 1) logits for the position after the block
            self.q_logits = torch.empty((n, blk - 1, spec.vocab), dtype=torch.float32, device="cuda")
            self.verify_ws = torch.empty(max(1, int(B_.lib().dflash_verify_workspace_bytes(n, blk, spec.vocab))),
                                         dtype=torch.uint8, device="cuda")
            self.p_logits = torch.empty((n, blk, spec.vocab), dtype=torch.float32, device="cuda")
        # target tokens: the first pass's drafts with a Geometric(p)-stopped
        # matched prefix, then uniformly random different tokens
        self.step()
        torch.cuda.synchronize()
        if temperature > 0:
            rng = np.random.default_rng(8)
            q = self.q_logits.cpu().numpy()
            p = np.concatenate([q + rng.normal(scale=0.5, size=q.shape).astype(np.float32),
                                rng.normal(size=(n, 1, spec.vocab)).astype(np.float32)], axis=1)
            self.p_logits.copy_(torch.from_numpy(p))
        K, r, bonus = I.gen_accept_construction(spec, 4)
        self.K = K
        tgt = I.make_targets(self.draft.cpu().numpy(), K, r, bonus, spec.vocab)
        self.target = torch.from_numpy(tgt).cuda()

    def _dev_bf16(self, bits):
        t = self.torch
        return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(t.bfloat16)

    def _ingest(self, feats):
        nonempty = [f for f in feats if f.shape[0]]
        dev = self._dev_bf16(np.concatenate(nonempty, axis=0)) if nonempty else None
        self.B.fuse_ctx(self.model, self.ctx, dev, [f.shape[0] for f in feats], self.ws)
        self.torch.cuda.synchronize()

    def step(self):
        B_, s = self.B, self.spec
        for b, c in enumerate(self.base):
            self.ctx.truncate(b, c)
        if self.temperature > 0:
            B_.step_sample(self.model, self.ctx, self.step_feats, self.n_new, self.anchors, s.block,
                           self.temperature, 1234, self.ws, draft=self.draft, logits=self.q_logits)
            if hasattr(self, "target"):
                B_.verify_sample(self.draft, self.q_logits, self.p_logits, s.block, self.temperature, 1234,
                                 ws=self.verify_ws, accept=self.accept, next_token=self.next_anchor)
            return
        if self.draft_only:
            B_.draft_block(self.model, self.ctx, self.anchors, s.block, self.ws, draft=self.draft)
        elif self.two_call:
            B_.fuse_ctx(self.model, self.ctx, self.step_feats, self.n_new, self.ws)
            B_.draft_block(self.model, self.ctx, self.anchors, s.block, self.ws, draft=self.draft)
        else:
            B_.step(self.model, self.ctx, self.step_feats, self.n_new, self.anchors, s.block, self.ws,
                    draft=self.draft)
        if self.denoise_steps > 1:
            B_.draft_refine(self.model, self.ctx, self.anchors, s.block, self.denoise_steps - 1, self.ws,
                            init_tokens=self.draft, draft=self.draft)
        if hasattr(self, "target"):
            B_.accept_len(self.draft, self.target, s.block, self.accept, self.next_anchor)

    def logits(self):
        t = self.torch
        s = self.spec
        for b, c in enumerate(self.base):
            self.ctx.truncate(b, c)
        if not self.draft_only:
            self.B.fuse_ctx(self.model, self.ctx, self.step_feats, self.n_new, self.ws)
        lg = t.empty((s.n_seqs, s.block - 1, s.vocab), dtype=t.float32, device="cuda")
        d = self.B.draft_block(self.model, self.ctx, self.anchors, s.block, self.ws, logits=lg)
        t.cuda.synchronize()
        return d.cpu().numpy(), lg.cpu().numpy()


class TrainWorkload:
    """Training-attention forward: every sequence's full context ingested,
    then train_blocks anchored blocks per sequence drafted in one call."""

    def __init__(self, spec, weights, torch, B_):
        self.spec, self.torch, self.B = spec, torch, B_
        I = _inputs()
        blk = spec.block
        self.denoise_steps = 1
        self.bseq, self.apos = [], []
        for b, T in enumerate(spec.ctx_lens):
            a = I.gen_train_anchors(T, spec.train_blocks, blk, seed=10 + b, prompt_len=spec.prompt_len)
            self.bseq += [b] * len(a)
            self.apos += [int(v) for v in a]
        self.n_blocks = len(self.bseq)
        self.cfg = B_.Config.from_spec(spec, max_block=max(blk, 16))
        self.model = B_.Model(self.cfg, B_.upload_weights(spec, weights))
        self.ctx = B_.Context(self.model, list(spec.ctx_lens))
        self.ws = B_.workspace(self.model, max(self.n_blocks, spec.n_seqs), blk, sum(spec.ctx_lens))
        self.host_feats = [I.gen_features(spec, 1, b, c) for b, c in enumerate(spec.ctx_lens)]
        self.feats = torch.from_numpy(np.ascontiguousarray(np.concatenate(self.host_feats, 0)).view(np.int16)) \
            .cuda().view(torch.bfloat16)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(6, spawn_key=(9,))))
        self.anchor_tok = rng.integers(0, spec.vocab - 1, size=self.n_blocks).astype(np.int32)
        self.anchors = torch.from_numpy(self.anchor_tok).cuda()
        self.draft = torch.empty((self.n_blocks, blk - 1), dtype=torch.int32, device="cuda")
        self.n_new = list(spec.ctx_lens)

    def step(self, logits=None):
        B_, s = self.B, self.spec
        for b in range(s.n_seqs):
            self.ctx.truncate(b, 0)
        B_.fuse_ctx(self.model, self.ctx, self.feats, self.n_new, self.ws)
        B_.draft_anchored(self.model, self.ctx, self.bseq, self.apos, self.anchors, s.block, self.ws,
                          draft=self.draft, logits=logits)

    def logits(self, blocks):
        t = self.torch
        lg = t.empty((self.n_blocks, self.spec.block - 1, self.spec.vocab), dtype=t.float32, device="cuda")
        self.step(logits=lg)
        t.cuda.synchronize()
        out = lg[blocks].cpu().numpy(), self.draft[blocks].cpu().numpy()
        del lg
        return out


class IngestWorkload:
    """The ingest phase: every sequence's whole context ingested from its
    target features (fusion + every layer's K/V into the cache) in one call."""

    def __init__(self, spec, weights, torch, B_):
        self.spec, self.torch, self.B = spec, torch, B_
        I = _inputs()
        self.denoise_steps = 1
        self.cfg = B_.Config.from_spec(spec, max_block=max(spec.block, 16))
        self.model = B_.Model(self.cfg, B_.upload_weights(spec, weights))
        self.ctx = B_.Context(self.model, list(spec.ctx_lens))
        self.ws = B_.workspace(self.model, spec.n_seqs, spec.block, sum(spec.ctx_lens))
        packed = np.concatenate([I.gen_features(spec, 1, b, c) for b, c in enumerate(spec.ctx_lens)], axis=0)
        self.feats = torch.from_numpy(np.ascontiguousarray(packed).view(np.int16)).cuda().view(torch.bfloat16)
        del packed
        self.n_new = list(spec.ctx_lens)

    def step(self):
        for b in range(self.spec.n_seqs):
            self.ctx.truncate(b, 0)
        self.B.fuse_ctx(self.model, self.ctx, self.feats, self.n_new, self.ws)


def ingest_work(spec):
    """Algorithmic (bytes, flops) of ingesting every context position: W_fc
    and the features, every layer's W_k / W_v, the K/V written to the cache
    (fp32-equivalent, 8 bytes per K and V element pair)."""
    T, L = sum(spec.ctx_lens), spec.n_layers
    fb, ff = stage_work(spec, "fusion", T)
    kb, kf = stage_work(spec, "kv_proj", T)
    return fb + L * kb + T * L * spec.n_kv_heads * spec.head_dim * 8, ff + L * kf


def _decode_rows(wl, stage: str) -> int:
    """Activation rows of one launch of `stage` (per layer for layer stages)."""
    s = wl.spec
    n = wl.n_blocks if isinstance(wl, TrainWorkload) else s.n_seqs
    if stage == "lm_head":
        return n * (s.block - 1)
    if stage in ("fusion", "kv_proj") and isinstance(wl, (TrainWorkload, IngestWorkload)):
        return sum(s.ctx_lens)
    return n * s.block


def lm_head_executed_flops(spec, n_blocks: int) -> float:
    """bf16 matrix-core flops one LM-head launch executes: every padded block
    row (anchor rows and row padding included: 16-row groups up to 32 rows,
    128-row groups above) against every vocabulary column, and two bf16
    products per multiply-add (the activations are hi/lo pairs)."""
    m = n_blocks * spec.block
    mp = (m + 15) // 16 * 16 if m <= 32 else (m + 127) // 128 * 128
    return 2.0 * 2.0 * mp * spec.vocab * spec.hidden


def stage_total(wl, stage: str):
    """Algorithmic (bytes, flops) of every launch of `stage` in one step."""
    s = wl.spec
    S = wl.denoise_steps
    rows = _decode_rows(wl, stage)
    if stage == "attention":
        if isinstance(wl, TrainWorkload):
            # the shared context is read once (bytes); each block attends to
            # its prefix and itself (flops)
            kb = sum(s.ctx_lens) + wl.n_blocks * s.block
            kf = sum(a + s.block for a in wl.apos)
        else:
            kb = kf = sum(c + s.block for c in s.ctx_lens)
        b, _ = stage_work(s, "attention", rows, kb)
        _, f = stage_work(s, "attention", rows, kf)
    else:
        b, f = stage_work(s, stage, rows)
    if stage not in ("lm_head", "fusion"):
        b, f = b * s.n_layers, f * s.n_layers
    if stage not in ("fusion", "kv_proj"):
        b, f = b * S, f * S
    return b, f


def train_step_work(wl):
    """Algorithmic (bytes, flops) of one training-forward step: ingest of every
    position (fusion + all layers' K/V), then the anchored pass."""
    by = fl = 0
    for st in ("fusion", "kv_proj", "qkv", "oproj", "gate_up", "down", "attention", "lm_head"):
        b, f = stage_total(wl, st)
        if st in ("qkv", "kv_proj"):
            # W_k / W_v bytes are shared by the ingest and the block pass
            b = b if st == "qkv" else 0
        by, fl = by + b, fl + f
    s = wl.spec
    by += s.n_layers * 2 * s.hidden * 2 + s.hidden * 2
    return by, fl


def measured_traffic(workload: str, stage: str):
    """HBM bytes per launch of `stage` from the committed rocprofv3 counter
    summary for this workload, if there is one and the kernel sources have not
    changed since it was taken; else None."""
    from block_diffusion_drafting_pass_amd import profsum
    got = profsum.read_traffic(os.path.join(ROOT, "profiles", f"{stage}_{workload}_traffic.txt"))
    if got is None or got[1] != profsum.kernel_sources_sha256():
        return None
    return got[0]


def copy_bandwidth(torch, nbytes=1 << 30, reps=10) -> float:
    """Achieved device-to-device copy bandwidth (read + write bytes / s), GB/s."""
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del x, y
    return 2 * nbytes / (ms * 1e-3) / 1e9


def time_steps(torch, run, steps: int):
    """Mean ms per step over `steps` back-to-back calls, bracketed by two events."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, (time.perf_counter() - w0) / steps * 1e3


def step_spread(torch, run, steps: int):
    """p10 / p50 / p90 of the per-step time (ms), one event between every two
    steps (a separate loop, so the headline timing carries no extra events)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        run()
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    return {"p10_ms": round(float(np.percentile(t, 10)), 4), "p50_ms": round(float(np.percentile(t, 50)), 4),
            "p90_ms": round(float(np.percentile(t, 90)), 4)}


def measured_counters(workload: str):
    """(executed bf16 flops per draft pass, MFMA busy share) from the committed
    rocprofv3 counter summary of this workload's draft pass, while the kernel
    sources are unchanged since it was taken; else None."""
    from block_diffusion_drafting_pass_amd import profsum
    got = profsum.read_counters(os.path.join(ROOT, "profiles", f"mfma_{workload}_counters.txt"))
    if got is None or got[2] != profsum.kernel_sources_sha256():
        return None
    return got[0], got[1]


def host_description() -> str:
    """CPU model and the BLAS library numpy runs on (for the oracle baseline)."""
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown BLAS"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api', '?')} {libs[0].get('version', '')}".strip()
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass
    return f"CPU {cpu}, BLAS {blas}"


# ----------------------------------------------------------------------------
# CPU oracle baseline
# ----------------------------------------------------------------------------

def _inputs():
    from block_diffusion_drafting_pass_amd import inputs as I
    return I


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        n = [i.get("num_threads", 0) for i in info if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(spec, weights, ws_target_s=10.0, max_reps=8, draft_only=False):
    """The oracle's step (append B, draft, accept; draft_only: draft, accept
    over the whole context) on one sequence, timed on the host cores until
    about ws_target_s seconds of work (1..max_reps steps)."""
    from oracle import dflash_oracle as O
    I = _inputs()
    sub = spec.with_(ctx_lens=spec.ctx_lens[:1])
    blk, c = sub.block, sub.ctx_lens[0]
    model = O.OracleModel.from_spec(sub, weights)
    ctx = O.OracleContext(model, 1)
    feats = I.gen_features(spec, 1, 0, c)
    anchors = I.gen_anchors(spec, 2)[:1]
    base = c if draft_only else c - blk
    t0 = time.perf_counter()
    O.fuse_ctx(model, ctx, 0, feats[:base])
    log(f"oracle ingest of {base} positions: {time.perf_counter() - t0:.1f} s")
    times, res = [], None
    while len(times) < max_reps and sum(times) < ws_target_s:
        O.truncate_ctx(ctx, 0, base)
        t0 = time.perf_counter()
        if not draft_only:
            O.fuse_ctx(model, ctx, 0, feats[base:])
        res = O.draft_block(model, ctx, anchors, blk)
        K, r, bonus = I.gen_accept_construction(sub, 4, n_seqs=1)
        O.accept_len(res.drafts, I.make_targets(res.drafts, K, r, bonus, sub.vocab))
        times.append(time.perf_counter() - t0)
        log(f"oracle step {len(times)}: {times[-1]:.2f} s")
    t = float(np.median(times))
    return {
        "value": (blk - 1) / t,
        "unit": "draft tokens/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": (f"{len(times)} oracle step(s) of sequence 0 ({'' if draft_only else f'append {blk}, '}draft, "
                   f"accept; context {c}), "
                   f"numpy float64, median {t:.2f} s/step; {len(os.sched_getaffinity(0))} host CPUs visible, "
                   f"{host_description()}"),
    }, res


def cpu_baseline_ingest(spec, weights, max_pos=512):
    """The oracle's ingest of the first max_pos positions of sequence 0."""
    from oracle import dflash_oracle as O
    I = _inputs()
    sub = spec.with_(ctx_lens=spec.ctx_lens[:1])
    model = O.OracleModel.from_spec(sub, weights)
    T = min(spec.ctx_lens[0], max_pos)
    feats = I.gen_features(spec, 1, 0, T)
    times = []
    while len(times) < 3 and sum(times) < 10.0:
        ctx = O.OracleContext(model, 1)
        t0 = time.perf_counter()
        O.fuse_ctx(model, ctx, 0, feats)
        times.append(time.perf_counter() - t0)
        log(f"oracle ingest of {T} positions: {times[-1]:.2f} s")
    t = float(np.median(times))
    return {
        "value": T / t,
        "unit": "ingested positions/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": (f"{len(times)} oracle ingest(s) of the first {T} positions of sequence 0 (fusion + every layer's "
                   f"K/V), numpy float64, median {t:.2f} s; {len(os.sched_getaffinity(0))} host CPUs visible, "
                   f"{host_description()}"),
    }


def cpu_baseline_train(spec, weights, wl, n_blk=2):
    """The oracle on sequence 0 of a training-forward workload: its ingest,
    then n_blk of its anchored blocks, extrapolated to all of its blocks."""
    from oracle import dflash_oracle as O
    I = _inputs()
    sub = spec.with_(ctx_lens=spec.ctx_lens[:1])
    model = O.OracleModel.from_spec(sub, weights)
    ctx = O.OracleContext(model, 1)
    T, blk = spec.ctx_lens[0], spec.block
    t0 = time.perf_counter()
    O.fuse_ctx(model, ctx, 0, I.gen_features(spec, 1, 0, T))
    t_ing = time.perf_counter() - t0
    log(f"oracle ingest of {T} positions: {t_ing:.1f} s")
    sel = [j for j in range(wl.n_blocks) if wl.bseq[j] == 0][:n_blk]
    t0 = time.perf_counter()
    res = O.draft_anchored(model, ctx, [0] * len(sel), [wl.apos[j] for j in sel], wl.anchor_tok[sel], blk)
    t_blk = time.perf_counter() - t0
    log(f"oracle anchored pass over {len(sel)} blocks: {t_blk:.1f} s")
    per_seq = t_ing + spec.train_blocks / len(sel) * t_blk
    return {
        "value": spec.train_blocks * (blk - 1) / per_seq,
        "unit": "drafted positions/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": (f"sequence 0: ingest of {T} positions ({t_ing:.1f} s) and {len(sel)} of its "
                   f"{spec.train_blocks} anchored blocks ({t_blk:.1f} s), extrapolated to all its blocks; numpy "
                   f"float64; {len(os.sched_getaffinity(0))} host CPUs visible, "
                   f"{host_description()}"),
    }, res, sel


# ----------------------------------------------------------------------------

def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="q8b_ctx1024",
                    help="tiny | q8b_ctx1024 (default) | q8b_ctx8192 | q8b_conc32 | q8b_l3_b32_ragged")
    ap.add_argument("--probe", default="lm_head", help="stage whose launches are timed for the roofline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--breakdown", action="store_true", help="also time every stage (extra passes)")
    ap.add_argument("--two-call", action="store_true",
                    help="step as dflash_fuse_ctx + dflash_draft_block instead of the fused dflash_step")
    ap.add_argument("--denoise-steps", type=int, default=1,
                    help="draft passes per block (1 = the single-pass drafter)")
    ap.add_argument("--phase", choices=("decode", "draft", "ingest"), default="decode",
                    help="decode: the steady-state step, append + draft + accept (default); draft: the draft "
                         "pass + accept alone over a resident context; ingest: whole-context ingest of every "
                         "sequence")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="sampled drafts at this temperature, verified losslessly (0 = greedy)")
    ap.add_argument("--no-pack", action="store_true",
                    help="stream the row-major weights instead of the packed copy (dflash_model_pack)")
    ap.add_argument("--block", type=int, default=0,
                    help="block size B (anchor + B - 1 masks) in place of the workload's own; the metric then "
                         "names it and no pass target is reported (the aims are stated at the workload's block)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step as one captured HIP graph (identical steps, so identical work)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the draft pass is built and "
              "measured on a single MI355X, with no multi-GPU path.", file=sys.stderr)
        return 2

    import torch
    from block_diffusion_drafting_pass_amd import binding as B_
    I = _inputs()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    B_.lib()  # fails loudly when the HIP library is missing
    torch.cuda.set_device(0)

    spec = I.spec(args.workload)
    block_override = args.block > 0 and args.block != spec.block
    if args.block > 0:
        if args.block < 2 or args.block > 64:
            print("--block must be in [2, 64]", file=sys.stderr)
            return 2
        spec = spec.with_(block=args.block)
    log(f"workload {spec.name}: layers {spec.n_layers}, ctx {spec.ctx_lens[:4]}..., "
        f"{spec.n_seqs} seqs, block {spec.block}")
    t0 = time.perf_counter()
    weights = I.gen_weights(spec, seed=0)
    log(f"weights generated in {time.perf_counter() - t0:.1f} s")
    copy_gbs = copy_bandwidth(torch)
    log(f"device copy bandwidth {copy_gbs:.0f} GB/s")

    S = args.denoise_steps
    if S < 1 or S > 65:
        print("--denoise-steps must be in [1, 65]", file=sys.stderr)
        return 2
    train = spec.train_blocks > 0
    ingest = args.phase == "ingest"
    if ingest and (train or S > 1 or args.two_call or args.temperature > 0 or args.graph):
        print("--phase ingest takes a decode workload and none of --denoise-steps, --two-call, --temperature, "
              "--graph", file=sys.stderr)
        return 2
    if ingest and args.probe == "lm_head":
        args.probe = "fusion"
    if train and (S > 1 or args.two_call or args.temperature > 0):
        print("--denoise-steps, --two-call and --temperature apply to decode workloads only", file=sys.stderr)
        return 2
    draft_only = args.phase == "draft"
    if draft_only and (train or S > 1 or args.two_call or args.temperature > 0):
        print("--phase draft takes a decode workload and none of --denoise-steps, --two-call, --temperature",
              file=sys.stderr)
        return 2
    if args.temperature > 0 and (S > 1 or args.two_call):
        print("--temperature combines with neither --denoise-steps nor --two-call", file=sys.stderr)
        return 2
    if ingest:
        wl = IngestWorkload(spec, weights, torch, B_)
    elif train:
        wl = TrainWorkload(spec, weights, torch, B_)
    else:
        wl = Workload(spec, weights, torch, B_, two_call=args.two_call, denoise_steps=S,
                      temperature=args.temperature, draft_only=draft_only)
    if not args.no_pack:
        # one-time layout copy of the streamed weights, outside the timed region
        # like the weight upload itself (results are bitwise identical)
        wl.model.pack()
        torch.cuda.synchronize()
        log(f"packed weight copy: {wl.model.pack_bytes() / 1e9:.2f} GB")
    log("workload resident; warming up")
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()

    n_launch = 64 * S if (train or ingest) else {"lm_head": S, "fusion": 1}.get(args.probe, spec.n_layers * S)
    run = wl.step
    if args.graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            wl.step()
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        run = g.replay
    # the headline: K steps between two events, nothing else recorded
    ms_step, wall_ms = time_steps(torch, run, args.steps)
    log(f"{args.steps} steps: {ms_step:.3f} ms/step (wall {wall_ms:.3f} ms/step)")
    spread = step_spread(torch, run, args.steps)
    log(f"per-step spread over another {args.steps} steps: {spread}")
    # the dominant kernel: library events around its launches, on eager steps
    # of their own (the probe's events are not captured into graphs)
    B_.probe_arm(wl.model, args.probe, n_launch * args.steps)
    for _ in range(args.steps):
        wl.step()
    probe_ms, probe_n, probe_missed = B_.probe_read(wl.model)

    # the draft pass alone over the resident context (phase D): after one step
    # every context position is ingested; each iteration is dflash_draft_block
    # + dflash_accept_len, which change no length
    phase_d = None
    decode = not (train or ingest)
    if decode and not draft_only and S == 1 and args.temperature == 0:
        wl.step()

        def run_d():
            B_.draft_block(wl.model, wl.ctx, wl.anchors, spec.block, wl.ws, draft=wl.draft)
            B_.accept_len(wl.draft, wl.target, spec.block, wl.accept, wl.next_anchor)

        for _ in range(args.warmup):
            run_d()
        d_ms, _ = time_steps(torch, run_d, args.steps)
        phase_d = {"ms_per_step": round(d_ms, 4), **step_spread(torch, run_d, args.steps)}
        log(f"draft pass alone: {d_ms:.3f} ms/step; {phase_d}")
    elif decode and draft_only:
        phase_d = {"ms_per_step": round(ms_step, 4), **spread}

    n, blk = spec.n_seqs, spec.block
    n_units = wl.n_blocks if train else n
    draft_tok_s = n_units * (blk - 1) / (ms_step * 1e-3)
    if ingest:
        draft_tok_s = sum(spec.ctx_lens) / (ms_step * 1e-3)
        by, fl = ingest_work(spec)
    elif train:
        by, fl = train_step_work(wl)
    elif draft_only:
        by, fl = pass_work(spec)
    else:
        by, fl = step_work(spec)
        if S > 1:
            pb_, pf_ = pass_work(spec)
            by, fl = by + (S - 1) * pb_, fl + (S - 1) * pf_

    # the probed stage's algorithmic work per launch: its per-step total over
    # the launches one step makes
    tb, tf = stage_total(wl, args.probe)
    per_step = max(probe_n, 1) / args.steps
    pb, pf = tb / per_step, tf / per_step
    avg_ms = probe_ms / max(probe_n, 1)
    ai = pf / pb
    ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai < ridge:
        achieved = pb / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = pf / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4)}
    roof.update({"traffic": measured_traffic(spec.name, args.probe), "kernel": args.probe,
                 "avg_launch_ms": round(avg_ms, 4), "launches_timed": probe_n, "alg_bytes_per_launch": pb,
                 "alg_flops_per_launch": pf})
    if args.probe == "lm_head":
        # what the matrix cores execute: with hi/lo activations and padded rows
        # a launch of a few hundred rows sits above the ridge though its
        # algorithmic intensity is below it
        ef = lm_head_executed_flops(spec, n_units)
        roof["executed"] = {"flops_per_launch": ef, "intensity": round(ef / pb, 1),
                            "bound": "mfma" if ef / pb >= ridge else "hbm",
                            "mfma_frac": round(ef / (avg_ms * 1e-3) / (MFMA_BF16_PEAK_TFS * 1e12), 4)}

    pass_target = None
    if phase_d is not None:
        pbd, pfd = pass_work(spec)
        t_d = phase_d["ms_per_step"] * 1e-3
        phase_d.update({"draft_tok_s": round(n * (blk - 1) / t_d, 1), "alg_bytes": pbd, "alg_flops": pfd,
                        "hbm_frac": round(pbd / t_d / (HBM_PEAK_GBS * 1e9), 4),
                        "mfma_frac": round(pfd / t_d / (MFMA_BF16_PEAK_TFS * 1e12), 5)})
        ctr = measured_counters(spec.name)
        phase_d["exec_mfma_frac"] = None if ctr is None else round(ctr[0] / t_d / (MFMA_BF16_PEAK_TFS * 1e12), 4)
        phase_d["mfma_busy"] = None if ctr is None else round(ctr[1], 4)
        if spec.name in PASS_TARGETS and not block_override:
            bound, aim = PASS_TARGETS[spec.name]
            frac = phase_d["hbm_frac"] if bound == "hbm" else phase_d["mfma_frac"]
            pass_target = {"phase": "D (draft pass + accept over a resident context)", "bound": bound,
                           "frac": frac, "target": aim, "met": bool(frac >= aim)}

    breakdown = None
    if args.breakdown:
        # per step: event-bracketed time of every launch of the stage (a stage
        # may be one launch per layer or one for all layers), its algorithmic
        # bytes and flops over all layers
        breakdown = {}
        reps = 10
        for st in (("fusion", "kv_proj") if ingest else
                   ("qkv", "attention", "oproj", "gate_up", "down", "lm_head", "fusion", "kv_proj")):
            B_.probe_arm(wl.model, st, 64 * S * reps)
            for _ in range(reps):
                wl.step()
            ms, cnt, _ = B_.probe_read(wl.model)
            if cnt == 0:  # e.g. the context K/V projection inside a fused dflash_step
                breakdown[st] = {"us_per_step": 0.0, "launches_per_step": 0}
                continue
            b_, f_ = stage_total(wl, st)
            st_ms = ms / reps
            breakdown[st] = {"us_per_step": round(st_ms * 1e3, 1), "launches_per_step": cnt // reps,
                             "GB_s": round(b_ / (st_ms * 1e-3) / 1e9, 1),
                             "TFLOP_s": round(f_ / (st_ms * 1e-3) / 1e12, 2)}
        log(f"breakdown: {json.dumps(breakdown)}")

    cpu = None
    parity = None
    if not args.no_cpu and ingest:
        log("timing the CPU oracle on the host cores")
        cpu = cpu_baseline_ingest(spec, weights)
    elif not args.no_cpu and train:
        log("timing the CPU oracle on the host cores")
        cpu, ref, sel = cpu_baseline_train(spec, weights, wl)
        lg_gpu, d_gpu = wl.logits(sel)
        from oracle import dflash_oracle as O
        sure = O.top2_gap(ref.logits) > 0.05
        parity = {"blocks": sel, "max_abs_logit_err": float(np.max(np.abs(lg_gpu - ref.logits))),
                  "drafts_equal_on_decided_rows": bool(np.all((d_gpu == ref.drafts)[sure])),
                  "decided_rows": int(sure.sum())}
        log(f"parity vs oracle (sequence 0, blocks {sel}): {parity}")
    elif not args.no_cpu:
        d_gpu, lg_gpu = wl.logits()
        log("timing the CPU oracle on the host cores")
        cpu, ref = cpu_baseline(spec, weights, draft_only=draft_only)
        from oracle import dflash_oracle as O
        sure = O.top2_gap(ref.logits) > 0.05
        parity = {"seq": 0, "max_abs_logit_err": float(np.max(np.abs(lg_gpu[:1] - ref.logits))),
                  "drafts_equal_on_decided_rows": bool(np.all((d_gpu[:1] == ref.drafts)[sure])),
                  "decided_rows": int(sure.sum())}
        log(f"parity vs oracle (sequence 0): {parity}")

    if ingest:
        metric = (f"context ingest: positions/sec (fusion + {spec.n_layers} layers' injected K/V), "
                  f"{n} x {spec.ctx_lens[0]} positions")
        workload = (f"{spec.name}: {spec.n_layers}-layer drafter, hidden {spec.hidden}, {spec.n_kv_heads} kv heads x "
                    f"{spec.head_dim}, fusion {spec.fused_width}->{spec.hidden}; {n} sequence(s) of "
                    f"{list(spec.ctx_lens)[:4]}{'...' if n > 4 else ''} positions; step = ingest every position "
                    f"(dflash_fuse_ctx)")
    elif train:
        metric = (f"training-attention forward: drafted positions/sec ({spec.train_blocks} anchored blocks of "
                  f"{blk} per sequence), {spec.n_layers}-layer, {n} x {spec.ctx_lens[0]} context")
        workload = (f"{spec.name}: {spec.n_layers}-layer drafter, hidden {spec.hidden}, "
                    f"{spec.n_q_heads}/{spec.n_kv_heads} heads x {spec.head_dim}, SwiGLU {spec.intermediate}, "
                    f"vocab {spec.vocab}, fusion {spec.fused_width}->{spec.hidden}; {n} training sequence(s) of "
                    f"{list(spec.ctx_lens)} positions (prompt {spec.prompt_len}), {wl.n_blocks} anchored blocks "
                    f"of {blk}; step = ingest every position + one anchored draft pass (dflash_fuse_ctx + "
                    f"dflash_draft_anchored)")
    else:
        metric = METRIC if not block_override else METRIC.replace("block 16", f"block {blk}")
        workload = (f"{spec.name}: {spec.n_layers}-layer drafter, hidden {spec.hidden}, "
                    f"{spec.n_q_heads}/{spec.n_kv_heads} heads x {spec.head_dim}, SwiGLU {spec.intermediate}, "
                    f"vocab {spec.vocab}, fusion {spec.fused_width}->{spec.hidden}; {n} sequence(s), "
                    f"context {spec.ctx_lens[0] if n == 1 else list(spec.ctx_lens)}, block {blk}; "
                    + (f"step = draft pass + accept scan over the resident context (dflash_draft_block + "
                       f"dflash_accept_len)" if draft_only else
                       f"step = append {blk} verified positions + draft pass + accept scan"
                       f"{' (two calls)' if args.two_call else ' (dflash_step)'}") +
                    f"{f' + {S - 1} refinement pass(es)' if S > 1 else ''}"
                    f"{f'; drafts sampled at temperature {args.temperature} and verified losslessly' if args.temperature > 0 else ''}")
    out = {
        "metric": metric,
        "value": round(draft_tok_s, 1),
        "unit": "ingested positions/s" if ingest else ("drafted positions/s" if train else "draft tokens/s"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "global_batch": n_units if train else n,
            "block": blk,
            "denoise_steps": S,
            "temperature": args.temperature,
            "seq_len": max(spec.ctx_lens),
            "parallelism": "single GPU",
            "packed_weights": not args.no_pack,
        },
        "step_spread": spread,
        "phase_d": phase_d,
        "pass_target": pass_target,
        "blocks_per_s": round(n_units / (ms_step * 1e-3), 1),
        "step_alg_bytes": by,
        "step_alg_flops": fl,
        "step_hbm_frac": round(by / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
        "step_mfma_frac": round(fl / (ms_step * 1e-3) / (MFMA_BF16_PEAK_TFS * 1e12), 5),
        "copy_bw_GBps": round(copy_gbs, 1),
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity_seq0": parity,
    }
    if breakdown is not None:
        out["breakdown"] = breakdown
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
