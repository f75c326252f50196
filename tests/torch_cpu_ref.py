"""A second formulation of the draft pass built from torch library routines
(float64, CPU), used only to pin the numpy oracle.

It differs from the oracle in every step that could hide a mistake:
RMSNorm is ``torch.nn.functional.rms_norm``; RoPE is a complex multiplication
(x_j + i x_{j+d/2}) * exp(i p w_j) via ``torch.polar``; attention is
``scaled_dot_product_attention`` with ``enable_gqa`` (its own head grouping);
the MLP uses ``F.silu``; linear maps use ``F.linear`` on [out][in] weights.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def _t(bits) -> torch.Tensor:
    b = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).astype(np.int32) << 16)
    return b.view(torch.float32).to(torch.float64)


def _rope_complex(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    # x: [heads][P][d]
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-torch.arange(0, half, dtype=torch.float64) * 2.0 / d)
    ang = pos.to(torch.float64)[:, None] * inv[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)  # e^{i angle}
    z = torch.complex(x[..., :half], x[..., half:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def torch_draft(cfg, weights, features, anchors, block, use_rope=True):
    """features[b]: [c_b][L_t*H] bf16 bits.  Returns (logits [n][B-1][V], drafts)."""
    nq, nkv, d, H = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.hidden
    W = {k: _t(v) for k, v in weights.items()}
    eps = cfg.rms_eps
    out_logits = []
    for b, anchor in enumerate(anchors):
        fe = _t(features[b]) if len(features[b]) else torch.zeros(0, cfg.n_target_layers * H, dtype=torch.float64)
        c = fe.shape[0]
        h = F.linear(fe, W["w_fc"])
        ctx_k, ctx_v = [], []
        for l in range(cfg.n_layers):
            k = F.linear(h, W[f"layers.{l}.wk"]).view(c, nkv, d).transpose(0, 1)
            v = F.linear(h, W[f"layers.{l}.wv"]).view(c, nkv, d).transpose(0, 1)
            if use_rope:
                k = _rope_complex(k, torch.arange(c), cfg.rope_theta)
            ctx_k.append(k)
            ctx_v.append(v)
        toks = torch.tensor([int(anchor)] + [cfg.mask_token_id] * (block - 1))
        x = W["embed"][toks]
        pos = torch.arange(c, c + block)
        for l in range(cfg.n_layers):
            p = f"layers.{l}."
            u = F.rms_norm(x, (H,), weight=W[p + "attn_norm"], eps=eps)
            q = F.linear(u, W[p + "wq"]).view(block, nq, d).transpose(0, 1)
            k = F.linear(u, W[p + "wk"]).view(block, nkv, d).transpose(0, 1)
            v = F.linear(u, W[p + "wv"]).view(block, nkv, d).transpose(0, 1)
            if use_rope:
                q = _rope_complex(q, pos, cfg.rope_theta)
                k = _rope_complex(k, pos, cfg.rope_theta)
            keys = torch.cat([ctx_k[l], k], dim=1)
            vals = torch.cat([ctx_v[l], v], dim=1)
            o = F.scaled_dot_product_attention(q[None], keys[None], vals[None], enable_gqa=(nq != nkv))[0]
            x = x + F.linear(o.transpose(0, 1).reshape(block, nq * d), W[p + "wo"])
            w = F.rms_norm(x, (H,), weight=W[p + "mlp_norm"], eps=eps)
            x = x + F.linear(F.silu(F.linear(w, W[p + "wgate"])) * F.linear(w, W[p + "wup"]), W[p + "wdown"])
        y = F.rms_norm(x[1:], (H,), weight=W["final_norm"], eps=eps)
        out_logits.append(F.linear(y, W["embed"]).numpy())
    logits = np.stack(out_logits)
    return logits, logits.argmax(-1)


def torch_anchored(cfg, weights, features, block_seq, anchor_pos, anchors, block):
    """Anchored blocks (training attention) as one packed sequence: every
    sequence's context rows, then every block's rows, through each layer in a
    single SDPA call whose boolean mask lets a row of block j see its own
    block and the rows of sequence block_seq[j]'s context before
    anchor_pos[j].  Context positions are keys only: their K/V come from the
    target features, not from a layer input.  Returns (logits [n][B-1][V],
    drafts)."""
    nq, nkv, d, H = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.hidden
    W = {k: _t(v) for k, v in weights.items()}
    eps = cfg.rms_eps
    n = len(block_seq)
    lens = [len(f) for f in features]
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    C = int(starts[-1])
    # context K/V of every sequence, packed: rows starts[s] .. starts[s+1]
    fe = torch.cat([_t(f) if len(f) else torch.zeros(0, cfg.n_target_layers * H, dtype=torch.float64)
                    for f in features], 0)
    h = F.linear(fe, W["w_fc"])
    ctx_pos = torch.cat([torch.arange(c) for c in lens]) if C else torch.zeros(0, dtype=torch.long)
    toks = torch.full((n, block), cfg.mask_token_id, dtype=torch.long)
    toks[:, 0] = torch.as_tensor(np.asarray(anchors, dtype=np.int64))
    x = W["embed"][toks.reshape(-1)]                     # [n*B][H]
    blk_pos = torch.cat([torch.arange(int(a), int(a) + block) for a in anchor_pos])
    R = n * block
    mask = torch.zeros(R, C + R, dtype=torch.bool)
    for j in range(n):
        rows = slice(j * block, (j + 1) * block)
        s0 = int(starts[int(block_seq[j])])
        mask[rows, s0: s0 + int(anchor_pos[j])] = True
        mask[rows, C + j * block: C + (j + 1) * block] = True
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        ck = F.linear(h, W[p + "wk"]).view(C, nkv, d).transpose(0, 1)
        cv = F.linear(h, W[p + "wv"]).view(C, nkv, d).transpose(0, 1)
        ck = _rope_complex(ck, ctx_pos, cfg.rope_theta)
        u = F.rms_norm(x, (H,), weight=W[p + "attn_norm"], eps=eps)
        q = _rope_complex(F.linear(u, W[p + "wq"]).view(R, nq, d).transpose(0, 1), blk_pos, cfg.rope_theta)
        k = _rope_complex(F.linear(u, W[p + "wk"]).view(R, nkv, d).transpose(0, 1), blk_pos, cfg.rope_theta)
        v = F.linear(u, W[p + "wv"]).view(R, nkv, d).transpose(0, 1)
        keys = torch.cat([ck, k], dim=1)
        vals = torch.cat([cv, v], dim=1)
        o = F.scaled_dot_product_attention(q[None], keys[None], vals[None], attn_mask=mask[None, None],
                                           enable_gqa=(nq != nkv))[0]
        x = x + F.linear(o.transpose(0, 1).reshape(R, nq * d), W[p + "wo"])
        w = F.rms_norm(x, (H,), weight=W[p + "mlp_norm"], eps=eps)
        x = x + F.linear(F.silu(F.linear(w, W[p + "wgate"])) * F.linear(w, W[p + "wup"]), W[p + "wdown"])
    x = x.view(n, block, H)
    y = F.rms_norm(x[:, 1:], (H,), weight=W["final_norm"], eps=eps)
    logits = F.linear(y, W["embed"]).numpy()
    return logits, logits.argmax(-1)
