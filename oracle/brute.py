"""Scalar-loop evaluation of the DFlash draft pass for tiny shapes.

TEST INFRASTRUCTURE ONLY.  This is a second, independent evaluation of the
same function as ``dflash_oracle`` (see that module's header for the pages it
follows and the readings it takes), written with Python floats, explicit index
loops and the ``math`` module only: no numpy in the arithmetic, no shared
helpers.  It exists to pin ``dflash_oracle``: a dropped term, a wrong sign, a
transposed operand or a wrong head mapping in either shows up as a mismatch.
It is far too slow for anything but a few hundred weights.
"""
from __future__ import annotations

import math
import struct
from typing import Dict, List, Sequence


def _bf16(bits) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _mat(weights, name) -> List[List[float]]:
    w = weights[name]
    return [[_bf16(w[i][j]) for j in range(len(w[0]))] for i in range(len(w))]


def _vec(weights, name) -> List[float]:
    return [_bf16(b) for b in weights[name]]


def _matvec(W: List[List[float]], x: List[float]) -> List[float]:
    out = []
    for row in W:
        acc = 0.0
        for a, b in zip(row, x):
            acc += a * b
        out.append(acc)
    return out


def _rmsnorm(x: List[float], g: List[float], eps: float) -> List[float]:
    ss = 0.0
    for t in x:
        ss += t * t
    r = 1.0 / math.sqrt(ss / len(x) + eps)
    return [g[i] * x[i] * r for i in range(len(x))]


def _rope_head(vec: List[float], pos: int, theta: float) -> List[float]:
    d = len(vec)
    half = d // 2
    out = [0.0] * d
    for j in range(half):
        ang = pos * theta ** (-2.0 * j / d)
        c, s = math.cos(ang), math.sin(ang)
        out[j] = vec[j] * c - vec[j + half] * s
        out[j + half] = vec[j + half] * c + vec[j] * s
    return out


def brute_draft(cfg, weights: Dict, features: Sequence, anchors: Sequence[int], block: int,
                use_rope: bool = True, block_tokens=None):
    """Full pipeline for tiny shapes: ingest each sequence's features as context,
    then draft one block per sequence.

    cfg: object with n_layers, hidden, n_q_heads, n_kv_heads, head_dim,
    intermediate, vocab, mask_token_id, rms_eps, rope_theta.  features[b] is a
    [c_b][L_t*H] array of bf16 bits (c_b may be 0).  Returns (logits, drafts)
    with logits[b][i-1][v] for block rows i = 1..B-1.
    """
    L, H = cfg.n_layers, cfg.hidden
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    Wfc = _mat(weights, "w_fc")
    E = _mat(weights, "embed")
    gF = _vec(weights, "final_norm")
    lay = []
    for l in range(L):
        p = f"layers.{l}."
        lay.append(dict(an=_vec(weights, p + "attn_norm"), mn=_vec(weights, p + "mlp_norm"),
                        q=_mat(weights, p + "wq"), k=_mat(weights, p + "wk"), v=_mat(weights, p + "wv"),
                        o=_mat(weights, p + "wo"), g=_mat(weights, p + "wgate"), u=_mat(weights, p + "wup"),
                        dn=_mat(weights, p + "wdown")))

    all_logits, all_drafts = [], []
    for b, anchor in enumerate(anchors):
        feats = features[b]
        c = len(feats)
        # injected context: ctxK[l][t][g] / ctxV[l][t][g] are d-vectors
        ctxK = [[None] * c for _ in range(L)]
        ctxV = [[None] * c for _ in range(L)]
        for t in range(c):
            f = [_bf16(x) for x in feats[t]]
            h = _matvec(Wfc, f)
            for l in range(L):
                kf = _matvec(lay[l]["k"], h)
                vf = _matvec(lay[l]["v"], h)
                heads_k, heads_v = [], []
                for g in range(nkv):
                    kh = kf[g * d:(g + 1) * d]
                    heads_k.append(_rope_head(kh, t, cfg.rope_theta) if use_rope else kh)
                    heads_v.append(vf[g * d:(g + 1) * d])
                ctxK[l][t] = heads_k
                ctxV[l][t] = heads_v

        if block_tokens is None:
            toks = [int(anchor)] + [cfg.mask_token_id] * (block - 1)
        else:
            toks = [int(anchor)] + [int(t) for t in block_tokens[b]]
        x = [list(E[tk]) for tk in toks]
        for l in range(L):
            P = lay[l]
            qs, ks, vs = [], [], []
            for i in range(block):
                u = _rmsnorm(x[i], P["an"], cfg.rms_eps)
                qf, kf, vf = _matvec(P["q"], u), _matvec(P["k"], u), _matvec(P["v"], u)
                pos = c + i
                qs.append([_rope_head(qf[h * d:(h + 1) * d], pos, cfg.rope_theta) if use_rope
                           else qf[h * d:(h + 1) * d] for h in range(nq)])
                ks.append([_rope_head(kf[g * d:(g + 1) * d], pos, cfg.rope_theta) if use_rope
                           else kf[g * d:(g + 1) * d] for g in range(nkv)])
                vs.append([vf[g * d:(g + 1) * d] for g in range(nkv)])
            newx = []
            for i in range(block):
                concat = []
                for h in range(nq):
                    g = (h * nkv) // nq
                    keys = [ctxK[l][t][g] for t in range(c)] + [ks[j][g] for j in range(block)]
                    vals = [ctxV[l][t][g] for t in range(c)] + [vs[j][g] for j in range(block)]
                    scores = []
                    for key in keys:
                        dot = 0.0
                        for e in range(d):
                            dot += qs[i][h][e] * key[e]
                        scores.append(dot / math.sqrt(d))
                    mx = max(scores)
                    ex = [math.exp(s - mx) for s in scores]
                    tot = sum(ex)
                    oh = [0.0] * d
                    for j, val in enumerate(vals):
                        pj = ex[j] / tot
                        for e in range(d):
                            oh[e] += pj * val[e]
                    concat += oh
                att = _matvec(P["o"], concat)
                newx.append([x[i][e] + att[e] for e in range(H)])
            x = newx
            for i in range(block):
                w = _rmsnorm(x[i], P["mn"], cfg.rms_eps)
                gt, up = _matvec(P["g"], w), _matvec(P["u"], w)
                a = [gt[j] / (1.0 + math.exp(-gt[j])) * up[j] for j in range(len(gt))]
                dn = _matvec(P["dn"], a)
                x[i] = [x[i][e] + dn[e] for e in range(H)]
        rows, drafts = [], []
        for i in range(1, block):
            y = _rmsnorm(x[i], gF, cfg.rms_eps)
            lg = _matvec(E, y)
            best = 0
            for vidx in range(1, len(lg)):
                if lg[vidx] > lg[best]:
                    best = vidx
            rows.append(lg)
            drafts.append(best)
        all_logits.append(rows)
        all_drafts.append(drafts)
    return all_logits, all_drafts
