"""Independent brute-force formulations used to pin the oracle.

These are written differently from the oracle on purpose:
  * routing sorts every logit with Python's sort by (-value, index) and takes
    the softmax with scipy (the biased router: scipy's expit/softmax scores,
    the same sort on score + bias);
  * alignment is a Python stable sort of the pair list by its key;
  * the layer computes EVERY expert for EVERY token densely (numpy einsum in
    fp64) and combines them through a dense [T, E'] gate matrix, so a wrong
    index, a transposed operand or a dropped term in the oracle shows up as
    a mismatch.
"""
from __future__ import annotations

import numpy as np
from scipy.special import softmax


def to_f64(t) -> np.ndarray:
    import torch
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def route(logits, K: int, S: int = 0, rsf: float = 1.0, renormalize: int = 1):
    lg = np.asarray(to_f64(logits), dtype=np.float64)
    T, E = lg.shape
    ids = np.zeros((T, K + S), np.int32)
    w = np.zeros((T, K + S), np.float32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:K]
        ids[t, :K] = order
        if renormalize:
            p = softmax(lg[t, order])
        else:
            p = softmax(lg[t])[order]
        w[t, :K] = p.astype(np.float32)
        for q in range(S):
            ids[t, K + q] = E + q
            w[t, K + q] = np.float32(1.0) / np.float32(rsf)
    return ids, w


def route_bias(logits, K: int, S: int = 0, rsf: float = 1.0, renormalize: int = 1, scoring: str = "sigmoid",
               bias=None):
    """Biased router written with library routines: scipy's expit / softmax
    for the fp64 scores, Python's sort by (-(score + bias), index) for the
    choice, weights from the unbiased scores."""
    from scipy.special import expit
    lg = np.asarray(to_f64(logits), dtype=np.float64)
    T, E = lg.shape
    b = np.zeros(E) if bias is None else np.asarray(bias, dtype=np.float32).astype(np.float64)
    ids = np.zeros((T, K + S), np.int32)
    w = np.zeros((T, K + S), np.float32)
    for t in range(T):
        sc = expit(lg[t]) if scoring == "sigmoid" else softmax(lg[t])
        order = sorted(range(E), key=lambda e: (-(float(sc[e]) + float(b[e])), e))[:K]
        ids[t, :K] = order
        sel = sc[order]
        w[t, :K] = (sel / sel.sum() if renormalize else sel).astype(np.float32)
        for q in range(S):
            ids[t, K + q] = E + q
            w[t, K + q] = np.float32(1.0) / np.float32(rsf)
    return ids, w


def align(topk_ids, adapter_ids, Ep: int, La: int, bm: int, lbm: int):
    ids = np.asarray(topk_ids).reshape(-1)
    T = np.asarray(topk_ids).shape[0]
    Kp = np.asarray(topk_ids).shape[1] if T else 1
    P = ids.size
    ad = [int(adapter_ids[f // Kp]) if La > 0 else -1 for f in range(P)]
    pairs = sorted(range(P), key=lambda f: (int(ids[f]), ad[f], f))
    rows, blocks = [], []
    items = []
    for e in range(Ep):
        grp = [f for f in pairs if ids[f] == e]
        start = len(rows)
        rows += grp
        pad = -len(grp) % bm
        rows += [P] * pad
        blocks += [e] * ((len(grp) + pad) // bm)
        if La > 0:
            for a in range(La):
                sub = [i for i, f in enumerate(grp) if ad[f] == a]
                if not sub:
                    continue
                s0 = start + sub[0]
                for q in range(0, len(sub), lbm):
                    items.append((s0 + q, min(lbm, len(sub) - q), a, e))
    return dict(sorted_ids=np.array(rows, np.int32), block_expert=np.array(blocks, np.int32),
                num_post_pad=len(rows), items=np.array(items, np.int32).reshape(-1, 4))


def silu(z):
    return z / (1.0 + np.exp(-z))


def layer_dense(x, w13, w2, gate, adapter_ids=None, a13=None, b13=None, a2=None, b2=None,
                rsf: float = 1.0):
    """out[t] = rsf * sum_e gate[t,e] * MLP_e(x[t]) with every expert computed densely.

    gate is a dense [T, E'] matrix holding each token's slot weights at its
    chosen experts and zero elsewhere."""
    X = to_f64(x)
    W13 = to_f64(w13)
    W2 = to_f64(w2)
    G = np.asarray(gate, np.float64)
    Ep, twoI, H = W13.shape
    I = twoI // 2
    g = np.einsum("th,enh->ten", X, W13)
    if a13 is not None:
        A13, B13, A2, B2 = map(to_f64, (a13, b13, a2, b2))
        ad = np.asarray(adapter_ids).astype(np.int64)
        m = (ad >= 0).astype(np.float64)
        sel = np.clip(ad, 0, None)
        u = np.einsum("th,tekh->tek", X, A13[sel]) * m[:, None, None]
        g = g + np.einsum("tek,tenk->ten", u, B13[sel])
    h = silu(g[..., :I]) * g[..., I:]
    y = np.einsum("tei,eni->ten", h, W2)
    if a13 is not None:
        v = np.einsum("tei,teki->tek", h, A2[sel]) * m[:, None, None]
        y = y + np.einsum("tek,tenk->ten", v, B2[sel])
    return rsf * np.einsum("te,ten->tn", G, y)


def gate_matrix(ids, w, Ep: int) -> np.ndarray:
    T, Kp = ids.shape
    G = np.zeros((T, Ep), np.float64)
    for t in range(T):
        for j in range(Kp):
            G[t, ids[t, j]] += float(w[t, j])
    return G
