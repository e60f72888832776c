"""fp64 MoE layer forward: routing, SwiGLU experts, gate-weighted combine.

Test infrastructure only.  The definition followed, step by step:

1. Router logits l[t,e] = sum_h x[t,h] * W_r[e,h] (no bias term).  Inputs are
   fp32 or bf16, so every product is exact in fp64; l is the correctly
   rounded exact sum (math.fsum).  For large inputs a BLAS fp64 product is
   used first, only to decide the selection: each approximate score is
   given an interval from the classical summation error bound
   gamma_n * sum|x*w|, and a token is certified only when its k selected
   intervals are strictly ordered and the k-th lies strictly above the
   interval of every unselected expert.  Certified tokens then take the
   selected experts' logits from fsum; every other token is recomputed with
   fsum in full.  So ids and gates always equal the all-fsum ones exactly.
   (The returned logits of unselected experts of certified tokens are the
   BLAS values, within the bound.)
2. Selection score s = l + b (b: optional selection-only bias, default 0).
   The k experts with the largest s are kept, ordered by (s descending,
   expert id ascending): equal scores go to the lower id.
3. Gates g = softmax of the selected logits l (not of s): exp(l_j - M) / sum,
   M the largest selected logit.  This equals the full softmax over all E
   experts renormalised over the selected set.  With renormalize=False the
   gate is the full-softmax probability itself.
4. Each selected expert e computes y = D_e (silu(G_e x) * (U_e x)) with
   silu(z) = z / (1 + exp(-z)), all in fp64.
5. out[t] = sum over j (in rank order) of [e_tj in mask] * g[t,j] * y[t,j].
   The mask (a bitset over expert ids) selects which experts this call
   computes; routing and gates ignore it, so the outputs for the parts of any
   partition of the experts add up to the unmasked output.

Routing is never changed by the cache and the output of the split-and-sum is
the exact MoE output (FreeToken explainer page, "how" section).  The softmax,
top-k renormalisation and SwiGLU are the textbook MoE layer; the pages name
no formula.
"""
import math

import numpy as np

from .formats import bf16_bits_to_f64

F32, BF16 = 0, 1
_U = 2.0 ** -53


def to_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    """Stored activations / router weights -> their exact fp64 values."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_bits_to_f64(a)
    raise ValueError(dtype)


def mask_has(mask, e: int) -> bool:
    if mask is None:
        return True
    return bool((int(mask[e >> 5]) >> (e & 31)) & 1)


def exact_logits_row(x_t: np.ndarray, wr: np.ndarray) -> np.ndarray:
    """Correctly rounded exact dot products of one token with every router row."""
    return np.array([math.fsum((x_t * wr[e]).tolist()) for e in range(wr.shape[0])])


def select_topk(s_t: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores, by (score desc, index asc)."""
    order = np.argsort(-s_t, kind="stable")
    return order[:k]


def _gamma(n: int) -> float:
    return n * _U / (1.0 - n * _U)


def approx_logits(x: np.ndarray, wr: np.ndarray):
    """BLAS fp64 logits and, per entry, a bound on their distance from the
    correctly rounded exact dot products: twice the classical bound
    gamma_H * sum_h |x w| on any order of floating-point summation."""
    H = x.shape[1]
    return x @ wr.T, 2.0 * _gamma(H) * (np.abs(x) @ np.abs(wr).T)


def certified_order(s: np.ndarray, slack: np.ndarray, k: int):
    """Given approximate scores s and radii slack (each exact score lies in
    [s - slack, s + slack]), return the top-k (score desc, id asc) of the
    exact scores if the intervals decide it, else None.

    Decided means: consecutive selected experts are strictly separated
    (lower end of the higher one above the upper end of the next), and the
    lower end of the k-th is above the upper end of EVERY unselected expert.
    Then the exact scores are strictly ordered the same way, with no ties."""
    order = np.argsort(-s, kind="stable")
    sel, rest = order[:k], order[k:]
    lo, hi = s - slack, s + slack
    if np.any(lo[sel[:-1]] <= hi[sel[1:]]):
        return None
    if rest.size and lo[sel[-1]] <= hi[rest].max():
        return None
    return sel


def route(x: np.ndarray, wr: np.ndarray, k: int, bias: np.ndarray = None,
          renormalize: bool = True, exact_all: bool = None):
    """x [T,H] f64, wr [E,H] f64, bias [T,E] or None.
    -> ids int32 [T,k], gates f64 [T,k], logits f64 [T,E]."""
    T, H = x.shape
    E = wr.shape[0]
    if exact_all is None:
        exact_all = T * E * H <= 2_000_000
    if exact_all:
        logits = np.stack([exact_logits_row(x[t], wr) for t in range(T)]) if T else np.zeros((0, E))
        certified = np.ones(T, dtype=bool)
    else:
        logits, bound = approx_logits(x, wr)
        certified = np.zeros(T, dtype=bool)
    b = np.zeros((T, E)) if bias is None else np.asarray(bias, dtype=np.float64)
    ids = np.zeros((T, k), dtype=np.int32)
    gates = np.zeros((T, k))
    for t in range(T):
        s = logits[t] + b[t]
        sel = select_topk(s, k)
        if not certified[t]:
            got = certified_order(s, bound[t] + 2.0 * _U * np.abs(s), k)
            if got is None or not renormalize:
                # undecided, or full-softmax gates that need every logit
                logits[t] = exact_logits_row(x[t], wr)
                s = logits[t] + b[t]
                sel = select_topk(s, k)
            else:
                # decided: the gates use the exact logits of the selection
                logits[t, sel] = exact_logits_row(x[t], wr[sel])
        ids[t] = sel
        ls = logits[t, sel]
        if renormalize:
            m = ls.max()
            ex = np.exp(ls - m)
            gates[t] = ex / ex.sum()
        else:
            m = logits[t].max()
            ex = np.exp(logits[t] - m)
            gates[t] = ex[sel] / ex.sum()
    return ids, gates, logits


def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(x_t: np.ndarray, G: np.ndarray, U: np.ndarray, D: np.ndarray,
                  quant=None) -> np.ndarray:
    """y = D (silu(G x) * (U x)); `quant`, when given, is applied to h before D
    (the prefill path's activation quantisation)."""
    a = G @ x_t
    b = U @ x_t
    h = silu(a) * b
    if quant is not None:
        h = quant(h)
    return D @ h


def experts_forward(x: np.ndarray, ids: np.ndarray, gates: np.ndarray, expert, mask=None,
                    x_quant=None, h_quant=None, y_quant=None, tokens=None) -> np.ndarray:
    """Steps 4-5 for given ids [T,k] and gates [T,k]: out[t] = sum over j in
    rank order of [e_tj in mask] g_tj y_tj.  A token may list an expert more
    than once; each listing adds its own term.  -> out [T,H] (rows outside
    `tokens` are NaN)."""
    T, H = x.shape
    out = np.full((T, H), np.nan)
    rows = range(T) if tokens is None else tokens
    for t in rows:
        acc = np.zeros(H)
        xt = x[t] if x_quant is None else x_quant(x[t])
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if not mask_has(mask, e):
                continue
            G, U, D = expert(e)
            y = swiglu_expert(xt, G, U, D, quant=h_quant)
            acc = acc + gates[t, j] * (y if y_quant is None else y_quant(y))
        out[t] = acc
    return out


def experts_forward_by_expert(x: np.ndarray, ids: np.ndarray, gates: np.ndarray, expert, tokens, mask=None,
                              x_quant=None, h_quant=None, y_quant=None) -> np.ndarray:
    """experts_forward for the rows `tokens`, visiting each expert once, for
    experts too large to keep decoded together: every y_tj is computed as
    there and the terms are added in the same rank order, so the result is
    the same bit for bit.  -> out [T,H] (rows outside `tokens` are NaN)."""
    T, H = x.shape
    want = {}
    for t in tokens:
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if mask_has(mask, e):
                want.setdefault(e, []).append((t, j))
    ys = {}
    for e in sorted(want):
        G, U, D = expert(e)
        for t, j in want[e]:
            xt = x[t] if x_quant is None else x_quant(x[t])
            y = swiglu_expert(xt, G, U, D, quant=h_quant)
            ys[(t, j)] = y if y_quant is None else y_quant(y)
    out = np.full((T, H), np.nan)
    for t in tokens:
        acc = np.zeros(H)
        for j in range(ids.shape[1]):
            if (t, j) in ys:
                acc = acc + gates[t, j] * ys[(t, j)]
        out[t] = acc
    return out


def moe_layer(x: np.ndarray, wr: np.ndarray, expert, k: int, bias=None, mask=None,
              renormalize: bool = True, x_quant=None, h_quant=None, tokens=None, y_quant=None):
    """Full layer.  `expert(e)` returns (G, U, D) in fp64.  `tokens` limits the
    output rows computed (routing is still per token, independent of others).
    x_quant / h_quant / y_quant mirror a storage precision of the activations,
    of h before the down projection, and of each expert output before the
    combine (identity when None).
    -> out [T,H] (rows outside `tokens` are NaN), ids, gates."""
    ids, gates, _ = route(x, wr, k, bias=bias, renormalize=renormalize)
    out = experts_forward(x, ids, gates, expert, mask=mask, x_quant=x_quant, h_quant=h_quant,
                          y_quant=y_quant, tokens=tokens)
    return out, ids, gates
