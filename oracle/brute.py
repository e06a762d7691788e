"""Brute-force checks in 50-digit decimal arithmetic for tiny inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle.attention``).  These routines write the
definitions out literally, with none of the oracle's structure, so that they
can pin it from outside:

* softmax as exp(s_j) / sum_k exp(s_k), with no max subtraction (the form the
  explainer's appendix on softmax starts from before it subtracts the max);
* attention O_i = sum_j softmax(s_i)_j v_j over the visible keys (causal: j <= i);
* gradients of L = sum_{i,c} O_ic dO_ic by central finite differences, with no
  use of any backward formula.

Inputs are Python floats or float64 arrays; each is converted exactly to Decimal.
"""
from __future__ import annotations

from decimal import Decimal, localcontext

import numpy as np

__all__ = ["softmax_decimal", "attention_decimal", "loss_decimal", "grads_fd_decimal"]

PREC = 50


def _D(x) -> Decimal:
    return Decimal(float(x))


def softmax_decimal(s) -> list:
    with localcontext() as ctx:
        ctx.prec = PREC
        ex = [_D(x).exp() for x in s]
        tot = sum(ex, Decimal(0))
        return [e / tot for e in ex]


def attention_decimal(q, k, v, scale, causal: bool, q_offset: int = 0, k_offset: int = 0):
    """O (list of lists of Decimal) and LSE (list of Decimal) by the literal definition.

    With offsets, query i sits at global position q_offset + i and key j at
    k_offset + j; a row that sees no key yields O = 0 and LSE = None.
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    with localcontext() as ctx:
        ctx.prec = PREC
        sc = _D(scale)
        O, L = [], []
        for i in range(q.shape[0]):
            keys = [j for j in range(k.shape[0]) if (not causal or k_offset + j <= q_offset + i)]
            if not keys:
                O.append([Decimal(0)] * v.shape[1])
                L.append(None)
                continue
            s = [sc * sum((_D(q[i, c]) * _D(k[j, c]) for c in range(q.shape[1])), Decimal(0))
                 for j in keys]
            ex = [x.exp() for x in s]
            tot = sum(ex, Decimal(0))
            O.append([sum((ex[t] / tot * _D(v[j, c]) for t, j in enumerate(keys)), Decimal(0))
                      for c in range(v.shape[1])])
            L.append(tot.ln())
        return O, L


def loss_decimal(q, k, v, do, scale, causal: bool, qD=None, kD=None, vD=None):
    """L = sum O o dO in Decimal; qD/kD/vD optionally override inputs with Decimal arrays."""
    with localcontext() as ctx:
        ctx.prec = PREC
        Q = qD if qD is not None else [[_D(x) for x in row] for row in np.asarray(q)]
        K = kD if kD is not None else [[_D(x) for x in row] for row in np.asarray(k)]
        V = vD if vD is not None else [[_D(x) for x in row] for row in np.asarray(v)]
        dO = [[_D(x) for x in row] for row in np.asarray(do)]
        sc = _D(scale)
        total = Decimal(0)
        for i in range(len(Q)):
            keys = [j for j in range(len(K)) if (not causal or j <= i)]
            s = [sc * sum((Q[i][c] * K[j][c] for c in range(len(Q[i]))), Decimal(0)) for j in keys]
            ex = [x.exp() for x in s]
            tot = sum(ex, Decimal(0))
            for c in range(len(V[0])):
                oc = sum((ex[t] / tot * V[j][c] for t, j in enumerate(keys)), Decimal(0))
                total += oc * dO[i][c]
        return total


def grads_fd_decimal(q, k, v, do, scale, causal: bool, h: str = "1e-15"):
    """Central finite differences of L w.r.t. every entry of q, k and v (as float64 arrays)."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    with localcontext() as ctx:
        ctx.prec = PREC
        hD = Decimal(h)
        base = {n: [[_D(x) for x in row] for row in a] for n, a in (("q", q), ("k", k), ("v", v))}
        out = {}
        for name in ("q", "k", "v"):
            arr = base[name]
            g = np.zeros((len(arr), len(arr[0])))
            for r in range(len(arr)):
                for c in range(len(arr[0])):
                    vals = []
                    for sgn in (1, -1):
                        pert = {n: [row[:] for row in base[n]] for n in base}
                        pert[name][r][c] = arr[r][c] + sgn * hD
                        vals.append(loss_decimal(None, None, None, do, scale, causal,
                                                 pert["q"], pert["k"], pert["v"]))
                    g[r, c] = float((vals[0] - vals[1]) / (2 * hD))
            out["d" + name] = g
        return out
