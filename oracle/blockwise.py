"""CPU float64 statements of the two blockwise schedules the GPU path uses,
kept so that the tests can show, on the CPU, that each schedule reaches the
plain definition in ``oracle.attention``.

TEST INFRASTRUCTURE ONLY: imported by the tests alone, never by the GPU
library, and sharing no code with it.

* ``online_head``: the tiled online-softmax recurrence of lattice-inference
  "src/attention/flash.rs" (``run_tiled_attention_head``), for one head and a
  per-row visibility matrix: per key tile, new row max, rescale factor
  ``exp(m_old - m_new)`` (0 while the old max is -inf), tile weights
  ``exp(s - m_new)`` (0 while the new max is -inf), running sum and running
  output; at the end divide by the sum, or output 0 when the sum is 0.
* ``split_partials`` / ``combine_partials``: the two-pass decode schedule
  named by nuvec-core "tests/attention_plan.rs" (first pass over key
  partitions, second pass reducing them): each key block yields its own
  maximum, sum of weights and unnormalised output; the reduce rescales every
  block to the common maximum (log-sum-exp) and divides once. Reading taken:
  a sink joins the reduce as one more logit with no value row.
"""
from __future__ import annotations

import numpy as np


def online_head(q, k, v, vis, scale, tile_q, tile_kv):
    """q [Lq,D], k [Lk,D], v [Lk,Dv], vis [Lq,Lk] bool -> out [Lq,Dv] (float64)."""
    Lq, Lk, Dv = q.shape[0], k.shape[0], v.shape[1]
    out = np.zeros((Lq, Dv))
    for q0 in range(0, Lq, tile_q):
        q1 = min(q0 + tile_q, Lq)
        o = np.zeros((q1 - q0, Dv))
        m = np.full(q1 - q0, -np.inf)
        l = np.zeros(q1 - q0)
        for k0 in range(0, Lk, tile_kv):
            k1 = min(k0 + tile_kv, Lk)
            s = scale * (q[q0:q1] @ k[k0:k1].T)
            s = np.where(vis[q0:q1, k0:k1], s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            old = np.isfinite(m)
            alpha = np.zeros_like(m)
            alpha[old] = np.exp(m[old] - m_new[old])
            fin = np.isfinite(m_new)
            p = np.where(fin[:, None], np.exp(s - np.where(fin, m_new, 0.0)[:, None]), 0.0)
            l = alpha * l + p.sum(axis=1)
            o = alpha[:, None] * o + p @ v[k0:k1]
            m = m_new
        good = l > 0
        out[q0:q1] = np.where(good[:, None], o / np.where(good, l, 1.0)[:, None], 0.0)
    return out


def split_partials(q_row, k, v, vis_row, scale, block):
    """One query row against key blocks of ``block`` keys.

    Returns a list of (m_b, l_b, o_b): the block's maximum visible score
    (-inf if none), the sum of exp(s - m_b) over its visible keys, and the
    unnormalised output sum of exp(s - m_b) * v.
    """
    Lk, Dv = k.shape[0], v.shape[1]
    parts = []
    for k0 in range(0, Lk, block):
        k1 = min(k0 + block, Lk)
        s = scale * (k[k0:k1] @ q_row)
        s = np.where(vis_row[k0:k1], s, -np.inf)
        m_b = s.max() if k1 > k0 else -np.inf
        if np.isfinite(m_b):
            w = np.exp(s - m_b)
            parts.append((m_b, w.sum(), w @ v[k0:k1]))
        else:
            parts.append((-np.inf, 0.0, np.zeros(Dv)))
    return parts


def combine_partials(parts, Dv, sink=None):
    """Log-sum-exp reduce of ``split_partials`` output, with an optional sink logit."""
    ms = [m for m, _, _ in parts]
    M = max(ms + ([sink] if sink is not None else []), default=-np.inf)
    if not np.isfinite(M):
        return np.zeros(Dv)
    L = 0.0
    acc = np.zeros(Dv)
    for m_b, l_b, o_b in parts:
        if np.isfinite(m_b):
            f = np.exp(m_b - M)
            L += l_b * f
            acc += o_b * f
    if sink is not None:
        L += np.exp(sink - M)
    return acc / L if L > 0 else np.zeros(Dv)
