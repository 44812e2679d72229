"""CPU float64 oracle for fused scaled-dot-product attention forward.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The GPU library never calls it, and
it shares no code with the GPU library.

What is computed is the plain definition of attention, one materialised
softmax row per query, in float64 on the exact values of the stored inputs:

* the direct formula of the nuvec-core fused-op tests ("tests/fast.rs",
  ``attention_fallback_matches_a_direct_formula``): scores are
  ``scale * q . k``, the row maximum is subtracted before ``exp``, the
  weights are divided by their sum and applied to ``v``; with a causal mask,
  query ``i`` of ``Lq`` sees key ``j`` of ``Lk`` iff ``j < i + Lk - Lq + 1``
  (the mask is aligned to the bottom-right corner);
* masked keys are excluded from the row, never given a finite sentinel score,
  and a row that sees no key outputs exactly zero (lattice-inference
  "src/attention/flash.rs", ``run_tiled_attention_head`` and its tests
  ``masked_key_below_finite_sentinel_does_not_dominate`` and
  ``all_masked_row_yields_zero_output_not_nan``);
* grouped-query heads: query head ``h`` reads key/value head
  ``h // (Hq / Hkv)`` (flash.rs, ``kv_head_index``);
* a boolean mask is one ``[Lq, Lk]`` matrix shared by every batch item and
  head, nonzero meaning "attend" (nuvec-core "tests/attention_plan.rs",
  ``attention()``; fast.rs, ``window_mask``);
* a sliding window (causal only) of w keys: query ``i`` at position
  ``pos = i + Lk - Lq`` sees key ``j`` iff ``pos - w < j <= pos``, the band of
  nuvec-core "tests/fast.rs" (``window_mask``, and the windowed-kernel tests
  ``windows_run_fused_and_equal_the_boolean_mask`` and
  ``window_errors_empty_inputs_and_full_windows``); a window of at least Lk
  keys is plain causal attention;
* an additive mask (nuvec-core "tests/fast.rs",
  ``attention_kernels_match_the_fallback``: a float mask of shape
  ``[1, Hq, Lq, Lk]`` in the input type, passed where a boolean mask could
  be) is added to the scaled scores, ``scale * q . k + mask[b, h, i, j]``;
  it broadcasts over batch items and heads. Reading taken: a key whose mask
  entry is ``-inf`` is excluded like a masked key, so a row whose every entry
  is ``-inf`` outputs zero, as an all-masked row does;
* an optional per-query-head sink is one extra logit in the softmax
  denominator with no value row. Reading taken: the sink is added as given,
  after scaling (it is not multiplied by ``scale``), and takes part in the row
  maximum. The pages name sinks but never print their formula, so this
  reading is parity unpinned beyond the closed forms the tests check.

Row-subset evaluation (``rows=``) computes the same rows one by one, so large
problems can be checked on sampled outputs.
"""
from __future__ import annotations

import numpy as np

MASK_NONE, MASK_CAUSAL, MASK_BOOL, MASK_ADDITIVE = 0, 1, 2, 3


def visible_keys(i: int, Lq: int, Lk: int, mask_kind: int, mask=None, window=None) -> np.ndarray:
    """Boolean [Lk] vector: which keys query row ``i`` may attend to."""
    j = np.arange(Lk)
    if window is not None:
        if mask_kind != MASK_CAUSAL or window < 1:
            raise ValueError("a window needs the causal mask and at least one key")
        pos = i + Lk - Lq
        return (j <= pos) & (j > pos - window)
    if mask_kind == MASK_NONE:
        return np.ones(Lk, dtype=bool)
    if mask_kind == MASK_CAUSAL:
        return j <= i + Lk - Lq
    if mask_kind == MASK_BOOL:
        return np.asarray(mask[i], dtype=bool).copy()
    if mask_kind == MASK_ADDITIVE:
        return np.ones(Lk, dtype=bool)   # -inf entries are dropped with the scores
    raise ValueError(f"unknown mask kind {mask_kind}")


def _visible_matrix(rows_i, Lq, Lk, mask_kind, mask, window=None):
    return np.stack([visible_keys(int(i), Lq, Lk, mask_kind, mask, window) for i in rows_i]) \
        if len(rows_i) else np.zeros((0, Lk), dtype=bool)


def head_probabilities(q_rows, k_head, rows_i, Lq, scale, mask_kind, mask=None, sink=None, window=None,
                       bias=None):
    """Softmax weights for some query rows of one head.

    q_rows [n, D], k_head [Lk, D] float64; bias [n, Lk] the additive mask rows
    (MASK_ADDITIVE only). Returns (p [n, Lk], p_sink [n]): the weight of every
    key (0 where masked) and the sink's share of the denominator (0 without a
    sink). A row with no visible key and no sink has all weights 0.
    """
    Lk = k_head.shape[0]
    s = scale * (q_rows @ k_head.T)                      # scores, [n, Lk]
    vis = _visible_matrix(rows_i, Lq, Lk, mask_kind, mask, window)
    if mask_kind == MASK_ADDITIVE:
        bias = np.asarray(bias, dtype=np.float64)
        vis = vis & ~np.isneginf(bias)
        s = s + np.where(vis, bias, 0.0)
    s_vis = np.where(vis, s, -np.inf)
    m = s_vis.max(axis=1) if Lk else np.full(len(rows_i), -np.inf)
    if sink is not None:
        m = np.maximum(m, sink)
    live = np.isfinite(m)                                # rows with something to normalise
    m_safe = np.where(live, m, 0.0)
    w = np.where(vis, np.exp(s_vis - m_safe[:, None]), 0.0)
    z = w.sum(axis=1)
    w_sink = np.exp(sink - m_safe) if sink is not None else np.zeros(len(rows_i))
    w_sink = np.where(live, w_sink, 0.0)
    z = z + w_sink
    z_safe = np.where(z > 0, z, 1.0)
    p = np.where((z > 0)[:, None], w / z_safe[:, None], 0.0)
    p_sink = np.where(z > 0, w_sink / z_safe, 0.0)
    return p, p_sink


def _bias(mask, B, Hq, Lq, Lk):
    """The additive mask broadcast to [B, Hq, Lq, Lk] (a read-only view)."""
    m = np.asarray(mask, dtype=np.float64)
    return np.broadcast_to(m.reshape((1,) * (4 - m.ndim) + m.shape), (B, Hq, Lq, Lk))


def sdpa(q, k, v, scale, mask_kind, mask=None, sinks=None, rows=None, window=None):
    """Attention forward in float64.

    q [B,Hq,Lq,D], k [B,Hkv,Lk,D], v [B,Hkv,Lk,Dv] (float64), mask [Lq,Lk]
    (bool, MASK_BOOL) or an additive float mask broadcastable to
    [B,Hq,Lq,Lk] (MASK_ADDITIVE), sinks [Hq] or None, window (causal only)
    None or the number of keys each query row reads back from its position.

    rows=None returns out [B,Hq,Lq,Dv]. rows = iterable of (b, h, i) returns
    [len(rows), Dv] for just those query rows.
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, Hq, Lq, D = q.shape
    Hkv, Lk, Dv = k.shape[1], k.shape[2], v.shape[3]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    group = Hq // Hkv
    bias = _bias(mask, B, Hq, Lq, Lk) if mask_kind == MASK_ADDITIVE else None
    if rows is None:
        out = np.zeros((B, Hq, Lq, Dv))
        for b in range(B):
            for h in range(Hq):
                hk = h // group
                sink = None if sinks is None else float(sinks[h])
                p, _ = head_probabilities(q[b, h], k[b, hk], np.arange(Lq), Lq, scale,
                                          mask_kind, mask, sink, window,
                                          None if bias is None else bias[b, h])
                out[b, h] = p @ v[b, hk]
        return out
    rows = [tuple(int(x) for x in r) for r in rows]
    out = np.zeros((len(rows), Dv))
    # group the requested rows by (b, h) so each head's keys are touched once
    by_head = {}
    for n, (b, h, i) in enumerate(rows):
        by_head.setdefault((b, h), []).append((n, i))
    for (b, h), items in by_head.items():
        hk = h // group
        idx = [n for n, _ in items]
        ii = np.array([i for _, i in items])
        sink = None if sinks is None else float(sinks[h])
        p, _ = head_probabilities(q[b, h, ii], k[b, hk], ii, Lq, scale, mask_kind, mask, sink, window,
                                  None if bias is None else bias[b, h, ii])
        out[idx] = p @ v[b, hk]
    return out


def probabilities(q, k, scale, mask_kind, mask=None, sinks=None, window=None):
    """All softmax weights: (p [B,Hq,Lq,Lk], p_sink [B,Hq,Lq])."""
    q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
    B, Hq, Lq, _ = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    group = Hq // Hkv
    bias = _bias(mask, B, Hq, Lq, Lk) if mask_kind == MASK_ADDITIVE else None
    p = np.zeros((B, Hq, Lq, Lk))
    ps = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            sink = None if sinks is None else float(sinks[h])
            p[b, h], ps[b, h] = head_probabilities(q[b, h], k[b, h // group], np.arange(Lq),
                                                   Lq, scale, mask_kind, mask, sink, window,
                                                   None if bias is None else bias[b, h])
    return p, ps
