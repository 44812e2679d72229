"""A second, loop-by-loop attention in pure Python floats (float64), written
independently of the oracle, for tiny shapes only. Test infrastructure."""
import math


def attention_loops(q, k, v, B, Hq, Hkv, Lq, Lk, D, Dv, scale, mask_kind, mask=None, sinks=None,
                    window=None):
    """q, k, v: nested lists [B][H][L][E]; mask: [Lq][Lk] of 0/1 (kind 2), or
    the additive mask [B][Hq][Lq][Lk] of floats (kind 3, -inf drops the key);
    sinks: [Hq]; window: with the causal mask, the keys a row reads back from
    its position. Returns nested list [B][Hq][Lq][Dv]."""
    g = Hq // Hkv
    out = []
    for b in range(B):
        ob = []
        for h in range(Hq):
            kh = h // g
            oh = []
            for i in range(Lq):
                keys = []
                for j in range(Lk):
                    if mask_kind == 1 and j > i + (Lk - Lq):
                        continue
                    if window is not None and j + window <= i + (Lk - Lq):
                        continue
                    if mask_kind == 2 and not mask[i][j]:
                        continue
                    if mask_kind == 3 and mask[b][h][i][j] == -math.inf:
                        continue
                    dot = 0.0
                    for c in range(D):
                        dot += q[b][h][i][c] * k[b][kh][j][c]
                    keys.append((j, scale * dot + (mask[b][h][i][j] if mask_kind == 3 else 0.0)))
                logits = [s for _, s in keys]
                if sinks is not None:
                    logits.append(sinks[h])
                if not keys:
                    oh.append([0.0] * Dv)
                    continue
                top = max(logits)
                denom = sum(math.exp(s - top) for s in logits)
                row = [0.0] * Dv
                for j, s in keys:
                    wgt = math.exp(s - top) / denom
                    for c in range(Dv):
                        row[c] += wgt * v[b][kh][j][c]
                oh.append(row)
            ob.append(oh)
        out.append(ob)
    return out
