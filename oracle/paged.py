"""CPU float64 oracle for paged-cache attention and the paged cache write.

TEST INFRASTRUCTURE ONLY (like oracle.attention): only the tests, the smoke
check and the benchmark's CPU leg may use it; it shares no code with the GPU
library.

Paged caches, as in nuvec-core "tests/fast.rs" (the ``paged`` helper and
``paged_attention_equals_contiguous_attention``): K and V caches of shape
[blocks, Hkv, bs, D]; a block table [B, max_blocks] of int32; lengths [B] of
int32. Key position j of sequence s lives in block table[s][j // bs], row
j % bs. Attention over a paged cache is attention over the keys gathered back
into order, with sequence s's length as its key count (causal alignment and
windows are relative to that length).

Hostile tables and lengths are clamped (fast.rs,
``paged_attention_clamps_hostile_tables_and_lengths``). The pages print no
rule for the clamp; the reading taken: a length is clamped to
[0, max_blocks * bs] and a table entry to [0, blocks - 1]. Parity is
unpinned beyond that reading.

The cache write (fast.rs, ``paged_write_matches_the_fallback_and_writes_in_place``,
``paged_write_skips_out_of_range_slots``): new rows [n, Hkv, D] go to slots
[n] of int32, slot = block * bs + row; a slot outside [0, blocks * bs) is
skipped.
"""
from __future__ import annotations

import numpy as np

from . import attention as orc


def gather(cache, table_row, length, bs):
    """Keys (or values) 0..length-1 of one sequence, [Hkv, length, D], from the
    clamped block table row."""
    blocks = cache.shape[0]
    pos = np.arange(length)
    blk = np.clip(np.asarray(table_row, dtype=np.int64)[pos // bs], 0, blocks - 1)
    return np.transpose(cache[blk, :, pos % bs, :], (1, 0, 2))


def paged_sdpa(q, kcache, vcache, table, lengths, scale, mask_kind, sinks=None, window=None):
    """q [B, Hq, Lq, D]; caches [blocks, Hkv, bs, D/Dv]; table [B, max_blocks];
    lengths [B]. mask_kind 0 (none) or 1 (causal); window needs causal.
    Returns out [B, Hq, Lq, Dv] in float64."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, Lq, _ = q.shape
    bs = kcache.shape[2]
    cap = np.asarray(table).shape[1] * bs
    Dv = vcache.shape[3]
    out = np.zeros((B, Hq, Lq, Dv))
    for b in range(B):
        n = int(min(max(int(lengths[b]), 0), cap))
        k = gather(np.asarray(kcache, np.float64), table[b], n, bs)[None]
        v = gather(np.asarray(vcache, np.float64), table[b], n, bs)[None]
        out[b] = orc.sdpa(q[b:b + 1], k, v, scale, mask_kind, None, sinks, window=window)[0]
    return out


def paged_write(cache, new, slots):
    """The cache after writing rows new[r] ([Hkv, D]) to slots[r]; invalid slots skipped."""
    out = np.array(cache, copy=True)
    blocks, _, bs, _ = out.shape
    for r, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if 0 <= slot < blocks * bs:
            out[slot // bs, :, slot % bs, :] = new[r]
    return out
