"""CPU check of the tile-load addresses of the pipelined prefill (csrc/prefill_fast.h)
and the key-split prefill (csrc/prefill_ksplit.h).

Each lane of each wavefront issues direct-to-LDS loads of one 16-byte chunk of
a K and a V row per tile. Its offset within the tile is kept as a 32-bit
unsigned byte offset; for the last, ragged tile, rows past the last key are
pulled back to the last key by subtracting whole rows from that unsigned
offset. This replays that arithmetic, modulo 2^32 as the kernel does it, for
every tile a workgroup issues, over ragged key counts, causal, windowed and
unmasked calls and strided rows, and checks that every load reads a key row in
[0, Lk) and a chunk inside the row, i.e. the unsigned offset never wraps.

80- and 96-wide rows (and the 64-wide V rows of the (96, 64) pair) sit in the
pipelined kernel's 128-wide LDS layout; a lane whose layout slot falls past the
row's real chunks loads a real chunk again, which the replay checks too.
"""
import itertools

import pytest

BN, NW, ROWS = 32, 4, 32
U32 = 1 << 32


FAST_PAIRS = [(64, 64), (80, 80), (96, 96), (128, 128), (96, 64)]   # the pipelined kernel's head pairs


def layout(D, Dv):
    """LDS row width (elements) of the pipelined kernel for a head pair."""
    return 64 if D <= 64 and Dv <= 64 else 128


def cfg(LW):
    rb = 2 * LW
    return dict(RB=rb, CPR=LW // 8, ROWS_PER_KB=1024 // rb)


def swz_k(LW, row):
    return row % (LW // 8)


def swz_v(LW, row):
    c = cfg(LW)
    rpl = 1 if c["RB"] >= 256 else 256 // c["RB"]
    nx = min(c["CPR"] // 4, 4)
    return 4 * ((row // rpl) % nx)


def src_chunk(slot, real):
    """The chunk a lane loads into layout slot `slot` of a row with `real` chunks."""
    return slot if slot < real else slot - real


def issued_tiles(Lq, Lk, qb, mask_kind, window, heads=4):
    """Key tiles (start keys) one workgroup of query block qb issues."""
    wph = NW // heads
    bm = wph * ROWS
    shift = Lk - Lq
    kend = Lk
    if mask_kind == 1:
        kend = min(Lk, min(qb * bm + bm, Lq) - 1 + shift + 1)
    kend = max(kend, 0)
    kbeg = 0
    if window > 0:
        kbeg = min(max(0, qb * bm + shift - window + 1), kend)
    tb = kbeg // BN
    ntiles = max((kend + BN - 1) // BN - tb, 0)
    return [(tb + t) * BN for t in range(ntiles)]


def check_tile(LW, Lk, k0, rs, swz, BN=BN, NW=NW, real=None):
    """Every lane's load of the tile at key k0 with row stride rs bytes, in an LDS
    layout of LW-wide rows holding `real` 16-byte chunks of each row (all of them
    by default)."""
    c = cfg(LW)
    real = c["CPR"] if real is None else real
    lpw = (BN * c["RB"] // 1024) // NW
    for w, it, lane in itertools.product(range(NW), range(lpw), range(64)):
        row = (w + NW * it) * c["ROWS_PER_KB"] + lane // c["CPR"]
        slot = lane % c["CPR"]
        chunk = src_chunk(slot ^ swz(LW, row), real) * 16
        off = (row * rs + chunk) % U32
        if k0 + BN > Lk:
            over = max(k0 + row - (Lk - 1), 0)
            off = (off - over * rs) % U32
        else:
            over = 0
        exact = (row - over) * rs + chunk          # what the offset must be, as a signed value
        assert off == exact, (LW, Lk, k0, rs, row, over)
        key = k0 + row - over
        assert 0 <= key <= Lk - 1, (LW, Lk, k0, row, key)
        assert 0 <= chunk < 16 * real


CALLS = [(1, 1), (5, 31), (40, 32), (40, 33), (97, 700), (130, 130), (333, 1297), (64, 96), (1040, 1297),
         (4096, 4096), (200, 1)]


@pytest.mark.parametrize("heads", [1, 4])
@pytest.mark.parametrize("D,Dv", FAST_PAIRS)
@pytest.mark.parametrize("mask_kind,window", [(0, 0), (1, 0), (1, 7), (1, 300), (2, 0)])
def test_every_issued_tile_reads_inside_the_keys(D, Dv, mask_kind, window, heads):
    # heads: query heads sharing a workgroup (4 under grouped queries; 1 gives 128-row blocks)
    LW = layout(D, Dv)
    for Lq, Lk in CALLS:
        nqb = -(-Lq // (ROWS * NW // heads))
        starts = set()   # the ragged last tile (the one that pulls rows back) and the first, per block
        for qb in range(nqb):
            tiles = issued_tiles(Lq, Lk, qb, mask_kind, window, heads)
            for k0 in tiles:
                assert k0 <= Lk - 1, "a tile starts past the last key"
            starts.update([t for t in tiles if t + BN > Lk] + tiles[:1])
        for k0 in sorted(starts):
            # K and V rows: contiguous, odd and the largest allowed strides
            for rs in [2 * D, 2 * D * 3 + 16 * 5, (1 << 26) - 16]:
                check_tile(LW, Lk, k0, rs, swz_k, real=D // 8)
            for rs in [2 * Dv, 2 * Dv * 3 + 16 * 5, (1 << 26) - 16]:
                check_tile(LW, Lk, k0, rs, swz_v, real=Dv // 8)


# --- V^T operand offsets -------------------------------------------------------------------------
# The pipelined kernel reads the V^T operand of each PV k-step with two transposed
# LDS reads per 32-column block. Their byte offsets are formed as one lane offset per
# block plus a key offset folded into the instruction; this replays that form against
# the direct per-read formula (row * RB + chunk permuted by the V swizzle of that row).

def swz_v_rows(LW, row):
    return swz_v(LW, row)


def acc_row32(i, kg):
    # 32x32 MFMA accumulator row of element i in lane group kg (KG = 2)
    return (i // 4) * 8 + kg * 4 + i % 4


@pytest.mark.parametrize("D,Dv", FAST_PAIRS)
def test_v_operand_offsets_fold_the_key_offset(D, Dv):
    MF, ACC, BN = 32, 16, 32
    LW = layout(D, Dv)
    RB, TILE = 2 * LW, BN * 2 * LW
    NPV, NDB = BN // 16, -(-Dv // MF)
    for lane in range(64):
        kg = lane // MF
        tr_e = (lane & 15) >> 2
        tr_c = lane & 3
        tr_chunk = ((lane >> 4) & 1) * 2 + (tr_c >> 1)
        tr_half = (tr_c & 1) * 8
        vk0 = acc_row32(0, kg) + tr_e
        for t8 in range(NPV):
            for half in (0, 4):
                i = 8 * t8 + half
                key = (i // ACC) * MF + acc_row32(i % ACC, kg) + tr_e
                kofs = (i // ACC) * MF + acc_row32(i % ACC, 0)
                assert key == vk0 + kofs and kofs % 8 == 0
                for db in range(NDB):
                    ch = db * 4 + tr_chunk
                    direct = TILE + key * RB + tr_half + ((ch ^ swz_v_rows(LW, key)) * 16)
                    folded = TILE + vk0 * RB + tr_half + (((db * 4 + tr_chunk) ^ swz_v_rows(LW, vk0)) * 16) + kofs * RB
                    assert folded == direct, (D, lane, t8, half, db)
                    assert TILE <= direct < 2 * TILE
                    # the slot read holds, as loaded, chunk src_chunk(slot ^ swizzle): for
                    # a real chunk that is the chunk itself (spare chunks feed columns at or
                    # past Dv, which are not stored)
                    held = src_chunk((ch ^ swz_v_rows(LW, key)) ^ swz_v_rows(LW, key), Dv // 8)
                    assert held == ch if ch < Dv // 8 else 8 * ch >= Dv


@pytest.mark.parametrize("D,Dv", FAST_PAIRS)
def test_k_operands_and_query_loads_stay_in_the_real_columns(D, Dv):
    # QK^T k-steps read chunks 2c + kg of K rows and elements 16c + 8kg .. +7 of
    # the query row, c < D / 16; output stores cover 8-column groups below Dv
    KW, MF = 16, 32
    for c in range(D // KW):
        for kg in (0, 1):
            assert 2 * c + kg < D // 8 and 16 * c + 8 * kg + 8 <= D
    stored = set()
    for db in range(-(-Dv // MF)):
        for g4 in range(4):
            if db * MF + g4 * 8 >= Dv:
                continue
            for kg in (0, 1):
                dv = db * MF + g4 * 8 + kg * 4
                assert dv + 4 <= Dv
                stored.update(range(dv, dv + 4))
    assert stored == set(range(Dv))


# --- the key-split prefill: 64-key steps loaded by eight wavefronts ---------------------------
# (head pairs (64,64), (128,128), (192,192), (192,128) and (256,256); 16 query rows per (head, row block) slot, so a workgroup's
# query block is 16, 32 or 64 rows for four, two or one heads per workgroup)

# the key-split kernel's head pairs
KS_PAIRS = [(64, 64), (80, 80), (96, 96), (128, 128), (96, 64), (192, 192), (192, 128), (256, 256)]


def ks_layout(width):
    # LDS row width of a K or V row: 192-wide rows sit in 256-wide ones
    return 64 if width <= 64 else 128 if width <= 128 else 256


def ks_swz_k(LW, row):
    return (row >> 1) % 8 if LW == 64 else row % (LW // 8)


def ks_swz_v(LW, row):
    return 2 * ((row >> 1) % 4) if LW == 64 else 2 * (row % 8)


@pytest.mark.parametrize("D,Dv", KS_PAIRS)
@pytest.mark.parametrize("heads", [1, 2, 4])
@pytest.mark.parametrize("mask_kind,window", [(0, 0), (1, 0), (1, 7), (1, 300), (2, 0)])
def test_key_split_steps_read_inside_the_keys(mask_kind, window, heads, D, Dv):
    KBN, KNW = 64, 8
    LW, LWV = ks_layout(D), ks_layout(Dv)
    bm = (4 // heads) * 16
    for Lq, Lk in CALLS:
        shift = Lk - Lq
        starts = set()   # the ragged last step and the first, per query block
        for qb in range(-(-Lq // bm)):
            kend = Lk
            if mask_kind == 1:
                kend = min(Lk, min(qb * bm + bm, Lq) - 1 + shift + 1)
            kend = max(kend, 0)
            kbeg = min(max(0, qb * bm + shift - window + 1), kend) if window > 0 else 0
            tb = kbeg // KBN
            steps = [(tb + t) * KBN for t in range(max((kend + KBN - 1) // KBN - tb, 0))]
            for k0 in steps:
                assert k0 <= Lk - 1, "a step starts past the last key"
            starts.update([t for t in steps if t + KBN > Lk] + steps[:1])
        for k0 in sorted(starts):
            for rs in [2 * D, 2 * D * 3 + 16 * 5, (1 << 26) - 16]:
                check_tile(LW, Lk, k0, rs, ks_swz_k, KBN, KNW, real=D // 8)
            for rs in [2 * Dv, 2 * Dv * 3 + 16 * 5, (1 << 26) - 16]:
                check_tile(LWV, Lk, k0, rs, ks_swz_v, KBN, KNW, real=Dv // 8)


@pytest.mark.parametrize("D,Dv", KS_PAIRS)
def test_key_split_lds_operand_offsets(D, Dv):
    # K operand reads fold four lane offsets plus constants; V^T transposed reads fold
    # eight lane offsets plus 256 bytes for the upper output blocks (256-wide layout)
    # and 16 rows for the second read. Both against the direct row * RB + swizzled
    # chunk formula, and each read lands on a slot that holds the real chunk it wants.
    LW, LWV = ks_layout(D), ks_layout(Dv)
    RB, RBV, SUB = 2 * LW, 2 * LWV, 32
    for kl in (0, 1):
        for lane in range(64):
            col, kg = lane % 16, lane // 16
            kb4 = [(SUB * kl + col) * RB + (((4 * c + kg) ^ ks_swz_k(LW, SUB * kl + col)) * 16) for c in range(4)]
            for c in range(-(-D // 32)):
                for nb in range(2):
                    if LW <= 128:
                        folded = kb4[c] + nb * (16 * RB)
                    else:
                        folded = (kb4[c] + nb * (16 * RB + 256) if c < 4
                                  else kb4[c - 4] + 256 + nb * (16 * RB - 256))
                    row = SUB * kl + 16 * nb + col
                    slot = (4 * c + kg) ^ ks_swz_k(LW, row)
                    assert slot < LW // 8
                    held = src_chunk(slot ^ ks_swz_k(LW, row), D // 8)
                    if 4 * c + kg < D // 8:
                        # the slot holds, as loaded, the chunk it is read for
                        assert held == 4 * c + kg
                    else:
                        # past an 80-wide row: a real chunk, against query elements the
                        # kernel loads as zeros (32c + 8kg onwards, at or past D)
                        assert held < D // 8 and 32 * c + 8 * kg >= D
                    assert folded == row * RB + slot * 16, (kl, lane, c, nb)
            vr = lane >> 2
            vsw = ks_swz_v(LWV, SUB * kl + vr) // 2
            vb8 = [(SUB * kl + vr) * RBV + ((2 * (d ^ vsw) + ((lane >> 1) & 1)) * 16) + (lane & 1) * 8
                   for d in range(8)]
            for db in range(Dv // 16):
                folded = vb8[db % 8] + (256 if db >= 8 else 0)
                for second in (0, 1):
                    row = SUB * kl + vr + 16 * second
                    # provider lane 4e + c of its 16-lane group: row 4g + e, columns 16 db + 4c
                    assert row - SUB * kl - 16 * second == 4 * (lane // 16) + (lane % 16) // 4
                    byte = 2 * (16 * db + 4 * (lane % 4))
                    slot = (byte // 16) ^ ks_swz_v(LWV, row)
                    assert src_chunk(slot ^ ks_swz_v(LWV, row), Dv // 8) == byte // 16 < Dv // 8
                    direct = row * RBV + slot * 16 + byte % 16
                    assert folded + 16 * RBV * second == direct, (kl, lane, db, second)
                    assert 0 <= direct and direct + 8 <= 64 * RBV
