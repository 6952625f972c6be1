"""The documented configuration menu of the grouped kernel, written out by the
tests as a specification.  The library's moe_variant_info / moe_cost_constants
are checked against it, and the oracle's cost-model inputs come from here (never
from the library)."""

# BLOCK_M, BLOCK_N gate/up, BLOCK_N down, BLOCK_K, waves M, N, K-split, split-K,
# streaming (non-temporal) weight loads, workgroups per CU, threads per workgroup
MENU = [
    (16, 16, 16, 256, 1, 1, 4, 1, 1, 2, 256),
    (32, 32, 32, 128, 1, 2, 2, 1, 1, 2, 256),
    (64, 64, 64, 64, 2, 2, 1, 1, 1, 2, 256),
    (128, 64, 128, 64, 2, 2, 1, 1, 0, 2, 256),
    (256, 128, 256, 32, 2, 2, 1, 1, 0, 1, 256),
    (16, 32, 32, 128, 1, 2, 2, 1, 1, 2, 256),
    (32, 16, 32, 256, 1, 1, 4, 1, 1, 2, 256),
    (64, 32, 64, 128, 2, 2, 1, 1, 1, 2, 256),
    (32, 64, 64, 64, 1, 4, 1, 1, 1, 2, 256),
    (64, 64, 64, 64, 2, 2, 1, 1, 0, 2, 256),
    (128, 64, 128, 64, 2, 2, 1, 1, 1, 2, 256),
    (32, 32, 32, 128, 1, 2, 2, 1, 0, 2, 256),
]
# workgroups per compute unit of the streaming class's persistent launch
WG_PER_CU = (2, 2)


def cost_constants(hidden: int, inter: int, num_cus: int) -> dict:
    """b, q1, q2, S1, S2 per configuration, per the definitions in include/moe.h:
    S = the persistent grid of the configuration's class."""
    grid = [min(num_cus * m[9], MAX_GRID) for m in MENU]
    return {
        "b": [m[0] for m in MENU],
        "q1": [-(-inter // m[1]) for m in MENU],
        "q2": [-(-hidden // m[2]) * m[7] for m in MENU],
        "S1": grid,
        "S2": grid,
    }


# The persistent grouped-FFN grid: min(CUs * workgroups per CU, MAX_GRID).
MAX_GRID = 512


def splits_tail(r: int, grid: int, stream: int, full_rounds: int = 0) -> bool:
    """Whether a streaming-class phase's last r (< grid) tiles are split by
    reduction stages across the whole grid (hybrid Stream-K): for streaming
    configurations when fewer than three quarters of the workgroups would be busy;
    for the cached one when the idle share of an unsplit phase,
    (grid - r) / (grid (F + 1)), exceeds one tenth.  The wide class never splits."""
    if r <= 0:
        return False
    if stream:
        return 4 * r < 3 * grid
    return 10 * (grid - r) > grid * (full_rounds + 1)


# The wide configuration (one workgroup per CU): BLOCK_M 256, BLOCK_N 256 in the
# down phase, 32-deep stages.  Its down phase splits the last round's tiles
# (include/moe.h, moe_grouped_down): after F >= 1 full rounds of the wide grid, a
# tail of 0 < r <= grid / 2 tiles is cut into P = min(grid // r, nst // 8) pieces
# per tile (no split when P < 2), nst = I / 32 stages per tile, which must be a
# multiple of 4 and at least 8.
WIDE = next(v for v, m in enumerate(MENU) if m[9] == 1)


def wide_pieces(total: int, grid: int, nst: int) -> int:
    F, r = divmod(total, grid)
    if F < 1 or r <= 0 or 2 * r > grid or nst % 4 or nst < 8:
        return 0
    P = min(grid // r, nst // 8)
    return P if P >= 2 else 0


def expert_major_tile(t: int, block_expert, ncol: int):
    """(row-block, column tile) of the wide configuration's tile t: the row-blocks
    of one expert form a run, and a run's tiles go column tile by column tile with
    its row-blocks fastest (block experts ascending, as the alignment step writes
    them)."""
    be = list(block_expert)
    b = t // ncol
    e = be[b]
    s0 = be.index(e)
    n = sum(1 for x in be if x == e)
    local = t - s0 * ncol
    return s0 + local % n, local // n


def pack_wide_bytes(E: int, H: int, I: int) -> int:
    """Bytes of the wide configuration's packed weight copy (include/moe.h,
    moe_pack_wide) for E experts: gate/up blocks of 128 W1 rows and 128 W3 rows,
    then down blocks of 256 W2 rows, each 32 bf16 values deep."""
    return 2 * E * (-(-I // 128) * 128) * H * 2 + E * (-(-H // 256) * 256) * I * 2


def pack_wide(w1, w3, w2):
    """The packed copy as uint16 words, written out from the header's description:
    per expert, per column tile, per 32-deep block, 256 rows of 32 values (rows past
    the matrix's end are zeros); gate/up for every expert first, then down."""
    import numpy as np
    E, I, H = w1.shape
    out = []
    for e in range(E):
        for n in range(-(-I // 128)):
            for kb in range(H // 32):
                blk = np.zeros((256, 32), np.uint16)
                r1 = w1[e, n * 128:(n + 1) * 128, kb * 32:(kb + 1) * 32]
                r3 = w3[e, n * 128:(n + 1) * 128, kb * 32:(kb + 1) * 32]
                blk[:r1.shape[0]] = r1
                blk[128:128 + r3.shape[0]] = r3
                out.append(blk)
    for e in range(E):
        for n in range(-(-H // 256)):
            for kb in range(I // 32):
                blk = np.zeros((256, 32), np.uint16)
                r2 = w2[e, n * 256:(n + 1) * 256, kb * 32:(kb + 1) * 32]
                blk[:r2.shape[0]] = r2
                out.append(blk)
    return np.concatenate([b.ravel() for b in out])
