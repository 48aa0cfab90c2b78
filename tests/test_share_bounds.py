"""Host replay of the balanced split's share arithmetic (decode_paged.hip,
paged_balanced_kernel): the work list is every (sequence, unit group, block),
cut into one contiguous share per workgroup in a virtual list where each
segment (sequence, unit group) is preceded by kSegmentCost empty items; the
shares are proportional to the workgroups' XCD weights once the list is long
enough, else equal and at least kMinPieceBlocks long.

A (b, h) gets one piece per share that holds blocks of its segment; the
workspace gives it ceil(blocks / 16) + 1 slots (api.cpp, plan), which the
replay checks over random batches, group counts and XCD weights.
"""

import numpy as np
import pytest

SEGMENT_COST = 4
MIN_PIECE = 16
ODD_SHARE = 1000


def bounds(vtotal, groups, even_share):
    """Virtual start of every share, k = 0 .. groups."""
    k = np.arange(groups + 1, dtype=np.int64)
    if vtotal >= groups * 2 * MIN_PIECE:
        weight = even_share * ((k + 1) // 2) + ODD_SHARE * (k // 2)
        return vtotal * weight // weight[-1]
    per = max(MIN_PIECE, -(-vtotal // groups))
    return np.minimum(vtotal, k * per)


def owners(lens, n_ug, groups, even_share):
    """For every segment (b, ug) with blocks, the share index of each block."""
    nb = -(-np.asarray(lens, dtype=np.int64) // 16)
    nonempty = (nb > 0).astype(np.int64)
    prefix = np.concatenate([[0], np.cumsum(nb)])
    seqs = np.concatenate([[0], np.cumsum(nonempty)])
    vprefix = n_ug * (prefix + SEGMENT_COST * seqs)
    bnd = bounds(int(vprefix[-1]), groups, even_share)
    out = []
    for b, n in enumerate(nb):
        if n == 0:
            continue
        for ug in range(n_ug):
            v = vprefix[b] + ug * (n + SEGMENT_COST) + SEGMENT_COST + np.arange(n)
            out.append(np.searchsorted(bnd, v, side="right") - 1)
    return out


def random_lens(rng):
    B = int(rng.integers(1, 200))
    kind = rng.integers(0, 3)
    if kind == 0:
        return rng.integers(0, 20000, B)
    if kind == 1:
        return rng.integers(0, 300, B)
    lens = rng.integers(0, 2000, B)
    lens[rng.integers(0, B)] = int(rng.integers(20000, 140000))
    return lens


@pytest.mark.parametrize("seed", range(6))
def test_pieces_per_row_within_workspace(seed):
    rng = np.random.default_rng(seed)
    for _ in range(50):
        lens = random_lens(rng)
        n_ug = int(rng.integers(1, 5))
        groups = int(rng.choice([64, 256, 512, 768]))
        even = int(rng.choice([1000, 1060, 1120]))
        for own in owners(lens, n_ug, groups, even):
            assert np.all(np.diff(own) >= 0)
            assert own[-1] - own[0] + 1 <= -(-len(own) // 16) + 1, (groups, even)


def test_every_block_has_one_share_and_shares_fill_the_list():
    # The GQA decode batch's shape of list (64 sequences, 512-8192 tokens)
    # on 256 eight-wave workgroups: every block lies in exactly one share,
    # the shares are contiguous and the even XCDs take the larger ones.
    rng = np.random.default_rng(7)
    lens = rng.integers(512, 8193, 64)
    own = np.concatenate(owners(lens, 1, 256, 1060))
    assert np.all(np.diff(own) >= 0)
    assert own[0] == 0 and own[-1] == 255
    sizes = np.bincount(own, minlength=256)
    assert sizes[0::2].mean() > sizes[1::2].mean()
