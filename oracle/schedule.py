"""Reference of the split-KV scheduler's partition -- test infrastructure.

The scheduler is this library's own design (the pages only say that a tile
scheduler spreads requests and blocks evenly over the cores, FlashMLA page
"为什么 FlashMLA 的解码内核能跑到 660 TFLOPS", section 设计 5).  This plain
Python version of the same partition lets tests compare the GPU metadata
bit for bit and check its properties.

Cost line: unit u with nb_u > 0 blocks occupies nb_u + penalty positions;
block k of unit u sits at C_u + penalty + k (C = exclusive prefix of costs).
With T = max(1, ceil(total / P)), part p owns the blocks whose position lies
in [p*T, (p+1)*T).
"""

from __future__ import annotations

from typing import List, Tuple


def blocks_per_unit(seqlens, s_q: int, topk: int, page: int = 64) -> List[int]:
    if topk > 0:
        return [(topk + page - 1) // page] * (len(seqlens) * s_q)
    return [(max(int(L), 0) + page - 1) // page for L in seqlens]


def schedule(nb: List[int], num_parts: int, penalty: int) -> Tuple[List[List[int]], List[int]]:
    """Returns (sched rows of 8 ints, num_splits prefix of length U+1)."""
    U = len(nb)
    C = [0] * (U + 1)
    for u in range(U):
        C[u + 1] = C[u] + (nb[u] + penalty if nb[u] > 0 else 0)
    total = C[U]
    T = max(1, -(-total // num_parts))

    def first_block_at(x):
        for u in range(U):
            if C[u + 1] > x:
                return u, max(0, x - C[u] - penalty)
        return U, 0

    sched = []
    for p in range(num_parts):
        ub, kb = first_block_at(p * T)
        ue, ke = first_block_at((p + 1) * T)
        s0 = p - (C[ub] + penalty) // T if ub < U else 0
        sched.append([ub, kb, ue, ke, s0, T, penalty, 0])
    splits = [0] * (U + 1)
    for u in range(U):
        n = 0
        if nb[u] > 0:
            n = (C[u] + penalty + nb[u] - 1) // T - (C[u] + penalty) // T + 1
        splits[u + 1] = splits[u] + n
    return sched, splits


def segments(nb: List[int], sched_row: List[int]):
    """(unit, first_block, end_block, split_index) segments of one part."""
    ub, kb, ue, ke, s0 = sched_row[:5]
    out = []
    u = ub
    while u < len(nb) and (u < ue or (u == ue and ke > 0)):
        k0 = kb if u == ub else 0
        k1 = ke if u == ue else nb[u]
        if k0 < k1:
            out.append((u, k0, k1, s0 if u == ub else 0))
        u += 1
    return out
