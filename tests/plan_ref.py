"""The split plan written out from its definition (include/mla_decode.h, "Split plan"), for
checking the plan the device makes.  Test infrastructure: pure Python, no GPU.

Every sequence with p_b = ceil(L_b / 64) pages is cut into ceil(p_b / c) items of c pages; c
is the smallest page count whose item count fits the target (or the longest sequence's pages
when none does), or ceil(ceil(max_seqlen / 64) / n) when n splits are forced; one item per
slot, slots in item order or XCD-major.
"""

from __future__ import annotations

import numpy as np


def _cdiv(a, b):
    return -(-a // b)


def expected_plan(lens, max_seqlen, target, slots, forced=0, xcd_major=False):
    lens = [min(max(int(L), 0), max_seqlen) for L in lens]
    B = len(lens)
    items = []  # (b, t0, t1, slot)
    work = np.tile(np.array([-1, 0, 0, -1], np.int64), (slots, 1))
    slot_end = np.zeros(slots, np.int64)
    pages = [_cdiv(L, 64) for L in lens]
    if forced:
        c = _cdiv(max(1, _cdiv(max_seqlen, 64)), forced)
    else:
        maxp = max(max(pages), 1)
        count = lambda cc: sum(_cdiv(p, cc) for p in pages)
        c = next((cc for cc in range(1, maxp + 1) if count(cc) <= target), maxp)
    for b, L in enumerate(lens):
        for j in range(_cdiv(pages[b], c)):
            t0 = j * c * 64
            items.append([b, t0, min(L, t0 + c * 64), -1])
    W = len(items)
    per = _cdiv(W, 8)
    for s in range(slots):
        item = s
        if xcd_major:
            x, g = s % 8, s // 8
            item = x * per + g if g < per else W
        if item < W:
            items[item][3] = s
            work[s] = (*items[item][:3], item)
            slot_end[s] = item + 1
    pages_per_item = c
    n_of = np.zeros(B, np.int64)
    for it in items:
        n_of[it[0]] += 1
    split_off = np.concatenate([[0], np.cumsum(n_of)]).astype(np.int64)
    return {"items": len(items), "pages": pages_per_item, "slots": slots,
            "target": 0 if forced else target,
            "work": work, "slot_end": slot_end,
            "item_table": np.array(items, np.int64).reshape(-1, 4), "split_off": split_off}


def check_plan(got, want):
    """Every table of the device's plan equals the one worked out from the definition."""
    for k in ("items", "pages", "slots", "target"):
        assert int(got[k]) == int(want[k]), (k, got[k], want[k])
    assert np.array_equal(np.asarray(got["split_off"], np.int64), want["split_off"]), "split_off"
    assert np.array_equal(np.asarray(got["item_table"], np.int64), want["item_table"]), "items"
    assert np.array_equal(np.asarray(got["work"], np.int64), want["work"]), "work"
    assert np.array_equal(np.asarray(got["slot_end"], np.int64), want["slot_end"]), "slot_end"
