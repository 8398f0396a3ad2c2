"""The group-maxima selection's bound, checked on the CPU.

The device selection (group_select_kernel) takes a lower bound L on T, the k-th largest group
maximum, from the first 12-bit digit of the group keys: d is the digit at which the count of
group keys from the top reaches k, and L = d << 52.  It then re-reads only the groups whose keys
reach L and selects among their keys >= L.  That is exact because k distinct keys reach T >= L,
so every top-k key is >= L and its group's maximum is too.  When too many groups or candidates
pass, it uses the exact T (and a second radix select).  This test runs that control flow in
NumPy (host logic, no GPU) and compares the result with the oracle's stable top-k on rows that
take every branch.  A mistake in the bound (the crossing digit off by one, a strict comparison,
a group admitted by its first logit instead of its maximum) fails it.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle

ADMIT_MAX = 256  # groups the bound may admit
RANK_MAX = 256   # candidates ranked directly


def keys_of(v):
    """64-bit keys orderable(value) << 32 | ~index: unsigned order = value desc, lower index first."""
    u = v.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = np.where(u == 0x80000000, np.uint64(0), u)  # -0.0 == +0.0
    u = np.where(u & np.uint64(0x80000000), (~u) & np.uint64(0xFFFFFFFF), u | np.uint64(0x80000000))
    idx = np.arange(len(v), dtype=np.uint64)
    return (u << np.uint64(32)) | ((~idx) & np.uint64(0xFFFFFFFF))


def select(v, k, gs=64):
    """Returns (indices of the top k, branch names taken)."""
    key = keys_of(v)
    gkeys = np.array([key[g:g + gs].max() for g in range(0, len(v), gs)], dtype=np.uint64)
    taken = []
    if k <= len(gkeys):
        digit = (gkeys >> np.uint64(52)).astype(np.int64)
        counts = np.bincount(digit, minlength=4096)
        above = np.concatenate([np.cumsum(counts[::-1])[::-1][1:], [0]])  # keys in higher digits
        d = int(np.nonzero(above + counts >= k)[0].max())  # the crossing digit from the top
        admitted = int(above[d] + counts[d])
        if admitted <= ADMIT_MAX:
            T = np.uint64(d) << np.uint64(52)
            taken.append("bound")
        else:
            T = np.sort(gkeys)[::-1][k - 1]
            taken.append("exact")
    else:
        T = np.uint64(0)
        taken.append("all groups")
    groups = np.nonzero(gkeys >= T)[0]
    cand = np.concatenate([key[g * gs:(g + 1) * gs] for g in groups])
    cand = cand[cand >= T]
    assert len(cand) >= k
    taken.append("rank" if len(cand) <= RANK_MAX else "second select")
    top = np.sort(cand)[::-1][:k]
    return ((~top) & np.uint64(0xFFFFFFFF)).astype(np.int64), taken


def rows():
    r = np.random.default_rng(3)
    v = 151936
    out = [("normal", (r.standard_normal(v) * 0.9).astype(np.float32), 40),
           ("all equal", np.full(v, 1.5, np.float32), 40),
           ("ramp", np.arange(v, dtype=np.float32) / v, 64),
           ("signed zeros", np.where(r.random(v) < 0.5, np.float32(-0.0), np.float32(0.0)), 7)]
    x = (r.standard_normal(v) * 0.1).astype(np.float32)
    x[: 100 * 64] = 7.0  # 100 groups of equal maxima: admitted, too many candidates
    out.append(("100 full groups", x, 40))
    x = (r.standard_normal(v) * 0.1).astype(np.float32)
    x[::64][:300] = 7.0  # 300 groups share the first digit: more than the bound may admit
    out.append(("300 groups", x, 40))
    x = (r.standard_normal(v) * 0.1).astype(np.float32)
    x[np.sort(r.choice(v // 64, 40, replace=False)) * 64 + 3] = 7.0 + np.arange(40) / 64
    out.append(("the top in 40 groups' third logits", x, 40))
    out.append(("fewer groups than k", (r.standard_normal(130) * 0.9).astype(np.float32), 5))
    return out


@pytest.mark.parametrize("name,v,k", rows(), ids=[r[0] for r in rows()])
def test_bound_selection_matches_the_oracle(name, v, k):
    got, taken = select(v, k)
    exp = oracle.topk_ref(v[None, :], k)[0][0]
    assert np.array_equal(got, exp), (name, taken)


def test_every_branch_is_taken():
    seen = set()
    for _, v, k in rows():
        seen.update(select(v, k)[1])
    assert seen == {"bound", "exact", "all groups", "rank", "second select"}
