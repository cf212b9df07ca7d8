"""Model of the sparse selection kernel's top-512 (sparse_gqa.hip), on the CPU.

The kernel ranks candidate blocks by key = mono(score) - mono(min score),
mono being the order-preserving map of fp32 bits to uint32.  A radix
select in 11-bit digits, most significant first, finds the 512th largest
key T and how many keys equal to T are taken (`need`).  The compaction
then writes every block whose key is above T and the `need` lowest-id
blocks whose key equals T, ids ascending.  The scores never hold -0 (the
scoring kernel adds +0 before storing).  The test checks these steps
against the definition of [Step-5] "Die eigentliche Attention liest
weiterhin originale K/V" as the oracle reads it: the 512 highest scores,
equal scores ranked by lower block id.
"""

import numpy as np
import pytest

BUDGET, DIGIT = 512, 11


def mono(f):
    u = np.asarray(f, np.float32).view(np.uint32).astype(np.uint64)
    return np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000).astype(np.uint64)


def model(sc):
    R = len(sc)
    if R <= BUDGET:
        return list(range(R))
    m = mono(sc)
    lo, hi = int(m.min()), int(m.max())
    bits = (hi - lo).bit_length()
    key = m - lo
    passes = (bits + DIGIT - 1) // DIGIT
    prefix = mask = 0
    need = BUDGET
    for p in range(passes):
        shift = DIGIT * (passes - 1 - p)
        live = (key & mask) == prefix
        hist = np.bincount(((key[live] >> shift) & 2047).astype(np.int64), minlength=2048)
        above = 0
        for d in range(2047, -1, -1):
            if above < need <= above + hist[d]:
                pick, left = d, need - above
            above += hist[d]
        prefix |= (pick << shift) & 0xFFFFFFFF
        mask |= (2047 << shift) & 0xFFFFFFFF
        need = left
    out, eq_seen = [], 0
    for r in range(R):
        if key[r] > prefix:
            out.append(r)
        elif key[r] == prefix:
            if eq_seen < need:
                out.append(r)
            eq_seen += 1
    return out


def definition(sc):
    order = sorted(range(len(sc)), key=lambda r: (-float(sc[r]), r))
    return sorted(order[:BUDGET])


def scores(kind, R, rng):
    if kind == "normal":
        sc = rng.standard_normal(R)
    elif kind == "heavy_ties":
        sc = np.round(rng.standard_normal(R) * 2)
    elif kind == "all_equal":
        sc = np.full(R, 0.5)
    elif kind == "relu_zeros":
        sc = np.maximum(rng.standard_normal(R), 0)
    elif kind == "full_span":
        sc = rng.standard_normal(R) * 1e30
    else:  # ties exactly at the 512th score
        sc = rng.standard_normal(R).astype(np.float32)
        sc[rng.choice(R, 40, replace=False)] = np.sort(sc)[::-1][BUDGET - 1]
    return (np.asarray(sc, np.float32) + np.float32(0.0)).astype(np.float32)


@pytest.mark.parametrize("kind", ["normal", "heavy_ties", "all_equal", "relu_zeros",
                                  "full_span", "threshold_ties"])
def test_model_matches_the_sorted_definition(kind):
    rng = np.random.default_rng(7)
    for R in (513, 600, 1000, 2047, 4096):
        sc = scores(kind, R, rng)
        got = model(sc)
        assert len(got) == BUDGET
        assert got == definition(sc)


def test_at_most_the_budget_takes_every_candidate():
    assert model(np.zeros(512, np.float32)) == list(range(512))
