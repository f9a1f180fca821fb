"""Host model of the task-queue schedule of mixed batches (the setup
kernel's per-sequence item lists, the XCD shares of the prefill-type list
and the main kernel's item -> (sequence, q-block, KV head) mapping), checked
over random batches: every q-block of every KV head is claimed exactly once
whatever order the workgroups of the eight XCDs draw in, the prefill-type
list holds exactly the sequences with q_len * G > 32, each (sequence, KV
head)'s q-blocks come most-keys-first and, except where a share boundary
cuts it, inside one XCD share.  Mirrors queue_setup_kernel, draw_prefill and
queue_mixed; no GPU."""
import numpy as np
import pytest

KCOLS = 32
THREADS = 1024


def setup_lists(q_lens, G, Hkv, BQ):
    B = len(q_lens)
    per = (B + THREADS - 1) // THREADS
    npf = np.zeros(B, np.int64)
    ndc = np.zeros(B, np.int64)
    for j, ql in enumerate(q_lens):
        if ql <= 0:
            continue
        if ql * G > KCOLS:
            npf[j] = (ql + BQ - 1) // BQ * Hkv
        else:
            ndc[j] = Hkv
    # the kernel: per-thread chunk sums, an inclusive scan over 1024 threads,
    # then a sequential exclusive scan inside each chunk
    cp = np.array([npf[min(B, t * per):min(B, t * per + per)].sum() for t in range(THREADS)])
    cd = np.array([ndc[min(B, t * per):min(B, t * per + per)].sum() for t in range(THREADS)])
    sp, sd = np.cumsum(cp), np.cumsum(cd)
    offp = np.zeros(B + 1, np.int64)
    offd = np.zeros(B + 1, np.int64)
    for t in range(THREADS):
        ep, ed = sp[t] - cp[t], sd[t] - cd[t]
        for j in range(min(B, t * per), min(B, t * per + per)):
            offp[j], offd[j] = ep, ed
            ep += npf[j]
            ed += ndc[j]
    offp[B], offd[B] = sp[-1], sd[-1]
    return offp, offd


def claim(which, ks, off, q_lens, Hkv, BQ):
    """Items ks of one list -> (b, g, i0, ntok) arrays: b is the one sequence
    whose range [off[b], off[b+1]) holds k (the kernel finds it by testing
    every range)."""
    b = np.searchsorted(off, ks, side="right") - 1
    assert np.all((off[b] <= ks) & (ks < off[b + 1]))
    r = ks - off[b]
    ql = q_lens[b]
    if which == 0:
        nb = (ql + BQ - 1) // BQ
        g = r // nb
        i0 = (nb - 1 - (r - g * nb)) * BQ
        ntok = np.minimum(BQ, ql - i0)
    else:
        g, i0, ntok = r, np.zeros_like(r), ql
    return b, g, i0, ntok


@pytest.mark.parametrize("seed", range(12))
def test_queue_lists_cover_every_item_once(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 3, 17, 300, 1500, 2500]))
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    Hkv = int(rng.choice([1, 2, 8]))
    BQ = max(1, 128 // G)
    kind = rng.random(B)
    q_lens = np.where(kind < 0.15, 0, np.where(kind < 0.6, rng.integers(1, 3, B),
                                                rng.integers(1, 700, B))).astype(np.int64)
    offp, offd = setup_lists(q_lens, G, Hkv, BQ)
    seen = {}
    last_i0 = {}
    for which, off in ((0, offp), (1, offd)):
        ks = np.arange(int(off[-1]), dtype=np.int64)
        bs, gs, i0s, ntoks = claim(which, ks, off, q_lens, Hkv, BQ)
        assert np.all((gs >= 0) & (gs < Hkv) & (i0s >= 0) & (ntoks >= 1) & (i0s + ntoks <= q_lens[bs]))
        for b, g, i0 in zip(bs.tolist(), gs.tolist(), i0s.tolist()):
            key = (b, i0, g)
            assert key not in seen
            seen[key] = which
            # q-blocks of one (sequence, head): most keys first
            if (b, g) in last_i0:
                assert i0 < last_i0[(b, g)]
            last_i0[(b, g)] = i0
    want = {}
    for b, ql in enumerate(q_lens):
        if ql <= 0:
            continue
        if ql * G > KCOLS:
            for qb in range((ql + BQ - 1) // BQ):
                for g in range(Hkv):
                    want[(b, qb * BQ, g)] = 0
        else:
            for g in range(Hkv):
                want[(b, 0, g)] = 1
    assert seen == want


SHARES = 8


def share_bounds(n):
    return [(y * n // SHARES, (y + 1) * n // SHARES) for y in range(SHARES)]


def draw_prefill(ctr, n, xcd):
    """draw_prefill of the kernel: the own share first, then the others."""
    for s in range(SHARES):
        y = (xcd + s) % SHARES
        lo, hi = y * n // SHARES, (y + 1) * n // SHARES
        if lo >= hi:
            continue
        k = ctr[y]
        ctr[y] += 1
        if lo + k < hi:
            return lo + k
    return -1


@pytest.mark.parametrize("seed", range(8))
def test_xcd_shares_claim_every_prefill_item_once(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.choice([0, 1, 5, 7, 8, 9, 100, 2048, 2051]))
    ctr = [0] * SHARES
    got = []
    # workgroups of random XCDs draw until every list is empty; an empty
    # draw ends that workgroup, as in the kernel
    alive = list(range(512))
    while alive:
        w = alive[int(rng.integers(0, len(alive)))]
        k = draw_prefill(ctr, n, w % SHARES)
        if k < 0:
            alive.remove(w)
        else:
            got.append(k)
    assert sorted(got) == list(range(n))
    assert sum(hi - lo for lo, hi in share_bounds(n)) == n


def test_mixed_24b_pairs_stay_in_one_share():
    # the serving mix: 8 prefill chunks of 1000 tokens (q-blocks of 32 at
    # G = 4) and 248 decode rows; each (sequence, KV head)'s 32 q-blocks are
    # contiguous in the prefill list, so a share boundary cuts at most one
    # pair per share
    q_lens = np.array([1000] * 8 + [1] * 248, np.int64)
    Hkv, BQ = 8, 32
    offp, _ = setup_lists(q_lens, 4, Hkv, BQ)
    n = int(offp[-1])
    ks = np.arange(n, dtype=np.int64)
    b, g, i0, _ = claim(0, ks, offp, q_lens, Hkv, BQ)
    share = np.zeros(n, np.int64)
    for y, (lo, hi) in enumerate(share_bounds(n)):
        share[lo:hi] = y
    pairs = {}
    for bb, gg, yy in zip(b.tolist(), g.tolist(), share.tolist()):
        pairs.setdefault((bb, gg), set()).add(yy)
    assert len(pairs) == 64
    assert sum(len(v) > 1 for v in pairs.values()) <= SHARES - 1
