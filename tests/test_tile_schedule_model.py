"""CPU model of the grouped GEMM's persistent tile schedule (gemm.hip): the
two tile lists (full tiles, and a segment's last tile when it fills at most
half of the block's rows), the run-time choice between one and two lists,
the per-XCD ranges of each list, and the decode of a tile id into (K slice,
segment, n-tile, m-tile).  The model follows the kernel's integer
arithmetic step by step; every tile of every segment must be visited
exactly once, for any grid size, K split and mix of segment lengths.  The
weight-gradient mode's schedule (XCD ranges split by k-tiles, m-tiles or
n-tiles fastest) is modelled the same way."""
import random

import pytest

BM = 256


def schedule(rows, NT, nsplit, grid):
    nseg = len(rows)
    nslots = grid >> 3
    heavy = [r // BM + (1 if r % BM > BM // 2 else 0) for r in rows]
    light = [1 if 0 < r % BM <= BM // 2 else 0 for r in rows]
    pre_h, pre_l = [0], [0]
    for s in range(nseg):
        pre_h.append(pre_h[-1] + heavy[s])
        pre_l.append(pre_l[-1] + light[s])
    h = pre_h[nseg] * NT * nsplit
    al = h + pre_l[nseg] * NT * nsplit
    two = ((h + 7) // 8 + nslots - 1) // nslots < ((al + 7) // 8 + nslots - 1) // nslots
    seg_tile = pre_h if two else [a + b for a, b in zip(pre_h, pre_l)]
    seg_lt = pre_l if two else [0] * (nseg + 1)
    tiles, ltiles = seg_tile[nseg] * NT, seg_lt[nseg] * NT
    nheavy, nlight = tiles * nsplit, ltiles * nsplit
    per, lper = (nheavy + 7) >> 3, (nlight + 7) >> 3
    seen = []
    for b in range(grid):
        xcd = b & 7
        hlen = min(max(nheavy - xcd * per, 0), per)
        llen = min(max(nlight - xcd * lper, 0), lper)
        it = b >> 3
        while True:
            i = it
            if i < hlen:
                LL = xcd * per + i
            elif i - hlen < llen:
                LL = nheavy + xcd * lper + (i - hlen)
            else:
                break
            lt = LL >= nheavy
            P = seg_lt if lt else seg_tile
            k = LL - (nheavy if lt else 0)
            tl = ltiles if lt else tiles
            ks = k // tl
            L = k - ks * tl
            found = [s for s in range(nseg) if P[s] * NT <= L < P[s + 1] * NT]
            assert len(found) == 1
            s = found[0]
            hm = seg_tile[s + 1] - seg_tile[s]
            m = 1 if lt else hm
            local = L - P[s] * NT
            seen.append((ks, s, local // m, local % m + (hm if lt else 0)))
            it += nslots
    return seen, two


def expected(rows, NT, nsplit):
    return sorted((ks, s, n, m) for ks in range(nsplit) for s, r in enumerate(rows)
                  for n in range(NT) for m in range((r + BM - 1) // BM))


@pytest.mark.parametrize("seed", range(4))
def test_every_tile_exactly_once(seed):
    rng = random.Random(seed)
    both = set()
    for _ in range(150):
        nseg = rng.randint(1, 130 if rng.random() < 0.1 else 12)
        rows = [rng.choice([0, 1, 64, 128, 129, 255, 256, 257, 384, 385, 1000,
                            rng.randint(0, 3000)]) for _ in range(nseg)]
        NT, nsplit, grid = rng.randint(1, 20), rng.choice([1, 1, 2, 4]), 8 * rng.randint(1, 32)
        seen, two = schedule(rows, NT, nsplit, grid)
        assert sorted(seen) == expected(rows, NT, nsplit)
        both.add(two)
    assert both == {False, True}


def test_large_prefill_down_shape_takes_two_lists():
    """The routed row counts of the seeded large prefill run (8 experts, in
    ascending order; 16 n-tiles in the down projection): 64 full m-tiles
    fill exactly four rounds of 256 blocks and the five half-empty ones
    follow, instead of a fifth round of full tiles."""
    rows = [1991, 1996, 1997, 2050, 2052, 2080, 2086, 2132]
    assert sum(rows) == 8192 * 2
    seen, two = schedule(rows, 16, 1, 256)
    assert two and sorted(seen) == expected(rows, 16, 1)


def test_split_lists_case_takes_two_lists():
    """The GPU parity case relu_E64_T16384_split_lists routes (by the
    oracle's top-k on its seeded inputs) into 256 full m-tiles plus
    half-empty ones, which makes both of its grouped GEMMs (one 256-column
    tile each way, 256 blocks) take the two-list schedule."""
    import numpy as np
    import oracle as O
    from synth import RUNS, make_inputs, scaled, to_f64
    run = scaled(RUNS["gpt2"], T=16384, d_model=256, d_ff=128, num_experts=64, top_k=4,
                 activation="relu", capacity_factor=None)
    inp = make_inputs(run)
    logits = O.router_logits(to_f64(inp["x"]), to_f64(inp["w_router"]), to_f64(inp["b_router"]))
    idx = np.argsort(-logits, axis=1, kind="stable")[:, :run.top_k]
    rows = [int(c) for c in np.bincount(idx.ravel(), minlength=run.num_experts)]
    seen, two = schedule(rows, 1, 1, 256)
    assert two and sorted(seen) == expected(rows, 1, 1)


def wgrad_schedule(kpad, mtw, NT, grid, nfast):
    """The weight-gradient schedule: every segment has mtw m-tiles and NT
    n-tiles, each tile reducing over the segment's kpad padded rows; XCD x
    takes the tile ids whose k-tile midpoints fall in its eighth of all
    k-tiles, and a tile id decodes with the m-tiles fastest or, when nfast,
    the n-tiles fastest."""
    nseg = len(kpad)
    kpos = [0]
    for p in kpad:
        kpos.append(kpos[-1] + p)
    Ts = mtw * NT
    W = (kpos[nseg] // 32) * Ts
    G = 8
    nslots = grid >> 3
    seen = []
    for b in range(grid):
        xcd = b & 7
        rng = []
        for e in (0, 1):
            X0 = 2 * (xcd + e) * W
            cnt = 0
            for sg in range(nseg):
                w = (kpos[sg + 1] - kpos[sg]) // 32
                X = X0 - 2 * G * ((kpos[sg] // 32) * Ts)
                c = ((X - 1) // (G * w) + 1) // 2 if X >= 1 else 0
                cnt += min(c, Ts)
            rng.append(cnt)
        first, end = rng
        it = b >> 3
        while first + it < end:
            LL = first + it
            s = LL // Ts
            local = LL - s * Ts
            nt, mt = (local % NT, local // NT) if nfast else (local // mtw, local % mtw)
            assert nt < NT and mt < mtw
            seen.append((s, nt, mt))
            it += nslots
    return seen


@pytest.mark.parametrize("nfast", [False, True])
def test_wgrad_every_tile_exactly_once(nfast):
    rng = random.Random(5 + nfast)
    for _ in range(200):
        nseg = rng.randint(1, 70 if rng.random() < 0.2 else 10)
        kpad = [64 * rng.choice([1, 1, 2, 17, rng.randint(1, 300)]) for _ in range(nseg)]
        mtw, NT, grid = rng.randint(1, 12), rng.randint(1, 12), 8 * rng.randint(1, 32)
        seen = wgrad_schedule(kpad, mtw, NT, grid, nfast)
        assert sorted(seen) == sorted((s, n, m) for s in range(nseg) for n in range(NT)
                                      for m in range(mtw))
