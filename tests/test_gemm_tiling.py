"""Host emulation of the prefill GEMM's index arithmetic (the 64-deep weight-block ring).

For real routings (the oracle's top-k and sort), every workgroup of the launch is mapped to
its work item the way the kernel does it (XCD-aware slices of the (group, N-tile, M-tile)
order), and every address the item forms is checked: activation and weight DMA sources
against their buffers (after the kernel's clamping), LDS destinations and operand reads
against their slots, output stores against the output.  The swizzle is checked to be a
bijection that the operand reads undo.  CPU only: this proves the launch geometry in bounds
before a GPU runs it.  The formulas are the kernel's, restated; see k_gemm.hip.
"""
import dataclasses

import numpy as np
import pytest

import moe_synth as S
from oracle import moe_oracle as O

TM = 128          # M-tile rows
RWN = 4           # wavefronts per workgroup, side by side over N
KSTEP = 32        # K per activation step
XCDS = 8


def routed_plan(wl, T, cf):
    """Counts, group offsets and the plan's tile list (group, first row) at tile height TM."""
    x = S.make_tokens(wl, T)
    L = S.make_layer(dataclasses.replace(wl, I=16))  # the router only
    ids, _ = O.route(O.router_logits(x, L.w_router, L.bias), wl.k, wl.renormalize)
    counts, offs, perm, _ = O.permute(ids, wl.E)
    offsets = list(offs) + [T * wl.k + s * T for s in range(1, wl.S + 1)]
    cap = int(np.ceil(cf * T * wl.k / wl.E)) if cf > 0 else 0
    touched = [e for e in range(wl.E) if counts[e] > 0] + [wl.E + s for s in range(wl.S)]
    tiles = []
    for g in touched:
        rows = (min(counts[g], cap) if cap else counts[g]) if g < wl.E else T
        tiles += [(g, m0) for m0 in range(0, rows, TM)]
    return np.asarray(offsets), np.asarray(perm), cap, tiles


def work_items(wl, T, N, n_blk, offsets, cap, tiles):
    """(g, r0, M, m0, n0) of every workgroup with work, and a check that each item of the
    (group, N-tile, M-tile) order is taken exactly once."""
    k, E, Sh = wl.k, wl.E, wl.S
    NT = -(-N // n_blk)
    bound = (T * k) // TM + min(T * k, E) + Sh * (-(-T // TM)) + 1
    max_tiles = (T * k) // 16 + E + Sh * (-(-T // 16)) + 1
    assert len(tiles) <= min(bound, max_tiles)
    grid = -(-(min(bound, max_tiles) * NT) // XCDS) * XCDS
    valid = len(tiles) * NT
    per = -(-valid // XCDS)
    wid = np.arange(grid)
    Lw = (wid % XCDS) * per + wid // XCDS
    live = (wid // XCDS < per) & (Lw < valid)
    Lw = Lw[live]
    assert np.array_equal(np.sort(Lw), np.arange(valid))
    tg = np.asarray([t[0] for t in tiles]); tm0 = np.asarray([t[1] for t in tiles])
    p = Lw // NT
    g = tg[p]
    r0 = offsets[g]
    M = offsets[g + 1] - r0
    if cap:
        M = np.where(g < E, np.minimum(M, cap), M)
    mt = -(-M // TM)
    first = p - tm0[p] // TM
    o = Lw - first * NT
    assert np.all((o >= 0) & (o < mt * NT))
    return g, r0, M, (o % mt) * TM, (o // mt) * n_blk


def check_item_addresses(wl, T, mode, tbn, w8, offsets, perm, cap, tiles):
    K, N = (wl.d, wl.I) if mode == 0 else (wl.I, wl.d)
    assert K % 64 == 0
    R = T * wl.k + wl.S * T
    n_blk = tbn // 2 if mode == 0 else tbn
    g, r0, M, m0, n0 = work_items(wl, T, N, n_blk, offsets, cap, tiles)
    ni = len(g)
    esz = 1 if w8 else 2
    ROW = 64 * esz                     # bytes of a weight row per 64-K block
    A_SLOT, B_SLOT = TM * 64, tbn * ROW
    LPR = ROW // 16; RPI = 64 // LPR; DMA_B = tbn // RPI // RWN
    swz = (lambda r: (r >> 2) & 3) if w8 else (lambda r: (r >> 1) & 7)
    wave = np.arange(RWN)[:, None]; lane = np.arange(64)[None, :]
    nk = K // KSTEP

    # activation DMA: two loads per wavefront per step
    for i in range(2):
        q = wave * 2 + i
        row = 16 * q + lane // 4                                 # (4, 64)
        assert np.all(q * 1024 + lane * 16 + 16 <= A_SLOT)
        chunk = (lane % 4) ^ ((row >> 2) & 3)
        assert np.all((nk - 1) * KSTEP + chunk * 8 + 8 <= K)
        m = np.minimum(m0[:, None, None] + row[None], (M - 1)[:, None, None])
        r = r0[:, None, None] + m
        assert np.all((r >= 0) & (r < R))
        if mode == 0:
            routed = (g < wl.E)[:, None, None]
            src = np.where(routed, perm[np.minimum(r, len(perm) - 1)] // wl.k, m)
            assert np.all((src >= 0) & (src < T))
    # weight DMA: DMA_B loads per wavefront per block
    for i in range(DMA_B):
        q = wave * DMA_B + i
        row = RPI * q + lane // LPR
        assert np.all(q * 1024 + lane * 16 + 16 <= B_SLOT)
        chunk = (lane % LPR) ^ swz(row)
        assert np.all((K // 64 - 1) * ROW + chunk * 16 + 16 <= K * esz)
        n = (row % (tbn // 2)) if mode == 0 else row
        n = np.minimum(n0[:, None, None] + n[None], N - 1)
        assert np.all((n >= 0) & (g[:, None, None] < wl.E + wl.S))
    # every 16-byte chunk of a row's block is fetched once, and the operand reads undo the
    # swizzle: logical chunk c of row r sits at physical chunk c ^ swz(r)
    for r in range(tbn):
        phys = np.arange(LPR); src = phys ^ swz(r)
        assert sorted(src) == list(range(LPR))
        assert all(src[c ^ swz(r)] == c for c in range(LPR))
    # operand reads inside the slots
    lr = lane % 16
    rd = ((lane // 16) ^ ((lr >> 2) & 3)) * 16
    for i in range(TM // 16):
        assert np.all((i * 16 + lr) * 64 + rd + 16 <= A_SLOT)
    tj = tbn // RWN // 16
    for j in range(tj):
        if mode == 0:
            brow = (0 if j < tj // 2 else tbn // 2) + wave * (tbn // RWN // 2) + (j % (tj // 2)) * 16 + lr
        else:
            brow = wave * (tbn // RWN) + j * 16 + lr
        for h in range(2):
            c = h * 4 + lane // 16
            off = (brow * ROW + ((c >> 1) ^ swz(brow)) * 16 + (c & 1) * 8 + 8) if w8 else \
                  (brow * ROW + (c ^ swz(brow)) * 16 + 16)
            assert np.all(off <= B_SLOT)
    # epilogue: 4 consecutive channels per lane, rows inside the group, channels inside N
    c4 = 4 * (lane // 16)
    for i in range(TM // 16):
        m = m0[:, None, None] + i * 16 + lr[None]
        inside = m < M[:, None, None]
        for j in range(tj // 2 if mode == 0 else tj):
            n = n0[:, None, None] + wave * (tbn // RWN // (2 if mode == 0 else 1)) + j * 16 + c4
            store = inside & (n < N)
            rows = np.broadcast_to(r0[:, None, None] + m, store.shape)[store]
            assert np.all(rows < R) and np.all(np.broadcast_to(n, store.shape)[store] + 4 <= N)
    return ni


CASES = [
    (S.DEEPSEEK_BF16, 2048, 0.0), (S.DEEPSEEK_BF16, 40, 0.0), (S.DEEPSEEK_BF16, 512, 1.0),
    (S.OLMOE_BF16, 300, 0.0), (S.OLMOE_STACK16, 2048, 2.0),
    # ragged N-tiles in both GEMMs (448 channels of gate/up, 320 of down)
    (S.Workload("tiling_ragged", 97, d=320, E=8, k=2, I=448, S=1, renormalize=True), 300, 0.0),
]


@pytest.mark.parametrize("wl,T,cf", CASES, ids=[f"{c[0].name}-T{c[1]}-cf{c[2]}" for c in CASES])
def test_ring64_addresses_stay_in_bounds(wl, T, cf):
    offsets, perm, cap, tiles = routed_plan(wl, T, cf)
    for mode in (0, 1):
        for tbn in (256, 128):
            for w8 in (False, True):
                assert check_item_addresses(wl, T, mode, tbn, w8, offsets, perm, cap, tiles) > 0


def test_emulation_catches_a_wrong_gather_rule():
    """The check is not vacuous: indexing x by sorted row instead of by token (the fault once
    made by a tile-width-dependent gather rule) reads past the end of x."""
    wl, T = S.DEEPSEEK_BF16, 512
    offsets, perm, cap, tiles = routed_plan(wl, T, 0.0)
    bad_perm = np.arange(len(perm)) * wl.k   # src = row index, not its token
    with pytest.raises(AssertionError):
        check_item_addresses(wl, T, 0, 256, False, offsets, bad_perm, cap, tiles)
