"""Host emulation of the index arithmetic of the grouped FFN's other kernels.

tests/test_gemm_tiling.py covers the 64-deep weight-block ring GEMM.  Here the same is done
for the 32-deep ring GEMM (K % 64 == 32), the general GEMM (K not a multiple of 32), the VALU
decode GEMV (every channel-group / K-step / row-chunk instance its dispatcher picks) and the
matrix-core GEMV: for real routings (the oracle's top-k and sort, with and without a capacity
limit) every workgroup is mapped to its work the way the kernel does it, and every global load,
LDS offset and store the work forms is checked against its buffer.  CPU only: the launch
geometry is proved in bounds before a GPU runs it.  The formulas are the kernels' own,
restated (k_gemm.hip, k_gemv.hip).
"""
import dataclasses

import numpy as np
import pytest

import moe_synth as S
from oracle import moe_oracle as O
from tests.test_gemm_tiling import XCDS, routed_plan, work_items

TM = 128


# ------------------------------------------------------------------------------------------
# shared pieces
# ------------------------------------------------------------------------------------------
def a_rows(wl, T, mode, g, r0, M, m, perm):
    """Source row of the A operand for tile rows m (clamped into the group): a token of x for
    gate/up (through perm for a routed expert), a row of h for down."""
    m = np.minimum(m, M - 1)
    r = r0 + m
    R = T * wl.k + wl.S * T
    assert np.all((r >= 0) & (r < R))
    if mode == 1:
        return r, R
    routed = g < wl.E
    src = np.where(routed, perm[np.minimum(r, len(perm) - 1)] // wl.k, m)
    return src, T


def epilogue_rows(wl, T, r0, M, m):
    R = T * wl.k + wl.S * T
    inside = m < M
    rows = (r0 + m)[inside]
    assert np.all(rows < R)
    return inside


# ------------------------------------------------------------------------------------------
# k_gemm_ring: 32-deep ring (K a multiple of 32)
# ------------------------------------------------------------------------------------------
def check_ring32(wl, T, mode, tbn, w8, offsets, perm, cap, tiles):
    K, N = (wl.d, wl.I) if mode == 0 else (wl.I, wl.d)
    assert K % 32 == 0
    n_blk = tbn // 2 if mode == 0 else tbn
    g, r0, M, m0, n0 = work_items(wl, T, N, n_blk, offsets, cap, tiles)
    g, r0, M, m0, n0 = (v[:, None, None] for v in (g, r0, M, m0, n0))
    esz = 1 if w8 else 2
    ROW = 32 * esz
    A_BYTES = TM * 32 * 2
    STAGE = A_BYTES + tbn * ROW
    LPR = ROW // 16
    RPI = 64 // LPR
    DMA = tbn // RPI // 4
    TJ = tbn // 4 // 16
    nk = K // 32
    wave = np.arange(4)[:, None]
    lane = np.arange(64)[None, :]
    lr = lane % 16
    # activation DMA: two loads per wavefront per stage
    for i in range(2):
        row = 16 * (wave * 2 + i) + lane // 4
        assert np.all((wave * 2 + i) * 1024 + lane * 16 + 16 <= A_BYTES)
        ca = ((lane % 4) ^ ((row >> 2) & 3)) * 8
        assert np.all((nk - 1) * 32 + ca + 8 <= K)
        src, rows = a_rows(wl, T, mode, g, r0, M, m0 + row[None], perm)
        assert np.all((src >= 0) & (src < rows))
    # weight DMA
    for i in range(DMA):
        row = RPI * (wave * DMA + i) + lane // LPR
        assert np.all(A_BYTES + (wave * DMA + i) * 1024 + lane * 16 + 16 <= STAGE)
        cb = (((lane % 2) ^ ((row >> 3) & 1)) if w8 else ((lane % 4) ^ ((row >> 2) & 3))) * 16
        assert np.all((nk - 1) * 32 * esz + cb + 16 <= K * esz)
        n = (row % (tbn // 2)) if mode == 0 else row
        n = np.minimum(n0 + n[None], N - 1)
        assert np.all((n >= 0) & (n < N) & (g < wl.E + wl.S))
    # the source-side swizzles are bijections the operand reads undo
    for r in range(tbn):
        if w8:
            phys = np.arange(2) ^ ((r >> 3) & 1)
            assert sorted(phys) == [0, 1]
        else:
            phys = np.arange(4) ^ ((r >> 2) & 3)
            assert sorted(phys) == [0, 1, 2, 3]
    # operand reads
    rd = ((lane // 16) ^ ((lr >> 2) & 3)) * 16
    for i in range(TM // 16):
        assert np.all((i * 16 + lr) * 64 + rd + 16 <= A_BYTES)
    for j in range(TJ):
        if mode == 0:
            brow = (0 if j < TJ // 2 else tbn // 2) + wave * (tbn // 8) + (j % (TJ // 2)) * 16 + lr
        else:
            brow = wave * (tbn // 4) + j * 16 + lr
        c = lane // 16
        if w8:
            off = A_BYTES + brow * 32 + (((c >> 1) ^ ((brow >> 3) & 1)) * 16) + (c & 1) * 8 + 8
        else:
            off = A_BYTES + brow * 64 + rd + 16
        assert np.all(off <= STAGE)
    # epilogue: 4 consecutive channels per lane
    c4 = 4 * (lane // 16)
    for i in range(TM // 16):
        m = m0 + i * 16 + lr[None]
        inside = epilogue_rows(wl, T, r0, M, m)
        for j in range(TJ // 2 if mode == 0 else TJ):
            n = n0 + wave * (tbn // 4 // (2 if mode == 0 else 1)) + j * 16 + c4
            st = inside & (n < N)
            assert np.all(np.broadcast_to(n, st.shape)[st] + 4 <= N)
    return g.shape[0]


# ------------------------------------------------------------------------------------------
# k_gemm: the general kernel (any K that is a multiple of 16)
# ------------------------------------------------------------------------------------------
def check_general(wl, T, mode, w8, offsets, perm, cap, tiles):
    K, N = (wl.d, wl.I) if mode == 0 else (wl.I, wl.d)
    assert K % 16 == 0
    BN, BK, PITCH = 128, 64, 72
    n_blk = BN // 2 if mode == 0 else BN
    g, r0, M, m0, n0 = work_items(wl, T, N, n_blk, offsets, cap, tiles)
    g, r0, M, m0, n0 = (v[:, None] for v in (g, r0, M, m0, n0))
    A_ELEMS = B_ELEMS = TM * PITCH
    tid = np.arange(256)[None, :]
    nk = -(-K // BK)
    cols = np.arange(nk) * BK
    # A loads: 4 rows per thread, chunk tid % 8 (8 elements), guarded by col < K
    for i in range(4):
        row = tid // 8 + 32 * i
        src, rows = a_rows(wl, T, mode, g, r0, M, m0 + row, perm)
        assert np.all((src >= 0) & (src < rows))
        col = cols[:, None] + (tid % 8) * 8                         # (nk, 256)
        assert np.all(col[col < K] + 8 <= K)
        assert np.all(row * PITCH + (tid % 8) * 8 + 8 <= A_ELEMS)
    # B loads: int8 4 chunks of 16 per row, bf16 8 chunks of 8
    cpr = 4 if w8 else 8
    for i in range(128 * cpr // 256):
        row = tid // cpr + (256 // cpr) * i
        n = (row % (BN // 2)) if mode == 0 else row
        n = np.minimum(n0 + n, N - 1)
        assert np.all((n >= 0) & (n < N))
        step = 16 if w8 else 8
        col = cols[:, None] + (tid % cpr) * step
        assert np.all(col[col < K] + step <= K)
        assert np.all(row * PITCH + (tid % cpr) * (16 if w8 else 8) + (16 if w8 else 8) <= B_ELEMS)
    # operand reads: 2 x 2 wavefronts of 64 x 64
    lane = np.arange(64)
    lr, lk = lane % 16, (lane // 16) * 8
    for wv in range(4):
        wm, wn = wv // 2, wv % 2
        for ks in (0, 32):
            for i in range(4):
                assert np.all((wm * 64 + i * 16 + lr) * PITCH + ks + lk + 8 <= A_ELEMS)
            for j in range(4):
                brow = ((0 if j < 2 else BN // 2) + wn * 32 + (j % 2) * 16 + lr) if mode == 0 \
                    else (wn * 64 + j * 16 + lr)
                assert np.all(brow * PITCH + ks + lk + 8 <= B_ELEMS)
        # epilogue: element stores
        for i in range(4):
            for v in range(4):
                m = m0 + wm * 64 + i * 16 + (lane[None] // 16) * 4 + v
                inside = epilogue_rows(wl, T, r0, M, m)
                for j in range(2 if mode == 0 else 4):
                    n = n0 + (wn * 32 if mode == 0 else wn * 64) + j * 16 + lr[None]
                    st = inside & (n < N)
                    assert np.all(np.broadcast_to(n, st.shape)[st] < N)
    return g.shape[0]


# ------------------------------------------------------------------------------------------
# the GEMVs: touched groups of the plan, one block per (N-block, group)
# ------------------------------------------------------------------------------------------
def touched_groups(wl, T, offsets, cap):
    E = wl.E
    counts = np.diff(offsets)[:E]
    g = [e for e in range(E) if counts[e] > 0] + [E + s for s in range(wl.S)]
    r0 = offsets[g]
    M = offsets[np.asarray(g) + 1] - r0
    if cap:
        M = np.where(np.asarray(g) < E, np.minimum(M, cap), M)
    slots = min(T * wl.k, E) + wl.S
    assert len(g) <= slots
    return np.asarray(g), r0, M


def gemv_instance(mode, T, K, wdt, act):
    """(CPG, MAXIT, MB) of the VALU GEMV for this matrix, as its dispatcher picks them."""
    V = {"f32": 4, "bf16": 8, "i8": 16}[wdt if act != "f32" else "f32"]
    nmat = 2 if mode == 0 else 1
    steps = -(-K // (8 * V))
    spw = -(-steps // 4)
    if spw <= 2:
        return (4 if nmat == 2 else 2), 2, 4
    if spw <= 4:
        c = 1 if (nmat == 1 or V == 16) else 2
        return c, 4, (1 if T == 1 else 2 if T == 2 else 4)
    if spw <= 8:
        if T <= 2:
            return 1, 8, T
        if T <= 4:
            return 1, 8, 4
        return 1, 8, (8 if mode == 0 else 4)
    return (1 if nmat == 2 else 2), 8, 8


def check_gemv(wl, T, mode, offsets, perm, cap):
    K, N = (wl.d, wl.I) if mode == 0 else (wl.I, wl.d)
    act = wl.act
    wdt = wl.wdt
    asz = 4 if act == "f32" else 2
    V = {"f32": 4, "bf16": 8, "i8": 16}[wdt if act != "f32" else "f32"]
    CPG, MAXIT, MB = gemv_instance(mode, T, K, wdt, act)
    STEP = 8 * V
    ROUND = 4 * MAXIT * STEP
    mb_max = min(T, MB)
    lds = mb_max * ROUND * asz
    row_bytes = ROUND * asz
    R = T * wl.k + wl.S * T
    G = wl.E + wl.S
    g, r0, M = touched_groups(wl, T, offsets, cap)
    NB = 8 * CPG
    lane = np.arange(64)
    q, lg = lane % 8, lane // 8
    rounds = -(-K // ROUND)
    for n0 in range(0, N, NB):
        for c in range(CPG):
            ch = np.minimum(n0 + c * 8 + lg, N - 1)
            assert np.all((g[:, None] * N + ch[None]) < G * N)
        for rd in range(rounds):
            k_round = rd * ROUND
            cols = min(ROUND, K - k_round)
            steps = -(-cols // STEP)
            spw = -(-steps // 4)
            chunks = cols * asz // 16
            ipr = -(-chunks // 64)
            for wave in range(4):
                s_lo, s_hi = wave * spw, min(steps, wave * spw + spw)
                for it in range(MAXIT):
                    col = k_round + (s_lo + it) * STEP + q * V
                    ok = (s_lo + it < s_hi) & (col < K)
                    assert np.all(col[ok] + V <= K)                    # weight load
                    xcol = (s_lo + it) * STEP + q * V                  # math read of a row
                    rd_bytes = 32 if V == 16 else 16
                    okx = (s_lo + it < s_hi) & (xcol < cols)
                    assert np.all(xcol[okx] * asz + (mb_max - 1) * row_bytes + rd_bytes <= lds)
        # row staging and stores, per group
        for gi in range(len(g)):
            for m0 in range(0, M[gi], mb_max):
                mb = min(mb_max, M[gi] - m0)
                for rd in range(rounds):
                    k_round = rd * ROUND
                    cols = min(ROUND, K - k_round)
                    chunks = cols * asz // 16
                    ipr = -(-chunks // 64)
                    for j in range(mb * ipr):
                        m, c0 = j // ipr, (j % ipr) * 64
                        r = r0[gi] + m0 + m
                        assert r < R
                        if mode == 0:
                            src = perm[r] // wl.k if g[gi] < wl.E else m0 + m
                            assert 0 <= src < T
                        else:
                            src = r
                        cc = c0 + lane
                        okc = cc < chunks
                        assert np.all(k_round + cc[okc] * (16 // asz) + 16 // asz <= K)
                        assert np.all(m * row_bytes + c0 * 16 + lane[okc] * 16 + 16 <= lds)
                for c in range(CPG):
                    n = n0 + c * 8 + lg
                    st = (q < mb)[:, None] & (n < N)[None, :]
                    rows = r0[gi] + m0 + q
                    assert np.all(np.broadcast_to(rows[:, None], st.shape)[st] < R)
    return (CPG, MAXIT, MB)


def check_gemv_mfma(wl, T, mode, offsets, perm, cap):
    K, N = (wl.d, wl.I) if mode == 0 else (wl.I, wl.d)
    assert K % 64 == 0 and wl.act == "bf16"
    w8 = wl.wdt == "i8"
    esz, wl_loads = (1, 1) if w8 else (2, 2)
    nbk = K // 64
    MAXB = 2 if nbk <= 8 else 4 if nbk <= 16 else 6 if nbk <= 24 else 8
    NTI = 2
    NC = 8 * NTI if mode == 0 else 16 * NTI
    RB = 4 * MAXB
    rounds = -(-nbk // RB)
    R = T * wl.k + wl.S * T
    G = wl.E + wl.S
    g, r0, M = touched_groups(wl, T, offsets, cap)
    lane = np.arange(64)
    lr, kq = lane % 16, lane // 16
    for n0 in range(0, N, NC):
        for j in range(NTI):
            ch = (n0 + 8 * j + lr % 8) if mode == 0 else (n0 + 16 * j + lr)
            ch = np.minimum(ch, N - 1)
            assert np.all((g[:, None] * N + ch[None]) < G * N)
        for rd in range(rounds):
            nb_r = min(RB, nbk - rd * RB)
            bpw = -(-nb_r // 4)
            kb_last = rd * RB + nb_r - 1
            for wave in range(4):
                kb0 = rd * RB + wave * bpw
                for it in range(MAXB):
                    blk = min(kb0 + it, kb_last)
                    for u in range(wl_loads):
                        assert np.all(kq * 16 * esz + blk * 64 * esz + 16 * u + 16 <= K * esz)
                    assert np.all(kq * 32 + blk * 128 + 32 <= K * 2)      # activation loads
        for gi in range(len(g)):
            for m0 in range(0, M[gi], 16):
                if mode == 0:
                    if g[gi] < wl.E:
                        r = r0[gi] + np.minimum(m0 + np.arange(16), M[gi] - 1)
                        src = perm[r] // wl.k
                    else:
                        src = np.minimum(m0 + lr, M[gi] - 1)
                    assert np.all((src >= 0) & (src < T))
                else:
                    src = r0[gi] + np.minimum(m0 + lr, M[gi] - 1)
                    assert np.all(src < R)
                mb = min(16, M[gi] - m0)
                t = np.arange(16 * NC)
                cc, chl = t // NC, t % NC
                st = (cc < mb) & (n0 + chl < N)
                assert np.all(r0[gi] + m0 + cc[st] < R)
    return MAXB


# ------------------------------------------------------------------------------------------
# cases: workloads and token counts that put each kernel on the real routings
# ------------------------------------------------------------------------------------------
RAGGED32 = S.Workload("idx_ragged32", 97, d=288, E=8, k=2, I=352, S=1, renormalize=True)
RAGGED16 = S.Workload("idx_ragged16", 97, d=272, E=8, k=2, I=208, S=1, renormalize=True)
WIDE_K = S.Workload("idx_wide_k", 98, d=16384, E=8, k=3, I=64, S=1, renormalize=True)


@pytest.mark.parametrize("wl,T,cf", [(RAGGED32, 300, 0.0), (RAGGED32, 40, 1.0),
                                     (dataclasses.replace(RAGGED32, name="idx_r32_i8", wdt="i8"), 300, 0.0)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_ring32_addresses_stay_in_bounds(wl, T, cf):
    offsets, perm, cap, tiles = routed_plan(wl, T, cf)
    for mode in (0, 1):
        for tbn in (256, 128):
            assert check_ring32(wl, T, mode, tbn, wl.wdt == "i8", offsets, perm, cap, tiles) > 0


@pytest.mark.parametrize("wl,T,cf", [(RAGGED16, 100, 0.0), (RAGGED16, 300, 1.0),
                                     (dataclasses.replace(RAGGED16, name="idx_r16_i8", wdt="i8"), 100, 0.0),
                                     (S.Workload("idx_edge", 96, d=16, E=3, k=1, I=16, S=1), 40, 0.0)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_general_gemm_addresses_stay_in_bounds(wl, T, cf):
    offsets, perm, cap, tiles = routed_plan(wl, T, cf)
    for mode in (0, 1):
        assert check_general(wl, T, mode, wl.wdt == "i8", offsets, perm, cap, tiles) > 0


GEMV_CASES = [(S.OLMOE_BF16, 1, 0.0), (S.OLMOE_BF16, 2, 0.0), (S.OLMOE_BF16, 4, 0.0),
              (S.OLMOE_BF16, 8, 0.0), (S.OLMOE_BF16, 24, 0.0), (S.OLMOE_BF16, 8, 1.0),
              (S.OLMOE_I8, 1, 0.0), (S.OLMOE_I8, 8, 0.0), (S.OLMOE_I8_ZIPF, 16, 1.0),
              (S.DEEPSEEK_BF16, 1, 0.0), (S.DEEPSEEK_BF16, 7, 0.0), (S.DEEPSEEK_I8, 4, 0.0),
              (S.TINY_F32, 16, 0.0), (S.TINY_F32, 200, 0.0), (RAGGED16, 7, 0.0), (WIDE_K, 5, 0.0)]


@pytest.mark.parametrize("wl,T,cf", GEMV_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_gemv_addresses_stay_in_bounds(wl, T, cf):
    offsets, perm, cap, _ = routed_plan(wl, T, cf)
    seen = {check_gemv(wl, T, mode, offsets, perm, cap) for mode in (0, 1)}
    assert seen


def test_gemv_instances_cover_the_dispatcher():
    """Every (CPG, MAXIT, MB) instance the dispatcher can pick for the workloads' matrices is
    reached by the cases above."""
    reached = set()
    for wl, T, _ in GEMV_CASES:
        for mode in (0, 1):
            K = wl.d if mode == 0 else wl.I
            reached.add((mode, gemv_instance(mode, T, K, wl.wdt, wl.act)))
    assert len(reached) >= 8, reached


MFV_CASES = [(S.OLMOE_BF16, 32, 0.0), (S.OLMOE_BF16, 64, 1.0), (S.OLMOE_I8, 24, 0.0),
             (S.OLMOE_I8_ZIPF, 48, 0.0), (S.DEEPSEEK_BF16, 8, 0.0), (S.DEEPSEEK_BF16, 16, 2.0),
             (S.DEEPSEEK_I8, 12, 0.0), (WIDE_K, 12, 0.0),
             (S.Workload("idx_mfv_small", 86, d=320, E=8, k=2, I=448, renormalize=True,
                         routing="zipf", zipf_alpha=2.0, router_std=0.05), 32, 0.0)]


@pytest.mark.parametrize("wl,T,cf", MFV_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_gemv_mfma_addresses_stay_in_bounds(wl, T, cf):
    offsets, perm, cap, _ = routed_plan(wl, T, cf)
    for mode in (0, 1):
        assert check_gemv_mfma(wl, T, mode, offsets, perm, cap) >= 2


def test_gemv_emulation_catches_a_wrong_row_rule():
    """Not vacuous: indexing x by sorted row instead of by token reads past the end of x."""
    wl, T = S.OLMOE_BF16, 8
    offsets, perm, cap, _ = routed_plan(wl, T, 0.0)
    with pytest.raises(AssertionError):
        check_gemv(wl, T, 0, offsets, np.arange(len(perm)) * wl.k * 2, cap)


# ------------------------------------------------------------------------------------------
# k_down_combine: the down projection and the combine in one launch (moe_forward, decode)
# ------------------------------------------------------------------------------------------
DC_MAX_LDS = 160 * 1024
DC_RING = 2
DC_STREAMS = {"i8": 4}  # slot streams per workgroup by weight type (else 2)


def down_combine_geom(wl, T):
    """(spw, slice, R, lds bytes) of the fused launch, as the launcher computes them."""
    f32, i8 = wl.act == "f32", wl.wdt == "i8"
    V, asz = (4, 4) if f32 else ((16, 2) if i8 else (8, 2))
    steps = -(-wl.I // (8 * V))
    spw = -(-steps // 4)
    slice_ = spw * 8 * V * asz
    R = T * wl.k + wl.S * T
    lds = 4 * R * slice_ + 4 * R * 8 * 4 + (R * 8 * 4 if i8 else 0) + T * wl.k * 8
    return spw, slice_, R, lds


def down_combine_fits(wl, T):
    spw, _, _, lds = down_combine_geom(wl, T)
    max_spw = 6 if wl.wdt == "i8" else 8
    return 1 <= T and T * 8 <= 256 and T * wl.k <= 256 and spw <= max_spw and lds <= DC_MAX_LDS


def routed_inv_perm(wl, T, cap):
    x = S.make_tokens(wl, T)
    L = S.make_layer(dataclasses.replace(wl, I=16))  # the router only
    ids, _ = O.route(O.router_logits(x, L.w_router, L.bias), wl.k, wl.renormalize)
    return O.permute_with_capacity(ids, wl.E, cap)[3]


def check_down_combine(wl, T, offsets, inv_perm, cap):
    """Every address of k_down_combine in bounds, and the combine reads only rows the ring
    wrote.  Returns the number of (group, row) sums the blocks form."""
    K, N = wl.I, wl.d
    f32, i8 = wl.act == "f32", wl.wdt == "i8"
    V, asz = (4, 4) if f32 else ((16, 2) if i8 else (8, 2))
    STEP = 8 * V
    spw, slice_, R, lds = down_combine_geom(wl, T)
    assert lds <= DC_MAX_LDS and spw <= 8
    MAXIT = spw
    G = wl.E + wl.S
    Tk = T * wl.k
    stage_end = 4 * R * slice_
    part_end = stage_end + 4 * R * 8 * 4
    scl_end = part_end + (R * 8 * 4 if i8 else 0)
    assert scl_end + Tk * 8 == lds
    g, r0, M = touched_groups(wl, T, offsets, cap)
    nslots = len(g)
    NG = DC_STREAMS.get(wl.wdt, 2)
    tid = np.arange(256 * NG)
    wave, lane = tid // 64, tid % 64
    q, lg = lane % 8, lane // 8
    ct, cc = tid // 8, tid % 8
    steps = -(-K // STEP)
    # (0) the combine's inputs
    assert np.all(tid[tid < Tk] < len(inv_perm))
    written = set()
    for n0 in range(0, N, 8):
        n = np.minimum(n0 + lg, N - 1)
        cn = n0 + cc
        ridx = np.minimum(ct, T - 1) * N + np.minimum(cn, N - 1)
        assert np.all((ridx >= 0) & (ridx < T * N))
        # (1) row staging, the kernel's incremental (row, piece) walk; the NG wavefronts of a
        #     K-slice take 64 pieces each in turn and together cover every piece once
        for w in range(4):
            s_lo = w * spw
            if s_lo >= steps:
                continue
            kw0 = s_lo * STEP
            cpr = slice_ // 16
            dr, dp = NG * 64 // cpr, NG * 64 % cpr
            ln = np.arange(64)
            covered = np.zeros(R * cpr, dtype=np.int64)
            for grp in range(NG):
                r, p = (grp * 64 + ln) // cpr, (grp * 64 + ln) % cpr
                for c0 in range(grp * 64, R * cpr, NG * 64):
                    c = c0 + ln
                    assert np.array_equal(r, c // cpr) and np.array_equal(p, c % cpr)
                    col = kw0 + p * (16 // asz)
                    col = np.where(col >= K, kw0, col)
                    live = r < R
                    assert np.all(r[live] * K + col[live] + 16 // asz <= R * K)
                    assert np.all(w * R * slice_ + c0 * 16 + ln[live] * 16 + 16 <= stage_end)
                    covered[c[live]] += 1
                    r, p = r + dr, p + dp
                    wrap = p >= cpr
                    p, r = np.where(wrap, p - cpr, p), np.where(wrap, r + 1, r)
            assert np.all(covered == 1)
        if n0 > 0:
            continue  # the ring's indexing below does not depend on n0 beyond n (checked)
        # (2) the weight rings, one per slot stream: issue order, then the rows each group's
        #     sums cover; every group is taken by exactly one stream
        issued, taken = [], []
        for grp in range(NG):
            mine = -(-(nslots - grp) // NG) if nslots > grp else 0
            if mine == 0:
                continue
            own = [grp + i * NG for i in range(mine)]
            taken += own
            issued += [own[min(j, mine - 1)] for j in range(DC_RING)]
            for i0 in range(0, mine, DC_RING):
                for j in range(DC_RING):
                    issued.append(own[min(i0 + j + DC_RING, mine - 1)])
        assert sorted(taken) == list(range(nslots))
        for sl in issued:
            assert 0 <= sl < nslots and 0 <= g[sl] < G
            for w in range(4):
                s_lo, s_hi = w * spw, min(steps, w * spw + spw)
                kw0 = s_lo * STEP
                for it in range(MAXIT):
                    col = kw0 + it * STEP + q * V
                    colc = np.where((s_lo + it < s_hi) & (col < K), col, np.where(q * V < K, q * V, 0))
                    assert np.all((g[sl] * N + n[lane]) * K + colc + V <= G * N * K)
                assert np.all(g[sl] * N + n[lane] < G * N)
        for sl in range(nslots):
            for w in range(4):
                s_lo, s_hi = w * spw, min(steps, w * spw + spw)
                kw0 = s_lo * STEP
                for m in range(M[sl]):
                    r = r0[sl] + m
                    assert r < R
                    for it in range(MAXIT):
                        xcol = it * STEP + q * V
                        ok = (s_lo + it < s_hi) & (kw0 + xcol < K)
                        rd_bytes = 32 if V == 16 else 16
                        assert np.all(xcol[ok] * asz + rd_bytes <= slice_)
                        assert np.all(w * R * slice_ + r * slice_ + xcol[ok] * asz + rd_bytes <= stage_end)
                    assert stage_end + ((w * R + r) * 8 + 7) * 4 + 4 <= part_end
                    if i8:
                        assert part_end + (r * 8 + 7) * 4 + 4 <= scl_end
                    written.add(int(r))
    # (3) the combine reads only rows the ring summed; stores stay in y
    for t in range(T):
        for j in range(wl.k):
            r = int(inv_perm[t * wl.k + j])
            assert r < 0 or r in written, (t, j, r)
        for s in range(wl.S):
            assert Tk + s * T + t in written
    live = (ct < T)[:, None] & ((np.arange(0, N, 8)[None, :] + cc[:, None]) < N)
    ys = ct[:, None] * N + np.arange(0, N, 8)[None, :] + cc[:, None]
    assert np.all(ys[live] < T * N)
    return len(written)


DC_CASES = [(S.OLMOE_BF16, 1, 0.0), (S.OLMOE_BF16, 8, 0.0), (S.OLMOE_BF16, 9, 0.0), (S.OLMOE_BF16, 8, 1.0),
            (S.OLMOE_I8, 1, 0.0), (S.OLMOE_I8, 8, 0.0), (S.OLMOE_I8_ZIPF, 9, 1.0),
            (S.DEEPSEEK_BF16, 1, 0.0), (S.DEEPSEEK_BF16, 6, 0.0), (S.DEEPSEEK_I8, 4, 0.0),
            (S.DEEPSEEK_I8, 5, 2.0), (S.TINY_F32, 16, 0.0), (S.TINY_F32, 3, 1.0), (RAGGED16, 7, 0.0),
            (RAGGED32, 5, 0.0), (WIDE_K, 5, 0.0)]


@pytest.mark.parametrize("wl,T,cf", DC_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_down_combine_addresses_stay_in_bounds(wl, T, cf):
    offsets, perm, cap, _ = routed_plan(wl, T, cf)
    inv_perm = routed_inv_perm(wl, T, cap)
    assert down_combine_fits(wl, T)
    assert check_down_combine(wl, T, offsets, inv_perm, cap) > 0


def test_down_combine_limits():
    """Where the fused launch stops: OLMoE-shaped layers through T=9, DeepSeek-shaped through T=6
    (the rows' slices fill the 160 KiB of LDS)."""
    assert down_combine_fits(S.OLMOE_BF16, 9) and not down_combine_fits(S.OLMOE_BF16, 10)
    assert down_combine_fits(S.OLMOE_I8, 9) and not down_combine_fits(S.OLMOE_I8, 10)
    assert down_combine_fits(S.DEEPSEEK_BF16, 6) and not down_combine_fits(S.DEEPSEEK_BF16, 7)


def test_down_combine_emulation_catches_a_dropped_row():
    """Not vacuous: a combine that read a dropped row (inv_perm kept at its sorted position
    past the capacity) is caught."""
    wl, T = S.OLMOE_BF16, 8
    offsets, perm, cap, _ = routed_plan(wl, T, 0.25)
    assert cap > 0
    full = routed_inv_perm(wl, T, 0)
    capped = routed_inv_perm(wl, T, cap)
    assert np.any(capped < 0)
    with pytest.raises(AssertionError):
        check_down_combine(wl, T, offsets, full, cap)
