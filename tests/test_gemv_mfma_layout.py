"""Host emulation of the matrix-core GEMV's operand layout (k_gemv_mfma).

Each lane's weight and activation fragments are built from the kernel's index formulas (row
lane % 16, K elements 16 * (lane / 16) + 8h .. +7 of every 64-K block, tiles of 8 gate + 8 up
rows or 16 down rows), multiplied with the matrix-core instruction's definition (lane l
supplies A[l % 16][8 * (l / 16) + e] and B[8 * (l / 16) + e][l % 16]; lane l receives
D[4 * (l / 16) + v][l % 16]), split over four wavefronts, reduced through the same LDS
indexing and passed through the epilogue's token / channel mapping.  The result must equal
the plain products, so a wrong lane index, K permutation or tile-row mapping fails here, on
the CPU.  CPU only; the formulas are the kernel's, restated (see k_gemv.hip).
"""
import numpy as np
import pytest

WAVES = 4


def silu(z):
    return z / (1.0 + np.exp(-z))


def emulate(mode, W, X, nti=2, up_row_offset=32):
    """W: [mats, N, K] (gate and up for mode 0), X: [M, K].  Returns out [M, N]."""
    mats, N, K = W.shape
    M = X.shape[0]
    nc = 8 * nti if mode == 0 else 16 * nti
    nbk = K // 64
    bpw = -(-nbk // WAVES)
    lane = np.arange(64)
    lr, kq = lane % 16, lane // 16
    e = np.arange(8)
    out = np.full((M, N), np.nan)
    for n0 in range(0, N, nc):
        for m0 in range(0, M, 16):
            red = np.zeros((WAVES, nti, 64, 4))
            for wave in range(WAVES):
                b_lo, b_hi = wave * bpw, min(nbk, wave * bpw + bpw)
                for j in range(nti):
                    if mode == 0:
                        mat, ch = lr // 8, n0 + 8 * j + lr % 8
                    else:
                        mat, ch = np.zeros_like(lr), n0 + 16 * j + lr
                    ch = np.minimum(ch, N - 1)
                    m = np.minimum(m0 + lr, M - 1)
                    acc = np.zeros((64, 4))
                    for blk in range(b_lo, b_hi):
                        for h in range(2):
                            kel = blk * 64 + 16 * kq[:, None] + 8 * h + e[None, :]  # [64, 8]
                            a_frag = W[mat[:, None], ch[:, None], kel]              # lane's A elements
                            b_frag = X[m[:, None], kel]                             # lane's B elements
                            A = np.zeros((16, 32)); B = np.zeros((32, 16))
                            for l in range(64):
                                A[l % 16, 8 * (l // 16):8 * (l // 16) + 8] = a_frag[l]
                                B[8 * (l // 16):8 * (l // 16) + 8, l % 16] = b_frag[l]
                            D = A @ B
                            for l in range(64):
                                acc[l] += D[4 * (l // 16) + np.arange(4), l % 16]
                    red[wave, j] = acc
            mb = min(16, M - m0)
            for t in range(16 * nc):
                c, chl = divmod(t, nc)
                n = n0 + chl
                if c >= mb or n >= N:
                    continue
                if mode == 0:
                    j, i = divmod(chl, 8)
                    v, lg = i % 4, 16 * (i // 4) + c
                    lu = lg + up_row_offset
                    gv = (red[0, j, lg, v] + red[1, j, lg, v]) + (red[2, j, lg, v] + red[3, j, lg, v])
                    uv = (red[0, j, lu, v] + red[1, j, lu, v]) + (red[2, j, lu, v] + red[3, j, lu, v])
                    out[m0 + c, n] = silu(gv) * uv
                else:
                    j, i = divmod(chl, 16)
                    v, l = i % 4, 16 * (i // 4) + c
                    out[m0 + c, n] = (red[0, j, l, v] + red[1, j, l, v]) + (red[2, j, l, v] + red[3, j, l, v])
    return out


def reference(mode, W, X):
    if mode == 0:
        return silu(X @ W[0].T) * (X @ W[1].T)
    return X @ W[0].T


# K = 192: three 64-K blocks (one wavefront idle); K = 320: 2/2/1/0 blocks; N ragged against
# the block's 16 (gate/up) and 32 (down) channels; M = 21: a full and a partial 16-token chunk
CASES = [(0, 40, 192, 21), (0, 40, 320, 5), (1, 40, 320, 21), (1, 64, 192, 16), (0, 16, 64, 1)]


@pytest.mark.parametrize("mode,N,K,M", CASES)
def test_lane_layout_reproduces_the_products(mode, N, K, M):
    rng = np.random.default_rng(N * K + M + mode)
    W = rng.standard_normal((2 if mode == 0 else 1, N, K))
    X = rng.standard_normal((M, K))
    np.testing.assert_allclose(emulate(mode, W, X), reference(mode, W, X), rtol=1e-12, atol=1e-12)


def test_emulation_catches_a_wrong_tile_row():
    """Not vacuous: reading the up channel from tile row i + 4 instead of i + 8 is caught."""
    rng = np.random.default_rng(7)
    W = rng.standard_normal((2, 16, 128))
    X = rng.standard_normal((3, 128))
    bad = emulate(0, W, X, up_row_offset=16)
    assert not np.allclose(bad, reference(0, W, X))
