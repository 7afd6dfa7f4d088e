"""Host-side model of every global access of the trailing products run as
three bf16 products (csrc/gemm_x3.hip, csrc/sweep.hip): the transposing
split of the factor into hi and lo (once per layer, the part above the
diagonal blocks), the product's operand loads (rows past M or
N clamped to the last valid row), its LDS panels and masked stores, and the sweep kernels' split-error
writes, checked against the buffers quantize_layer carves from its workspace,
for the tested and configured shapes.  (The kernels' index formulas are
restated here; a change to them must be mirrored, which is the point.)"""
import numpy as np
import pytest

SBW, XT, XK, TT = 1024, 128, 64, 64


def cdiv(a, b):
    return -(-a // b)


def flushes(m, n, B, superblock):
    """(ec, r0, K, c0, N) of every flush that runs as bf16 products."""
    out = []
    for s0 in range(0, n, SBW):
        s1 = min(s0 + SBW, n)
        if not superblock:
            g0 = s0
            while g0 < s1:
                i = g0
                for _ in range(2):
                    if i < s1:
                        i += min(B, s1 - i)
                if s1 - i > 0 and (i - g0) % 64 == 0:
                    out.append((g0 - s0, g0, i - g0, i, s1 - i))
                g0 = i
        if s1 < n and (s1 - s0) % 64 == 0:
            out.append((0, s0, s1 - s0, s1, n - s1))
    return out


def check(m, n, B, superblock):
    lde, ldu = 2 * SBW, 2 * n
    ecat, ut, vsz, usz = m * 2 * SBW, n * 2 * n, m * n, n * n
    assert n % 4 == 0 and ldu % 8 == 0
    # split_t_kernel (once per layer): tile (j0, k0) skipped unless k0 lies
    # in an earlier granule than j0 (granules of SBW columns on the
    # superblock path, 64 on the paired one); reads U[k][j], writes Ut[j][k]
    # (hi) and Ut[j][n + k] (lo)
    gran = SBW if superblock else 64
    written = set()
    for bx in range(cdiv(n, TT)):
        for by in range(cdiv(n, TT)):
            j0, k0 = bx * TT, by * TT
            if k0 // gran >= j0 // gran:
                continue
            written.add((bx, by))
            kk = k0 + np.arange(TT)[:, None]
            jj = j0 + np.arange(TT)[None, :]
            ok = (kk < n) & (jj < n)
            assert (kk * n + jj)[ok].max() < usz
            assert (jj * ldu + kk + n)[ok].max() < ut
    for ec, r0, K, c0, N in flushes(m, n, B, superblock):
        assert K % XK == 0 and r0 % XK == 0 and c0 + N <= n and r0 + K <= c0
        # gemm_x3_kernel loads: A row min(r, M-1) at ec (hi) and ec + SBW (lo);
        # Bt = Ut + c0 ldu + r0: row min(j, N-1) at 0 (hi) and n (lo), 16
        # bytes at k0 + 8 c8
        last_a = (m - 1) * lde + ec + SBW + (K - XK) + 56 + 7
        last_b = (c0 + N - 1) * ldu + r0 + n + (K - XK) + 56 + 7
        assert last_a < ecat and last_b < ut
        assert ec + K <= SBW  # the hi segment does not run into the lo one
        # every Ut entry read (rows c0.., columns r0..r0+K-1) was written:
        # the flush's factor rows end at a granule boundary at or before c0
        assert (r0 + K) % gran == 0
        for j in {c0, c0 + N - 1}:
            for k in {r0, r0 + K - 1}:
                assert (j // TT, k // TT) in written
        # masked stores into V's columns c0.. (row < M, column < N)
        assert (m - 1) * n + c0 + N - 1 < vsz
    # split-error writes of the sweep kernels: row r, block column (in its superblock) + c, + SBW
    for s0 in range(0, n, SBW):
        s1 = min(s0 + SBW, n)
        for i in range(s0, s1, B):
            w = min(B, s1 - i)
            assert (m - 1) * 2 * SBW + (i - s0) + w - 1 + SBW < ecat


def test_lds_indexes_in_bounds():
    """gemm_x3_kernel's four LDS panels of XT rows x XP bf16: the stores
    (row q / 8, piece q % 8) and the fragment reads (row 64 wr + 32 h + l % 32,
    k 16 ks + 8 (l / 32) .. + 7) stay inside a panel."""
    XP = XK + 8
    q = np.arange(1024)
    st = (q >> 3) * XP + 8 * (q & 7) + 7
    assert st.max() < XT * XP
    lane = np.arange(64)
    for wr in range(2):
        for h in range(2):
            for ks in range(XK // 16):
                rd = (wr * 64 + (lane & 31)) * XP + 32 * h * XP + 16 * ks + 8 * (lane >> 5) + 7
                assert rd.max() < XT * XP
    assert 4 * XT * XP * 2 * 2 <= 160 * 1024  # two workgroups per CU


@pytest.mark.parametrize("m,n,B", [(130, 2048, 128), (70, 1400, 64), (40, 2600, 128), (40, 4500, 128),
                                   (24, 4224, 64), (256, 1024, 128), (4096, 4096, 128), (4096, 11008, 128)])
def test_superblock_path_in_bounds(m, n, B):
    check(m, n, B, superblock=True)


@pytest.mark.parametrize("m,n,B", [(33000, 2176, 128), (12288, 4096, 128), (22016, 4096, 128),
                                   (49152, 12288, 128), (11008, 4096, 128), (300, 100, 64)])
def test_paired_path_in_bounds(m, n, B):
    check(m, n, B, superblock=False)


def test_short_last_block_stays_fp32():
    """A flush whose K is not a multiple of 64 is not run as bf16 products."""
    fl = flushes(40, 1100, 100, superblock=False)
    assert all(K % 64 == 0 for _, _, K, _, _ in fl)


def test_tile_order_is_a_bijection():
    """gemm_x3_kernel's tile order (XCD x takes tiles [x P, (x + 1) P) of an
    order walking bands of 8 tile rows column by column) covers every tile of
    the grid exactly once, and workgroups past the tiles exit."""
    for tM in range(1, 50):
        for tN in range(1, 30):
            T = tM * tN
            P = cdiv(T, 8)
            seen = set()
            for b in range(8 * P):
                t = (b % 8) * P + b // 8
                if t >= T:
                    continue
                band = t // (8 * tN)
                rows = min(8, tM - band * 8)
                within = t - band * 8 * tN
                tm, tn = band * 8 + within % rows, within // rows
                assert 0 <= tm < tM and 0 <= tn < tN
                seen.add((tm, tn))
            assert len(seen) == T
