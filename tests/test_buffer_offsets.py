"""Buffer-resource offsets of the kernels that put part of an address in the
scalar offset (CPU model, no GPU).

A raw buffer load is range-checked on its lane offset only: a lane offset at
or past the resource's extent returns zeros, but the scalar offset is added
after the check, so a lane offset inside the extent plus a scalar offset can
read past the end of the buffer.  The large GEMM kernel puts the K step in
the scalar offset of its activation (buffer-to-LDS) and weight loads, and the
fused loss kernel its K step and 8-row block; both must turn every load whose
lane offset plus scalar offset would leave the buffer (prefetches past the
last step, rows past M or N, channels past K) into an out-of-range lane
offset.  These tests restate the offset arithmetic of those loads, lane by
lane, for the edge tiles of ragged shapes (last tile row and column, last K
step and the two prefetch steps after it, every K slice of a split), and
check that no load both passes the range check and ends past the extent.
The formulas are the ones in gemm_large_kernel (load_x, fetch_w) and
loss_fused_kernel (load_x); a change there must be mirrored here."""
from __future__ import annotations

import numpy as np
import pytest

OOB = 0x80000000
BK = 64


def swz(row, chunk):
    return chunk ^ ((row >> 1) & 7)


def escapes(voff, soff, size, extent):
    """Loads that pass the lane-offset range check but end past the extent."""
    voff = np.asarray(voff, np.int64)
    return (voff < extent) & (voff + soff + size > extent)


def large_kernel_escapes(M, N, K, TBM, NB, splits=1):
    """gemm_large_kernel: 4 waves; the activation tile is TBM x 64 fp16 (wave w
    loads rows TBM/4 w .. in 1 KiB loads of 8 rows), the weight loads are
    128-bit words of 32 channels of row wn + 32 b + lane % 32, half lane / 32."""
    ktail = K % BK != 0
    nsteps = -(-K // BK)
    spp = -(-nsteps // splits)
    TBN = 128 * NB
    lane = np.arange(64)
    bad = 0
    last_m = ((M - 1) // TBM) * TBM
    last_n = ((N - 1) // TBN) * TBN
    for m0 in sorted({0, last_m}):
        rows_m = min(TBM, M - m0)
        x_extent = rows_m * K * 2
        for n0 in sorted({0, last_n}):
            rows_n = min(TBN, N - n0)
            w_extent = rows_n * (K // 2)
            for split in range(splits):
                s0, s1 = split * spp, min(nsteps, split * spp + spp)
                for step in range(s0, s1 + 2):  # the loop prefetches two steps ahead
                    for wave in range(4):
                        xrows = TBM // 4
                        for j in range(xrows // 8):
                            row = xrows * wave + 8 * j + (lane >> 3)
                            chunk = swz(row, lane & 7)
                            off = np.where(step < nsteps, row * K * 2 + chunk * 16, OOB)
                            if ktail:
                                off = np.where(step * BK + 8 * chunk >= K, OOB, off)
                            bad += escapes(off, step * BK * 2, 16, x_extent).sum()
                        fi, fh = lane & 31, lane >> 5
                        k0 = step * BK + 32 * fh
                        kin = (step < nsteps) & ((not ktail) | (k0 < K))
                        for b in range(NB):
                            row = wave * 32 * NB + 32 * b + fi
                            woff = np.where(kin, row * (K // 2) + fh * 16, OOB)
                            bad += escapes(woff, step * (BK // 2), 16, w_extent).sum()
    return int(bad)


@pytest.mark.parametrize("M,N,K", [(2048, 28672, 8192), (2048, 8192, 28672), (261, 44280, 128), (261, 44280, 96),
                                   (513, 44280, 96), (65, 512, 544), (1000, 4104, 4096), (300, 1032, 2080),
                                   (4096, 4096, 4096)])
@pytest.mark.parametrize("TBM,NB", [(256, 2), (256, 1), (128, 2), (128, 1), (64, 1)])
def test_large_kernel_loads_stay_in_their_buffers(M, N, K, TBM, NB):
    for splits in (1, 3):
        assert large_kernel_escapes(M, N, K, TBM, NB, splits) == 0, (M, N, K, TBM, NB, splits)


def test_model_catches_an_unguarded_prefetch():
    """The same model with the step guard taken out of the activation loads
    (lane offset kept in range past the last step) finds loads that leave the
    buffer: the check can fail."""
    M, K, TBM = 256, 4096, 256
    nsteps = K // BK
    lane = np.arange(64)
    extent = M * K * 2
    bad = 0
    for step in (nsteps, nsteps + 1):
        row = (TBM // 4) * 3 + 8 * 7 + (lane >> 3)
        off = row * K * 2 + swz(row, lane & 7) * 16
        bad += escapes(off, step * BK * 2, 16, extent).sum()
    assert bad > 0


def loss_kernel_escapes(M, K, rows_m_list):
    """loss_fused_kernel's activation tile (64-channel steps, 512-row tiles of
    8 waves): wave w, load j, lane l reads row 64 w + 8 j + l / 8 with the
    8-row block and the step in the scalar offset."""
    TK = 64
    ktail = K % TK != 0
    nsteps = -(-K // TK)
    lane = np.arange(64)
    bad = 0
    for rows_m in rows_m_list:
        extent = rows_m * K * 2
        for step in range(max(0, nsteps - 2), nsteps + 2):
            for wave in range(8):
                xrow = 64 * wave + (lane >> 3)
                for j in range(8):
                    chunk = swz(xrow + 8 * (j & 1), lane & 7)
                    off = np.where((step < nsteps) & (xrow + 8 * j < rows_m), xrow * K * 2 + chunk * 16, OOB)
                    if ktail:
                        off = np.where(step * TK + 8 * chunk >= K, OOB, off)
                    bad += escapes(off, step * TK * 2 + 8 * j * K * 2, 16, extent).sum()
    return int(bad)


@pytest.mark.parametrize("K", [4096, 11008, 2080, 544, 96])
def test_loss_kernel_loads_stay_in_their_buffers(K):
    assert loss_kernel_escapes(512, K, [512, 500, 37, 1]) == 0
