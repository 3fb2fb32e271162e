"""CPU model of every global-memory and LDS address the stream kernels
(tgemm_stream, forward and dX) compute for their direct-to-LDS loads, checked
against the buffers' sizes for each shape the GPU tests run on them, before
any of those shapes reaches the GPU.  A direct-to-LDS load has no range
check: an address past its buffer would fault.  (The stores are guarded by
row and column tests and checked on the GPU against a canary border.)

The model restates the kernel's offsets (set_loads / issue in tgemm_stream):
  Q load i of wave w, lane l: tile row r = 16 (kALoads w + i) + l / 4, row
    m = min(m0 + r, R - 1), offset m * ldq + 16 ((l % 4) ^ ((r >> 1) % 4)),
    based at Q + 64 s for step s; 16 bytes into LDS at stage + 1024 (kALoads
    w + i) + 16 l.
  packed load i < units(w): dword d = 64 (first_unit(w) + i) + l of the step;
    forward: column n = min(n0 + d / 4, Cc - 1), offset n kb + 4 (d % 4),
    based at Wp + 16 s; dX: contraction row d / (BN / 16), byte
    min(n0 / 4 + 4 (d % (BN / 16)), kb - 4), offset row kb + byte, based at
    Wp + 64 s kb; 4 bytes into LDS at the packed stage + 256 u + 4 l.
"""
import numpy as np
import pytest

from shapes import DX_STREAM_SHAPES, STREAM_SHAPES
from ternary_weight_int8_amd import binding as B

WAVES, BM, BK, LP = 8, 512, 64, 64
A_STAGE = BM * LP
A_LOADS = A_STAGE // 1024 // WAVES
Q_STAGES, D_STAGES, P_STAGES = 3, 3, 2


def geo(op):
    bn = 144 if op == "fwd" else 160
    units = (bn * BK // 16) // 64
    q, r = divmod(units, WAVES)

    def units_of(w):
        return q + (1 if w >= WAVES - r else 0)

    def first_unit(w):
        return q * w + (w - (WAVES - r) if w > WAVES - r else 0)

    return bn, units, units_of, first_unit


def row_layout_bytes(bn):
    # decoded dX stage: 64 contraction rows of bn bytes; an odd number of
    # 16-byte chunks per row (144 bytes) adds a 128-byte shift per second
    # block of 16 rows, twice an odd number (160) a 16-byte one
    chunks = bn // 16
    extra = 0
    if chunks % 2 == 1:
        extra = 128
    elif (chunks // 2) % 2 == 1:
        extra = 16
    return 64 * bn + extra


@pytest.mark.parametrize("op,M,N,K", [("fwd",) + s for s in STREAM_SHAPES + [(16384, 3456, 1280)]]
                         + [("dx",) + s for s in DX_STREAM_SHAPES + [(16384, 3456, 1280)]])
def test_stream_load_addresses_stay_in_their_buffers(op, M, N, K):
    pl = B.plan(op, M, N, K)
    assert pl.kernel == B.KERNEL_STREAM
    R, Cc, L = pl.out_rows, pl.out_cols, pl.contraction
    assert L % BK == 0
    nk = L // BK
    bn, units, units_of, first_unit = geo(op)
    assert (pl.tile_rows, pl.tile_cols) == (BM, bn)
    ldq = L
    kb = K // 4                                   # packed row stride
    q_bytes = R * L                               # A [M][K] or dC [M][N]
    w_bytes = (N * kb) if op == "fwd" else (L * kb)
    tiles_c = -(-Cc // bn)
    tiles = tiles_c * -(-R // BM)
    assert tiles == pl.tiles
    lane = np.arange(64)
    # every tile position some workgroup takes (coverage is tested elsewhere)
    for pos in range(tiles):
        m0, n0 = pos // tiles_c * BM, pos % tiles_c * bn
        for w in range(WAVES):
            for i in range(A_LOADS):
                r = 16 * (A_LOADS * w + i) + (lane >> 2)
                m = np.minimum(m0 + r, R - 1)
                off = m * ldq + 16 * ((lane & 3) ^ ((r >> 1) & 3))
                for s in (0, nk - 1):
                    hi = 64 * s + off.max() + 16
                    assert 0 <= 64 * s + off.min() and hi <= q_bytes, (op, pos, w, i, s, hi, q_bytes)
            for i in range(units_of(w)):
                d = 64 * (first_unit(w) + i) + lane
                if op == "fwd":
                    n = np.minimum(n0 + (d >> 2), Cc - 1)
                    off = n * kb + 4 * (d & 3)
                    base = [16 * s for s in (0, nk - 1)]
                else:
                    per_row = bn // 16
                    kw = n0 // 4 + 4 * (d % per_row)
                    off = (d // per_row) * kb + np.where(kw + 4 <= kb, kw, kb - 4)
                    base = [BK * s * kb for s in (0, nk - 1)]
                for b in base:
                    assert b + off.min() >= 0 and b + off.max() + 4 <= w_bytes, (op, pos, w, i, b, w_bytes)


@pytest.mark.parametrize("op", ["fwd", "dx"])
def test_stream_lds_destinations_stay_in_their_stages(op):
    bn, units, units_of, first_unit = geo(op)
    wd_stage = bn * LP if op == "fwd" else row_layout_bytes(bn)
    off_wd = Q_STAGES * A_STAGE
    off_wp = off_wd + D_STAGES * wd_stage
    wp_stage = units * 256
    lds = off_wp + P_STAGES * wp_stage
    assert lds <= 160 * 1024
    assert B.plan(op, 16384, 3456, 1280).lds_bytes >= lds
    lane = np.arange(64)
    for w in range(WAVES):
        for st in range(Q_STAGES):
            for i in range(A_LOADS):
                a = st * A_STAGE + w * (A_LOADS * 1024) + 1024 * i + 16 * lane
                assert a.min() >= st * A_STAGE and a.max() + 16 <= (st + 1) * A_STAGE
        seen = set()
        for ps in range(P_STAGES):
            for i in range(units_of(w)):
                u = first_unit(w) + i
                assert u < units
                seen.add(u)
                p = off_wp + ps * wp_stage + 256 * u + 4 * lane
                assert p.min() >= off_wp + ps * wp_stage and p.max() + 4 <= off_wp + (ps + 1) * wp_stage
    # the waves' units tile the packed stage exactly once
    allu = sorted(first_unit(w) + i for w in range(WAVES) for i in range(units_of(w)))
    assert allu == list(range(units))
