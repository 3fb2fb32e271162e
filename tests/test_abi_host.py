"""The C-ABI library on a host without a GPU: exports, validation, launch plan.

Validation runs before any HIP call, so every error path here is exercised
without a device and without launching anything.
"""
import ctypes
import os
import re

import pytest

from ternary_weight_int8_amd import binding as B
from golden_io import read_kv
from shapes import (DW_SHAPES, DX_SHAPES, DX_STREAM_SHAPES, FWD_SHAPES, SKINNY_DX_SHAPES, SKINNY_SHAPES,
                    SPLIT_DX_SHAPES, STREAM_SHAPES, TILES)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ternary_gemm.h")

GEMMS = ("ternary_gemm_s8", "ternary_gemm_s8_dx", "ternary_gemm_s8_dw")
FAKE = (0x10000, 0x20000000, 0x40000000)    # three distinct, never-dereferenced addresses


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_exports():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for st in (B.OK, B.ERR_NULL, B.ERR_DIM, B.ERR_PACK, B.ERR_BOUND, B.ERR_ALIAS, B.ERR_HIP, B.ERR_KIND,
               B.ERR_SCRATCH):
        s = B.status_str(st)
        assert s and s != "unknown status"
    assert B.status_str(12345) == "unknown status"


@pytest.mark.parametrize("name", GEMMS)
@pytest.mark.parametrize("which", [0, 1, 2])
def test_null_pointer_rejected(name, which):
    ptrs = list(FAKE)
    ptrs[which] = None
    assert B.call_raw(name, *ptrs, 4, 4, 4) == B.ERR_NULL


@pytest.mark.parametrize("name", GEMMS)
@pytest.mark.parametrize("dims", [(0, 4, 4), (4, 0, 4), (4, 4, 0), (-1, 4, 4), (1 << 40, 1 << 40, 4)])
def test_bad_dims_rejected(name, dims):
    assert B.call_raw(name, *FAKE, *dims) == B.ERR_DIM


@pytest.mark.parametrize("name", GEMMS[:2])
@pytest.mark.parametrize("K", [1, 2, 3, 6, 97])
def test_packed_dim_must_be_multiple_of_4(name, K):
    assert B.call_raw(name, *FAKE, 3, 5, K) == B.ERR_PACK


def test_dw_needs_no_packing():
    # K % 4 != 0 is fine for dW; with these fake pointers the call gets as far
    # as the launch only on a GPU host, so compare with the plan instead
    assert B.plan("dw", 3, 5, 7).out_rows == 7


def test_contraction_bounds():
    b = read_kv("bounds.txt")
    tern, i8 = b["ternary_max_contraction"], b["dw_max_contraction"]
    # forward: contraction K; largest multiple of 4 under the bound passes the check
    assert B.plan("fwd", 1, 1, tern - tern % 4).contraction == tern - tern % 4
    assert B.call_raw("ternary_gemm_s8", *FAKE, 1, 1, tern + 1 + (4 - (tern + 1) % 4) % 4) == B.ERR_BOUND
    # dX: contraction N
    assert B.plan("dx", 1, tern, 4).contraction == tern
    assert B.call_raw("ternary_gemm_s8_dx", *FAKE, 1, tern + 1, 4) == B.ERR_BOUND
    # dW: contraction M
    assert B.plan("dw", i8, 1, 1).contraction == i8
    assert B.call_raw("ternary_gemm_s8_dw", *FAKE, i8 + 1, 1, 1) == B.ERR_BOUND


def test_alias_rejected():
    base = 0x100000
    M, N, K = 8, 8, 16
    # output starts inside A
    assert B.call_raw("ternary_gemm_s8", base, base + 4096, base + 8, M, N, K) == B.ERR_ALIAS
    # output covers Wpacked
    assert B.call_raw("ternary_gemm_s8", base, base + 4096, base + 4000, M, N, K) == B.ERR_ALIAS
    assert B.call_raw("ternary_gemm_s8_dx", base, base + 4096, base + 4096 + 16, M, N, K) == B.ERR_ALIAS
    assert B.call_raw("ternary_gemm_s8_dw", base, base + 4096, base + 4096, M, N, K) == B.ERR_ALIAS


def _coverage(op, M, N, K, cus=None, xcds=None):
    pl = B.plan(op, M, N, K, cus=cus, xcds=xcds)
    seen = []
    for wg in range(pl.workgroups):
        for it in range(pl.tiles_per_workgroup):
            t = B.tile_of(pl, wg, it)
            if t is None:
                # a workgroup's tiles are a prefix of its iterations
                assert all(B.tile_of(pl, wg, j) is None for j in range(it, pl.tiles_per_workgroup))
                break
            r0, c0 = t
            assert r0 % pl.tile_rows == 0 and c0 % pl.tile_cols == 0
            assert 0 <= r0 < pl.out_rows and 0 <= c0 < pl.out_cols
            seen.append((r0, c0))
    want = {(r, c) for r in range(0, pl.out_rows, pl.tile_rows)
            for c in range(0, pl.out_cols, pl.tile_cols)}
    assert len(seen) == len(set(seen)) == pl.tiles and set(seen) == want
    return pl


@pytest.mark.parametrize("op,M,N,K", [
    ("fwd", 1, 16, 16), ("fwd", 300, 272, 96), ("fwd", 16384, 3456, 1280),
    ("fwd", 2048, 2048, 65536), ("fwd", 8191, 4001, 1040), ("fwd", 77, 4099, 32),
    ("fwd", 4100, 900, 84), ("dw", 16384, 3456, 1280), ("dx", 16384, 3456, 1280), ("dx", 1782, 3456, 1280),
    ("dx", 1782, 3456, 1280), ("dx", 1, 1, 4), ("dw", 1782, 3456, 1280), ("dw", 5, 3, 7)]
    + [("fwd",) + s for s in STREAM_SHAPES] + [("dx",) + s for s in DX_STREAM_SHAPES]
    + [("fwd",) + s for s in SKINNY_SHAPES] + [("dx",) + s for s in SKINNY_DX_SHAPES])
def test_every_output_tile_covered_once(op, M, N, K):
    pl = _coverage(op, M, N, K)
    assert pl.lds_bytes <= 160 * 1024
    if pl.kernel == B.KERNEL_STREAM:
        assert pl.threads_per_workgroup == 512
        assert pl.workgroups == 256 and pl.xcds == 8
        per_xcd = -(-pl.tiles // 8)
        assert pl.tiles_per_workgroup == -(-per_xcd // 32)
    elif pl.kernel == B.KERNEL_SKINNY:
        assert pl.threads_per_workgroup == 512 and pl.tile_rows in (16, 32) and pl.tile_rows >= M
        assert pl.workgroups == pl.tiles and pl.tiles_per_workgroup == 1
    else:
        assert pl.threads_per_workgroup == (512 if pl.kernel == B.KERNEL_SPLIT else 256)
        assert pl.workgroups == pl.tiles and pl.tiles_per_workgroup == 1


def test_parity_shapes_reach_every_tile_and_path():
    # the GPU parity shape lists exercise every tile shape on both load paths,
    # and every kernel on each load path it serves
    kernels = {"fwd": {(B.KERNEL_TILED, 0), (B.KERNEL_TILED, 1), (B.KERNEL_STREAM, 1),
                       (B.KERNEL_SKINNY, 1)},
               "dx": {(B.KERNEL_TILED, 0), (B.KERNEL_TILED, 1), (B.KERNEL_STREAM, 1), (B.KERNEL_SKINNY, 1),
                      (B.KERNEL_SPLIT, 0), (B.KERNEL_SPLIT, 1)},
               "dw": {(B.KERNEL_TILED, 0), (B.KERNEL_TILED, 1), (B.KERNEL_SPLIT, 0),
                      (B.KERNEL_SPLIT, 1)}}
    for op, shapes in (("fwd", FWD_SHAPES + STREAM_SHAPES + SKINNY_SHAPES),
                       ("dx", DX_SHAPES + DX_STREAM_SHAPES + SKINNY_DX_SHAPES),
                       ("dw", DW_SHAPES)):
        seen, seen_k = set(), set()
        for s in shapes:
            pl = B.plan(op, *s)
            seen.add((pl.tile_rows, pl.tile_cols, pl.fast_path))
            seen_k.add((pl.kernel, pl.fast_path))
        for tile in TILES:
            for fast in (0, 1):
                assert (*tile, fast) in seen, (op, tile, fast)
        assert kernels[op] <= seen_k, (op, kernels[op] - seen_k)


def test_kernel_choice():
    assert B.plan("fwd", 16384, 3456, 1280).kernel == B.KERNEL_STREAM
    assert B.plan("fwd", 16384, 3456, 1408).kernel == B.KERNEL_STREAM
    assert B.plan("fwd", 16384, 3454, 1280).kernel == B.KERNEL_STREAM   # N % 4 != 0: 4-byte stores
    assert B.plan("fwd", 6144, 3456, 1280).kernel == B.KERNEL_STREAM    # 288 tiles of 512 x 144
    assert B.plan("fwd", 16384, 3456, 1280, align=8).kernel == B.KERNEL_TILED   # A not 16-byte aligned
    assert B.plan("fwd", 16384, 3456, 1280, align=2).kernel == B.KERNEL_TILED   # A misaligned
    assert B.plan("fwd", 16384, 3456, 1296).kernel == B.KERNEL_TILED    # K % 64 != 0
    assert B.plan("fwd", 2048, 2048, 65536).kernel == B.KERNEL_TILED    # 60 tiles of 512 x 144
    assert B.plan("dx", 16384, 3456, 1280).kernel == B.KERNEL_STREAM
    assert B.plan("dx", 16384, 3456, 1288).kernel == B.KERNEL_TILED    # K % 16 != 0
    assert B.plan("dx", 16384, 3400, 1280).kernel == B.KERNEL_TILED    # N % 64 != 0
    # 32 tiles of 512 x 160 are too few for the stream kernel, and 126 of
    # 128 x 144 would leave half the CUs idle: 560 tiles of 64 x 64; 216 tiles
    # of 128 x 144 take the contraction split between two halves of a workgroup
    pl = B.plan("dx", 1782, 3456, 1280)
    assert (pl.kernel, pl.tile_rows, pl.tile_cols, pl.threads_per_workgroup) == (B.KERNEL_TILED, 64, 64, 256)
    pl = B.plan("dx", 3000, 3456, 1280)
    assert (pl.kernel, pl.tile_rows, pl.tile_cols, pl.threads_per_workgroup) == (B.KERNEL_SPLIT, 128, 144, 512)
    assert B.plan("dx", 4100, 80, 3904).kernel == B.KERNEL_TILED     # 924 tiles fill the CUs
    assert B.plan("dx", 4100, 80, 912).kernel == B.KERNEL_TILED      # 2 steps
    for s in DX_STREAM_SHAPES:
        assert B.plan("dx", *s).kernel == B.KERNEL_STREAM, s
    assert B.plan("dw", 16384, 3456, 1280).kernel == B.KERNEL_SPLIT
    assert B.plan("dw", 80, 3904, 4112).kernel == B.KERNEL_TILED   # short contraction
    assert B.plan("fwd", 300, 272, 96).kernel == B.KERNEL_TILED
    for s in STREAM_SHAPES:
        assert B.plan("fwd", *s).kernel == B.KERNEL_STREAM, s
    for s in SKINNY_SHAPES:
        assert B.plan("fwd", *s).kernel == B.KERNEL_SKINNY, s
    assert B.plan("fwd", 33, 16384, 16384).kernel != B.KERNEL_SKINNY   # more than 32 rows
    assert B.plan("fwd", 27, 16384, 16352).kernel == B.KERNEL_TILED    # K % 64 != 0
    assert B.plan("fwd", 27, 16384, 16384, align=8).kernel == B.KERNEL_TILED
    for s in SKINNY_DX_SHAPES:
        assert B.plan("dx", *s).kernel == B.KERNEL_SKINNY, s
    assert B.plan("dx", 27, 16384 + 32, 16384).kernel == B.KERNEL_TILED   # N % 64 != 0
    assert B.plan("dx", 27, 16384, 16392).kernel == B.KERNEL_SPLIT        # K % 16 != 0: not skinny
    assert B.plan("dx", 33, 16384, 16384).kernel != B.KERNEL_SKINNY       # more than 32 rows
    assert B.plan("dx", 27, 16384, 16384, align=8).kernel == B.KERNEL_TILED
    assert B.plan("dw", 27, 16384, 16384).kernel != B.KERNEL_SKINNY


def test_skinny_plan():
    # column blocks of 64, 32, 16: the widest that leaves 128 workgroups or more
    for (M, N, K), (rows, cols) in {(27, 16384, 16384): (32, 64), (16, 8192, 1280): (16, 64),
                                    (27, 8191, 1280): (32, 32), (1, 4096, 256): (16, 32),
                                    (32, 4095, 64): (32, 16), (17, 3456, 1280): (32, 16)}.items():
        pl = B.plan("fwd", M, N, K)
        assert pl.kernel == B.KERNEL_SKINNY and (pl.tile_rows, pl.tile_cols) == (rows, cols), (M, N, K)
        assert pl.tiles == pl.workgroups == -(-N // cols)
        # 8 waves' partial sums of the tile, rows padded by one 16-byte quad;
        # above 8 rows the same memory first holds each wave's A tile (rows x 256 B)
        red, tiles = 8 * rows * (cols // 4 + 1) * 16, (8 * rows * 256 if M > 8 else 0)
        assert pl.lds_bytes == max(red, tiles)
        # the XCD-contiguous order: workgroup b (XCD b % 8) takes a run of blocks
        q, r = divmod(pl.tiles, 8)
        x, j = 3 % 8, 3 // 8
        assert B.tile_of(pl, 3) == (0, (x * (q + 1) + j if x < r else r * (q + 1) + (x - r) * q + j) * cols)
    # dX: column blocks of 64 (K % 64 == 0 and 128 or more blocks) or 16; the
    # waves' tiles (64 contraction rows of the block's columns) share the
    # memory of the reduction buffer
    for (M, N, K), (rows, cols, tile) in {(27, 16384, 16384): (32, 64, 64 * 64), (5, 8192, 8192): (16, 64, 64 * 64),
                                          (27, 3456, 1280): (32, 16, 64 * 16 + 256),
                                          (1, 64, 4096): (16, 16, 64 * 16 + 256)}.items():
        pl = B.plan("dx", M, N, K)
        assert pl.kernel == B.KERNEL_SKINNY and (pl.tile_rows, pl.tile_cols) == (rows, cols), (M, N, K)
        assert pl.tiles == pl.workgroups == K // cols
        assert pl.lds_bytes == max(8 * rows * (cols // 4 + 1) * 16, 8 * tile)


def test_tile_query_out_of_range():
    pl = B.plan("fwd", 300, 272, 96)
    with pytest.raises(B.TernaryGemmError):
        B.tile_of(pl, pl.workgroups)
    with pytest.raises(B.TernaryGemmError):
        B.tile_of(pl, 0, 1)
    pl = B.plan("fwd", 15000, 3460, 192)            # 750 tiles over 256 workgroups
    assert pl.tiles == 750 and pl.tiles_per_workgroup == 3
    assert B.tile_of(pl, 0, pl.tiles_per_workgroup - 1) is not None
    assert sum(B.tile_of(pl, wg, pl.tiles_per_workgroup - 1) is None
               for wg in range(pl.workgroups)) == 256 * pl.tiles_per_workgroup - 750


def test_stream_schedule_mirror():
    # a CPU mirror of the stream kernel's own schedule (written from its
    # description: eight contiguous runs of row-major tile positions, workgroup
    # b on run b % 8 taking every 32nd position from b / 8) gives the same tiles
    pl = B.plan("fwd", 16300, 3450, 640)
    tiles_c = -(-pl.out_cols // pl.tile_cols)
    q, r = divmod(pl.tiles, 8)
    for wg in range(pl.workgroups):
        x, j = wg % 8, wg // 8
        start, cnt = x * q + min(x, r), q + (x < r)
        for it in range(pl.tiles_per_workgroup):
            pos = j + it * 32
            want = None if pos >= cnt else ((start + pos) // tiles_c * pl.tile_rows,
                                            (start + pos) % tiles_c * pl.tile_cols)
            assert B.tile_of(pl, wg, it) == want


def test_same_xcd_tiles_share_rows():
    # workgroups on one XCD (b, b + 8, ...) work on neighbouring positions of
    # one run at the same time: in the headline plan the tiles in flight on an
    # XCD span at most four row panels
    pl = B.plan("fwd", 16384, 3456, 1280)
    for x in range(8):
        for it in range(pl.tiles_per_workgroup):
            rows = {B.tile_of(pl, wg, it)[0] for wg in range(x, pl.workgroups, 8)}
            assert len(rows) <= 4, (x, it, rows)


def test_headline_plan():
    pl = B.plan("fwd", 16384, 3456, 1280)
    assert (pl.kernel, pl.tile_rows, pl.tile_cols) == (B.KERNEL_STREAM, 512, 144)
    assert pl.tiles == 32 * 24 and pl.workgroups == 256 and pl.tiles_per_workgroup == 3
    assert pl.threads_per_workgroup == 512 and pl.lds_bytes <= 160 * 1024
    assert pl.fast_path == 1
    assert B.plan("fwd", 16384, 3456, 1280, align=2).fast_path == 0
    assert B.plan("fwd", 300, 272, 96).fast_path == 1        # 96 % 16 == 0
    assert B.plan("fwd", 300, 272, 100).fast_path == 0


def test_wrappers_refuse_host_tensors():
    torch = pytest.importorskip("torch")
    A = torch.zeros((4, 16), dtype=torch.int8)
    Wp = torch.zeros((4, 4), dtype=torch.uint8)
    with pytest.raises(ValueError, match="device"):
        B.ternary_gemm_s8(A, Wp)
    with pytest.raises(TypeError):
        B.ternary_gemm_s8(A.to(torch.int16), Wp)


# ---------------------------------------------------------------------------
# scaled entry points: argument checks (no GPU: every case below returns
# before anything is launched)
# ---------------------------------------------------------------------------

SCALED = ("ternary_gemm_s8_scaled", "ternary_gemm_s8_dx_scaled", "ternary_gemm_s8_dw_scaled")


def _scaled_args(name, base=0x100000):
    # inputs, then scales, then the output, far apart; the second scale is a
    # float for the forward and dX, a device address for dW
    a, b, s0, out = base, base + (1 << 20), base + (2 << 20), base + (4 << 20)
    s1 = base + (3 << 20) if name.endswith("dw_scaled") else 0.5
    return [a, b, s0, s1, out]


def test_scaled_status_string():
    assert "TGEMM_OUT_F32" in B.status_str(B.ERR_KIND)


@pytest.mark.parametrize("name", SCALED)
@pytest.mark.parametrize("which", [0, 1, 2, 3, 4])
def test_scaled_null_pointer_rejected(name, which):
    args = _scaled_args(name)
    if which == 3 and not name.endswith("dw_scaled"):
        return  # the weight scale is a value, not a pointer
    args[which] = None
    assert B.call_raw_scaled(name, *args, B.OUT_BF16, 4, 4, 4) == B.ERR_NULL


@pytest.mark.parametrize("name", SCALED)
@pytest.mark.parametrize("kind", [0, 3, -1, 7])
def test_scaled_kind_rejected(name, kind):
    assert B.call_raw_scaled(name, *_scaled_args(name), kind, 4, 4, 4) == B.ERR_KIND


@pytest.mark.parametrize("name", SCALED)
def test_scaled_checks_as_plain(name):
    # the plain calls' checks still apply: dimensions, packing, bounds
    args = _scaled_args(name)
    assert B.call_raw_scaled(name, *args, B.OUT_F32, 0, 4, 4) == B.ERR_DIM
    if not name.endswith("dw_scaled"):
        assert B.call_raw_scaled(name, *args, B.OUT_F32, 3, 5, 6) == B.ERR_PACK
    else:
        assert B.call_raw_scaled(name, *args, B.OUT_F32, 131072, 4, 4) == B.ERR_BOUND


def test_scaled_output_overlapping_a_scale_rejected():
    M, N, K = 8, 8, 16
    a, b, s0, _, _ = _scaled_args("ternary_gemm_s8_scaled")
    # bf16 output of 8 x 8 (128 bytes) ending inside the row scales
    assert B.call_raw_scaled("ternary_gemm_s8_scaled", a, b, s0, 0.5, s0 - 64, B.OUT_BF16,
                             M, N, K) == B.ERR_ALIAS
    # dW: output over the column scales of dC
    a, b, s0, s1, _ = _scaled_args("ternary_gemm_s8_dw_scaled")
    assert B.call_raw_scaled("ternary_gemm_s8_dw_scaled", a, b, s0, s1, s1 + 4, B.OUT_F32,
                             M, N, K) == B.ERR_ALIAS
    # a bf16 output right after the row scales does not overlap them
    assert B.plan("fwd", M, N, K).out_rows == M


# ---------------------------------------------------------------------------
# packer and quantizer: argument checks (all on the host, before any launch)
# ---------------------------------------------------------------------------

def test_pack_weights_checks():
    f = B.lib().ternary_pack_weights
    a, b = 0x100000, 0x40000000
    assert f(None, b, 4, 8, None) == B.ERR_NULL and f(a, None, 4, 8, None) == B.ERR_NULL
    assert f(a, b, 0, 8, None) == B.ERR_DIM and f(a, b, 4, -4, None) == B.ERR_DIM
    assert f(a, b, 4, 6, None) == B.ERR_PACK
    assert f(a, a + 4 * 8 - 1, 4, 8, None) == B.ERR_ALIAS    # output ends inside the input
    assert f(a, a - 4, 4, 8, None) == B.ERR_ALIAS            # output runs into the input


@pytest.mark.parametrize("name", ["ternary_quantize_rows", "ternary_quantize_cols"])
def test_quantize_checks(name):
    f = getattr(B.lib(), name)
    x, q, s = 0x100000, 0x20000000, 0x40000000
    assert f(None, B.IN_F32, q, s, 4, 8, None) == B.ERR_NULL
    assert f(x, B.IN_F32, None, s, 4, 8, None) == B.ERR_NULL
    assert f(x, B.IN_F32, q, None, 4, 8, None) == B.ERR_NULL
    for kind in (0, 3, -1):
        assert f(x, kind, q, s, 4, 8, None) == B.ERR_KIND
    assert f(x, B.IN_BF16, q, s, 0, 8, None) == B.ERR_DIM and f(x, B.IN_BF16, q, s, 4, 0, None) == B.ERR_DIM
    # Q inside X (32 float32 = 128 bytes), the scale inside X or Q
    assert f(x, B.IN_F32, x + 100, s, 4, 8, None) == B.ERR_ALIAS
    assert f(x, B.IN_BF16, q, x + 60, 4, 8, None) == B.ERR_ALIAS
    assert f(x, B.IN_F32, q, q + 30, 4, 8, None) == B.ERR_ALIAS
    assert B.status_str(B.ERR_KIND).endswith("TGEMM_IN_BF16") or "kind" in B.status_str(B.ERR_KIND)


def test_binding_fails_loudly_without_the_library(tmp_path, monkeypatch):
    # the product path has no fallback: with the library absent, the first
    # call raises instead of computing anything some other way
    import importlib
    from ternary_weight_int8_amd import binding as Bfresh
    Bfresh = importlib.reload(Bfresh)
    monkeypatch.setattr(Bfresh, "LIB", str(tmp_path / "absent.so"))
    monkeypatch.setattr(Bfresh, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        Bfresh.lib()
    with pytest.raises(RuntimeError, match="not built"):
        Bfresh.plan("fwd", 4, 4, 4)
    importlib.reload(Bfresh)


# ---------------------------------------------------------------------------
# dX with a workspace
# ---------------------------------------------------------------------------

def _splits(M, N, K):
    blocks = K // 256
    return -(-256 // blocks)


def test_dx_workspace_size():
    # S = ceil(256 / (K / 256)) splits of M x K int32 partials, for few rows,
    # whole 64-row steps, 256-column blocks too few to fill the chip, every
    # wave with a step in every split, and 16-byte aligned operands
    assert B.ternary_gemm_dx_workspace(27, 16384, 16384) == 4 * 27 * 16384 * 4
    assert B.ternary_gemm_dx_workspace(1, 16384, 16384) == 4 * 1 * 16384 * 4
    assert B.ternary_gemm_dx_workspace(16, 4096, 8192) == 8 * 16 * 8192 * 4
    assert B.ternary_gemm_dx_workspace(5, 131072, 256) == 256 * 5 * 256 * 4
    assert B.ternary_gemm_dx_workspace(27, 3456, 1280) == 0       # 52 splits of 54 steps
    assert B.ternary_gemm_dx_workspace(33, 16384, 16384) == 0     # more than 32 rows
    assert B.ternary_gemm_dx_workspace(27, 16384 + 16, 16384) == 0
    assert B.ternary_gemm_dx_workspace(27, 16384, 16384 + 64) == 0
    assert B.ternary_gemm_dx_workspace(27, 16384, 65536) == 0     # 256 blocks: no split
    assert B.ternary_gemm_dx_workspace(27, 16384, 16384, align=8) == 0
    assert B.ternary_gemm_dx_workspace(27, 2048, 16384) > 0       # 32 steps: 8 per split
    assert B.ternary_gemm_dx_workspace(27, 1984, 16384) == 0      # 31 steps
    for M, N, K in SPLIT_DX_SHAPES:
        assert B.ternary_gemm_dx_workspace(M, N, K) == _splits(M, N, K) * M * K * 4, (M, N, K)


def test_dx_workspace_query_checks():
    L, b = B.lib(), ctypes.c_int64(-1)
    assert L.ternary_gemm_dx_workspace(27, 64, 256, 256, None) == B.ERR_NULL
    assert L.ternary_gemm_dx_workspace(0, 64, 256, 256, ctypes.byref(b)) == B.ERR_DIM
    assert L.ternary_gemm_dx_workspace(1, 64, 6, 256, ctypes.byref(b)) == B.ERR_PACK
    tern = read_kv("bounds.txt")["ternary_max_contraction"]
    assert L.ternary_gemm_dx_workspace(1, tern + 1, 4, 256, ctypes.byref(b)) == B.ERR_BOUND
    assert b.value == -1                                          # untouched on error


def test_dx_ws_checks():
    # the plain dX call's checks, then the workspace's: a negative size is
    # ERR_DIM, overlap with an input, the output or the row scales ERR_ALIAS;
    # every case is refused on the host, before any launch
    L = B.lib()
    M, N, K = 27, 16384, 16384
    dC, Wp, dX, rs, ws = 0x10000000, 0x20000000, 0x40000000, 0x50000000, 0x60000000
    big = 1 << 24
    f = L.ternary_gemm_s8_dx_ws
    for args in ((None, Wp, dX), (dC, None, dX), (dC, Wp, None)):
        assert f(*args, M, N, K, ws, big, None) == B.ERR_NULL
    assert f(dC, Wp, dX, 0, N, K, ws, big, None) == B.ERR_DIM
    assert f(dC, Wp, dX, M, N, 6, ws, big, None) == B.ERR_PACK
    assert f(dC, Wp, dX, M, N, K, ws, -1, None) == B.ERR_DIM
    for w in (dC + 64, Wp + N * K // 4 - 16, dX + 100, dX - big + 16):
        assert f(dC, Wp, dX, M, N, K, w, big, None) == B.ERR_ALIAS, hex(w)
    g = L.ternary_gemm_s8_dx_scaled_ws
    assert g(dC, Wp, None, 1.0, dX, B.OUT_F32, M, N, K, ws, big, None) == B.ERR_NULL
    assert g(dC, Wp, rs, 1.0, dX, 7, M, N, K, ws, big, None) == B.ERR_KIND
    assert g(dC, Wp, rs, 1.0, dX, B.OUT_F32, M, N, K, ws, -5, None) == B.ERR_DIM
    assert g(dC, Wp, rs, 1.0, dX, B.OUT_BF16, M, N, K, rs - 8, 64, None) == B.ERR_ALIAS
    assert g(dC, Wp, rs, 1.0, dX, B.OUT_BF16, M, N, K, dX + M * K * 2 - 4, 64, None) == B.ERR_ALIAS


@pytest.mark.parametrize("cus,xcds", [(64, 4), (80, 8), (304, 8), (256, 1)])
def test_plans_follow_the_machine(cus, xcds):
    # on a machine with other CU / XCD counts the persistent kernels launch
    # one workgroup per CU, the order still covers every tile once, and the
    # tile counts that choose a kernel scale with the CUs
    for op, shape in (("fwd", (16384, 3456, 1280)), ("fwd", (16300, 3450, 640)), ("dx", (16384, 3456, 1280)),
                      ("fwd", (300, 272, 96)), ("dw", (1782, 3456, 1280))):
        pl = _coverage(op, *shape, cus=cus, xcds=xcds)
        assert pl.xcds == xcds
        if pl.kernel == B.KERNEL_STREAM:
            assert pl.workgroups == cus
            assert pl.tiles_per_workgroup == -(-(-(-pl.tiles // xcds)) // (cus // xcds))
    # at least one 512 x 144 tile per CU: 768 tiles take the stream kernel up to 768 CUs
    assert B.plan("fwd", 16384, 3456, 1280, cus=768, xcds=8).kernel == B.KERNEL_STREAM
    assert B.plan("fwd", 16384, 3456, 1280, cus=776, xcds=8).kernel == B.KERNEL_TILED
    # the split dX kernel serves outputs of at most one 128 x 144 tile per CU
    assert B.plan("dx", 1782, 3456, 1280, cus=64, xcds=8).kernel == B.KERNEL_TILED
    with pytest.raises(B.TernaryGemmError):
        B.plan("fwd", 300, 272, 96, cus=100, xcds=8)     # CUs not a multiple of the XCDs


def test_noalloc_argument_checks_before_any_device_call():
    # pointer and dimension errors return before the call touches a device
    f = B.lib().ternary_gemm_s8_dx_noalloc
    x = 1 << 20
    assert f(None, x, x, 4, 4, 4, None) == B.ERR_NULL
    assert f(x, None, x, 4, 4, 4, None) == B.ERR_NULL
    assert f(x, x, None, 4, 4, 4, None) == B.ERR_NULL
    assert f(x, x, x, 0, 4, 4, None) == B.ERR_DIM
    assert f(x, x, x, 4, 4, 6, None) == B.ERR_PACK
    assert "scratch" in B.status_str(B.ERR_SCRATCH)
