"""Shapes (M, N, K) for the GPU parity tests: every tile shape of each product
on both load paths (fast: vector loads; slow: guarded byte loads), with ragged
edges in all three dimensions, plus degenerate edge shapes."""

FWD_SHAPES = [
    (8200, 3900, 80), (8200, 3900, 84),    # 256 x 128 tile
    (4100, 900, 80), (4100, 900, 84),      # 128 x 144
    (4100, 3900, 80), (4100, 3900, 84),
    (300, 272, 96), (299, 271, 100),       # 64 x 64
    (1, 1, 4), (1, 4097, 36), (1000, 1, 64), (65, 65, 68)]

DX_SHAPES = [  # contraction N; the fast path needs N % 16 == K % 16 == 0
    (8200, 80, 3904), (8200, 84, 3900),
    (4100, 80, 912), (4100, 84, 900),
    (4100, 80, 3904), (4100, 84, 3900),
    (300, 96, 272), (299, 100, 268),
    (1, 1, 4), (1, 16, 16), (27, 3456, 1280), (1, 4, 4100),
    # 128 x 144 tiles leaving more than half the CUs idle: 64 x 64 tiles; the
    # pages' backward batch, a ragged last step, odd step counts on the byte
    # path, a long contraction
    (1782, 3456, 1280), (1782, 3440, 1296), (1500, 1030, 1152), (1300, 900, 1436), (640, 8192, 2048),
    # 128 x 144 tiles filling more than half of the CUs but not all of them:
    # the contraction split between two halves of a workgroup, on the vector
    # and the byte path
    (3000, 3456, 1280), (2600, 3450, 1284)]

DW_SHAPES = [  # contraction M; the fast path needs N % 16 == K % 16 == 0
    (80, 3904, 8208), (81, 3901, 8201),
    (80, 912, 4112), (80, 901, 4101),
    (80, 3904, 4112), (80, 3901, 4101),
    (96, 272, 304), (97, 271, 299),
    (1, 1, 1), (1782, 5, 7), (1782, 16, 16), (27, 3456, 1280),
    (1088, 912, 4112), (1000, 901, 4101)]   # long contractions: the split dW kernel

TILES = ((256, 128), (128, 144), (64, 64))

# Shapes for the streaming forward kernel (K % 64 == 0, at least 256 tiles of
# 512 x 144): interior tiles only, ragged M and N on both store paths (N % 4
# != 0 has no 16-byte stores), tile counts that do not split evenly between
# the workgroups, and one or two steps per tile.
STREAM_SHAPES = [(16300, 3450, 640), (15000, 3460, 192), (4096, 4608, 64), (8192, 2304, 128),
                 (40000, 1000, 2112)]

# Shapes for the streaming dX kernel (contraction N % 64 == 0, K % 16 == 0, at
# least 256 tiles of 512 x 160): the timed shape, ragged M with a last column
# tile of 16 or 144 of its 160 columns, and one or two contraction steps.
DX_STREAM_SHAPES = [(16300, 3456, 1296), (15000, 2048, 1424), (8192, 64, 5120), (4096, 128, 10240)]

# Shapes for the skinny forward kernel (M <= 32, K % 64 == 0): one and two
# 16-row blocks, column blocks of 16, 32 and 64 with ragged last blocks (N % 4
# != 0 has no 16-byte stores), contractions that end inside a super-step of
# 256 (one, two or three 64-steps left) or in a whole one, fewer super-steps
# than waves, and the pages' row count at their weight shapes.
SKINNY_SHAPES = [(1, 16, 64), (16, 100, 192), (17, 3456, 1280), (27, 3456, 1280), (27, 1280, 3456),
                 (32, 4099, 2112), (5, 8200, 4160), (1, 16384, 16384), (27, 16384, 16384),
                 (32, 65, 64), (2, 4096, 512), (31, 8256, 768)]

# Shapes for the skinny dX kernel (M <= 32, contraction N % 64 == 0, K % 16
# == 0): column blocks of 16 and 64, one and two 16-row blocks, fewer steps
# than waves, the pages' 27-row backward at their weight shapes, and the
# skinny workload's weights.
SKINNY_DX_SHAPES = [(1, 64, 16), (16, 128, 48), (17, 640, 1296), (27, 3456, 1280), (27, 1280, 3456),
                    (32, 192, 8192), (5, 8192, 8192), (27, 16384, 16384), (2, 4096, 4112), (31, 64, 8208)]

# dX with a workspace, shapes that take the split kernel (M <= 32, N % 64 == 0,
# K % 256 == 0, K / 256 < 256 column blocks): the pages' 27 rows at 16384^2
# (4 splits), one row, one 16-row block with 8 splits, 17 rows with exactly one
# step per wave and split, 32 rows with 16 splits, 256 splits of one column
# block, splits of unequal length (33 and 100 steps over 4 and 6 splits; 300
# workgroups)
SPLIT_DX_SHAPES = [(27, 16384, 16384), (1, 16384, 16384), (16, 4096, 8192), (17, 2048, 16384),
                   (32, 8192, 4096), (5, 131072, 256), (27, 2112, 16384), (3, 6400, 12800)]
