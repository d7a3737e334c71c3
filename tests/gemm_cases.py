"""Shapes of the W4A8 GEMM parity tests (M, K, N, group size), each with the
launch plan it is meant to reach: (kernel family, strips per block or
large-M tile, K parts per block or K splits across blocks), as
qoq_w4a8_gemm_plan reports it.  The
pins make a plan change that would drop a kernel variant from the parity
tests fail on the CPU (tests/test_gemm_plans.py)."""

SMALL = [
    (16, 256, 256, 128, ('strip', 1, 8)),  # the tiny workload shape
    (1, 128, 16, 128, ('strip', 1, 8)),
    (17, 384, 40, 128, ('skinny32', 1, 4)),
    (63, 256, 200, 128, ('skinny64', 1, 4)),
    (64, 512, 96, 128, ('skinny64', 1, 4)),
    (65, 256, 130, 128, ('skinny64', 1, 4)),
    (130, 640, 72, 128, ('skinny64', 1, 4)),
    (257, 384, 300, 128, ('large', 1, 1)),
    (5, 256, 48, 0, ('strip', 1, 8)),
    (70, 384, 100, 0, ('skinny64', 1, 4)),
    (200, 2048, 96, 128, ('skinny64', 1, 4)),  # skinny 64-row tiles: 4 row blocks of one strip, K split over 4 waves
    (97, 1920, 40, 128, ('skinny64', 1, 4)),  # ... 15 groups: K parts of 3 and 4 groups per wave
    (256, 1024, 50, 0, ('skinny64', 1, 4)),  # ... per-channel, 4 row blocks
    (300, 2048, 96, 128, ('large', 1, 4)),  # large-M kernel, K split in 4 (INT32 partials + reduction)
    (290, 1920, 40, 128, ('large', 1, 2)),  # ... K split in 2 with an odd group count per split
    (270, 1024, 50, 0, ('large', 1, 2)),  # ... per-channel with a K split
    (300, 640, 520, 128, ('large', 1, 1)),  # small 64x256 tiles, ragged M and N
    (520, 512, 300, 128, ('large', 1, 1)),  # small tiles, ragged M and N
    (16, 512, 9615, 128, ('strip', 3, 2)),  # strip kernel: 3 strips x 2 K parts per block, dead waves past N
    (1, 256, 27990, 0, ('strip', 7, 1)),  # strip kernel: 7 strips per block, per-channel, ragged N
    (12, 384, 200, 128, ('strip', 1, 8)),  # strip kernel: odd row count, K split in 8 with empty parts
    (16, 10112, 40, 128, ('strip', 1, 8)),  # strip kernel: activations and metadata fill all 160 KB of LDS
    (16, 10240, 40, 128, ('skinny16', 1, 8)),  # one group more exceeds LDS: K-split skinny kernel instead
    (16, 2048, 20000, 128, ('strip', 5, 1)),  # strip kernel, 5 strips per block: second activation copy after the barrier
    (8, 1024, 3000, 128, ('strip', 1, 8)),  # strip kernel, 8 rows: groups padded to 16 LDS rows, group-major copies, K in 8 parts
    (15, 2048, 5000, 0, ('strip', 2, 4)),  # ... per-channel, 15 rows, 2 strips x 4 K parts
    (13, 4096, 28672, 128, ('strip', 7, 1)),  # ... 13 rows, 7 strips per block (the decode layout), rows 13-15 repeat row 12
    (9, 10112, 100, 128, ('strip', 1, 8)),  # ... 9 rows padded to 16: activations and metadata fill all 160 KB of LDS
    (8, 10240, 100, 128, ('strip', 1, 8)),  # ... one group more: 8 rows keep the dense layout (padded would exceed LDS)
    (8, 14336, 4096, 0, ('strip', 1, 8)),  # ... dense 8-row groups at K = 14336 (the 8B down projection), per-channel
    (15, 10752, 100, 128, ('strip', 1, 8)),  # ... 15 dense rows fill the LDS
    (15, 10880, 100, 128, ('skinny16', 1, 8)),  # ... one group more: neither layout fits, K-split skinny kernel instead
    (7, 1664, 17000, 0, ('strip', 5, 1)),  # ... per-channel, odd row count, copies running into padding
    (512, 256, 24576, 128, ('large', 0, 1)),  # big 128x512 tiles (192 of them), 2 groups
    (520, 384, 24400, 0, ('large', 0, 1)),  # ... per-channel, ragged M and N, 3 groups
    (768, 640, 16384, 128, ('large', 0, 1)),  # ... 5 groups: the four-slot LDS ring wraps
    (512, 1024, 24576, 128, ('large', 0, 1)),  # ... 8 groups: 192 tiles fill one round, so no K split
    (256, 1024, 12288, 128, ('large', 1, 1)),  # small tiles, 192 of them: no K split (a split would need 2 rounds)
    (640, 1024, 4096, 0, ('large', 1, 1)),  # ... per-channel, 160 tiles, ragged last row tile
    (256, 512, 4096, 128, ('skinny64', 4, 4)),  # up to 256 rows in one round of skinny blocks (4 strips, K split in LDS)
    (200, 384, 4000, 0, ('skinny64', 4, 4)),  # ... per-channel, ragged M and N (252 blocks)
    (80, 256, 14336, 128, ('skinny64', 7, 4)),  # skinny 64-row tiles at most 7 strips per block; rows past M repeat row M-1
    (192, 640, 4096, 128, ('skinny64', 4, 4)),  # 3 row blocks of 4 strips (192 blocks): strip count from the activation-aware cost
    (161, 384, 2000, 0, ('skinny64', 2, 4)),  # ... per-channel, 2 strips per block, ragged last row block and last strip block
    (250, 1024, 160, 128, ('skinny64', 1, 4)),  # ... one strip per block, 4 row blocks, rows past M in the last
    (50, 384, 30000, 0, ('skinny64', 4, 4)),  # ... per-channel, ragged N
    (64, 8192, 2000, 128, ('skinny64', 1, 8)),  # 8 K parts per skinny block (two waves per SIMD), 8 groups each, ragged N
    (48, 8320, 1000, 0, ('skinny64', 1, 8)),  # ... per-channel, 65 groups: K parts of 8 and 9 groups
    (64, 8192, 4100, 128, ('skinny64', 2, 8)),  # ... 2 strips per block, the last block with one valid strip
    (20, 16384, 520, 128, ('skinny32', 1, 8)),  # ... 32-row tiles, rows past M repeat row M-1
    (1024, 8320, 4096, 128, ('large', 2, 1)),  # K-set 128x128 tile (two sets of 4 waves), odd group count: the last step has one group
    (1000, 8192, 4000, 0, ('large', 2, 1)),  # ... per-channel, ragged M and N
    (512, 32768, 2048, 128, ('large', 2, 4)),  # ... with K split in 4 across blocks (64 groups per split)
    (384, 32768, 2048, 0, ('large', 2, 4)),  # ... per-channel, K split in 4
    (40, 256, 32768, 128, ('skinny64', 4, 4)),  # skinny 64-row tiles, 4 strips per block; rows past M repeat row M-1
    (40, 1024, 20000, 128, ('ring', 5, 1)),  # ring kernel (one strip per wave, activations through an LDS ring): one batch of 8 groups
    (33, 2048, 28000, 0, ('ring', 7, 1)),  # ... per-channel, two batches, rows past M
    (24, 5120, 24000, 128, ('ring', 6, 1)),  # ... 32-row tiles, five batches
    (16, 10240, 20000, 128, ('ring', 5, 2)),  # ... 16-row tiles where the strip kernel's LDS is too small: two waves a strip (K halves)
    (64, 1024, 32768, 128, ('ring', 8, 1)),  # ... eight strips per block (256 blocks)
    (60, 3072, 17000, 0, ('ring', 5, 1)),  # ... per-channel, three batches, dead waves past N in the last block
    (48, 8192, 20000, 0, ('ring', 5, 1)),  # ring kernel, 64-row tiles at 64 groups: one wave a strip, per-channel
    (64, 8192, 17000, 128, ('ring', 5, 1)),  # ... 64 rows, 8 batches, dead waves past N in the last block
    (20, 8192, 24000, 128, ('ring', 6, 2)),  # ring kernel, K halves over two waves a strip (64 groups on, up to 32 rows)
    (24, 8192, 20000, 0, ('ring', 5, 2)),  # ... per-channel, 32-row tiles, rows past M
    (12, 16384, 20000, 0, ('ring', 5, 2)),  # ... per-channel, 16-row tiles (neither strip layout fits LDS)
    (30, 8192, 32768, 128, ('ring', 8, 2)),  # ... 8 strips a block (16 waves)
    (20, 8192, 17000, 0, ('ring', 5, 2)),  # ... per-channel, ragged N: the last block has 3 live strips (4 dead waves)
    (16, 12288, 17000, 128, ('ring', 5, 2)),  # ... 16-row tiles, 96 groups, ragged N
]
