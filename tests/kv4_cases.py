"""Shapes of the KV4 attention parity tests, with the launch plan each one is
meant to reach: (query heads per workgroup, token chunks).  The attention has
one kernel per (heads per workgroup R in {1, 2, 4}, token-split or not); the
plan pins below make a change of the launch plan that would drop one of those
kernels from the tests fail on the CPU (tests/test_kv4_plans.py) instead of
passing unnoticed on the GPU."""

# (B, H, Hkv, T, lengths, peak, plan) for the single-pass entry
PLAIN = [
    (2, 4, 4, 64, [64, 17], 1.0, (1, 1)),          # full and partial unroll rounds
    (3, 8, 2, 200, [200, 1, 0], 1.0, (1, 1)),      # GQA, a single token, an empty sequence
    (1, 2, 1, 1000, [999], 4.0, (1, 1)),           # sharp softmax, T not a multiple of 64
    (4, 4, 4, 256, [256, 255, 129, 64], 1.0, (1, 1)),
    (4, 16, 2, 96, [96, 50, 1, 33], 1.0, (1, 1)),  # 8 heads per kv head: eight 1-head blocks each, XCD-grouped
    (32, 32, 8, 100, [100, 1, 77, 64] * 8, 1.0, (2, 1)),  # 2 heads a block (512 blocks; 4 heads give 256)
    (1, 6, 2, 128, [128], 1.0, (1, 1)),            # 3 heads per kv head: one head per block
    (1, 8, 2, 9000, [9000], 1.0, (1, 1)),          # 4 heads per kv head, few blocks: one head a block
    (1, 4, 1, 20000, [19999], 1.0, (1, 1)),        # ... and one per block
    (64, 8, 2, 150, [150, 3] * 32, 1.0, (1, 1)),   # 4 heads per kv head, 512 one-head blocks
    (128, 32, 8, 70, [70, 69] * 64, 1.0, (4, 1)),  # 4 heads a block (1024 blocks)
]

# (B, H, Hkv, T, lengths, peak, plan) for the token-split entry
SPLIT = [
    (1, 32, 8, 4096, [4096], 1.0, (2, 16)),             # 16 chunks of 256 tokens, two heads a workgroup
    (2, 32, 32, 3000, [3000, 1], 1.0, (1, 12)),         # MHA, 12 chunks of 256; one token: 11 empty chunks
    (4, 32, 32, 4096, [4096, 3000, 1025, 0], 1.0, (1, 4)),  # 4 chunks of 1024; 1025: a one-token chunk
    (3, 8, 2, 1000, [1000, 0, 513], 1.0, (2, 4)),       # empty sequence; 513 = two chunks and one token
    (1, 2, 1, 1000, [999], 4.0, (2, 4)),                # sharp softmax across chunks
    (1, 6, 2, 2000, [1777], 1.0, (1, 8)),               # 3 heads per kv head: one a workgroup
    (1, 4, 1, 32768, [32768], 1.0, (2, 128)),           # the longest cache: 128 chunks
    (1, 32, 8, 32768, [30001], 1.0, (2, 32)),           # 1024-token chunks; the last three partial or empty
    (4, 64, 8, 8192, [8192, 5000, 8191, 1], 1.0, (4, 8)),  # four heads a workgroup, 1024-token chunks
    (2, 8, 1, 20000, [20000, 8191], 1.0, (2, 79)),      # 8-head groups, chunk ends inside a sequence
]

# (B, H, Hkv, T, split, plan) for the query edge cases, one per kernel family
EDGE = [
    (1, 8, 2, 1500, False, (1, 1)),
    (1, 8, 2, 1500, True, (2, 6)),
    (32, 32, 8, 100, False, (2, 1)),
    (2, 32, 32, 3000, True, (1, 12)),
    (64, 32, 8, 300, False, (4, 1)),
    (4, 64, 8, 8192, True, (4, 8)),
]
