"""Exact linear projections of an INT32 product acc = x8 @ w8^T, for checking
every accumulator of products too large for the oracle to form one output at
a time.  Observed side: the accumulators under test; expected side: the
oracle's operands only (its activation codes and its weight encode, taken in
chunks of output channels).  Test infrastructure."""

import numpy as np

import oracle as O

CHUNK = 2048


def project_observed(acc, r_list, c_list):
    """acc^T r and acc c of the GPU accumulators, exactly (float64 sums of
    integers below 2^53), in row chunks."""
    M, N = acc.shape
    rt = [np.zeros(N) for _ in r_list]
    ac = [np.zeros(M) for _ in c_list]
    for m0 in range(0, M, 512):
        a = acc[m0:m0 + 512].astype(np.float64)
        for i, r in enumerate(r_list):
            rt[i] += r[m0:m0 + 512].astype(np.float64) @ a
        for i, c in enumerate(c_list):
            ac[i][m0:m0 + 512] = a @ c.astype(np.float64)
    return [v.astype(np.int64) for v in rt], [v.astype(np.int64) for v in ac]


def project_expected(x8, W, group_size, r_list, c_list):
    """The same projections from the oracle's operands, in int64."""
    N = W.shape[0]
    x = x8.astype(np.int64)
    u = [x.T @ r for r in r_list]                  # x8^T r, per r (K)
    rt = [np.zeros(N, np.int64) for _ in r_list]
    wc = [np.zeros(x.shape[1], np.int64) for _ in c_list]
    for n0 in range(0, N, CHUNK):
        enc = O.encode_weight_g128(W[n0:n0 + CHUNK]) if group_size else O.encode_weight_per_channel(W[n0:n0 + CHUNK])
        w8 = enc["w8"].astype(np.int64)
        for i in range(len(r_list)):
            rt[i][n0:n0 + CHUNK] = w8 @ u[i]
        for i, c in enumerate(c_list):
            wc[i] += w8.T @ c[n0:n0 + CHUNK]
    ac = [x @ v for v in wc]
    return rt, ac
