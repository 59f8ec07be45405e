"""Pure-Python brute force used to pin the oracle on tiny inputs.

Every score is materialised; O = sum_j e^{s_ij} v_j / sum_j e^{s_ij} and
LSE = ln sum_j e^{s_ij} are evaluated WITHOUT max-shifting, with math.exp and
math.fsum, so that no formula path is shared with the oracle (inputs are small
N(0,1) values, so the exponentials stay in range).
"""

import math


def brute_attention(q, k, v, q_idx, k_idx, scale, causal, seg_q=None, seg_k=None):
    """q: [Nq][Hq][d] nested lists; k, v: [Nk][Hkv][d].  Returns (O [Nq][Hq][d],
    LSE [Hq][Nq]) with O = 0 and LSE = -inf for rows without any visible key."""
    nq, hq, d = len(q), len(q[0]), len(q[0][0])
    hkv = len(k[0])
    group = hq // hkv
    o = [[[0.0] * d for _ in range(hq)] for _ in range(nq)]
    lse = [[-math.inf] * nq for _ in range(hq)]
    for i in range(nq):
        for h in range(hq):
            g = h // group
            weights = []
            for j in range(len(k)):
                if causal and k_idx[j] > q_idx[i]:
                    continue
                if seg_q is not None and seg_q[i] != seg_k[j]:
                    continue
                s = scale * math.fsum(q[i][h][t] * k[j][g][t] for t in range(d))
                weights.append((math.exp(s), j))
            if not weights:
                continue
            z = math.fsum(w for w, _ in weights)
            for t in range(d):
                o[i][h][t] = math.fsum(w * v[j][g][t] for w, j in weights) / z
            lse[h][i] = math.log(z)
    return o, lse


def brute_segment_ids(pos_row):
    """Sample index per token by walking the row: a new sample starts at pos == 0."""
    out = []
    cur = -1
    for p in pos_row:
        if p == 0:
            cur += 1
        out.append(cur)
    return out
