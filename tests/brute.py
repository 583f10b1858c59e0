"""Pure-Python brute force of softmax attention for tiny inputs (a pin of the oracle).

Independent of oracle/: Python floats, math.exp and math.fsum (exactly rounded
sums), nested lists.  Follows the plain definition: for query i the logits are
s_ij = scale * sum_c q[i][c] * k[j][c] over the visible keys j; the output is
sum_j exp(s_ij - M) v_j / sum_j exp(s_ij - M) with M = max_j s_ij, and
LSE = M + log(sum_j exp(s_ij - M)).
"""
import math


def _tolist(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to(torch.float64).tolist()
    except ImportError:
        pass
    return x.tolist() if hasattr(x, "tolist") else x


def attention(q, k, v, q_off=0, kv_off=0, causal=False, scale=None):
    """q [B][nq][Hq][d], k/v [B][nkv][Hkv][d] -> (O [B][nq][Hq][d], LSE [B][Hq][nq])."""
    q, k, v = _tolist(q), _tolist(k), _tolist(v)
    B, nq, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    nkv, Hkv = len(k[0]), len(k[0][0])
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = [[[[0.0] * d for _ in range(Hq)] for _ in range(nq)] for _ in range(B)]
    L = [[[0.0] * nq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(nq):
                js = [j for j in range(nkv) if (not causal) or kv_off + j <= q_off + i]
                s = [scale * math.fsum(q[b][i][h][c] * k[b][j][g][c] for c in range(d)) for j in js]
                M = max(s)
                w = [math.exp(x - M) for x in s]
                den = math.fsum(w)
                for c in range(d):
                    O[b][i][h][c] = math.fsum(w[t] * v[b][j][g][c] for t, j in enumerate(js)) / den
                L[b][h][i] = M + math.log(den)
    return O, L
