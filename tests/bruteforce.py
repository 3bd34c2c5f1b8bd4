"""Pure-Python brute-force attention on tiny inputs (pins the oracle).

Written independently of oracle/: explicit loops over query rows and keys,
``math.exp`` and ``math.fsum`` (exactly rounded sums). The definition
followed is softmax(Q K^T * scale) V per row, with causal rows seeing keys
0..i (mlqm.cn/news/343191 chapter 1 and §3.1), and packed sequences kept
apart by their prefix offsets (lnrk.cn/news/11729 §1).
"""
import math


def row(qrow, keys, vals, scale, biases=None):
    """Output and log-sum-exp of one query row against the list of visible keys."""
    logits = []
    for n, kr in enumerate(keys):
        x = scale * math.fsum(a * b for a, b in zip(qrow, kr))
        if biases is not None:
            x += biases[n]
        logits.append(x)
    mx = max(logits)
    ws = [math.exp(x - mx) for x in logits]
    tot = math.fsum(ws)
    D = len(vals[0])
    out = [math.fsum(ws[j] / tot * vals[j][d] for j in range(len(keys))) for d in range(D)]
    return out, mx + math.log(tot)


def padded(q, k, v, causal, scale):
    """q,k,v nested lists [B][S][H][D] -> (O [B][S][H][D], LSE [B][H][S])."""
    B, S, H = len(q), len(q[0]), len(q[0][0])
    O = [[[None] * H for _ in range(S)] for _ in range(B)]
    L = [[[None] * S for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(S):
                n = i + 1 if causal else S
                keys = [k[b][j][h] for j in range(n)]
                vals = [v[b][j][h] for j in range(n)]
                O[b][i][h], L[b][h][i] = row(q[b][i][h], keys, vals, scale)
    return O, L


def packed(q, k, v, cu, causal, scale):
    """q,k,v nested lists [T][H][D], cu prefix offsets -> (O [T][H][D], LSE [H][T])."""
    T, H = len(q), len(q[0])
    O = [[None] * H for _ in range(T)]
    L = [[None] * T for _ in range(H)]
    for s in range(len(cu) - 1):
        a, e = cu[s], cu[s + 1]
        for h in range(H):
            for i in range(a, e):
                last = i if causal else e - 1
                keys = [k[j][h] for j in range(a, last + 1)]
                vals = [v[j][h] for j in range(a, last + 1)]
                O[i][h], L[h][i] = row(q[i][h], keys, vals, scale)
    return O, L


def sees(i, j, causal, window, n_global):
    """Key j visible to query i (local indices): window of `window` keys ending at i
    (|i - j| < window without causality); the first n_global rows see every key."""
    if i < n_global:
        return True
    if causal and j > i:
        return False
    if window > 0 and (i - j >= window or j - i >= window):
        return False
    return True


def padded_ext(q, k, v, causal, scale, window, n_global, slopes):
    """Like padded() with the window / global-row mask and ALiBi slopes (or None)."""
    B, S, H = len(q), len(q[0]), len(q[0][0])
    O = [[[None] * H for _ in range(S)] for _ in range(B)]
    L = [[[None] * S for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(S):
                js = [j for j in range(S) if sees(i, j, causal, window, n_global)]
                bias = None if slopes is None else [-slopes[h] * abs(i - j) for j in js]
                O[b][i][h], L[b][h][i] = row(q[b][i][h], [k[b][j][h] for j in js],
                                             [v[b][j][h] for j in js], scale, bias)
    return O, L


def decode(q, kc, vc, lens, causal, scale):
    """KV-cache decode: q [B][Sq][H][D], caches [B][H][S_max][D], valid lengths per sequence.
    Query row i sits at position L - Sq + i; under causality it sees keys up to there.
    Returns (O [B][Sq][H][D], LSE [B][H][Sq]); rows with no visible key give zeros and -inf."""
    B, Sq, H = len(q), len(q[0]), len(q[0][0])
    Dv = len(vc[0][0][0])
    O = [[[None] * H for _ in range(Sq)] for _ in range(B)]
    L_ = [[[None] * Sq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        L = lens[b]
        for h in range(H):
            for i in range(Sq):
                js = [j for j in range(L) if not causal or j <= L - Sq + i]
                if not js:
                    O[b][i][h], L_[b][h][i] = [0.0] * Dv, -math.inf
                    continue
                O[b][i][h], L_[b][h][i] = row(q[b][i][h], [kc[b][h][j] for j in js],
                                              [vc[b][h][j] for j in js], scale)
    return O, L_
