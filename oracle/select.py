"""Candidate selector: one path through the per-position top-K (test infrastructure only).

Sources: FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", spec table ("Draft" row:
candidate selector, top 16, rank 256; "Weights" row: two 248320 x 256 selector
codebooks) and section "How it is used" (one coherent path through the top 16
candidates per position); Mindket kit page, section "For newcomers and experts"
(a small selector picks a single consistent path).

The pages name the selector but do not fix its objective.  The objective used
here: a path picks one candidate c_t (index into the top-K list) per proposal
position t = 0..P-1 and scores

    sum_t lp[t, c_t]  +  s * sum_{t<P-1} < A[id[t, c_t]], B[id[t+1, c_{t+1}]] >

with lp the candidate log-probabilities, A and B the two codebooks and s the pair
scale (1/sqrt(rank)).  The maximiser is found by dynamic programming (Viterbi);
ties go to the lowest candidate index, at the last position and for every
predecessor.
"""
import itertools
import numpy as np


def pair_scores(ids, A, B, s, dtype=np.float64):
    """ids [P, K] -> T [P-1, K, K], T[t, i, j] = s * <A[ids[t,i]], B[ids[t+1,j]]>."""
    ids = np.asarray(ids)
    P, K = ids.shape
    A = np.asarray(A, dtype=dtype)
    B = np.asarray(B, dtype=dtype)
    T = np.empty((P - 1, K, K), dtype=dtype)
    for t in range(P - 1):
        T[t] = dtype(s) * (A[ids[t]] @ B[ids[t + 1]].T)
    return T


def viterbi(lp, T, dtype=np.float64):
    """lp [P, K] candidate scores, T [P-1, K, K] transition scores -> (path idx [P], best score).

    delta[0] = lp[0];  delta[t+1][j] = lp[t+1][j] + max_i (delta[t][i] + T[t][i][j]),
    psi[t+1][j] = the lowest i attaining that max;  the final index is the lowest
    argmax of delta[P-1]; the path is read back through psi.
    """
    lp = np.asarray(lp, dtype=dtype)
    T = np.asarray(T, dtype=dtype)
    P, K = lp.shape
    delta = lp[0].copy()
    psi = np.zeros((P, K), dtype=np.int64)
    for t in range(P - 1):
        cand = delta[:, None] + T[t]            # [i, j]
        best_i = np.argmax(cand, axis=0)        # first (lowest) index of the max
        delta = lp[t + 1] + cand[best_i, np.arange(K)]
        psi[t + 1] = best_i
    j = int(np.argmax(delta))
    best = delta[j]
    path = np.empty(P, dtype=np.int64)
    path[P - 1] = j
    for t in range(P - 1, 0, -1):
        j = int(psi[t, j])
        path[t - 1] = j
    return path, best


def path_score(lp, T, path):
    """Score of one explicit path (used by brute force and by tie-band checks)."""
    P = len(path)
    sc = sum(lp[t, path[t]] for t in range(P))
    sc += sum(T[t, path[t], path[t + 1]] for t in range(P - 1))
    return sc


def brute_force(lp, T):
    """Enumerate all K^P paths.  Returns (best path, best score, second-best score).

    Among exactly equal scores the winner is the path that is smallest when read
    from the last position backwards (the same tie rule as the Viterbi above).
    Vectorised over the last P-2 positions; loops over the first two.
    """
    lp = np.asarray(lp, dtype=np.float64)
    T = np.asarray(T, dtype=np.float64)
    P, K = lp.shape
    assert P >= 3
    # tail[i2, ..., i_{P-1}] = sum_{t>=2} lp[t, i_t] + sum_{t>=2} T[t, i_t, i_{t+1}]
    tail = lp[P - 1].copy()
    for t in range(P - 2, 1, -1):
        # prepend axis for position t
        tail = lp[t].reshape((K,) + (1,) * tail.ndim) + tail[None, ...] \
            + T[t].reshape((K, K) + (1,) * (tail.ndim - 1))
    top = [-np.inf, -np.inf]          # best and second-best score seen
    best_path = None
    for i0, i1 in itertools.product(range(K), range(K)):
        head = lp[0, i0] + lp[1, i1] + T[0, i0, i1]
        tot = head + tail + T[1, i1].reshape((K,) + (1,) * (tail.ndim - 1))
        flat = tot.reshape(-1)
        two = np.partition(flat, flat.size - 2)[-2:]
        top = sorted(top + [float(two[0]), float(two[1])])[-2:]
        mx = flat.max()
        if mx >= top[1]:
            for f in np.flatnonzero(flat == mx):
                rest = np.unravel_index(f, tot.shape)
                p = (i0, i1) + tuple(int(r) for r in rest)
                cur = None if best_path is None else path_score(lp, T, best_path)
                if cur is None or mx > cur or (mx == cur and p[::-1] < tuple(best_path)[::-1]):
                    best_path = p
    return np.array(best_path, dtype=np.int64), top[1], top[0]
