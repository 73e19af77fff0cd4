"""Trellis-coded quantization with a Viterbi search (oracle, test infrastructure only).

Pingala-8 post, "Trick 3: trellis coding": the encoder carries a state from one step to the
next; the state decides which subset (coset) of values the next step may use; the bits written
pick a value inside the subset and set the next state; the decoder tracks the state.  The best
path is found by the Viterbi algorithm, dynamic programming that keeps, for every state, the
cheapest path ending there.

Readings (the post gives the toy in full but not its 8-state trellis):
* one weight per step; S = 2^m states; from state s one branch bit u leads to the state
  ((s << 1) | u) mod S (a shift register; the post's toy is the case S = 2, where the bit
  written becomes the next state);
* branch (s, u) carries a coset of C values, ``values[s, u, :]``; the within-coset index v is
  written with u, code = u | (v << 1), and is the nearest value of the coset (the smaller index
  on a tie), since it does not affect the state;
* cost = sum of squared errors; the path starts in ``start_state``; ties between paths go to
  the predecessor with the smaller state index, and the path ends in the cheapest state (the
  smaller index on a tie).
"""

import numpy as np


def predecessors(s, S):
    """The two states that lead to s, and the branch bit: ((s >> 1) + j S/2 for j = 0, 1; s & 1)."""
    return (s >> 1), (s >> 1) + S // 2, s & 1


def coset_choice(t, coset):
    """Nearest value of a coset to each target t (the smaller index on a tie): (index, value)."""
    t = np.asarray(t, dtype=np.float64)
    d = (t[..., None] - np.asarray(coset, dtype=np.float64)) ** 2
    v = np.argmin(d, axis=-1)
    return v, np.take_along_axis(np.broadcast_to(coset, d.shape), v[..., None], axis=-1)[..., 0]


def viterbi(T, values, start_state=0):
    """Cheapest path through the trellis for each row of targets T (rows x n).

    values: S x 2 x C reconstruction values of branch (s, u).  Returns dict(codes (rows x n,
    u | v << 1), recon (rows x n), cost (rows), states (rows x (n + 1), the state before each
    step and the final one)).
    """
    T = np.atleast_2d(np.asarray(T, dtype=np.float64))
    values = np.asarray(values, dtype=np.float64)
    S = values.shape[0]
    if S < 2 or S & (S - 1) or values.shape[1] != 2:
        raise ValueError("values must be S x 2 x C with S a power of two >= 2")
    rows, n = T.shape
    cost = np.full((rows, S), np.inf)
    cost[:, start_state] = 0.0
    took_upper = np.zeros((n, rows, S), dtype=bool)
    for k in range(n):
        # branch metric of (s, u): distance to the nearest value of its coset
        bm = np.min((T[:, k, None, None, None] - values[None]) ** 2, axis=3)  # rows x S x 2
        new = np.empty((rows, S))
        for s in range(S):
            p0, p1, u = predecessors(s, S)
            c0 = cost[:, p0] + bm[:, p0, u]
            c1 = cost[:, p1] + bm[:, p1, u]
            up = c1 < c0
            new[:, s] = np.where(up, c1, c0)
            took_upper[k, :, s] = up
        cost = new
    end = np.argmin(cost, axis=1)
    states = np.zeros((rows, n + 1), dtype=np.int64)
    codes = np.zeros((rows, n), dtype=np.int64)
    recon = np.zeros((rows, n))
    s = end.copy()
    states[:, n] = s
    for k in range(n - 1, -1, -1):
        up = took_upper[k, np.arange(rows), s]
        p = (s >> 1) + up * (S // 2)
        u = s & 1
        v, val = coset_choice(T[:, k], values[p, u])
        codes[:, k] = u | (v << 1)
        recon[:, k] = val
        states[:, k] = p
        s = p
    if not np.all(states[:, 0] == start_state):
        raise AssertionError("traceback did not return to the start state")
    return {"codes": codes, "recon": recon, "cost": cost[np.arange(rows), end], "states": states}


def greedy(T, values, start_state=0):
    """Round each step to the nearest value the current state allows, following its state."""
    T = np.atleast_2d(np.asarray(T, dtype=np.float64))
    values = np.asarray(values, dtype=np.float64)
    S = values.shape[0]
    rows, n = T.shape
    s = np.full(rows, start_state, dtype=np.int64)
    codes = np.zeros((rows, n), dtype=np.int64)
    recon = np.zeros((rows, n))
    states = np.zeros((rows, n + 1), dtype=np.int64)
    states[:, 0] = s
    for k in range(n):
        allowed = values[s].reshape(rows, -1)          # rows x (2 C), index u * C + v
        d = (T[:, k, None] - allowed) ** 2
        j = np.argmin(d, axis=1)
        C = values.shape[2]
        u, v = j // C, j % C
        codes[:, k] = u | (v << 1)
        recon[:, k] = allowed[np.arange(rows), j]
        s = ((s << 1) | u) % S
        states[:, k + 1] = s
    return {"codes": codes, "recon": recon, "cost": np.sum((T - recon) ** 2, axis=1), "states": states}


def decode(codes, values, start_state=0):
    """Reconstruction from codes: follow the states from start_state."""
    codes = np.atleast_2d(np.asarray(codes, dtype=np.int64))
    values = np.asarray(values, dtype=np.float64)
    S = values.shape[0]
    rows, n = codes.shape
    s = np.full(rows, start_state, dtype=np.int64)
    recon = np.zeros((rows, n))
    for k in range(n):
        u, v = codes[:, k] & 1, codes[:, k] >> 1
        recon[:, k] = values[s, u, v]
        s = ((s << 1) | u) % S
    return recon
