"""Oracle: the Ulysses re-layout between sequence shards and head shards.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition (Keryc Ulysses SP article, "Como funciona", steps 1 and 3; aitoolresearcher
review, section 3, steps 1 and 3; DeepSpeed-Ulysses notes, "Method", all-to-all table):
P ranks; rank s holds the contiguous token range [s*S_l, (s+1)*S_l) for all H heads,
as an array X[s][t][h][d].  After the all-to-all, rank g holds every token for the
head subset [g*H/P, (g+1)*H/P):

    Y[g][s*S_l + t][h'][d] = X[s][t][g*H/P + h'][d]

The inverse (the second all-to-all, step 5) maps Y back to X.  Both are bitwise
copies: they work on any numpy dtype, including raw bf16 bit patterns (uint16).
"""

import numpy as np


def seq_to_head(x, group=None):
    """X [P][S_l][H][D] -> Y [P][P*S_l][H/P][D], or Y[group] if group is given."""
    P, S_l, H, D = x.shape
    if H % P:
        raise ValueError("head count must be divisible by the number of ranks")
    Hp = H // P
    y = np.empty((P, P * S_l, Hp, D), dtype=x.dtype)
    for g in range(P):
        for s in range(P):
            y[g, s * S_l:(s + 1) * S_l] = x[s, :, g * Hp:(g + 1) * Hp]
    return y if group is None else y[group].copy()


def head_to_seq(y, P=None, out=None, group=None):
    """Inverse re-layout.

    group None: y is [P][P*S_l][H/P][D] -> X [P][S_l][H][D].
    group g:    y is rank g's share [P*S_l][H/P][D]; only heads
                [g*H/P, (g+1)*H/P) of ``out`` (shape [P][S_l][H][D]) are written.
    """
    if group is None:
        P, S, Hp, D = y.shape
        S_l = S // P
        x = np.empty((P, S_l, P * Hp, D), dtype=y.dtype)
        for g in range(P):
            for s in range(P):
                x[s, :, g * Hp:(g + 1) * Hp] = y[g, s * S_l:(s + 1) * S_l]
        return x
    if out is None:
        raise ValueError("group form writes into an existing sequence-sharded array")
    P = out.shape[0]
    S, Hp, D = y.shape
    S_l = S // P
    for s in range(P):
        out[s, :, group * Hp:(group + 1) * Hp] = y[s * S_l:(s + 1) * S_l]
    return out


def seq_to_head_elementwise(x):
    """The same map as ``seq_to_head`` written one element at a time.

    Only for tiny arrays: it is the brute-force restatement used to pin the
    block-copy form above (global token = s*S_l + t, global head = g*H/P + h').
    """
    P, S_l, H, D = x.shape
    Hp = H // P
    y = np.empty((P, P * S_l, Hp, D), dtype=x.dtype)
    for s in range(P):
        for t in range(S_l):
            for h in range(H):
                for d in range(D):
                    g, hp = divmod(h, Hp)
                    y[g, s * S_l + t, hp, d] = x[s, t, h, d]
    return y
