"""Seeded synthetic inputs for the attention share, shared by tests, benchmark and
smoke check.

This module holds none of the method's arithmetic: only random draws, rounding
to bf16, packed-document lengths and the position_ids they imply.  Both the HIP
path and the CPU oracle receive exactly these arrays.

Workloads (all draws on the CPU with torch's generator, in float32, then rounded
to bf16 with round-to-nearest-even; draw order q, k, v, dO):

* ring example: ``torch.manual_seed(0)``; q, k, v = randn(3, 32, 16) float32,
  as in the four-device simulation of the Ring Attention glossary page.
* causal single device: [4096][8][128] bf16, position_ids 0..4095.
* Ulysses share: sequence-sharded [8 ranks][4096][32 heads][128] bf16.
* packed long context: q [131072][4][128], k, v [131072][1][128], 16 documents
  with lengths multinomial(131072, uniform) drawn with numpy seed 1.
* ring merge: [262144][2][128] bf16, one document.
"""

import numpy as np
import torch


def ring_example():
    """q, k, v of the Ring Attention page's simulation (float32 [32][16] each)."""
    torch.manual_seed(0)
    q, k, v = torch.randn(3, 32, 16)
    return q, k, v


def generator(seed):
    g = torch.Generator()
    g.manual_seed(int(seed))
    return g


def normal(shape, gen, dtype=torch.bfloat16):
    """N(0, 1) draw in float32 on the CPU, rounded to ``dtype``."""
    return torch.randn(tuple(shape), generator=gen, dtype=torch.float32).to(dtype)


def doc_lengths(total, n_docs, seed):
    """Packed document lengths: multinomial(total, uniform over n_docs), numpy seed."""
    rng = np.random.default_rng(int(seed))
    return rng.multinomial(int(total), [1.0 / n_docs] * n_docs).astype(np.int64)


def position_ids(lengths):
    """position_ids restarting at 0 for each packed document (int32)."""
    return np.concatenate([np.arange(int(L), dtype=np.int32) for L in lengths]) \
        if len(lengths) else np.zeros(0, dtype=np.int32)


def attention_case(S, Hq, Hkv, D, seed, lengths=None, dtype=torch.bfloat16, Sk=None):
    """q [S][Hq][D], k, v [Sk][Hkv][D], dO [S][Hq][D] and int32 position_ids."""
    g = generator(seed)
    Sk = S if Sk is None else Sk
    q = normal((S, Hq, D), g, dtype)
    k = normal((Sk, Hkv, D), g, dtype)
    v = normal((Sk, Hkv, D), g, dtype)
    do = normal((S, Hq, D), g, dtype)
    n = max(S, Sk)
    pos = position_ids([n] if lengths is None else lengths)
    return q, k, v, do, pos


# ---- the five named workloads -------------------------------------------------

CAUSAL_4K = dict(S=4096, Hq=8, Hkv=8, D=128, seed=2)
ULYSSES_SP8 = dict(P=8, S_local=4096, H=32, D=128, seed=3)
PACKED_128K = dict(S=131072, Hq=4, Hkv=1, D=128, seed=4, n_docs=16, doc_seed=1)
RING_256K = dict(S=262144, H=2, D=128, seed=5, n_blocks=16)


def causal_4k():
    c = CAUSAL_4K
    return attention_case(c["S"], c["Hq"], c["Hkv"], c["D"], c["seed"])


def ulysses_sp8(P=None, S_local=None, H=None, D=None, seed=None):
    """Sequence-sharded x_q, x_k, x_v, dO [P][S_local][H][D] bf16 and position_ids."""
    c = dict(ULYSSES_SP8)
    for key, val in (("P", P), ("S_local", S_local), ("H", H), ("D", D), ("seed", seed)):
        if val is not None:
            c[key] = val
    g = generator(c["seed"])
    shp = (c["P"], c["S_local"], c["H"], c["D"])
    xs = [normal(shp, g) for _ in range(4)]
    return xs[0], xs[1], xs[2], xs[3], position_ids([c["P"] * c["S_local"]])


def packed_128k():
    c = PACKED_128K
    lengths = doc_lengths(c["S"], c["n_docs"], c["doc_seed"])
    q, k, v, do, pos = attention_case(c["S"], c["Hq"], c["Hkv"], c["D"], c["seed"],
                                      lengths=lengths)
    return q, k, v, do, pos, lengths


def ring_256k(with_do=False):
    """q, k, v (and, drawn after them, dO) of the 256K single-document ring case."""
    c = RING_256K
    g = generator(c["seed"])
    shp = (c["S"], c["H"], c["D"])
    q, k, v = (normal(shp, g) for _ in range(3))
    if with_do:
        return q, k, v, normal(shp, g), position_ids([c["S"]])
    return q, k, v, position_ids([c["S"]])


# ---- the benchmark's layer: the packed 128K input as the Ulysses SP=8 layer holds it ----

BENCH_LAYER = dict(P=8, S=131072, Hq=32, Hkv=8, D=128, seed=4, n_docs=16, doc_seed=1)


def bench_layer(device):
    """Sequence-sharded x_q [8][16384][32][128], x_k, x_v [8][16384][8][128] and dO like
    x_q (bf16 N(0, 1), drawn on `device` with a torch generator seeded 4, in the order
    x_q, x_k, x_v, dO, float32 then rounded to bf16), the int32 position_ids of the 16
    packed documents (lengths multinomial over 131072 tokens, numpy seed 1) on `device`,
    and the lengths.  Rank g's share (heads [4g, 4g + 4) of x_q, head g of x_k, x_v) is
    the packed long-context workload."""
    c = BENCH_LAYER
    lengths = doc_lengths(c["S"], c["n_docs"], c["doc_seed"])
    g = torch.Generator(device=device)
    g.manual_seed(c["seed"])
    P, S_l = c["P"], c["S"] // c["P"]

    def draw(H):
        return torch.randn((P, S_l, H, c["D"]), generator=g, device=device,
                           dtype=torch.float32).to(torch.bfloat16)

    xq, xk, xv = draw(c["Hq"]), draw(c["Hkv"]), draw(c["Hkv"])
    xdo = draw(c["Hq"])
    pos = torch.from_numpy(position_ids(lengths)).to(device)
    return xq, xk, xv, xdo, pos, lengths


def share_of(x, P, group):
    """Rank `group`'s head slice of a sequence-sharded [P][S_l][H][D] tensor, in global
    token order: [P S_l][H/P][D] (plain tensor slicing, no arithmetic)."""
    Pp, S_l, H, D = x.shape
    hp = H // P
    return x[:, :, group * hp:(group + 1) * hp].reshape(Pp * S_l, hp, D)
