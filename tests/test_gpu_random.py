"""GPU parity over seeded random calls through the C ABI, on shapes nobody picked by
hand: blockattn forward and backward against the fp64 oracle; the re-layouts
bit-exact against the oracle's index map (odd rank counts and head dims, both
dtypes, one rank's share); lse_merge against the oracle's merge (every dtype pair,
empty partials); the fused Ulysses entry points bit-identical to the explicit
re-layout chain.

Each case draws a sequence length, query / key-value head counts (GQA ratios 1, 2,
4, 8), a packed-document mix (multinomial lengths, one-token documents allowed),
causal or not, and for causal calls a ring-style query block and key block at
global offsets (rows with no visible key included).  Bars as in
test_gpu_parity.py: O within 2e-2 abs + 1e-2 rel, LSE within 1e-3, gradients within
5e-2 of the reference's max-norm.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from sequence_parallelism_amd import inputs

pytestmark = pytest.mark.gpu

O_ATOL, O_RTOL, LSE_ATOL, GRAD_REL = 2e-2, 1e-2, 1e-3, 5e-2
DEV = "cuda:0"
# case counts (environment overrides for longer sweeps; the defaults run in about a minute)
N_CASES = int(os.environ.get("USP_RANDOM_CASES", "48"))        # small calls (S <= 1600)
N_SPLIT = int(os.environ.get("USP_RANDOM_SPLIT_CASES", "16"))  # S in [2048, 4096], 1-4 query
                                                               # heads: split key / query ranges


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def draw_case(i, split=False):
    """Case i of the sweep (independent of the others' draws)."""
    rng = np.random.default_rng(2026 + 7919 * i + (104729 if split else 0))
    S = int(rng.integers(2048, 4097)) if split else int(rng.integers(1, 1601))
    hq = int(rng.choice([1, 2, 4] if split else [1, 2, 4, 8]))
    hkv = int(rng.choice([d for d in (1, 2, 4, 8) if d <= hq and hq % d == 0]))
    causal = bool(rng.random() < 0.8)
    lengths = None
    if causal and S > 1:
        n_docs = int(rng.integers(1, min(6, S) + 1))
        share = rng.dirichlet(np.full(n_docs, 0.4))                          # skewed mix
        lengths = rng.multinomial(S - n_docs, share) + 1                      # every doc >= 1
        lengths = [int(x) for x in lengths]
    qa, qb, ka, kb = 0, S, 0, S
    if causal and rng.random() < 0.5:   # ring-style block pair at global offsets
        qa, qb = sorted(int(x) for x in rng.integers(0, S + 1, size=2))
        ka, kb = sorted(int(x) for x in rng.integers(0, S + 1, size=2))
        if qb == qa:   # at least one query row (the key block may be empty)
            if qa < S:
                qb = qa + 1
            else:
                qa = qb - 1
    return dict(S=S, hq=hq, hkv=hkv, causal=causal, lengths=lengths, qa=qa, qb=qb, ka=ka, kb=kb,
                seed=int(rng.integers(1 << 30)))


@pytest.mark.parametrize("i,split", [(i, False) for i in range(N_CASES)] +
                         [(i, True) for i in range(N_SPLIT)])
def test_random_call_fwd_bwd(usp, i, split):
    c = draw_case(i, split)
    print("random case", i, "split" if split else "small", c, flush=True)
    S, hq, hkv, causal = c["S"], c["hq"], c["hkv"], c["causal"]
    qa, qb, ka, kb = c["qa"], c["qb"], c["ka"], c["kb"]
    if qb <= qa:
        pytest.skip("empty query block")
    q, k, v, do, pos = inputs.attention_case(S, hq, hkv, 128, seed=c["seed"], lengths=c["lengths"])
    qs, ks, vs, dos = q[qa:qb], k[ka:kb], v[ka:kb], do[qa:qb]
    qd, kd, vd, dod = (t.to(DEV).contiguous() for t in (qs, ks, vs, dos))
    posd = torch.from_numpy(pos).to(DEV) if causal else None
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd, q_start=qa, k_start=ka, causal=causal)
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd, q_start=qa, k_start=ka, causal=causal)
    torch.cuda.synchronize()

    kw = dict(pos=pos, q_start=qa, k_start=ka, causal=True) if causal else dict(causal=False)
    args = (f64(qs), f64(ks), f64(vs))
    ref_o, ref_l = oracle.attention_fwd(*args, **kw)
    og = f64(o)
    err = np.abs(og - ref_o)
    assert np.all(err <= O_ATOL + O_RTOL * np.abs(ref_o)), ("o", float(err.max()))
    lg = lse.detach().cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lg), fin), "lse finiteness"
    assert np.all(lg[~fin] == ref_l[~fin])
    if fin.any():
        assert np.abs(lg[fin] - ref_l[fin]).max() <= LSE_ATOL, ("lse", float(np.abs(lg[fin] - ref_l[fin]).max()))
    assert np.all(og[np.repeat(~fin.T[:, :, None], og.shape[2], axis=2)] == 0), "rows with no key: O = 0"

    grads = oracle.attention_bwd(*args, f64(dos), **kw)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), grads):
        den = max(np.abs(r).max(), 1e-3)
        rel = np.abs(f64(g) - r).max() / den
        assert rel <= GRAD_REL, (name, float(rel))


# ---- re-layouts: bit-exact against the oracle's index map -------------------------------

N_PERM = int(os.environ.get("USP_RANDOM_PERMUTE_CASES", "24"))


def draw_permute(i):
    rng = np.random.default_rng(91 + 6151 * i)
    P = int(rng.choice([1, 2, 3, 4, 5, 8]))
    S_l = int(rng.integers(0, 300))
    H = P * int(rng.integers(1, 5))
    D = int(rng.choice([1, 3, 8, 16, 64, 128, 130]))
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    group = int(rng.integers(-1, P))
    return P, S_l, H, D, dtype, group, int(rng.integers(1 << 30))


@pytest.mark.parametrize("i", range(N_PERM))
def test_random_permute_bitexact(usp, i):
    P, S_l, H, D, dtype, group, seed = draw_permute(i)
    print("random permute", i, P, S_l, H, D, dtype, group, flush=True)
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    x = inputs.normal((P, S_l, H, D), inputs.generator(seed), dtype)
    xb = x.view(bits).numpy()
    ref = oracle.seq_to_head(xb, group=None if group < 0 else group)
    xd = x.to(DEV)
    y = usp.seq_to_head(xd, P, group=group)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().view(bits).numpy(), ref)
    if group < 0:
        back = usp.head_to_seq(y, P, H)
        torch.cuda.synchronize()
        assert torch.equal(back.cpu().view(bits), x.view(bits))
    else:   # one rank's share writes only its head slice of an existing array
        fill = inputs.normal((P, S_l, H, D), inputs.generator(seed + 1), dtype)
        out = fill.to(DEV)
        usp.head_to_seq(y, P, H, out=out, group=group)
        torch.cuda.synchronize()
        ref_out = oracle.head_to_seq(ref, out=fill.view(bits).numpy().copy(), group=group)
        assert np.array_equal(out.cpu().view(bits).numpy(), ref_out)


# ---- lse_merge: against the oracle's cumulative-softmax merge ---------------------------

N_MERGE = int(os.environ.get("USP_RANDOM_MERGE_CASES", "12"))


@pytest.mark.parametrize("i", range(N_MERGE))
def test_random_lse_merge(usp, i):
    rng = np.random.default_rng(313 + 2357 * i)
    S, H = int(rng.integers(1, 700)), int(rng.integers(1, 9))
    D = int(rng.choice([1, 5, 64, 127, 128, 256]))
    adt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    pdt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    print("random merge", i, S, H, D, adt, pdt, flush=True)
    g = inputs.generator(int(rng.integers(1 << 30)))
    oa, ob = inputs.normal((S, H, D), g, adt), inputs.normal((S, H, D), g, pdt)
    la, lb = inputs.normal((H, S), g, torch.float32) * 6, inputs.normal((H, S), g, torch.float32) * 6
    # empty partials (0, -inf) on either side, and on both at once
    ea, eb = rng.random((H, S)) < 0.1, rng.random((H, S)) < 0.1
    la[torch.from_numpy(ea)] = -float("inf")
    lb[torch.from_numpy(eb)] = -float("inf")
    oa[torch.from_numpy(ea.T)] = 0
    ob[torch.from_numpy(eb.T)] = 0
    ref_o, ref_l = oracle.lse_merge(f64(oa), f64(la), f64(ob), f64(lb))
    oad, obd, lad, lbd = (t.to(DEV) for t in (oa, ob, la, lb))
    usp.lse_merge(oad, lad, obd, lbd)
    torch.cuda.synchronize()
    rel = 1e-6 if adt == torch.float32 else 2.0 ** -8   # one rounding to the accumulator's type
    assert np.all(np.abs(f64(oad) - ref_o) <= 1e-5 + rel * np.abs(ref_o))
    lg = lad.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lg), fin) and np.all(lg[~fin] == ref_l[~fin])
    if fin.any():
        assert np.abs(lg[fin] - ref_l[fin]).max() <= LSE_ATOL


# ---- fused Ulysses entry points: bit-identical to the explicit re-layout chain ----------

N_FUSED = int(os.environ.get("USP_RANDOM_FUSED_CASES", "10"))


@pytest.mark.parametrize("i", range(N_FUSED))
def test_random_fused_ulysses_matches_unfused(usp, i):
    from test_gpu_ulysses_fused import fused, unfused
    rng = np.random.default_rng(577 + 4099 * i)
    P = int(rng.choice([1, 2, 4, 8]))
    S_l = 256 * int(rng.integers(1, 3))   # the fused calls take whole 256-row shards
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    causal = bool(rng.random() < 0.8)
    S = P * S_l
    lengths = None
    if causal:
        n_docs = int(rng.integers(1, min(5, S) + 1))
        lengths = [int(x) for x in rng.multinomial(S - n_docs, rng.dirichlet(np.full(n_docs, 0.5))) + 1]
    g_rank = int(rng.integers(0, P))
    print("random fused", i, P, S_l, P * hq, P * hkv, causal, lengths, g_rank, flush=True)
    gen = inputs.generator(int(rng.integers(1 << 30)))
    xq = inputs.normal((P, S_l, P * hq, 128), gen)
    xk = inputs.normal((P, S_l, P * hkv, 128), gen)
    xv = inputs.normal((P, S_l, P * hkv, 128), gen)
    xdo = inputs.normal((P, S_l, P * hq, 128), gen)
    xqd, xkd, xvd, xdod = (t.to(DEV) for t in (xq, xk, xv, xdo))
    posd = torch.from_numpy(inputs.position_ids(lengths)).to(DEV) if causal else None
    outs_f, lse_f = fused(usp, xqd, xkd, xvd, xdod, posd, P, g_rank, causal)
    outs_u, lse_u = unfused(usp, xqd, xkd, xvd, xdod, posd, P, g_rank, causal)
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "dq", "dk", "dv"), outs_f, outs_u):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
    assert torch.equal(lse_f, lse_u)
