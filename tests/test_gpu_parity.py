"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle on the
same seeded inputs.

Bars: permutes bit-exact; fp32 attention within 1e-5 absolute; bf16 attention
O within 2e-2 abs + 1e-2 rel (elementwise), LSE within 1e-3 abs, gradients within
5e-2 of the reference's max-norm; plus a diagnostic on O's max-normalised error.
"""

import numpy as np
import pytest
import torch

import oracle
from sequence_parallelism_amd import inputs

pytestmark = pytest.mark.gpu

O_ATOL, O_RTOL, LSE_ATOL, GRAD_REL, O_NORM_REL = 2e-2, 1e-2, 1e-3, 5e-2, 1e-2
DEV = "cuda:0"


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def say(*a):
    print(*a, flush=True)


def check_o(o_gpu, o_ref, what):
    o = f64(o_gpu)
    err = np.abs(o - o_ref)
    assert np.all(err <= O_ATOL + O_RTOL * np.abs(o_ref)), (what, float(err.max()))
    scale = max(np.abs(o_ref).max(), 1e-30)
    assert err.max() / scale <= O_NORM_REL, (what, "normalised", float(err.max() / scale))


def check_lse(lse_gpu, lse_ref, what):
    l = lse_gpu.detach().cpu().numpy().astype(np.float64)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(l), fin), what
    assert np.all(l[~fin] == lse_ref[~fin]), what
    if fin.any():
        assert np.abs(l[fin] - lse_ref[fin]).max() <= LSE_ATOL, (what, np.abs(l[fin] - lse_ref[fin]).max())


def check_grad(g_gpu, g_ref, what):
    """max |g - ref| <= 5e-2 * max |ref|.  Where the exact gradient is identically
    zero (one-token documents: dS = P (dP - D) = 0), the max-norm is floored at
    1e-3 so that rounding noise of order 1e-7 is not divided by zero."""
    g = f64(g_gpu) if isinstance(g_gpu, torch.Tensor) else g_gpu
    den = max(np.abs(g_ref).max(), 1e-3)
    rel = np.abs(g - g_ref).max() / den
    assert rel <= GRAD_REL, (what, float(rel))


def to_dev(*ts):
    return [t.to(DEV).contiguous() for t in ts]


# ---- permutes -------------------------------------------------------------------------

@pytest.mark.parametrize("P,S_l,H,D,dtype", [
    (8, 37, 32, 128, torch.bfloat16),    # ragged token count
    (4, 5, 8, 3, torch.bfloat16),        # 12-byte runs -> narrow vectors
    (2, 9, 6, 16, torch.float32),
    (1, 7, 4, 128, torch.bfloat16),
    (8, 64, 8, 128, torch.float32),      # one head per rank
])
def test_permute_bitexact_small(usp, P, S_l, H, D, dtype):
    say("permute", P, S_l, H, D, dtype)
    g = inputs.generator(100 + P + S_l)
    x = inputs.normal((P, S_l, H, D), g, dtype)
    xb = x.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy()
    ref = oracle.seq_to_head(xb)
    (xd,) = to_dev(x)
    y = usp.seq_to_head(xd, P)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy(), ref)
    back = usp.head_to_seq(y, P, H)
    torch.cuda.synchronize()
    assert torch.equal(back.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       x.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))
    # per-rank shares and the group inverse
    out = torch.zeros_like(xd)
    for grp in range(P):
        yg = usp.seq_to_head(xd, P, group=grp)
        torch.cuda.synchronize()
        assert np.array_equal(yg.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy(), ref[grp])
        usp.head_to_seq(yg, P, H, out=out, group=grp)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), x)


def test_permute_bitexact_ulysses_sp8_full(usp):
    """Full-size Ulysses share: [8][4096][32][128] bf16, all ranks and rank 0."""
    say("permute ulysses sp8 full")
    xq, xk, xv, xdo, _ = inputs.ulysses_sp8()
    for x in (xq, xk):
        xb = x.view(torch.int16).numpy()
        ref = oracle.seq_to_head(xb)
        (xd,) = to_dev(x)
        y = usp.seq_to_head(xd, 8)
        y0 = usp.seq_to_head(xd, 8, group=0)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().view(torch.int16).numpy(), ref)
        assert np.array_equal(y0.cpu().view(torch.int16).numpy(), ref[0])
        back = usp.head_to_seq(y, 8, 32)
        torch.cuda.synchronize()
        assert torch.equal(back.cpu(), x)
        del xd, y, y0, back
        torch.cuda.empty_cache()


def test_permute_empty(usp):
    x = torch.empty((4, 0, 8, 128), dtype=torch.bfloat16, device=DEV)
    y = usp.seq_to_head(x, 4)
    torch.cuda.synchronize()
    assert y.shape == (4, 0, 2, 128)


# ---- forward ------------------------------------------------------------------------------

def test_fwd_fp32_ring_example(usp):
    """The Ring Attention page's four-device example: one call, and block by block
    (query block i against key blocks in ring order, merged with lse_merge)."""
    say("fwd fp32 ring example")
    q, k, v = inputs.ring_example()
    ref_o, ref_l = oracle.attention_fwd(q.numpy()[:, None], k.numpy()[:, None], v.numpy()[:, None])
    qd, kd, vd = to_dev(q[:, None], k[:, None], v[:, None])
    o, lse = usp.blockattn_fwd(qd, kd, vd, causal=False)
    torch.cuda.synchronize()
    assert np.abs(f64(o) - ref_o).max() <= 1e-5
    assert np.abs(f64(lse) - ref_l).max() <= 1e-5
    n, blk = 4, 8
    out = torch.empty_like(qd)
    for i in range(n):
        acc = torch.zeros((blk, 1, 16), dtype=torch.float32, device=DEV)
        acc_l = torch.full((1, blk), -float("inf"), dtype=torch.float32, device=DEV)
        for step in range(n):
            j = (i - step) % n
            po, pl = usp.blockattn_fwd(qd[i * blk:(i + 1) * blk], kd[j * blk:(j + 1) * blk],
                                       vd[j * blk:(j + 1) * blk], causal=False)
            usp.lse_merge(acc, acc_l, po, pl)
        out[i * blk:(i + 1) * blk] = acc
    torch.cuda.synchronize()
    assert np.abs(f64(out) - ref_o).max() <= 1e-5


@pytest.mark.parametrize("S,Hq,Hkv,lengths,causal", [
    (300, 4, 2, None, True),                  # ragged tail, GQA 2:1
    (257, 2, 2, None, False),                 # non-causal, ragged
    (640, 4, 1, [100, 1, 250, 7, 282], True),  # packed docs incl. a 1-token doc
    (128, 1, 1, None, True),                  # exactly one tile
    (1, 2, 1, None, True),                    # one token
    (1000, 8, 8, [512, 488], True),
])
def test_fwd_bf16_small(usp, S, Hq, Hkv, lengths, causal):
    say("fwd bf16", S, Hq, Hkv, lengths, causal)
    q, k, v, _, pos = inputs.attention_case(S, Hq, Hkv, 128, seed=S + Hq, lengths=lengths)
    ref_o, ref_l = oracle.attention_fwd(f64(q), f64(k), f64(v), pos=pos, causal=causal)
    qd, kd, vd = to_dev(q, k, v)
    posd = torch.from_numpy(pos).to(DEV)
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd, causal=causal)
    o32, lse32 = usp.blockattn_fwd(qd, kd, vd, posd, causal=causal, o_dtype=torch.float32)
    torch.cuda.synchronize()
    check_o(o, ref_o, "o bf16")
    check_lse(lse, ref_l, "lse")
    check_o(o32, ref_o, "o f32")
    assert torch.equal(lse, lse32)


def test_fwd_offsets_and_empty_rows(usp):
    """Ring-style call: query block and key block at global offsets; the block
    above the diagonal has rows with no visible key (O = 0, LSE = -inf)."""
    say("fwd offsets")
    S = 1024
    q, k, v, _, pos = inputs.attention_case(S, 2, 1, 128, seed=7)
    qd, kd, vd = to_dev(q, k, v)
    posd = torch.from_numpy(pos).to(DEV)
    for qa, qb, ka, kb in ((512, 1024, 0, 512), (256, 512, 256, 768), (0, 256, 512, 1024),
                           (300, 700, 200, 650)):
        ref_o, ref_l = oracle.attention_fwd(f64(q[qa:qb]), f64(k[ka:kb]), f64(v[ka:kb]), pos=pos,
                                            q_start=qa, k_start=ka, causal=True)
        o, lse = usp.blockattn_fwd(qd[qa:qb], kd[ka:kb], vd[ka:kb], posd, q_start=qa, k_start=ka,
                                   causal=True, o_dtype=torch.float32)
        torch.cuda.synchronize()
        check_lse(lse, ref_l, ("lse", qa, ka))
        assert np.abs(f64(o) - ref_o).max() <= O_ATOL
    o, lse = usp.blockattn_fwd(qd[:64], kd[:0], vd[:0], posd, causal=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(lse == -float("inf"))


def test_fwd_large_logits(usp):
    """Scores of magnitude ~100s: the running max keeps everything finite."""
    say("fwd large logits")
    q, k, v, _, pos = inputs.attention_case(384, 2, 2, 128, seed=9, lengths=[200, 184])
    q = (q.float() * 30).to(torch.bfloat16)
    ref_o, ref_l = oracle.attention_fwd(f64(q), f64(k), f64(v), pos=pos, causal=True)
    assert np.abs(ref_l).max() > 50
    qd, kd, vd = to_dev(q, k, v)
    o, lse = usp.blockattn_fwd(qd, kd, vd, torch.from_numpy(pos).to(DEV))
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    check_o(o, ref_o, "o")
    say("  max |lse - ref|", float(np.abs(lse.cpu().numpy().astype(np.float64) - ref_l).max()),
        "at max |lse|", float(np.abs(ref_l).max()))
    check_lse(lse, ref_l, "lse")


def test_bwd_large_logits(usp):
    """Gradients with scores of magnitude ~100s (q scaled by 30, as in the forward's
    large-logit test): P is sharply peaked, so an error in a score's exponent shows
    directly in P, dS and the gradients."""
    say("bwd large logits")
    q, k, v, do, pos = inputs.attention_case(384, 2, 2, 128, seed=9, lengths=[200, 184])
    q = (q.float() * 30).to(torch.bfloat16)
    args = (f64(q), f64(k), f64(v))
    qd, kd, vd, dod = to_dev(q, k, v, do)
    posd = torch.from_numpy(pos).to(DEV)
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd)
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(*args, f64(do), pos=pos, causal=True)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        say("  ", name, "max |err| / max |ref|",
            float(np.abs(f64(got) - ref).max() / max(np.abs(ref).max(), 1e-3)))
        check_grad(got.cpu(), ref, name)


def test_large_logits_long_gqa(usp):
    """Large logits (q scaled by 30) on the 8-wave kernels: 32768 rows in two documents,
    4 query heads on 1 key/value head; every output against the oracle.  (The gradient
    tolerance is relative to the max norm of the whole tensor: keys seen by few rows,
    under attention this peaked, carry the bf16 rounding of the O the backward receives,
    which enters D = <dO, O>, at a larger share of their own small gradients.)"""
    say("large logits, 32k gqa")
    S = 32768
    q, k, v, do, pos = inputs.attention_case(S, 4, 1, 128, seed=11, lengths=[20000, 12768])
    q = (q.float() * 30).to(torch.bfloat16)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    posd = torch.from_numpy(pos).to(DEV)
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd)
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd)
    torch.cuda.synchronize()
    args = (f64(q), f64(k), f64(v))
    ref_o, ref_l = oracle.attention_fwd(*args, pos=pos, causal=True)
    check_o(o.cpu(), ref_o, "o")
    check_lse(lse.cpu(), ref_l, "lse")
    rq, rk, rv = oracle.attention_bwd(*args, f64(do), pos=pos, causal=True)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        say("  ", name, "max |err| / max |ref|",
            float(np.abs(f64(got) - ref).max() / max(np.abs(ref).max(), 1e-3)))
        check_grad(got.cpu(), ref, name)


def test_fwd_causal_4k_full(usp):
    """Single-device causal attention, [4096][8][128] bf16, every output."""
    say("fwd causal 4k")
    q, k, v, do, pos = inputs.causal_4k()
    ref_o, ref_l = oracle.attention_fwd(f64(q), f64(k), f64(v), pos=pos, causal=True)
    qd, kd, vd = to_dev(q, k, v)
    o, lse = usp.blockattn_fwd(qd, kd, vd, torch.from_numpy(pos).to(DEV))
    torch.cuda.synchronize()
    check_o(o, ref_o, "o")
    check_lse(lse, ref_l, "lse")


def test_fwd_future_keys_do_not_change_earlier_rows(usp):
    say("fwd future perturbation")
    q, k, v, _, pos = inputs.attention_case(512, 2, 1, 128, seed=11)
    qd, kd, vd = to_dev(q, k, v)
    posd = torch.from_numpy(pos).to(DEV)
    o1, l1 = usp.blockattn_fwd(qd, kd, vd, posd)
    k2, v2 = kd.clone(), vd.clone()
    k2[300:] = 3.0
    v2[300:] = -2.0
    o2, l2 = usp.blockattn_fwd(qd, k2, v2, posd)
    torch.cuda.synchronize()
    assert torch.equal(o1[:300], o2[:300]) and torch.equal(l1[:, :300], l2[:, :300])


# ---- backward -------------------------------------------------------------------------------

@pytest.mark.parametrize("S,Hq,Hkv,lengths,causal", [
    (300, 4, 2, None, True),
    (257, 2, 2, None, False),
    (640, 4, 1, [100, 1, 250, 7, 282], True),
    (1, 2, 1, None, True),
    (1000, 2, 2, [512, 488], True),
])
def test_bwd_bf16_small(usp, S, Hq, Hkv, lengths, causal):
    say("bwd bf16", S, Hq, Hkv, lengths, causal)
    q, k, v, do, pos = inputs.attention_case(S, Hq, Hkv, 128, seed=3 * S + Hq, lengths=lengths)
    rq, rk, rv = oracle.attention_bwd(f64(q), f64(k), f64(v), f64(do), pos=pos, causal=causal)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    posd = torch.from_numpy(pos).to(DEV)
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd, causal=causal)
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd, causal=causal)
    torch.cuda.synchronize()
    check_grad(dq, rq, "dq")
    check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")


def test_bwd_empty_and_invisible(usp):
    """Calls whose gradients are all zero, written over NaN-filled outputs: no query rows
    (every key block still writes dK = dV = 0), no keys (dQ = 0), and a ring pair whose
    keys all lie after its queries (nothing visible)."""
    say("bwd empty / invisible")
    S = 1024
    q, k, v, do, pos = inputs.attention_case(S, 4, 2, 128, seed=9)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    posd = torch.from_numpy(pos).to(DEV)
    nan = lambda t: torch.full_like(t, float("nan"))
    cases = (((0, 0), (0, 300)), ((0, 64), (0, 0)), ((0, 256), (512, 1024)))
    for (qa, qb), (ka, kb) in cases:
        qs, ks, vs, ds = qd[qa:qb], kd[ka:kb], vd[ka:kb], dod[qa:qb]
        o, lse = usp.blockattn_fwd(qs, ks, vs, posd, q_start=qa, k_start=ka, causal=True)
        dq, dk, dv = usp.blockattn_bwd(qs, ks, vs, o, lse, ds, posd, q_start=qa, k_start=ka, causal=True,
                                       dq=nan(qs), dk=nan(ks), dv=nan(vs))
        torch.cuda.synchronize()
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert torch.all(t == 0), (name, qa, qb, ka, kb)


def test_fwd_bwd_causal_4k_full(usp):
    say("bwd causal 4k")
    q, k, v, do, pos = inputs.causal_4k()
    rq, rk, rv = oracle.attention_bwd(f64(q), f64(k), f64(v), f64(do), pos=pos, causal=True)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    posd = torch.from_numpy(pos).to(DEV)
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd)
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd)
    torch.cuda.synchronize()
    check_grad(dq, rq, "dq")
    check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")


# ---- merge ------------------------------------------------------------------------------------

@pytest.mark.parametrize("adt,pdt,D", [(torch.float32, torch.float32, 128),
                                       (torch.float32, torch.bfloat16, 128),
                                       (torch.bfloat16, torch.float32, 64),
                                       (torch.bfloat16, torch.bfloat16, 128),
                                       (torch.float32, torch.float32, 7)])
def test_lse_merge_random(usp, adt, pdt, D):
    say("merge", adt, pdt, D)
    S, H = 333, 3
    g = inputs.generator(21)
    oa = inputs.normal((S, H, D), g, adt)
    ob = inputs.normal((S, H, D), g, pdt)
    la = inputs.normal((H, S), g, torch.float32) * 4
    lb = inputs.normal((H, S), g, torch.float32) * 4
    la[0, :10] = -float("inf")
    lb[0, 5:15] = -float("inf")
    oa[:10, 0] = 0
    ob[5:15, 0] = 0
    ref_o, ref_l = oracle.lse_merge(f64(oa), f64(la), f64(ob), f64(lb))
    oad, obd, lad, lbd = to_dev(oa, ob, la, lb)
    usp.lse_merge(oad, lad, obd, lbd)
    torch.cuda.synchronize()
    # fp32 accumulator: fp32 rounding; bf16 accumulator: one bf16 rounding (u = 2^-8)
    rel = 1e-6 if adt == torch.float32 else 2.0 ** -8
    assert np.all(np.abs(f64(oad) - ref_o) <= 1e-5 + rel * np.abs(ref_o))
    check_lse(lad, ref_l, "merge lse")


# ---- split key / query ranges (calls too small to fill the GPU with whole tiles) ---------

@pytest.mark.parametrize("S,Hq,Hkv,lengths,causal", [
    (3000, 4, 2, None, True),                     # ragged tail, GQA 2:1: 16 chunks per tile
    (2500, 2, 1, None, False),                    # non-causal
    (4200, 2, 2, [1500, 1, 2000, 699], True),     # packed docs incl. a 1-token doc
    (2048, 1, 1, [2048], True),                   # the smallest split call
])
def test_split_paths_fwd_bwd(usp, S, Hq, Hkv, lengths, causal):
    """Sizes whose 256-row tiles leave CUs idle: the forward and dQ kernels split key
    ranges, the dK/dV kernel splits query-tile ranges, and combine passes merge the
    partials; checked against the oracle over the whole sequence."""
    say("split paths", S, Hq, Hkv, causal)
    q, k, v, do, pos = inputs.attention_case(S, Hq, Hkv, 128, seed=41, lengths=lengths)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    posd = torch.from_numpy(pos).to(DEV) if causal else None
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd, causal=causal)
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd, causal=causal)
    torch.cuda.synchronize()
    kw = dict(pos=pos, causal=True) if causal else dict(causal=False)
    args = (f64(q), f64(k), f64(v))
    ref_o, ref_l = oracle.attention_fwd(*args, **kw)
    check_o(o.cpu(), ref_o, "o")
    check_lse(lse.cpu(), ref_l, "lse")
    rq, rk, rv = oracle.attention_bwd(*args, f64(do), **kw)
    check_grad(dq.cpu(), rq, "dq")
    check_grad(dk.cpu(), rk, "dk")
    check_grad(dv.cpu(), rv, "dv")
    # fp32 partial output (the ring's o_dtype) through the same split path
    o32, lse32 = usp.blockattn_fwd(qd, kd, vd, posd, causal=causal, o_dtype=torch.float32)
    torch.cuda.synchronize()
    check_o(o32.cpu(), ref_o, "o fp32")
    assert torch.equal(lse32, lse)
