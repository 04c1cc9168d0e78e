"""GPU parity of the striped layout (Ultralytics glossary "Ring Attention", section
"Como funciona la atencion en anillo", the Striped Attention remark; rank r of P
holds tokens r, r + P, ...): the stripe permutes bit-exact against the oracle, every
stripe pair's attention against the oracle's strided attention, and the ring over
stripes -- forward pairs merged by lse_merge, backward pairs with the merged O and
LSE, partial gradients summed -- against the oracle's attention of the original
sequence.  The partial-gradient sums are fp32 torch additions in the tests
(plumbing around the library calls)."""

import numpy as np
import pytest
import torch

import oracle
from sequence_parallelism_amd import inputs
from test_gpu_parity import DEV, check_grad, check_lse, check_o, f64, say, to_dev
from test_gpu_workloads import sample_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("P,S,H,D,dtype", [
    (4, 148, 3, 5, torch.float32),      # 60-byte rows: 4-byte vectors
    (4, 148, 3, 5, torch.bfloat16),     # 30-byte rows: 2-byte vectors
    (8, 4096, 2, 128, torch.bfloat16),  # 512-byte rows: 16-byte vectors
    (16, 65536, 2, 128, torch.bfloat16),
])
def test_stripe_permute_bitexact(usp, P, S, H, D, dtype):
    say("stripe permute", P, S, H, D, dtype)
    x = inputs.normal((S, H, D), inputs.generator(21), dtype)
    xd = x.to(DEV)
    y = usp.seq_to_stripe(xd, P)
    back = usp.stripe_to_seq(y)
    torch.cuda.synchronize()
    as_int = lambda t: t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    want = oracle.seq_to_stripe(as_int(x), P)
    assert np.array_equal(as_int(y), want)
    assert np.array_equal(as_int(back), as_int(x))


def test_stripe_permute_empty(usp):
    x = torch.empty((0, 2, 128), dtype=torch.bfloat16, device=DEV)
    assert usp.seq_to_stripe(x, 4).shape == (4, 0, 2, 128)


def _stripes(usp, P, *ts):
    return [usp.seq_to_stripe(t, P) for t in ts]


def striped_ring(usp, qd, kd, vd, dod, posd, P, q_ranks=None, backward=True):
    """Ring over P stripes: forward pairs (i, j) merged per query stripe i in ring order,
    then backward pairs with the merged O and LSE.  Returns, in stripe layout, O (bf16),
    LSE [P][H][n], and fp32 dQ, dK, dV (None without backward)."""
    qs, ks, vs, dos = _stripes(usp, P, qd, kd, vd, dod)
    n, H, D = qs.shape[1:]
    Hkv = ks.shape[2]
    q_ranks = range(P) if q_ranks is None else q_ranks
    acc = torch.zeros((P, n, H, D), dtype=torch.float32, device=DEV)
    acc_l = torch.full((P, H, n), -float("inf"), dtype=torch.float32, device=DEV)
    po = torch.empty((n, H, D), dtype=torch.float32, device=DEV)
    pl = torch.empty((H, n), dtype=torch.float32, device=DEV)
    for i in q_ranks:
        for step in range(P):
            j = (i - step) % P
            usp.striped_attn_fwd(qs[i], ks[j], vs[j], P, i, j, posd, o=po, lse=pl)
            usp.lse_merge(acc[i], acc_l[i], po, pl)
    o = acc.to(torch.bfloat16)
    if not backward:
        torch.cuda.synchronize()
        return o, acc_l, None, None, None
    dq = torch.zeros((P, n, H, D), dtype=torch.float32, device=DEV)
    dk = torch.zeros((P, n, Hkv, D), dtype=torch.float32, device=DEV)
    dv = torch.zeros_like(dk)
    pq = torch.empty((n, H, D), dtype=torch.bfloat16, device=DEV)
    pk = torch.empty((n, Hkv, D), dtype=torch.bfloat16, device=DEV)
    pv = torch.empty_like(pk)
    for i in q_ranks:
        for j in range(P):
            usp.striped_attn_bwd(qs[i], ks[j], vs[j], o[i], acc_l[i], dos[i], P, i, j, posd,
                                 dq=pq, dk=pk, dv=pv)
            dq[i] += pq.float()
            dk[j] += pk.float()
            dv[j] += pv.float()
    torch.cuda.synchronize()
    return o, acc_l, dq, dk, dv


def unstripe(t):
    """[P][n][...] -> [P n][...] on the host (token i + P a is stripe i, row a)."""
    P, n = t.shape[:2]
    return t.transpose(0, 1).reshape((P * n,) + tuple(t.shape[2:]))


def test_striped_pairs_fwd_small(usp):
    """Every stripe pair of a packed causal input against the oracle's strided attention."""
    P, S, Hq, Hkv, D = 4, 1024, 4, 2, 128
    lengths = [300, 1, 450, 273]
    say("striped pairs", P, S)
    q, k, v, _, pos = inputs.attention_case(S, Hq, Hkv, D, seed=22, lengths=lengths)
    qd, kd, vd = to_dev(q, k, v)
    posd = torch.from_numpy(pos).to(DEV)
    qs, ks, vs = _stripes(usp, P, qd, kd, vd)
    q64, k64, v64 = (oracle.seq_to_stripe(f64(t), P) for t in (q, k, v))
    for i in range(P):
        for j in range(P):
            o, lse = usp.striped_attn_fwd(qs[i], ks[j], vs[j], P, i, j, posd)
            ref_o, ref_l = oracle.striped_pair_fwd(q64[i], k64[j], v64[j], P, i, j, pos=pos)
            torch.cuda.synchronize()
            check_o(o.cpu(), ref_o, ("pair", i, j))
            check_lse(lse.cpu(), ref_l, ("pair lse", i, j))


@pytest.mark.parametrize("P,lengths,Hq,Hkv", [
    (4, [300, 1, 450, 273], 4, 2),    # packed documents
    (8, [2048], 2, 2),                # one causal document
])
def test_striped_ring_fwd_bwd_small(usp, P, lengths, Hq, Hkv):
    S, D = sum(lengths), 128
    say("striped ring", P, S)
    q, k, v, do, pos = inputs.attention_case(S, Hq, Hkv, D, seed=23, lengths=lengths)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    posd = torch.from_numpy(pos).to(DEV)
    o, lse, dq, dk, dv = striped_ring(usp, qd, kd, vd, dod, posd, P)
    args = (f64(q), f64(k), f64(v))
    ref_o, ref_l = oracle.attention_fwd(*args, pos=pos, causal=True)
    check_o(unstripe(o).cpu(), ref_o, "o")
    check_lse(lse.permute(1, 2, 0).reshape(Hq, S).cpu(), ref_l, "lse")
    rq, rk, rv = oracle.attention_bwd(*args, f64(do), pos=pos, causal=True)
    check_grad(unstripe(dq).cpu(), rq, "dq")
    check_grad(unstripe(dk).cpu(), rk, "dk")
    check_grad(unstripe(dv).cpu(), rv, "dv")


def test_striped_ring_256k_sampled(usp):
    """[262144][2][128] in one document over 16 stripes: the first and the last query
    stripe against all key stripes, sampled rows against the oracle."""
    P = 16
    say("striped ring 256k")
    q, k, v, pos = inputs.ring_256k()
    S, H, D = q.shape
    n = S // P
    qd, kd, vd = to_dev(q, k, v)
    posd = torch.from_numpy(pos).to(DEV)
    o, lse, _, _, _ = striped_ring(usp, qd, kd, vd, qd, posd, P, q_ranks=(0, P - 1), backward=False)
    q64, k64, v64 = f64(q), f64(k), f64(v)
    for i in (0, P - 1):
        rows = sample_rows(n, 12, 31 + i)
        tokens = i + P * rows
        ref_o, ref_l = oracle.attention_fwd(q64, k64, v64, pos=pos, causal=True, rows=tokens)
        check_o(o[i][rows].cpu(), ref_o, ("stripe", i))
        check_lse(lse[i][:, rows].cpu(), ref_l, ("stripe lse", i))
