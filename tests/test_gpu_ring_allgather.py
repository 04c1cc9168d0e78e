"""GPU parity of two compositions of the same entry points:

* ring backward through the merge: the forward runs query block i against key
  blocks 0..i with fp32 partials merged by lse_merge; the backward then calls
  blockattn_bwd on every (i, j) pair with the FINAL merged O and LSE of block i
  (so P and D are those of the whole row) and sums the partial gradients: dQ_i
  over j, dK_j and dV_j over i.  Exact in exact arithmetic (the Ring Attention
  page's blockwise decomposition, differentiated).
* all-gather-KV: rank r's local query shard (rows r*S/P .. (r+1)*S/P, q_start set
  accordingly) against the full K and V; the ranks' dK, dV partials sum to the
  full gradients.

The partial-gradient sums are fp32 torch additions in the tests (plumbing around
the library calls)."""

import numpy as np
import pytest
import torch

import oracle
from sequence_parallelism_amd import inputs
from test_gpu_parity import DEV, check_grad, check_lse, check_o, f64, say, to_dev
from test_gpu_workloads import sample_rows

pytestmark = pytest.mark.gpu


def ring_fwd_bwd(usp, qd, kd, vd, dod, posd, nb):
    """Blockwise ring forward (merged fp32 partials) and backward over block pairs;
    returns O (bf16), LSE, and fp32 dQ, dK, dV."""
    S, H, D = qd.shape
    Hkv = kd.shape[1]
    blk = S // nb
    acc = torch.zeros((S, H, D), dtype=torch.float32, device=DEV)
    acc_l = torch.full((H, S), -float("inf"), dtype=torch.float32, device=DEV)
    po = torch.empty((blk, H, D), dtype=torch.float32, device=DEV)
    pl = torch.empty((H, blk), dtype=torch.float32, device=DEV)
    for i in range(nb):
        qs = slice(i * blk, (i + 1) * blk)
        for j in range(i + 1):
            ks = slice(j * blk, (j + 1) * blk)
            usp.blockattn_fwd(qd[qs], kd[ks], vd[ks], posd, q_start=i * blk, k_start=j * blk,
                              o=po, lse=pl)
            usp.lse_merge(acc[qs], acc_l[:, qs], po, pl)
    o = acc.to(torch.bfloat16)
    dq = torch.zeros((S, H, D), dtype=torch.float32, device=DEV)
    dk = torch.zeros((S, Hkv, D), dtype=torch.float32, device=DEV)
    dv = torch.zeros_like(dk)
    pq = torch.empty((blk, H, D), dtype=torch.bfloat16, device=DEV)
    pk = torch.empty((blk, Hkv, D), dtype=torch.bfloat16, device=DEV)
    pv = torch.empty_like(pk)
    for i in range(nb):
        qs = slice(i * blk, (i + 1) * blk)
        for j in range(i + 1):
            ks = slice(j * blk, (j + 1) * blk)
            usp.blockattn_bwd(qd[qs], kd[ks], vd[ks], o[qs], acc_l[:, qs], dod[qs], posd,
                              q_start=i * blk, k_start=j * blk, dq=pq, dk=pk, dv=pv)
            dq[qs] += pq.float()
            dk[ks] += pk.float()
            dv[ks] += pv.float()
    torch.cuda.synchronize()
    return o, acc_l, dq, dk, dv


def test_ring_bwd_blockwise_small(usp):
    """S = 2048 in 4 ring blocks, 2 query heads sharing 1 key/value head, one causal
    document: every output against the full oracle backward."""
    say("ring bwd small")
    S, nb = 2048, 4
    q, k, v, do, pos = inputs.attention_case(S, 2, 1, 128, seed=21)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    posd = torch.from_numpy(pos).to(DEV)
    o, lse, dq, dk, dv = ring_fwd_bwd(usp, qd, kd, vd, dod, posd, nb)
    ro, rl = oracle.attention_fwd(f64(q), f64(k), f64(v), pos=pos, causal=True)
    check_o(o.cpu(), ro, "ring o")
    check_lse(lse.cpu(), rl, "ring lse")
    # the backward reference uses the bf16 O that the ring produced (D = <dO, O>)
    rdq, rdk, rdv = oracle.attention_bwd(f64(q), f64(k), f64(v), f64(do), pos=pos, causal=True)
    check_grad(dq, rdq, "ring dq")
    check_grad(dk, rdk, "ring dk")
    check_grad(dv, rdv, "ring dv")


def test_ring_bwd_256k(usp):
    """The 256K ring (16 blocks of 16384, 136 block pairs each way): sampled dQ rows,
    and dK, dV of the last 256 keys (seen only by the last 256 rows)."""
    say("ring bwd 256k")
    q, k, v, do, pos = inputs.ring_256k(with_do=True)
    S, nb, tail = 262144, 16, 256
    qd, kd, vd, dod = to_dev(q, k, v, do)
    posd = torch.from_numpy(pos).to(DEV)
    o, lse, dq, dk, dv = ring_fwd_bwd(usp, qd, kd, vd, dod, posd, nb)
    rows = sample_rows(S, 24, 5, tile=S // nb)
    rdq, _, _ = oracle.attention_bwd(f64(q), f64(k), f64(v), f64(do), pos=pos, causal=True,
                                     rows=rows)
    check_grad(dq[rows], rdq, "ring 256k dq rows")
    t = slice(S - tail, S)
    _, rdk, rdv = oracle.attention_bwd(f64(q[t]), f64(k), f64(v), f64(do[t]), pos=pos,
                                       q_start=S - tail, causal=True)
    check_grad(dk[t], rdk[S - tail:], "ring 256k dk tail")
    check_grad(dv[t], rdv[S - tail:], "ring 256k dv tail")


@pytest.mark.parametrize("lengths", [None, [700, 1300, 2096]])
def test_allgather_kv_fwd_bwd(usp, lengths):
    """S = 4096 over P = 4 ranks, 4 query heads sharing 2 key/value heads: each
    rank's shard against the full K, V; O, LSE and dQ rows against the oracle, and
    the ranks' dK, dV partials summed against the full gradients."""
    say("all-gather kv", lengths)
    S, P = 4096, 4
    q, k, v, do, pos = inputs.attention_case(S, 4, 2, 128, seed=22, lengths=lengths)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    posd = torch.from_numpy(pos).to(DEV)
    ro, rl = oracle.attention_fwd(f64(q), f64(k), f64(v), pos=pos, causal=True)
    rdq, rdk, rdv = oracle.attention_bwd(f64(q), f64(k), f64(v), f64(do), pos=pos, causal=True)
    n = S // P
    dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros_like(dk)
    for r in range(P):
        rs = slice(r * n, (r + 1) * n)
        o, lse = usp.blockattn_fwd(qd[rs], kd, vd, posd, q_start=r * n)
        check_o(o.cpu(), ro[rs], f"ag o rank {r}")
        check_lse(lse.cpu(), rl[:, rs], f"ag lse rank {r}")
        dq_r, dk_r, dv_r = usp.blockattn_bwd(qd[rs], kd, vd, o, lse, dod[rs], posd, q_start=r * n)
        check_grad(dq_r, rdq[rs], f"ag dq rank {r}")
        dk += dk_r.float()
        dv += dv_r.float()
    torch.cuda.synchronize()
    check_grad(dk, rdk, "ag dk sum")
    check_grad(dv, rdv, "ag dv sum")
