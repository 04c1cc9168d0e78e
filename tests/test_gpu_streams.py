"""Calls on caller-supplied streams: two forward + backward calls in flight at once on
two side streams (each with its own outputs and workspace) give bit-identical results
to the same call on the default stream.  Every launch of a call goes to the stream it
is given and the library keeps no state between calls; the kernels are deterministic
(no accumulation by atomics), so equality is exact."""

import pytest
import torch

from sequence_parallelism_amd import inputs
from test_gpu_parity import DEV, say

pytestmark = pytest.mark.gpu


def _fwd_bwd(usp, qd, kd, vd, dod, posd):
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd, causal=True)
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd, causal=True)
    return o, lse, dq, dk, dv


def test_concurrent_side_streams_match_default(usp):
    say("two side streams at once")
    S = 8192
    q, k, v, do, pos = inputs.attention_case(S, 4, 1, 128, seed=61, lengths=[3000, 100, 5092])
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    posd = torch.from_numpy(pos).to(DEV)
    ref = _fwd_bwd(usp, qd, kd, vd, dod, posd)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        r1 = _fwd_bwd(usp, qd, kd, vd, dod, posd)
    with torch.cuda.stream(s2):
        r2 = _fwd_bwd(usp, qd, kd, vd, dod, posd)
    torch.cuda.synchronize()
    for got in (r1, r2):
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), name
