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


def test_explicit_stream_argument_matches_default(usp):
    """Calls given a side stream that is NOT current, with no preallocated outputs or
    workspace: the binding allocates those while the side stream is current, so work
    that the current stream enqueues right after the call (here: allocations of the
    same sizes, filled with NaN) cannot take their memory while the side-stream kernels
    still use it.  Results equal the default-stream call bit for bit."""
    say("explicit stream argument")
    S = 8192
    q, k, v, do, pos = inputs.attention_case(S, 4, 1, 128, seed=62, lengths=[5000, 3192])
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    posd = torch.from_numpy(pos).to(DEV)
    ref = _fwd_bwd(usp, qd, kd, vd, dod, posd)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd, stream=side)
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd, stream=side)
    # the current stream now allocates and overwrites memory of the sizes the calls
    # allocated; with the temporaries on the side stream none of it can alias them
    junk = [torch.full_like(t, float("nan")) for t in (o, lse, dq, dk, dv)]
    junk += [torch.full((usp.bwd_workspace_bytes(S, S, 4, 1, 128),), 255, dtype=torch.uint8, device=DEV)]
    side.synchronize()
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), ref):
        assert torch.equal(a, b), name
    del junk
