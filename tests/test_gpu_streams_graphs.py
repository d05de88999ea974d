"""Execution-model checks of the library on the GPU: calls are asynchronous on
the given stream and carry no per-call state, so (1) a call captured in a
HIP graph replays to the eager result, replay after replay, with eager work
and synchronisations in between; (2) concurrent calls on two streams give
the same results as serial calls."""

import pytest
import torch

import joint_attention_rope_amd as kl
from helpers import random_fp8_inputs, random_inputs, to_device

pytestmark = pytest.mark.gpu


def _eager(q, k, v, pos, fp8_scales=None):
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if fp8_scales is None:
        kl.klein_rope4d_attn_fwd(q, k, v, pos, out)
    else:
        kl.klein_rope4d_attn_fwd_fp8(q, k, v, pos, out, *fp8_scales)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("fp8", [False, True])
def test_graph_capture_replays_match_eager(fp8):
    inp = (random_fp8_inputs if fp8 else random_inputs)(1, 600, 4, 128, seed=81)
    q, k, v, pos = to_device(inp)
    ref = _eager(q, k, v, pos, inp.descale)
    out = torch.zeros_like(ref)
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            if inp.descale is None:
                kl.klein_rope4d_attn_fwd(q, k, v, pos, out)
            else:
                kl.klein_rope4d_attn_fwd_fp8(q, k, v, pos, out, *inp.descale)
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        _eager(q, k, v, pos, inp.descale)           # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"


def test_two_streams_concurrently():
    a = random_inputs(2, 900, 6, 128, seed=82)
    b = random_inputs(1, 1300, 5, 64, seed=83)
    ta, tb = to_device(a), to_device(b)
    ra, rb = _eager(*ta), _eager(*tb)
    oa, ob = torch.empty_like(ra), torch.empty_like(rb)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(s1):
            kl.klein_rope4d_attn_fwd(*ta, oa)
        with torch.cuda.stream(s2):
            kl.klein_rope4d_attn_fwd(*tb, ob)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ra.view(torch.int16))
    assert torch.equal(ob.view(torch.int16), rb.view(torch.int16))
