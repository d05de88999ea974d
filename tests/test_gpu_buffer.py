"""GPU checks of the buffer klein_rope4d_attn_fwd and klein_rope4d_attn_fwd_fp8
keep per device.

With the buffer the plain entry points make the call of
klein_rope4d_attn_fwd_ws (keys rotated once, the split-KV schedule), so
their results must equal that call's bit for bit, whatever buffer the
previous calls left behind (a smaller one is replaced, one dtype's layout
follows the other's).  The limit picks the schedule: a shape that needs more
runs the per-tile kernels.  Calls on two streams, or from two host threads,
share the buffer and must come out as if run one after the other.  Under
graph capture the call records the per-tile kernels (a graph must not hold
the address of a buffer a later call may free), and replays must equal them
while eager calls on the buffer run between the replays.
"""

import threading

import pytest
import torch

import joint_attention_rope_amd as kl
from helpers import random_fp8_inputs, random_inputs, run_attention, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# 576 query tiles each: not whole rounds of a 256-CU GPU, so the schedule
# splits the last round and the buffer holds keys and partials
SPLIT_BF16 = (2, 4608, 16, 128)
SPLIT_FP8 = (1, 6000, 24, 64)


@pytest.fixture(autouse=True)
def default_limit():
    kl.klein_set_buffer_limit(kl.KLEIN_DEFAULT_BUFFER_LIMIT)
    yield
    kl.klein_set_buffer_limit(kl.KLEIN_DEFAULT_BUFFER_LIMIT)


def make(shape, fp8, seed):
    return (random_fp8_inputs if fp8 else random_inputs)(*shape, seed=seed)


def dtype_of(inp):
    return kl.KLEIN_DTYPE_BF16 if inp.descale is None else kl.KLEIN_DTYPE_FP8_E4M3


def call_plain(tensors, inp, out):
    q, k, v, pos = tensors
    if inp.descale is None:
        kl.klein_rope4d_attn_fwd(q, k, v, pos, out)
    else:
        kl.klein_rope4d_attn_fwd_fp8(q, k, v, pos, out, *inp.descale)


def run_ws(inp):
    q, k, v, pos = to_device(inp, DEV)
    B, S, H, D = q.shape
    ws = torch.empty(kl.klein_attn_workspace_size(B, S, H, D, dtype_of(inp)), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    kl.klein_rope4d_attn_fwd_ws(q, k, v, pos, out, ws, dtype=dtype_of(inp),
                                descales=inp.descale or (1.0, 1.0, 1.0))
    torch.cuda.synchronize()
    return out


def bits(t):
    return t.view(torch.int16)


def keys_bytes(shape, fp8):
    B, S, H, D = shape
    return (B * S * H * D * (1 if fp8 else 2) + 255) // 256 * 256


@pytest.mark.parametrize("fp8", [False, True])
def test_plain_entry_is_the_workspace_call(fp8):
    shape = SPLIT_FP8 if fp8 else SPLIT_BF16
    inp = make(shape, fp8, seed=301 + fp8)
    print(f"[case] plain vs workspace {shape} fp8={fp8}", flush=True)
    assert kl.klein_attn_workspace_size(*shape, dtype_of(inp)) > keys_bytes(shape, fp8)
    got = run_attention(inp)
    assert torch.equal(bits(got), bits(run_ws(inp)))


def test_buffer_replaced_by_larger_and_shared_by_both_dtypes():
    cases = [((1, 700, 3, 128), False), (SPLIT_BF16, False), (SPLIT_FP8, True),
             ((1, 700, 3, 128), False), ((1, 2100, 3, 64), True)]
    for i, (shape, fp8) in enumerate(cases):
        inp = make(shape, fp8, seed=310 + i)
        print(f"[case] call {i}: {shape} fp8={fp8}", flush=True)
        assert torch.equal(bits(run_attention(inp)), bits(run_ws(inp))), f"call {i}"


def test_limit_selects_the_schedule():
    inp = make(SPLIT_BF16, False, seed=320)
    need = kl.klein_attn_workspace_size(*SPLIT_BF16)
    per_tile = run_attention(inp, path="per-tile")
    ws = run_ws(inp)
    kl.klein_set_buffer_limit(need - 1)
    assert torch.equal(bits(run_attention(inp)), bits(per_tile))
    kl.klein_set_buffer_limit(need)
    assert torch.equal(bits(run_attention(inp)), bits(ws))


def test_two_streams_share_the_buffer_in_order():
    a, b = make(SPLIT_BF16, False, seed=330), make(SPLIT_FP8, True, seed=331)
    ra, rb = run_ws(a), run_ws(b)
    ta, tb = to_device(a, DEV), to_device(b, DEV)
    oa, ob = torch.empty_like(ra), torch.empty_like(rb)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for i in range(3):
        with torch.cuda.stream(s1):
            call_plain(ta, a, oa)
        with torch.cuda.stream(s2):
            call_plain(tb, b, ob)
    torch.cuda.synchronize()
    assert torch.equal(bits(oa), bits(ra))
    assert torch.equal(bits(ob), bits(rb))


def test_two_threads_share_the_buffer_in_order():
    a, b = make(SPLIT_BF16, False, seed=340), make(SPLIT_FP8, True, seed=341)
    ra, rb = run_ws(a), run_ws(b)
    jobs = [(to_device(a, DEV), a, torch.empty_like(ra)),
            (to_device(b, DEV), b, torch.empty_like(rb))]
    errors = []
    torch.cuda.synchronize()

    def worker(tensors, inp, out):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for _ in range(3):
                    call_plain(tensors, inp, out)
            stream.synchronize()
        except Exception as e:           # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=j) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    torch.cuda.synchronize()
    assert torch.equal(bits(jobs[0][2]), bits(ra))
    assert torch.equal(bits(jobs[1][2]), bits(rb))


def test_graph_capture_records_the_per_tile_kernels():
    inp = make(SPLIT_BF16, False, seed=350)
    tensors = to_device(inp, DEV)
    ref = run_attention(inp, path="per-tile")
    out = torch.zeros_like(ref)
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            call_plain(tensors, inp, out)
    torch.cuda.synchronize()
    eager = torch.empty_like(ref)
    for i in range(3):
        out.zero_()
        call_plain(tensors, inp, eager)             # the buffer schedule, between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(ref)), f"replay {i}"
    assert torch.equal(bits(eager), bits(run_ws(inp)))


def test_limit_zero_frees_and_allocates_nothing():
    inp = make(SPLIT_BF16, False, seed=360)
    tensors = to_device(inp, DEV)
    out = torch.empty(SPLIT_BF16, dtype=torch.bfloat16, device=DEV)
    ref = run_attention(inp, path="per-tile")
    need = kl.klein_attn_workspace_size(*SPLIT_BF16)
    call_plain(tensors, inp, out)                       # holds a buffer now
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    kl.klein_set_buffer_limit(0)
    free1, _ = torch.cuda.mem_get_info()
    assert free1 - free0 >= need                        # the buffer went back to the device
    call_plain(tensors, inp, out)
    torch.cuda.synchronize()
    free2, _ = torch.cuda.mem_get_info()
    assert free2 >= free1 - (4 << 20)                   # and no new one was taken
    assert torch.equal(bits(out), bits(ref))
