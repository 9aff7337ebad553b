"""The entry points under HIP graph capture (through torch.cuda.CUDAGraph), for callers that
launch the forward from captured code: a captured mifa_fwd (key-split and 8-wave tile-pair launch
shapes) and a captured mifa_attention_splitkv_noalloc (whose partials live in the library's static
array, so the capture needs no allocation).  Each graph is replayed several times, with new input
values copied in, eager launches and synchronisations between the replays; every replay must equal
an eager call on the same inputs bit for bit (same kernels, deterministic)."""
import pytest
import torch

from io_aware_softmax_mifa_amd import binding
from io_aware_softmax_mifa_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[graph] {msg}", flush=True)


def replay_and_compare(call, inputs, outputs, fresh_inputs, name):
    """call(stream) launches into `outputs` from `inputs`; fresh_inputs(i) gives new input values."""
    stream = torch.cuda.current_stream().cuda_stream
    call(stream)  # eager first: per-device set-up (LDS limits, the static array's address)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(torch.cuda.current_stream().cuda_stream)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for i in range(3):
        for t, new in zip(inputs, fresh_inputs(i)):
            t.copy_(new)
        for t in outputs:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outputs]
        for t in outputs:
            t.fill_(float("nan"))
        call(torch.cuda.current_stream().cuda_stream)  # eager, same inputs
        torch.cuda.synchronize()
        for a, b in zip(got, outputs):
            assert torch.equal(a, b), f"{name}: replay {i} differs from the eager call"
        say(f"{name}: replay {i} equals the eager call")


@pytest.mark.parametrize("B,H,N,d", [(4, 8, 1024, 64), (4, 16, 2048, 64)])
def test_captured_forward(B, H, N, d):
    """B=4 H=8 N=1024: the key-split launch; B=4 H=16 N=2048: the 8-wave tile-pair launch."""
    q, k, v = (t.cuda() for t in W.make_inputs(B, H, N, d, seed=6000 + N))
    o = torch.empty(B, H, N, d, device="cuda")
    lse = torch.empty(B, H, N, device="cuda")
    scale = W.fp32_scale(d)

    def call(stream):
        st = binding.mifa_fwd_raw(q, k, v, o, lse, B, H, N, d, True, scale, stream)
        assert st == 0, binding.mifa_status_string(st)

    def fresh(i):
        return [t.cuda() for t in W.make_inputs(B, H, N, d, seed=6100 + 10 * i + N)]

    say(f"forward B={B} H={H} N={N} d={d} causal")
    replay_and_compare(call, [q, k, v], [o, lse], fresh, f"fwd B={B} H={H} N={N}")


def test_captured_splitkv_noalloc():
    B, H, Nq, Nk, d = 1, 8, 16, 8192, 128
    q, k, v = (t.cuda() for t in W.make_rect_inputs(B, H, Nq, Nk, d, 6200))
    o = torch.empty(B, H, Nq, d, device="cuda")
    lse = torch.empty(B, H, Nq, device="cuda")
    scale = W.fp32_scale(d)

    def call(stream):
        st = binding.mifa_attention_splitkv_noalloc_raw(q, k, v, o, lse, B, H, Nq, Nk, d, True, scale, stream)
        assert st == 0, binding.mifa_status_string(st)

    def fresh(i):
        return [t.cuda() for t in W.make_rect_inputs(B, H, Nq, Nk, d, 6300 + i)]

    say(f"split-KV noalloc B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal")
    replay_and_compare(call, [q, k, v], [o, lse], fresh, "splitkv noalloc")
