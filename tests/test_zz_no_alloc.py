"""flash_gau_forward_noalloc against flash_gau_forward, both through the C ABI.

The allocation-free entry point runs the same kernels on the library's fixed scratch array instead
of a caller's workspace, so its output must equal flash_gau_forward's bit for bit. Two calls in a
row, the second on a smaller problem, check that the array's left-over contents from the first
call do not leak into the second.
"""

import numpy as np
import pytest
import torch

from efficient_transformer_attention_amd import flashgau as fg
from efficient_transformer_attention_amd import inputs as gen


def _upload(inp, tdt):
    def up(a, t=tdt):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(t).contiguous()
    return [up(inp.X), up(inp.W_u), up(inp.W_v), up(inp.W_z), up(inp.gamma, torch.float32),
            up(inp.beta, torch.float32), up(inp.W_o)]


def _both(shape, dtype, seed, side=None):
    B, n, d, e, s, c, causal = shape
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dt = fg.BF16 if dtype == "bf16" else fg.F32
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=seed, beta_std=0.1)
    args = _upload(inp, tdt)
    ptrs = [t.data_ptr() for t in args]
    stream = torch.cuda.current_stream().cuda_stream
    if side is not None:
        side.wait_stream(torch.cuda.current_stream())
        stream = side.cuda_stream
    nbytes = fg.workspace_size(B, n, d, e, s, c, causal, dt)
    assert nbytes <= fg.noalloc_scratch_bytes()
    ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    ref = torch.empty((B, n, d), dtype=tdt, device="cuda")
    got = torch.full((B, n, d), float("nan"), dtype=tdt, device="cuda")
    print(f"noalloc: shape {shape} {dtype} seed {seed} stream {stream:#x}", flush=True)
    assert fg.forward_raw(*ptrs, c, causal, B, n, d, e, s, dt, ref.data_ptr(), ws.data_ptr(),
                          nbytes, stream) == fg.OK
    assert fg.forward_noalloc_raw(*ptrs, c, causal, B, n, d, e, s, dt, got.data_ptr(),
                                  stream) == fg.OK
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_forward_twice_in_a_row():
    # first a larger problem (33 MiB of scratch), then a smaller one on the same array
    first = (4, 1024, 512, 1024, 128, 256, True)
    second = (2, 256, 256, 512, 64, 64, False)
    ref, got = _both(first, "bf16", 1)
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))
    ref, got = _both(second, "bf16", 2)
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))
    # and an fp32 problem after both
    ref, got = _both((1, 512, 256, 512, 128, 128, False), "f32", 3)
    assert torch.equal(ref.view(torch.int32), got.view(torch.int32))


@pytest.mark.gpu
def test_noalloc_rejects_a_problem_beyond_its_scratch():
    B, n, d, e, s, c = 8, 4096, 768, 1536, 128, 256
    X = torch.zeros((B, n, d), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((d, e), dtype=torch.bfloat16, device="cuda")
    Wz = torch.zeros((d, s), dtype=torch.bfloat16, device="cuda")
    Wo = torch.zeros((e, d), dtype=torch.bfloat16, device="cuda")
    g = torch.ones((4, s), dtype=torch.float32, device="cuda")
    O = torch.empty_like(X)
    rc = fg.forward_noalloc_raw(X.data_ptr(), W.data_ptr(), W.data_ptr(), Wz.data_ptr(), g.data_ptr(),
                                g.data_ptr(), Wo.data_ptr(), c, 1, B, n, d, e, s, fg.BF16, O.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    assert rc == fg.ERR_TOO_LARGE


@pytest.mark.gpu
def test_noalloc_on_a_created_stream():
    # the call takes the scratch copy of the device its stream belongs to (asked of the stream)
    side = torch.cuda.Stream()
    ref, got = _both((2, 512, 256, 512, 64, 128, True), "bf16", 4, side=side)
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))


@pytest.mark.gpu
def test_noalloc_replayed_from_a_hip_graph():
    # the callers it is for: a forward captured into a HIP graph with no allocation during
    # capture. One eager call first (the per-device scratch address is looked up then, outside
    # the capture); every replay, with eager work and synchronisations between, must equal
    # flash_gau_forward bit for bit.
    B, n, d, e, s, c, causal = 2, 512, 256, 512, 64, 128, True
    inp = gen.make_inputs(B, n, d, e, s, c, causal, "bf16", seed=5, beta_std=0.1)
    args = _upload(inp, torch.bfloat16)
    ptrs = [t.data_ptr() for t in args]
    ref = fg.flash_gau_forward(*args, c, causal)
    O = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    assert fg.forward_noalloc_raw(*ptrs, c, causal, B, n, d, e, s, fg.BF16, O.data_ptr(),
                                  side.cuda_stream) == fg.OK
    torch.cuda.synchronize()
    assert torch.equal(O.view(torch.int16), ref.view(torch.int16))
    print("noalloc: graph capture", flush=True)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        rc = fg.forward_noalloc_raw(*ptrs, c, causal, B, n, d, e, s, fg.BF16, O.data_ptr(),
                                    side.cuda_stream)
    assert rc == fg.OK
    for rep in range(3):
        O.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(O.view(torch.int16), ref.view(torch.int16)), rep
