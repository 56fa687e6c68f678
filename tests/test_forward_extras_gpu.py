"""GPU checks around the forward's boundary: the weight transpose is exact, the packed-weights
entry point returns bitwise what flash_gau_forward does, and the forward writes nothing outside O
and its workspace (guard bands of 0xFF bytes around both stay untouched), and calls on another
stream keep the memory they allocate until their kernels are done.
"""

import numpy as np
import pytest

from efficient_transformer_attention_amd import flashgau as fg
from efficient_transformer_attention_amd import inputs as gen

pytestmark = pytest.mark.gpu

SHAPES = {
    # name: (B, n, d, e, s, chunk, causal, dtype)
    "ragged_causal_bf16": (2, 216, 200, 136, 24, 72, True, "bf16"),
    "ragged_noncausal_fp32": (3, 144, 40, 88, 136, 48, False, "f32"),
    "c2_causal_bf16": (4, 1024, 512, 1024, 128, 256, True, "bf16"),
    "one_chunk_causal_bf16": (2, 256, 128, 256, 128, 256, True, "bf16"),
}
GUARD = 4096  # bytes on each side


def _torch():
    import torch
    return torch


def _setup(name, seed=0):
    torch = _torch()
    B, n, d, e, s, c, causal, dtype = SHAPES[name]
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=seed, beta_std=0.1)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def up(a, t=tdt):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(t).contiguous()

    args = [up(inp.X), up(inp.W_u), up(inp.W_v), up(inp.W_z), up(inp.gamma, torch.float32),
            up(inp.beta, torch.float32), up(inp.W_o)]
    dt = fg.BF16 if dtype == "bf16" else fg.F32
    print(f"[gpu case] {name}", flush=True)
    return (B, n, d, e, s, c, causal, dt, tdt), args


def _bits(t):
    torch = _torch()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("name", ["ragged_causal_bf16", "ragged_noncausal_fp32"])
def test_weight_transpose_is_exact(name):
    torch = _torch()
    (B, n, d, e, s, c, causal, dt, tdt), args = _setup(name)
    X, W_u, W_v, W_z, g, b, W_o = args
    ws = torch.empty(fg.workspace_size(B, n, d, e, s, c, causal, dt), dtype=torch.uint8, device="cuda")
    fg.flash_gau_forward(*args, c, causal, workspace=ws)
    packed = fg.pack_weights(W_u, W_v, W_z, W_o)
    torch.cuda.synchronize()
    v = fg.workspace_views(ws, B, n, d, e, s, c, causal, dt)
    want_cat = torch.cat([W_u, W_v, W_z], dim=1).t().contiguous()
    assert torch.equal(_bits(v["WCAT_T"]), _bits(want_cat))
    assert torch.equal(_bits(v["WO_T"]), _bits(W_o.t().contiguous()))
    esz = 2 if dt == fg.BF16 else 4
    cat_bytes = (2 * e + s) * d * esz
    wo_off = (cat_bytes + 255) // 256 * 256
    assert torch.equal(_bits(packed[:cat_bytes].view(tdt).view(2 * e + s, d)), _bits(want_cat))
    assert torch.equal(_bits(packed[wo_off:wo_off + d * e * esz].view(tdt).view(d, e)),
                       _bits(W_o.t().contiguous()))


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_packed_weights_forward_is_bitwise_the_forward(name):
    torch = _torch()
    (B, n, d, e, s, c, causal, dt, tdt), args = _setup(name, seed=3)
    X, W_u, W_v, W_z, g, b, W_o = args
    ref = fg.flash_gau_forward(*args, c, causal)
    packed = fg.pack_weights(W_u, W_v, W_z, W_o)
    nbytes = fg.workspace_size(B, n, d, e, s, c, causal, dt)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.full_like(ref, float("nan"))
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(2):  # twice: the second call reuses everything the first left
        rc = fg.forward_packed_raw(X.data_ptr(), packed.data_ptr(), packed.numel(), g.data_ptr(),
                                   b.data_ptr(), c, causal, B, n, d, e, s, dt, out.data_ptr(),
                                   ws.data_ptr(), nbytes, stream)
        assert rc == fg.OK
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref))
    # a packed buffer one byte short is refused before anything runs
    rc = fg.forward_packed_raw(X.data_ptr(), packed.data_ptr(), packed.numel() - 1, g.data_ptr(),
                               b.data_ptr(), c, causal, B, n, d, e, s, dt, out.data_ptr(),
                               ws.data_ptr(), nbytes, stream)
    assert rc == fg.ERR_WORKSPACE


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_forward_writes_only_its_output_and_workspace(name):
    torch = _torch()
    (B, n, d, e, s, c, causal, dt, tdt), args = _setup(name, seed=1)
    esz = 2 if dt == fg.BF16 else 4
    ref = fg.flash_gau_forward(*args, c, causal)
    o_bytes = B * n * d * esz
    nbytes = fg.workspace_size(B, n, d, e, s, c, causal, dt)
    o_buf = torch.full((o_bytes + 2 * GUARD,), 0xFF, dtype=torch.uint8, device="cuda")
    w_buf = torch.full((nbytes + 2 * GUARD,), 0xFF, dtype=torch.uint8, device="cuda")
    O = o_buf[GUARD:GUARD + o_bytes].view(tdt).view(B, n, d)
    ws = w_buf[GUARD:GUARD + nbytes]
    fg.flash_gau_forward(*args, c, causal, out=O, workspace=ws)
    torch.cuda.synchronize()
    for buf, size in ((o_buf, o_bytes), (w_buf, nbytes)):
        assert bool((buf[:GUARD] == 0xFF).all())
        assert bool((buf[GUARD + size:] == 0xFF).all())
    assert torch.equal(_bits(O), _bits(ref))


def _delay(stream, torch):
    # queue a few milliseconds of matrix products on `stream` (operands made and finished first)
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    buf = torch.empty_like(a)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(4):
            torch.mm(a, a, out=buf)
    return a, buf


def _scribble(nbytes, torch):
    # allocations on the current stream of about the size just freed, overwritten at once
    return [torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda") for _ in range(2)]


def test_calls_on_another_stream_keep_their_allocations():
    # A call given `stream=` but no workspace allocates the workspace on torch's current stream
    # and drops it on return, while its kernels run later on the given stream (here held back by
    # queued products). New allocations on the current stream, filled at once, must not receive
    # that memory before those kernels finish, or the kernels' late writes would land in them:
    # the fills stay intact, and the results equal a plain call's bit for bit.
    torch = _torch()
    (B, n, d, e, s, c, causal, dt, tdt), args = _setup("c2_causal_bf16")
    O_ref = fg.flash_gau_forward(*args, c, causal)
    dO = torch.randn(B, n, d, device="cuda").to(tdt)
    g_ref = fg.flash_gau_backward(*args, dO, c, causal)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    keep = _delay(side, torch)
    O = fg.flash_gau_forward(*args, c, causal, stream=side.cuda_stream)
    junk = _scribble(fg.workspace_size(B, n, d, e, s, c, causal, dt), torch)
    side.synchronize()
    torch.cuda.synchronize()
    assert all(bool((j == 0x7F).all()) for j in junk)
    assert torch.equal(_bits(O), _bits(O_ref))

    keep = _delay(side, torch)
    g = fg.flash_gau_backward(*args, dO, c, causal, stream=side.cuda_stream)
    junk = _scribble(fg.backward_workspace_size(B, n, d, e, s, c, causal, dt), torch)
    side.synchronize()
    torch.cuda.synchronize()
    assert all(bool((j == 0x7F).all()) for j in junk)
    del keep, junk
    for k in fg.GRAD_NAMES:
        assert torch.equal(_bits(g[k]), _bits(g_ref[k])), k


def test_calls_on_two_streams_at_once_match_sequential_calls():
    # the library keeps no state between calls besides the allocation-free entry point's scratch:
    # two problems run concurrently on two streams, each with its own workspace, give bit for bit
    # what they give one after the other
    torch = _torch()
    (B, n, d, e, s, c, causal, dt, tdt), a1 = _setup("c2_causal_bf16", seed=1)
    _, a2 = _setup("c2_causal_bf16", seed=2)
    dO1 = torch.randn(B, n, d, device="cuda").to(tdt)
    dO2 = torch.randn(B, n, d, device="cuda").to(tdt)
    O1 = fg.flash_gau_forward(*a1, c, causal)
    O2 = fg.flash_gau_forward(*a2, c, not causal)
    g1 = fg.flash_gau_backward(*a1, dO1, c, causal)
    g2 = fg.flash_gau_backward(*a2, dO2, c, not causal)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = {}
    for rep in range(3):
        with torch.cuda.stream(s1):
            outs["O1"] = fg.flash_gau_forward(*a1, c, causal)
            outs["g1"] = fg.flash_gau_backward(*a1, dO1, c, causal)
        with torch.cuda.stream(s2):
            outs["O2"] = fg.flash_gau_forward(*a2, c, not causal)
            outs["g2"] = fg.flash_gau_backward(*a2, dO2, c, not causal)
        torch.cuda.synchronize()
        assert torch.equal(_bits(outs["O1"]), _bits(O1)), rep
        assert torch.equal(_bits(outs["O2"]), _bits(O2)), rep
        for k in fg.GRAD_NAMES:
            assert torch.equal(_bits(outs["g1"][k]), _bits(g1[k])), (rep, k)
            assert torch.equal(_bits(outs["g2"][k]), _bits(g2[k])), (rep, k)
