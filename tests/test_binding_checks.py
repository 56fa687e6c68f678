"""The Python binding rejects malformed tensors before the library sees a pointer.

The C ABI receives raw addresses and cannot know the sizes of the buffers behind them, so the
binding checks shapes, dtypes, devices and layout first. The library's entry points are replaced
by functions that fail the test if they are reached: a check that lets a bad tensor through shows
up as that failure instead of an out-of-bounds write on the GPU.
"""

import pytest
import torch

from efficient_transformer_attention_amd import flashgau as fg

B, n, d, e, s, c = 2, 64, 32, 48, 16, 16


def _inputs(device="cpu", dtype=torch.bfloat16):
    X = torch.zeros((B, n, d), dtype=dtype, device=device)
    W_u = torch.zeros((d, e), dtype=dtype, device=device)
    W_v = torch.zeros((d, e), dtype=dtype, device=device)
    W_z = torch.zeros((d, s), dtype=dtype, device=device)
    g = torch.ones((4, s), dtype=torch.float32, device=device)
    b = torch.zeros((4, s), dtype=torch.float32, device=device)
    W_o = torch.zeros((e, d), dtype=dtype, device=device)
    return [X, W_u, W_v, W_z, g, b, W_o]


@pytest.fixture
def no_launch(monkeypatch):
    def boom(*a, **k):
        raise AssertionError("the library's entry point was reached")
    for name in ("forward_raw", "forward_rope_raw", "forward_train_raw", "backward_raw",
                 "backward_saved_raw", "decode_step_raw"):
        monkeypatch.setattr(fg, name, boom)


@pytest.mark.parametrize("slot,shape", [(1, (d, e + 8)), (2, (d + 8, e)), (3, (d, s + 8)),
                                        (6, (e, d + 8)), (4, (3, s))])
def test_forward_rejects_misshapen_weights(no_launch, slot, shape):
    args = _inputs()
    args[slot] = torch.zeros(shape, dtype=args[slot].dtype)
    with pytest.raises(ValueError):
        fg.flash_gau_forward(*args, c, True)


def test_forward_rejects_mixed_dtypes(no_launch):
    args = _inputs()
    args[2] = args[2].float()
    with pytest.raises(TypeError):
        fg.flash_gau_forward(*args, c, True)


def test_forward_rejects_cpu_tensors(no_launch):
    with pytest.raises(ValueError, match="same GPU"):
        fg.flash_gau_forward(*_inputs(), c, True)


@pytest.mark.parametrize("slot,shape", [(1, (d, e + 8)), (6, (e + 8, d))])
def test_forward_train_checks_its_weights(no_launch, slot, shape):
    args = _inputs()
    args[slot] = torch.zeros(shape, dtype=args[slot].dtype)
    ws = torch.empty(1, dtype=torch.uint8)
    with pytest.raises(ValueError):
        fg.flash_gau_forward_train(*args, c, True, ws)


def test_backward_checks_dO_shape(no_launch):
    args = _inputs()
    dO = torch.zeros((B, n, d + 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fg.flash_gau_backward(*args, dO, c, True)


# ---------------------------------------------------------------- output and workspace buffers

def _gpu_inputs():
    return _inputs(device="cuda")


@pytest.mark.gpu
@pytest.mark.parametrize("bad", ["shape", "dtype", "layout", "device"])
def test_forward_checks_out(no_launch, bad):
    args = _gpu_inputs()
    out = {"shape": torch.empty((B, n, d + 8), dtype=torch.bfloat16, device="cuda"),
           "dtype": torch.empty((B, n, d), dtype=torch.float32, device="cuda"),
           "layout": torch.empty((B, d, n), dtype=torch.bfloat16, device="cuda").transpose(1, 2),
           "device": torch.empty((B, n, d), dtype=torch.bfloat16)}[bad]
    with pytest.raises((ValueError, TypeError)):
        fg.flash_gau_forward(*args, c, True, out=out)


@pytest.mark.gpu
@pytest.mark.parametrize("bad", ["small", "dtype", "device"])
def test_forward_checks_workspace(no_launch, bad):
    args = _gpu_inputs()
    nbytes = fg.workspace_size(B, n, d, e, s, c, True, fg.BF16)
    ws = {"small": torch.empty(nbytes - 256, dtype=torch.uint8, device="cuda"),
          "dtype": torch.empty(nbytes, dtype=torch.float32, device="cuda"),
          "device": torch.empty(nbytes, dtype=torch.uint8)}[bad]
    with pytest.raises((ValueError, TypeError)):
        fg.flash_gau_forward(*args, c, True, workspace=ws)


@pytest.mark.gpu
def test_backward_checks_gradient_buffers(no_launch):
    args = _gpu_inputs()
    dO = torch.zeros((B, n, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fg.flash_gau_backward(*args, dO, c, True,
                              out={"dW_u": torch.empty((d, e - 8), dtype=torch.bfloat16, device="cuda")})
    with pytest.raises(TypeError):
        fg.flash_gau_backward(*args, dO, c, True,
                              out={"dgamma": torch.empty((4, s), dtype=torch.bfloat16, device="cuda")})
    with pytest.raises(ValueError):
        fg.flash_gau_backward(*args, dO, c, True, out={"dZ": torch.empty(1, device="cuda")})


@pytest.mark.gpu
def test_decode_checks_out(no_launch):
    args = _gpu_inputs()
    packed = torch.empty(fg.packed_weights_size(d, e, s, fg.BF16), dtype=torch.uint8, device="cuda")
    st = fg.DecodeState(B, d, e, s, c, torch.bfloat16, torch.device("cuda"))
    x = torch.zeros((B, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fg.flash_gau_decode_step(x, packed, args[4], args[5], c, 0, n, st,
                                 out=torch.empty((B, d + 8), dtype=torch.bfloat16, device="cuda"))
