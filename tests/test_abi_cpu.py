"""C-ABI checks that need no GPU: the library loads, exports what include/flashgau.h declares,
sizes its workspace as documented, and rejects every invalid call on the host before any launch.

Every flash_gau_forward call here is built to fail one validation rule, so no kernel is ever
launched (the addresses passed are never dereferenced). Those calls pass fake device addresses;
where a GPU is visible they are skipped, so that a regression in the host-side validation can
never launch a kernel on unmapped addresses.
"""

import ctypes
import os
import re

import pytest

from efficient_transformer_attention_amd import flashgau as fg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashgau.h")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover - torch missing
        return False


GPU_VISIBLE = _gpu_visible()


def _fake_addresses_allowed():
    if GPU_VISIBLE:
        pytest.skip("fake device addresses are only passed to the library where no GPU is visible")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*|size_t)\s+(\w+)\s*\(", text, re.M)))


def test_header_declares_the_documented_entry_points():
    assert _declared_functions() == sorted(fg.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(fg.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_workspace_enum_matches_binding():
    text = open(HEADER).read()
    names = re.findall(r"FLASHGAU_WS_(\w+)\s*(?:=\s*0)?,", text)
    assert tuple(names) == fg.WS_NAMES


def _expected_layout(B, n, d, e, s, c, causal, esz, ng):
    G = n // c
    M = B * n
    counts = [(2 * e + s) * d, d * e, M * e, M * s, M * s, M * s, M * s, M * c,
              (B * G if causal else B) * e * s, M * e, B * ng * e * s]
    off, offs = 0, []
    for cnt in counts:
        offs.append(off)
        off += (cnt * esz + 255) // 256 * 256
    return offs, off


@pytest.mark.parametrize("args,ng,gs", [
    ((8, 256, 64, 1536, 16, 8, True, fg.BF16), 16, 2),       # two chunks per group
    ((8, 256, 64, 1536, 16, 8, False, fg.BF16), 16, 2),
    ((128, 64, 32, 2048, 128, 16, True, fg.BF16), 1, 4),     # one group per sequence
    ((128, 64, 32, 2048, 128, 16, False, fg.BF16), 1, 4),
    ((128, 64, 32, 2048, 128, 16, True, fg.F32), 1, 4),
    ((8, 4096, 768, 1536, 128, 256, True, fg.BF16), 16, 1),  # one chunk per group
])
def test_state_groups_cover_every_carry_branch(args, ng, gs):
    """The GPU parity cases with these shapes reach each branch of the carry walk: the chunk
    grouping is ceil(2048 / (B * state tiles)) groups, at most one per chunk."""
    B, n, d, e, s, c, causal, dt = args
    G = n // c
    got = fg.state_groups(*args)
    assert got == ng
    assert -(-G // got) == gs


@pytest.mark.parametrize("name,args", [
    ("c1", (1, 512, 256, 512, 128, 128, False, fg.F32)),
    ("c3", (8, 4096, 768, 1536, 128, 256, True, fg.BF16)),
    ("c4nc", (2, 8192, 768, 1536, 128, 512, False, fg.BF16)),
    ("c5", (1, 32768, 1024, 2048, 128, 512, True, fg.BF16)),
    ("ragged", (3, 72, 200, 136, 24, 24, True, fg.BF16)),
])
def test_workspace_size_and_offsets(name, args):
    B, n, d, e, s, c, causal, dt = args
    esz = 2 if dt == fg.BF16 else 4
    ng = fg.state_groups(*args)
    G = n // c
    assert 1 <= ng <= G
    gs = -(-G // ng)
    assert -(-G // gs) == ng  # every group non-empty
    offs, total = _expected_layout(B, n, d, e, s, c, causal, esz, ng)
    assert fg.workspace_size(*args) == total
    got = fg.workspace_offsets(*args)
    assert [got[k] for k in fg.WS_NAMES] == offs
    assert all(o % 256 == 0 for o in offs)


def test_empty_problem_needs_no_workspace_and_succeeds_without_pointers():
    assert fg.workspace_size(0, 256, 64, 128, 128, 64, True, fg.BF16) == 0
    assert fg.workspace_size(4, 0, 64, 128, 128, 64, True, fg.BF16) == 0
    rc = fg.forward_raw(None, None, None, None, None, None, None, 64, 1, 0, 256, 64, 128, 128,
                        fg.BF16, None, None, 0, None)
    assert rc == fg.OK


@pytest.mark.parametrize("shape,code", [
    ((2, 100, 64, 128, 128, 64), fg.ERR_BAD_SHAPE),   # n % chunk != 0
    ((-1, 128, 64, 128, 128, 64), fg.ERR_BAD_SHAPE),  # negative batch
    ((1, 128, 64, 128, 128, 0), fg.ERR_BAD_SHAPE),    # chunk 0
    ((1, 128, 0, 128, 128, 64), fg.ERR_BAD_SHAPE),    # d 0
    ((1, 128, 60, 128, 128, 64), fg.ERR_UNSUPPORTED),  # d not a multiple of 8
    ((1, 120, 64, 128, 128, 12), fg.ERR_UNSUPPORTED),  # chunk not a multiple of 8
    ((1, 128, 64, 100, 128, 64), fg.ERR_UNSUPPORTED),  # e not a multiple of 8
    ((1, 1 << 31, 64, 128, 128, 64), fg.ERR_BAD_SHAPE),  # B*n beyond int32
])
def test_shape_validation(shape, code):
    with pytest.raises(fg.FlashGauError) as ei:
        fg.workspace_size(*shape, True, fg.BF16)
    assert ei.value.code == code


def test_unknown_dtype():
    with pytest.raises(fg.FlashGauError) as ei:
        fg.workspace_size(1, 128, 64, 128, 128, 64, True, 7)
    assert ei.value.code == fg.ERR_UNSUPPORTED


# Fake, well-separated, 256-aligned addresses: never dereferenced because every call below fails
# one host-side rule.
SHAPE = dict(B=1, n=128, d=64, e=128, s=128, chunk=64)


def _call(**over):
    _fake_addresses_allowed()
    B, n, d, e, s, c = (SHAPE[k] for k in ("B", "n", "d", "e", "s", "chunk"))
    ws = fg.workspace_size(B, n, d, e, s, c, True, fg.BF16)
    base = 1 << 40
    ptrs = dict(X=base, W_u=base + (1 << 30), W_v=base + (2 << 30), W_z=base + (3 << 30),
                gamma=base + (4 << 30), beta=base + (5 << 30), W_o=base + (6 << 30),
                O=base + (7 << 30), workspace=base + (8 << 30), workspace_bytes=ws)
    ptrs.update(over)
    return fg.forward_raw(ptrs["X"], ptrs["W_u"], ptrs["W_v"], ptrs["W_z"], ptrs["gamma"],
                          ptrs["beta"], ptrs["W_o"], c, 1, B, n, d, e, s, fg.BF16, ptrs["O"],
                          ptrs["workspace"], ptrs["workspace_bytes"], None)


@pytest.mark.parametrize("which", ["X", "W_u", "W_v", "W_z", "gamma", "beta", "W_o", "O", "workspace"])
def test_null_pointer_rejected(which):
    assert _call(**{which: None}) == fg.ERR_NULL_PTR


@pytest.mark.parametrize("which,delta", [("X", 8), ("W_o", 2), ("O", 4), ("workspace", 8), ("gamma", 2)])
def test_misaligned_pointer_rejected(which, delta):
    base = {"X": 1 << 40, "W_o": (1 << 40) + (6 << 30), "O": (1 << 40) + (7 << 30),
            "workspace": (1 << 40) + (8 << 30), "gamma": (1 << 40) + (4 << 30)}[which]
    assert _call(**{which: base + delta}) == fg.ERR_MISALIGNED


def test_small_workspace_rejected():
    assert _call(workspace_bytes=1024) == fg.ERR_WORKSPACE


@pytest.mark.parametrize("over", [
    dict(O=1 << 40),                                  # O is X
    dict(O=(1 << 40) + 256),                           # O starts inside X
    dict(workspace=(1 << 40) + (6 << 30)),             # workspace is W_o
    dict(O=(1 << 40) + (8 << 30) + 4096),              # O inside the workspace
    dict(workspace=(1 << 40) + (4 << 30)),             # workspace over gamma
])
def test_aliasing_rejected(over):
    assert _call(**over) == fg.ERR_ALIASING


def test_strerror_covers_every_code():
    texts = {c: fg.strerror(c) for c in range(-8, 1)}
    assert len(set(texts.values())) == 9
    assert fg.strerror(-99) == "unknown error"


# ------------------------------------------------------------------------------ decoding

def test_decode_state_enum_matches_binding():
    text = open(HEADER).read()
    names = re.findall(r"FLASHGAU_DS_(\w+)\s*(?:=\s*0)?,", text)
    assert tuple(names) == fg.DS_NAMES


@pytest.mark.parametrize("B,d,e,s,c,dt", [(8, 768, 1536, 128, 256, fg.BF16), (3, 64, 136, 24, 8, fg.F32),
                                          (17, 40, 88, 16, 4, fg.BF16), (0, 64, 64, 8, 1, fg.BF16)])
def test_decode_state_layout(B, d, e, s, c, dt):
    esz = 2 if dt == fg.BF16 else 4
    sizes = [B * s * e * 4, B * c * s * esz, B * c * s * esz, B * c * e * esz, B * e * esz,
             B * s * esz, B * s * esz, B * e * esz]
    off, offs = 0, []
    for nbytes in sizes:
        offs.append(off)
        off += (nbytes + 255) // 256 * 256
    assert fg.decode_state_size(B, d, e, s, c, dt) == off
    got = fg.decode_state_offsets(B, d, e, s, c, dt)
    assert [got[k] for k in fg.DS_NAMES] == offs


def test_packed_weights_layout_matches_forward_workspace():
    # the packed weights are the first two buffers of the forward's workspace
    d, e, s = 200, 136, 24
    for dt, esz in ((fg.BF16, 2), (fg.F32, 4)):
        wcat = ((2 * e + s) * d * esz + 255) // 256 * 256
        assert fg.packed_weights_size(d, e, s, dt) == wcat + (d * e * esz + 255) // 256 * 256
        ws = fg.workspace_offsets(2, 216, d, e, s, 72, True, dt)
        assert ws["WCAT_T"] == 0 and ws["WO_T"] == wcat


@pytest.mark.parametrize("args,code", [
    ((2, 64, 100, 24, 8), fg.ERR_UNSUPPORTED),   # e not a multiple of 8
    ((2, 60, 96, 24, 8), fg.ERR_UNSUPPORTED),    # d not a multiple of 8
    ((2, 64, 96, 24, 0), fg.ERR_BAD_SHAPE),      # chunk 0
    ((-1, 64, 96, 24, 8), fg.ERR_BAD_SHAPE),     # negative batch
    ((2, 64, 96, 4096, 64), fg.ERR_UNSUPPORTED),  # chunk + 2 s beyond the attention kernel's LDS
])
def test_decode_shape_validation(args, code):
    with pytest.raises(fg.FlashGauError) as ei:
        fg.decode_state_size(*args, fg.BF16)
    assert ei.value.code == code


DEC = dict(B=2, d=64, e=96, s=24, c=8)


def _dcall(t=3, n=16, **over):
    _fake_addresses_allowed()
    B, d, e, s, c = (DEC[k] for k in ("B", "d", "e", "s", "c"))
    st = fg.decode_state_size(B, d, e, s, c, fg.BF16)
    pk = fg.packed_weights_size(d, e, s, fg.BF16)
    base = 1 << 40
    ptrs = dict(x=base, packed=base + (1 << 30), gamma=base + (2 << 30), beta=base + (3 << 30),
                o=base + (4 << 30), state=base + (5 << 30), packed_bytes=pk, state_bytes=st)
    ptrs.update(over)
    return fg.decode_step_raw(ptrs["x"], ptrs["packed"], ptrs["packed_bytes"], ptrs["gamma"],
                              ptrs["beta"], c, t, n, ptrs.get("rope_base", 0.0), B, d, e, s, fg.BF16,
                              ptrs["o"], ptrs["state"], ptrs["state_bytes"], None)


@pytest.mark.parametrize("t,n", [(16, 16), (-1, 16), (0, 0), (20, 16)])
def test_decode_position_must_lie_in_the_sequence(t, n):
    assert _dcall(t=t, n=n) == fg.ERR_BAD_SHAPE


@pytest.mark.parametrize("which", ["x", "packed", "gamma", "beta", "o", "state"])
def test_decode_null_pointer_rejected(which):
    assert _dcall(**{which: None}) == fg.ERR_NULL_PTR


@pytest.mark.parametrize("which", ["x", "packed", "o", "state"])
def test_decode_misaligned_pointer_rejected(which):
    base = {"x": 1 << 40, "packed": (1 << 40) + (1 << 30), "o": (1 << 40) + (4 << 30),
            "state": (1 << 40) + (5 << 30)}[which]
    assert _dcall(**{which: base + 8}) == fg.ERR_MISALIGNED


def test_decode_small_buffers_rejected():
    assert _dcall(state_bytes=256) == fg.ERR_WORKSPACE
    assert _dcall(packed_bytes=256) == fg.ERR_WORKSPACE


@pytest.mark.parametrize("over", [
    dict(o=1 << 40),                            # o is x
    dict(state=(1 << 40) + (1 << 30) + 512),     # state inside the packed weights
    dict(o=(1 << 40) + (5 << 30) + 1024),        # o inside the state
    dict(state=(1 << 40) + (2 << 30)),           # state over gamma
])
def test_decode_aliasing_rejected(over):
    assert _dcall(**over) == fg.ERR_ALIASING


def test_decode_empty_batch_succeeds_without_pointers():
    rc = fg.decode_step_raw(None, None, 0, None, None, 8, 0, 16, 0.0, 0, 64, 96, 24, fg.BF16, None, None, 0,
                            None)
    assert rc == fg.OK


def test_pack_weights_validation():
    _fake_addresses_allowed()
    base = 1 << 40
    pk = fg.packed_weights_size(64, 96, 24, fg.BF16)
    w = [base, base + (1 << 30), base + (2 << 30), base + (3 << 30)]
    assert fg.pack_weights_raw(*w, 64, 96, 24, fg.BF16, None, pk, None) == fg.ERR_NULL_PTR
    assert fg.pack_weights_raw(*w, 64, 96, 24, fg.BF16, base + (4 << 30), 256, None) == fg.ERR_WORKSPACE
    assert fg.pack_weights_raw(*w, 64, 96, 24, fg.BF16, base + 8 + (4 << 30), pk, None) == fg.ERR_MISALIGNED
    assert fg.pack_weights_raw(*w, 64, 96, 24, fg.BF16, base + 256, pk, None) == fg.ERR_ALIASING
    assert fg.pack_weights_raw(*w, 64, 100, 24, fg.BF16, base + (4 << 30), pk, None) == fg.ERR_UNSUPPORTED


@pytest.mark.parametrize("base", [-1.0, float("nan"), float("inf")])
def test_decode_rotary_base_validated(base):
    assert _dcall(rope_base=base) == fg.ERR_BAD_SHAPE


@pytest.mark.parametrize("base", [0.0, -5.0, float("nan"), float("inf")])
def test_forward_rope_base_validated(base):
    _fake_addresses_allowed()
    base_ptr = 1 << 40
    B, n, d, e, s, c = 1, 128, 64, 128, 128, 64
    ws = fg.workspace_size(B, n, d, e, s, c, True, fg.BF16)
    rc = fg.forward_rope_raw(base_ptr, base_ptr + (1 << 30), base_ptr + (2 << 30), base_ptr + (3 << 30),
                             base_ptr + (4 << 30), base_ptr + (5 << 30), base_ptr + (6 << 30), c, 1, base,
                             B, n, d, e, s, fg.BF16, base_ptr + (7 << 30), base_ptr + (8 << 30), ws, None)
    assert rc == fg.ERR_BAD_SHAPE


# ----------------------------------------------------------------------------------- backward

def test_backward_workspace_holds_the_forward_layout_first():
    for args in ((1, 128, 64, 128, 128, 64, True, fg.BF16), (2, 216, 200, 136, 24, 72, False, fg.F32),
                 (8, 4096, 768, 1536, 128, 256, True, fg.BF16)):
        fwd = fg.workspace_size(*args)
        bwd = fg.backward_workspace_size(*args)
        assert bwd > fwd
        assert bwd % 256 == 0
    assert fg.backward_workspace_size(0, 128, 64, 128, 128, 64, True, fg.BF16) == 0


def test_backward_split_plan_is_quick_and_stable():
    # The backward splits its weight-gradient sums into token ranges chosen on the host (a replay
    # of the launch's tile schedule per candidate count). For any shape the choice must come back
    # quickly, hold at least one fp32 copy of the weight gradients, and be the same when asked
    # again (the second answer comes from the library's per-shape cache).
    import random
    import time
    rng = random.Random(0)
    seen = 0
    for _ in range(80):
        c = 8 * rng.randint(1, 64)
        n = c * rng.randint(1, 64)
        B = rng.randint(1, 16)
        d, e, s = (8 * rng.randint(1, 256) for _ in range(3))
        dt = rng.choice([fg.BF16, fg.F32])
        causal = rng.random() < 0.5
        t0 = time.perf_counter()
        try:
            bwd = fg.backward_workspace_size(B, n, d, e, s, c, causal, dt)
        except fg.FlashGauError:
            continue
        assert time.perf_counter() - t0 < 0.25
        seen += 1
        fwd = fg.workspace_size(B, n, d, e, s, c, causal, dt)
        assert bwd >= fwd + 4 * (3 * d * e + d * s)
        assert fg.backward_workspace_size(B, n, d, e, s, c, causal, dt) == bwd
    assert seen >= 60


@pytest.mark.parametrize("shape,code", [
    ((1, 100, 64, 128, 128, 64), fg.ERR_BAD_SHAPE),   # chunk does not divide n
    ((1, 128, 60, 128, 128, 64), fg.ERR_UNSUPPORTED),  # d not a multiple of 8
    ((1, 128, 64, 128, 128, 0), fg.ERR_BAD_SHAPE),     # chunk 0
    ((-1, 128, 64, 128, 128, 64), fg.ERR_BAD_SHAPE),
])
def test_backward_shape_validation(shape, code):
    with pytest.raises(fg.FlashGauError) as ei:
        fg.backward_workspace_size(*shape, True, fg.BF16)
    assert ei.value.code == code


def _bcall(**over):
    _fake_addresses_allowed()
    B, n, d, e, s, c = (SHAPE[k] for k in ("B", "n", "d", "e", "s", "chunk"))
    ws = fg.backward_workspace_size(B, n, d, e, s, c, True, fg.BF16)
    base = 1 << 40
    names = ("X", "W_u", "W_v", "W_z", "gamma", "beta", "W_o", "dO", "dX", "dW_u", "dW_v", "dW_z",
             "dgamma", "dbeta", "dW_o", "workspace")
    ptrs = {k: base + (i << 30) for i, k in enumerate(names)}
    ptrs["workspace_bytes"] = ws
    ptrs["rope_base"] = 0.0
    ptrs.update(over)
    return fg.backward_raw(*(ptrs[k] for k in names[:8]), c, 1, ptrs["rope_base"], B, n, d, e, s,
                           fg.BF16, *(ptrs[k] for k in names[8:15]), ptrs["workspace"],
                           ptrs["workspace_bytes"], None)


@pytest.mark.parametrize("which", ["X", "W_u", "W_v", "W_z", "gamma", "beta", "W_o", "dO", "dX",
                                   "dW_u", "dW_v", "dW_z", "dgamma", "dbeta", "dW_o", "workspace"])
def test_backward_null_pointer_rejected(which):
    assert _bcall(**{which: None}) == fg.ERR_NULL_PTR


@pytest.mark.parametrize("which,delta", [("X", 8), ("dO", 2), ("dX", 4), ("dW_o", 8),
                                         ("dgamma", 2), ("workspace", 8)])
def test_backward_misaligned_pointer_rejected(which, delta):
    names = ("X", "W_u", "W_v", "W_z", "gamma", "beta", "W_o", "dO", "dX", "dW_u", "dW_v", "dW_z",
             "dgamma", "dbeta", "dW_o", "workspace")
    assert _bcall(**{which: (1 << 40) + (names.index(which) << 30) + delta}) == fg.ERR_MISALIGNED


def test_backward_small_workspace_rejected():
    assert _bcall(workspace_bytes=4096) == fg.ERR_WORKSPACE


@pytest.mark.parametrize("over", [
    dict(dX=1 << 40),                                   # dX is X
    dict(dW_u=(1 << 40) + (10 << 30)),                   # dW_u is dW_v
    dict(workspace=(1 << 40) + (7 << 30)),               # workspace is dO
    dict(dgamma=(1 << 40) + (15 << 30) + 4096),          # dgamma inside the workspace
    dict(dbeta=(1 << 40) + (12 << 30)),                  # dbeta is dgamma
])
def test_backward_aliasing_rejected(over):
    assert _bcall(**over) == fg.ERR_ALIASING


@pytest.mark.parametrize("base", [-1.0, float("nan"), float("inf")])
def test_backward_rope_base_validated(base):
    assert _bcall(rope_base=base) == fg.ERR_BAD_SHAPE


def test_backward_rejects_shapes_beyond_its_descriptor_ranges():
    # a chunk's value block read as one operand (e x chunk elements) must stay under 4 GiB
    with pytest.raises(fg.FlashGauError) as ei:
        fg.backward_workspace_size(1, 32768, 64, 65536, 128, 32768, True, fg.BF16)
    assert ei.value.code == fg.ERR_BAD_SHAPE
    # the same widths with a short chunk are fine
    assert fg.backward_workspace_size(1, 1024, 64, 1024, 128, 256, True, fg.BF16) > 0


def _tcall(**over):
    _fake_addresses_allowed()
    B, n, d, e, s, c = (SHAPE[k] for k in ("B", "n", "d", "e", "s", "chunk"))
    ws = fg.backward_workspace_size(B, n, d, e, s, c, True, fg.BF16)
    base = 1 << 40
    names = ("X", "W_u", "W_v", "W_z", "gamma", "beta", "W_o", "O", "workspace")
    ptrs = {k: base + (i << 30) for i, k in enumerate(names)}
    ptrs["workspace_bytes"] = ws
    ptrs["rope_base"] = 0.0
    ptrs.update(over)
    return fg.forward_train_raw(*(ptrs[k] for k in names[:7]), c, 1, ptrs["rope_base"], B, n, d, e, s,
                                fg.BF16, ptrs["O"], ptrs["workspace"], ptrs["workspace_bytes"], None)


@pytest.mark.parametrize("which", ["X", "W_u", "W_v", "W_z", "gamma", "beta", "W_o", "O", "workspace"])
def test_forward_train_null_pointer_rejected(which):
    assert _tcall(**{which: None}) == fg.ERR_NULL_PTR


def test_forward_train_needs_the_backward_workspace():
    fwd = fg.workspace_size(1, 128, 64, 128, 128, 64, True, fg.BF16)
    assert _tcall(workspace_bytes=fwd) == fg.ERR_WORKSPACE


@pytest.mark.parametrize("over,code", [
    (dict(O=(1 << 40) + 4), fg.ERR_MISALIGNED),
    (dict(O=1 << 40), fg.ERR_ALIASING),                       # O is X
    (dict(workspace=(1 << 40) + (6 << 30)), fg.ERR_ALIASING),  # workspace is W_o
    (dict(rope_base=-1.0), fg.ERR_BAD_SHAPE),
])
def test_forward_train_validation(over, code):
    assert _tcall(**over) == code


def test_backward_saved_validates_like_the_backward():
    _fake_addresses_allowed()
    B, n, d, e, s, c = (SHAPE[k] for k in ("B", "n", "d", "e", "s", "chunk"))
    ws = fg.backward_workspace_size(B, n, d, e, s, c, True, fg.BF16)
    base = 1 << 40
    ptrs = [base + (i << 30) for i in range(16)]
    args = lambda p, wsb: (*p[:8], c, 1, 0.0, B, n, d, e, s, fg.BF16, *p[8:15], p[15], wsb, None)
    assert fg.backward_saved_raw(*args(ptrs, 1024)) == fg.ERR_WORKSPACE
    bad = list(ptrs)
    bad[7] = None  # dO
    assert fg.backward_saved_raw(*args(bad, ws)) == fg.ERR_NULL_PTR
    bad = list(ptrs)
    bad[8] = ptrs[0]  # dX is X
    assert fg.backward_saved_raw(*args(bad, ws)) == fg.ERR_ALIASING


def test_workspace_bytes_returns_the_size_or_zero():
    for args in ((8, 4096, 768, 1536, 128, 256, True, fg.BF16), (1, 512, 256, 512, 128, 128, False, fg.F32),
                 (3, 72, 200, 136, 24, 24, True, fg.BF16)):
        assert fg.workspace_bytes(*args) == fg.workspace_size(*args) > 0
    assert fg.workspace_bytes(0, 256, 64, 128, 128, 64, True, fg.BF16) == 0   # empty
    assert fg.workspace_bytes(2, 100, 64, 128, 128, 64, True, fg.BF16) == 0   # n % chunk
    assert fg.workspace_bytes(1, 128, 60, 128, 128, 64, True, fg.BF16) == 0   # d % 8
    assert fg.workspace_bytes(1, 128, 64, 128, 128, 64, True, 7) == 0          # dtype


def test_noalloc_rejects_problems_beyond_its_scratch():
    # the size check precedes any HIP call, so it needs no device; the addresses are never used
    _fake_addresses_allowed()
    assert fg.noalloc_scratch_bytes() == 64 << 20
    args = (8, 4096, 768, 1536, 128, 256, True, fg.BF16)
    assert fg.workspace_bytes(*args) > fg.noalloc_scratch_bytes()
    base = 1 << 40
    rc = fg.forward_noalloc_raw(*(base + (i << 30) for i in range(7)), 256, 1, 8, 4096, 768, 1536,
                                128, fg.BF16, base + (7 << 30), None)
    assert rc == fg.ERR_TOO_LARGE
    # an empty problem succeeds without touching the device
    assert fg.forward_noalloc_raw(None, None, None, None, None, None, None, 64, 1, 0, 256, 64, 128,
                                  128, fg.BF16, None, None) == fg.OK


def test_score_buffer_limit():
    # chunk = n keeps n*n scores per sequence: 2^33 elements is the most the forward materialises
    assert fg.workspace_size(1, 65536, 64, 128, 128, 65536, True, fg.BF16) > 2 * 65536 ** 2
    with pytest.raises(fg.FlashGauError) as ei:
        fg.workspace_size(1, 131072, 64, 128, 128, 131072, True, fg.BF16)
    assert ei.value.code == fg.ERR_UNSUPPORTED
    assert "score buffer" in fg.strerror(fg.ERR_UNSUPPORTED)
    # the same sequence in chunks of 512 is fine
    assert fg.workspace_size(1, 131072, 64, 128, 128, 512, True, fg.BF16) > 0
