#!/usr/bin/env python3
"""Benchmark of one FLASH layer forward on one MI355X (the HIP library through its C ABI).

Default workload: causal, bf16 storage with fp32 accumulation, B = 8, n = 4096, d = 768,
e = 1536, s = 128, chunk 256, seeded synthetic inputs (X ~ N(0,1), weights ~ N(0, 1/fan_in),
gamma ~ N(1, 0.02), beta = 0). A step is one full forward call: all seven kernels (pack, proj,
scores, states, carry, mix, out) over the whole batch, with inputs already resident in HBM.

Prints one JSON line. Before anything is timed, forward calls run untimed for --settle-ms (the
host has just spent seconds generating inputs with the GPU idle, and the first calls after that
run on clocks that are still ramping; `settle_ms` in the line records it), then --warmup untimed
calls. `value` is tokens/s = B*n / (wall time of one step), timed over exactly --steps calls
between two device synchronisations, with nothing else on the stream. Two separate passes follow
outside the timed region: calls that launch every kernel with its own start and stop HIP events
on the library's stream (per-kernel durations; the roofline object reports the kernel that takes
the longest), and
at least 50 calls each bracketed by two events (`step_ms_quantiles`). The CPU baseline is the fp64 oracle timed on the
host on one sequence of the same batch; its output also checks the GPU's on that sequence.

`configs` holds one row per workload of inputs.WORKLOADS (the eight configurations, the headline
among them): the same measurement with shorter settle and step counts, tokens/s, fraction of the
dtype's dense matrix peak, the dominant kernel with its roofline fraction, and the max relative
error of one sampled sequence (the batch's last) against the fp64 oracle.

For a causal workload the line also carries a "decode" object: the same batch and dimensions
decoded one token per sequence per step (flash_gau_decode_step), timed over one whole chunk of
positions (c .. 2c-1, the last step folding the chunk into the state) after chunk 0 has filled the
state untimed, with its HBM roofline (algorithmic bytes per step, see decode_bytes) and the
oracle's decode step timed on the host. The "backward" object times flash_gau_backward on the same
batch (2 x the forward's algorithmic FLOPs), with the oracle's backward on one sequence as its CPU
baseline and parity check, and (saved_activations) a training step that keeps the forward's
intermediates: flash_gau_forward_train, then flash_gau_backward_saved. Two more objects time the same layer with the rotary
embedding (flash_gau_forward_rope) and compare FLASH-Quad (chunk = n: one quadratic chunk, no
global term) with FLASH (the workload's chunk) on longer causal sequences of the same width.
"""

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/sec per FLASH layer fwd (n=4096 causal bf16); % bf16 MFMA peak"
PEAK = {"bf16": 2500.0, "f32": 157.3}  # dense matrix-core TFLOP/s of MI355X
HBM_PEAK = 8000.0  # GB/s


def alg_flops(B, n, d, e, s, c, causal):
    """Algorithmic FLOPs of one layer forward, split by kernel (multiply-add = 2)."""
    N = B * n
    proj = 2 * N * d * (e + s)  # V and the heads; the gate's GEMM runs in the mix kernel
    gate = 2 * N * d * e
    if causal:
        # query i of a chunk sees i+1 keys: scores and P·V over (c+1)/2 keys on average
        scores = N * (c + 1) * s
        pv = N * (c + 1) * e
        n_state = N - B * c  # the last chunk's summary and the first chunk's read-out are unused
    else:
        scores = 2 * N * c * s
        pv = 2 * N * c * e
        n_state = N
    states = 2 * n_state * s * e
    readout = 2 * n_state * s * e
    out = 2 * N * e * d
    return {"pack": 0, "proj": proj, "scores_states": scores + states, "carry": 0,
            "mix": gate + pv + readout, "out": out}


def state_branch(B, n, c, causal, ng):
    """Which code path the cross-chunk sum takes (ng: chunk groups per sequence of the states
    stage, as flashgau_state_groups reports): "none" (causal with one chunk: no global term),
    "one_group" (the states stage walks every chunk of a sequence and writes the states itself,
    no carry launch), "chunk_per_group" (causal, one chunk per group: the states stage writes chunk
    totals, the carry stage writes every state), "groups" (causal, several chunks per group: the
    states stage writes in-group prefixes and group totals, the carry stage adds earlier groups'
    totals in place), "noncausal_groups" (group totals summed by the carry stage)."""
    G = n // c
    if causal and G == 1:
        return "none"
    if ng == 1:
        return "one_group"
    if not causal:
        return "noncausal_groups"
    gs = -(-G // ng)
    return "chunk_per_group" if gs == 1 else "groups"


def alg_bytes(B, n, d, e, s, c, causal, esz, ng):
    """Bytes each kernel must move at least once between HBM and the chip, for the code path the
    problem takes (ng: chunk groups per sequence of the states stage; see state_branch). A causal
    sequence's last chunk feeds no state, so its K_lin and V are not read by the states stage; chunk
    0's state is zero and the mix stage does not need it."""
    N = B * n
    G = n // c
    gs = -(-G // ng)
    es = e * s
    branch = state_branch(B, n, c, causal, ng)
    pc = (c * (c + 1) // 2) if causal else c * c  # P entries written by scores, read by mix, per chunk
    if branch == "none":
        st_in = st_out = carry = mix_lin = 0
    else:
        if causal:
            st_in = (N - B * c) * (e + s)       # every chunk but the last of each sequence
            mix_lin = (N - B * c) * s + B * (G - 1) * es  # Q_lin and the states of chunks 1..G-1
        else:
            st_in = N * (e + s)
            mix_lin = N * s + B * es
        if branch == "one_group":
            st_out = B * G * es if causal else B * es
            carry = 0
        elif branch == "chunk_per_group":
            st_out = B * (G - 1) * es                  # totals of chunks 0..G-2
            carry = B * (G - 1) * es + B * G * es      # read them, write every chunk's state
        elif branch == "groups":
            st_out = B * G * es + B * (ng - 1) * es    # in-group prefixes + totals of groups 0..ng-2
            carry = B * (ng - 1) * es + 2 * B * (G - gs) * es  # totals read; later groups' states updated
        else:  # noncausal_groups
            st_out = B * ng * es
            carry = B * ng * es + B * es
    return {
        "pack": 2 * ((2 * e + s) * d + e * d) * esz,
        "proj": (N * d + (e + s) * d + N * (e + 4 * s)) * esz,
        "scores_states": (2 * N * s + B * G * pc + st_in + st_out) * esz,
        "carry": carry * esz,
        "mix": (N * e + B * G * pc + mix_lin + N * d + e * d + N * e) * esz,
        "out": (N * e + e * d + N * d) * esz,
    }


PROFILE_BYTES = os.path.join(ROOT, "profiles", "flash_layer_c3_hbm_bytes.txt")
# the forward's sources, hashed in this order
LIB_SOURCES = tuple(os.path.join(ROOT, "efficient_transformer_attention_amd", "csrc", f)
                    for f in ("flashgau.hip", "kernels.h", "common.h"))


def forward_source_sha():
    import hashlib
    h = hashlib.sha256()
    for f in LIB_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """Per-launch HBM-side bytes (FETCH_SIZE + WRITE_SIZE, copy-calibrated) of `kernel` from the
    committed rocprofv3 summary, or None when the summary is for another workload or the library
    source has changed since the counters were taken."""
    if workload != "c3_causal_bf16_n4096" or not os.path.exists(PROFILE_BYTES):
        return None
    sha = forward_source_sha()
    text = open(PROFILE_BYTES).read()
    if f"library source sha256: {sha}" not in text:
        return None
    for line in text.splitlines():
        parts = line.split()
        if parts and parts[0] == kernel and len(parts) == 6:
            return int(parts[5])
    return None


BOUND = {"pack": "hbm", "proj": "mfma", "scores_states": "hbm", "carry": "hbm", "mix": "mfma",
         "out": "mfma"}


class HipEvents:
    def __init__(self, count):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.handles = []
        for _ in range(count):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.handles.append(h.value)

    def ms(self, a, b):
        out = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return out.value

    def close(self):
        for h in self.handles:
            self.hip.hipEventDestroy(ctypes.c_void_p(h))


def cpu_baseline(inp, seconds):
    """Times the fp64 oracle on sequence 0 of the batch until `seconds` have passed (at least
    one run); returns the baseline record and the oracle output for that sequence."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    times = []
    ref = None
    t_start = time.perf_counter()
    while not times or time.perf_counter() - t_start < seconds:
        t0 = time.perf_counter()
        ref = oracle.flash_forward(inp.X[:1], inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta,
                                   inp.W_o, inp.chunk, inp.causal)
        times.append(time.perf_counter() - t0)
    n = inp.X.shape[1]
    med = statistics.median(times)
    rec = {"value": n / med, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"sequence 0 of {inp.X.shape[0]} ({n} tokens) of the same workload, "
                     f"fp64 NumPy oracle, median of {len(times)} runs ({med:.2f} s each); "
                     f"host has {os.cpu_count()} logical CPUs"}
    return rec, ref


def _train_pair(fg, torch, dev, args, dO, c, causal, ws, grads, steps, dtype):
    """A training step without the backward's recompute, timed with events around each half:
    flash_gau_forward_train, then flash_gau_backward_saved on its workspace (10 untimed pairs
    first). grads: the gradient tensors to write (flash_gau_backward's dict)."""
    B, n, d = args[0].shape
    e, s = args[1].shape[1], args[3].shape[1]
    O = torch.empty_like(args[0])
    for _ in range(10):
        fg.flash_gau_forward_train(*args, c, causal, ws, out=O)
        fg.flash_gau_backward(*args, dO, c, causal, workspace=ws, out=grads, saved=True)
    torch.cuda.synchronize(dev)
    t_f = t_b = 0.0
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    for _ in range(steps):
        e0.record()
        fg.flash_gau_forward_train(*args, c, causal, ws, out=O)
        e1.record()
        fg.flash_gau_backward(*args, dO, c, causal, workspace=ws, out=grads, saved=True)
        e2.record()
        torch.cuda.synchronize(dev)
        t_f += e0.elapsed_time(e1)
        t_b += e1.elapsed_time(e2)
    t_f, t_b = t_f / steps, t_b / steps
    step_flops = 3.0 * sum(alg_flops(B, n, d, e, s, c, causal).values())
    return {"forward_train_ms": round(t_f, 4), "backward_saved_ms": round(t_b, 4),
            "train_step_tokens_per_s": round(B * n / ((t_f + t_b) * 1e-3), 1),
            "frac_bf16_peak": round(step_flops / ((t_f + t_b) * 1e-3) / 1e12 / PEAK["bf16"], 4)
            if dtype == "bf16" else None}


def train_measure(inp, dtype, torch, fg, dev, steps=10, settle_s=0.5):
    """Only the training pair (no recomputing backward is called), for a kernel trace of the pair
    alone: untimed pairs for settle_s seconds (the clocks ramp up after the host has generated
    the inputs), then _train_pair's 10 untimed and `steps` timed pairs."""
    from efficient_transformer_attention_amd import inputs as gen
    B, n, d = inp.X.shape
    e, s, c, causal = inp.W_u.shape[1], inp.W_z.shape[1], inp.chunk, inp.causal
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def up(a, t=tdt):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(t).contiguous()

    args = [up(inp.X), up(inp.W_u), up(inp.W_v), up(inp.W_z), up(inp.gamma, torch.float32),
            up(inp.beta, torch.float32), up(inp.W_o)]
    dO = up(gen.make_output_grad(B, n, d, dtype))
    dt = fg.BF16 if dtype == "bf16" else fg.F32
    ws = torch.empty((fg.backward_workspace_size(B, n, d, e, s, c, causal, dt),), dtype=torch.uint8,
                     device=dev)
    O = fg.flash_gau_forward_train(*args, c, causal, ws)
    grads = fg.flash_gau_backward(*args, dO, c, causal, workspace=ws, saved=True)
    settle_pairs = 1
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        fg.flash_gau_forward_train(*args, c, causal, ws, out=O)
        fg.flash_gau_backward(*args, dO, c, causal, workspace=ws, out=grads, saved=True)
        torch.cuda.synchronize(dev)
        settle_pairs += 1
    rec = _train_pair(fg, torch, dev, args, dO, c, causal, ws, grads, steps, dtype)
    rec.update(steps=steps, settle_pairs=settle_pairs)
    return rec


def backward_measure(inp, dtype, torch, fg, dev, cpu_seconds, steps=10, with_saved=True):
    """Times flash_gau_backward on the whole batch (dO drawn by inputs.make_output_grad) and the
    fp64 oracle's backward on sequence 0; checks the GPU gradients of a call whose dO is zero on
    every other sequence against that oracle run. Algorithmic work: every contraction of the
    forward has two gradient contractions of its size, so 2 x the forward's algorithmic FLOPs
    (the recomputed forward intermediates are not counted)."""
    import oracle
    from efficient_transformer_attention_amd import inputs as gen
    B, n, d = inp.X.shape
    e, s, c, causal = inp.W_u.shape[1], inp.W_z.shape[1], inp.chunk, inp.causal
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def up(a, t=tdt):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(t).contiguous()

    args = [up(inp.X), up(inp.W_u), up(inp.W_v), up(inp.W_z), up(inp.gamma, torch.float32),
            up(inp.beta, torch.float32), up(inp.W_o)]
    dO_np = gen.make_output_grad(B, n, d, dtype)
    dO = up(dO_np)
    dt = fg.BF16 if dtype == "bf16" else fg.F32
    ws = torch.empty((fg.backward_workspace_size(B, n, d, e, s, c, causal, dt),), dtype=torch.uint8,
                     device=dev)
    out = fg.flash_gau_backward(*args, dO, c, causal, workspace=ws)
    # warm-up: dO was just drawn on the host, with the GPU idle; ~20 ms of work lets the clocks
    # settle before the timed calls
    for _ in range(15):
        fg.flash_gau_backward(*args, dO, c, causal, workspace=ws, out=out)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(steps):
        fg.flash_gau_backward(*args, dO, c, causal, workspace=ws, out=out)
    torch.cuda.synchronize(dev)
    ms = (time.perf_counter() - t0) * 1e3 / steps
    flops = 2.0 * sum(alg_flops(B, n, d, e, s, c, causal).values())
    # a training step without the backward's recompute: forward_train, then backward_saved
    training = None
    if with_saved:
        training = _train_pair(fg, torch, dev, args, dO, c, causal, ws, out, steps, dtype)
    rec = {"workload": f"backward of the same layer and batch", "steps": steps,
           "ms_per_step": round(ms, 4), "tokens_per_s": round(B * n / (ms * 1e-3), 1),
           "alg_gflop": round(flops / 1e9, 2),
           "achieved_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
           "frac_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK["bf16"], 4) if dtype == "bf16" else None,
           "saved_activations": training}
    if cpu_seconds > 0:
        dO_np[1:] = 0.0
        g = fg.flash_gau_backward(*args, up(dO_np), c, causal, workspace=ws, out=out)
        torch.cuda.synchronize(dev)
        got = {k: v.float().cpu().numpy().astype(np.float64) for k, v in g.items()}
        times, ref = [], None
        t_start = time.perf_counter()
        while not times or time.perf_counter() - t_start < cpu_seconds:
            t1 = time.perf_counter()
            ref = oracle.flash_backward(inp.X[:1], inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta,
                                        inp.W_o, dO_np[:1], c, causal)
            times.append(time.perf_counter() - t1)
        med = statistics.median(times)
        rec["cpu_baseline"] = {"value": n / med, "unit": "tokens/s", "kind": "oracle",
                               "sample": f"backward of sequence 0 ({n} tokens), fp64 NumPy oracle, "
                                         f"median of {len(times)} runs ({med:.2f} s each)"}
        rec["max_rel_err_seq0"] = {
            k: float(np.abs((got[k][:1] if k == "dX" else got[k]) - ref[k]).max() / np.abs(ref[k]).max())
            for k in fg.GRAD_NAMES}
    return rec


def decode_bytes(B, d, e, s, c, esz, i):
    """Algorithmic HBM bytes of one decoding step at position i of its chunk (B sequences): the
    packed weights once, the token in and out, the cache rows 0..i and the fp32 state read, the
    new cache row and the per-step scratch (u, the query heads, y) written and read back, and
    after the chunk's last token the fold (cache read, state read and written)."""
    w = ((2 * e + s) * d + d * e) * esz
    io = 2 * B * d * esz
    reads = B * (i + 1) * (s + e) * esz + B * s * e * 4
    writes = B * (2 * s + e) * esz + 2 * B * (2 * e + 2 * s) * esz
    fold = (B * c * (s + e) * esz + 2 * B * s * e * 4) if i == c - 1 else 0
    return w + io + reads + writes + fold


def decode_measure(inp, dtype, torch, fg, dev, cpu_seconds):
    """Times one chunk of causal decoding steps (positions c .. 2c-1, after chunk 0 has filled the
    state untimed) for the workload's batch and dimensions. Returns the record for the JSON line."""
    B, n, d, e, s = inp.shape
    c = inp.chunk
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    esz = 2 if dtype == "bf16" else 4

    def up(a, t=tdt):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(t).contiguous()

    W = [up(a) for a in (inp.W_u, inp.W_v, inp.W_z, inp.W_o)]
    gamma, beta = up(inp.gamma, torch.float32), up(inp.beta, torch.float32)
    packed = fg.pack_weights(*W)
    state = fg.DecodeState(B, d, e, s, c, tdt, dev)
    xs = up(inp.X[:, : 2 * c]).transpose(0, 1).contiguous()  # [2c, B, d]: one contiguous token row per step
    o = torch.empty((B, d), dtype=tdt, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    dt = fg.BF16 if dtype == "bf16" else fg.F32

    def step(t):
        rc = fg.decode_step_raw(xs[t].data_ptr(), packed.data_ptr(), packed.numel(), gamma.data_ptr(),
                                beta.data_ptr(), c, t, n, 0.0, B, d, e, s, dt, o.data_ptr(),
                                state.buf.data_ptr(), state.buf.numel(), stream)
        if rc != fg.OK:
            raise fg.FlashGauError(rc, "flash_gau_decode_step")

    print(f"[bench] decode: {c} untimed steps, then {c} timed", file=sys.stderr, flush=True)
    for t in range(c):
        step(t)
    torch.cuda.synchronize()
    after_chunk0 = state.buf.clone()
    ev = HipEvents(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.hip.hipEventRecord(ctypes.c_void_p(ev.handles[0]), ctypes.c_void_p(stream))
    for t in range(c, 2 * c):
        step(t)
    ev.hip.hipEventRecord(ctypes.c_void_p(ev.handles[1]), ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev.ms(ev.handles[0], ev.handles[1])

    # The same chunk of steps captured once into a HIP graph and replayed from the same state:
    # the usual way a serving loop removes the host's launch cost from decoding.
    state.buf.copy_(after_chunk0)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap):
        for t in range(c, 2 * c):
            rc = fg.decode_step_raw(xs[t].data_ptr(), packed.data_ptr(), packed.numel(),
                                    gamma.data_ptr(), beta.data_ptr(), c, t, n, 0.0, B, d, e, s, dt,
                                    o.data_ptr(), state.buf.data_ptr(), state.buf.numel(),
                                    cap.cuda_stream)
            if rc != fg.OK:
                raise fg.FlashGauError(rc, "flash_gau_decode_step")
    torch.cuda.synchronize()
    ev.hip.hipEventRecord(ctypes.c_void_p(ev.handles[0]), ctypes.c_void_p(stream))
    graph.replay()
    ev.hip.hipEventRecord(ctypes.c_void_p(ev.handles[1]), ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    graph_ms = ev.ms(ev.handles[0], ev.handles[1])
    ev.close()
    nbytes = sum(decode_bytes(B, d, e, s, c, esz, i) for i in range(c)) / c
    us_step = gpu_ms * 1e3 / c
    achieved = nbytes / (us_step * 1e-6) / 1e9
    us_graph = graph_ms * 1e3 / c
    rec = {"metric": "decode tokens/s (causal, one token per sequence per step)",
           "value": round(B * c / (wall), 1), "unit": "tokens/s", "steps": c, "batch": B,
           "positions": [c, 2 * c - 1], "us_per_step": round(us_step, 2),
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK, 4),
                        "bytes_per_step": int(nbytes)},
           "hip_graph": {"us_per_step": round(us_graph, 2),
                         "tokens_per_s": round(B / (us_graph * 1e-6), 1),
                         "achieved_gbs": round(nbytes / (us_graph * 1e-6) / 1e9, 1)}}
    if cpu_seconds > 0:
        import oracle
        st = oracle.decode_init(B, s, e, c)
        times, t = [], 0
        t_start = time.perf_counter()
        while t < c + 8 and (t < c or time.perf_counter() - t_start < cpu_seconds):
            t1 = time.perf_counter()
            oracle.decode_step(st, inp.X[:, t], t, n, inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta,
                               inp.W_o, c)
            times.append(time.perf_counter() - t1)
            t += 1
        med = statistics.median(times)
        rec["cpu_baseline"] = {"value": round(B / med, 1), "unit": "tokens/s", "kind": "oracle",
                               "sample": f"fp64 oracle decode_step for the same {B} sequences, "
                                         f"median of {len(times)} steps ({med * 1e3:.1f} ms each)"}
    rec["batch_sweep"] = [decode_batch_point(Bx, n, d, e, s, c, dtype, torch, fg, dev)
                          for Bx in (32, 128)]
    return rec


def decode_batch_point(B, n, d, e, s, c, dtype, torch, fg, dev):
    """The same decoding step at a larger batch (the widths and sequence length of the workload,
    seeded synthetic tokens and weights for 2c positions): one chunk untimed, one chunk timed between
    HIP events. The weights are read once per step whatever the batch, so the HBM fraction grows
    with B until the state and cache reads dominate."""
    from efficient_transformer_attention_amd import inputs as gen
    inp = gen.make_inputs(B, 2 * c, d, e, s, c, True, dtype, seed=11)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    esz = 2 if dtype == "bf16" else 4

    def up(a, t=tdt):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(t).contiguous()

    packed = fg.pack_weights(*[up(a) for a in (inp.W_u, inp.W_v, inp.W_z, inp.W_o)])
    gamma, beta = up(inp.gamma, torch.float32), up(inp.beta, torch.float32)
    state = fg.DecodeState(B, d, e, s, c, tdt, dev)
    xs = up(inp.X).transpose(0, 1).contiguous()
    o = torch.empty((B, d), dtype=tdt, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    dt = fg.BF16 if dtype == "bf16" else fg.F32

    def step(t):
        rc = fg.decode_step_raw(xs[t].data_ptr(), packed.data_ptr(), packed.numel(), gamma.data_ptr(),
                                beta.data_ptr(), c, t, n, 0.0, B, d, e, s, dt, o.data_ptr(),
                                state.buf.data_ptr(), state.buf.numel(), stream)
        if rc != fg.OK:
            raise fg.FlashGauError(rc, "flash_gau_decode_step")

    for t in range(c):
        step(t)
    ev = HipEvents(2)
    torch.cuda.synchronize()
    ev.hip.hipEventRecord(ctypes.c_void_p(ev.handles[0]), ctypes.c_void_p(stream))
    for t in range(c, 2 * c):
        step(t)
    ev.hip.hipEventRecord(ctypes.c_void_p(ev.handles[1]), ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    us_step = ev.ms(ev.handles[0], ev.handles[1]) * 1e3 / c
    ev.close()
    nbytes = sum(decode_bytes(B, d, e, s, c, esz, i) for i in range(c)) / c
    achieved = nbytes / (us_step * 1e-6) / 1e9
    return {"batch": B, "us_per_step": round(us_step, 2), "tokens_per_s": round(B / (us_step * 1e-6), 1),
            "bytes_per_step": int(nbytes), "hbm_frac": round(achieved / HBM_PEAK, 4)}


def time_forward(fg, torch, dev, B, n, d, e, s, c, causal, dtype, rope_base=None, steps=20,
                 warmup=50, seed=0):
    """Average time (us) of one forward call (flash_gau_forward, or flash_gau_forward_rope when
    rope_base is given) over `steps` calls after `warmup` calls, between two HIP events. The
    inputs are generated on the host first, which leaves the GPU idle for seconds: a few warm-up
    calls would time the clocks ramping back up."""
    from efficient_transformer_attention_amd import inputs as gen
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dt = fg.BF16 if dtype == "bf16" else fg.F32

    def up(a, t=tdt):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(t).contiguous()

    X, Wu, Wv, Wz, Wo = (up(a) for a in (inp.X, inp.W_u, inp.W_v, inp.W_z, inp.W_o))
    gamma, beta = up(inp.gamma, torch.float32), up(inp.beta, torch.float32)
    nbytes = fg.workspace_size(B, n, d, e, s, c, causal, dt)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    O = torch.empty((B, n, d), dtype=tdt, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    ptrs = (X.data_ptr(), Wu.data_ptr(), Wv.data_ptr(), Wz.data_ptr(), gamma.data_ptr(),
            beta.data_ptr(), Wo.data_ptr())

    def call():
        if rope_base is None:
            rc = fg.forward_raw(*ptrs, c, causal, B, n, d, e, s, dt, O.data_ptr(), ws.data_ptr(),
                                nbytes, stream)
        else:
            rc = fg.forward_rope_raw(*ptrs, c, causal, rope_base, B, n, d, e, s, dt, O.data_ptr(),
                                     ws.data_ptr(), nbytes, stream)
        if rc != fg.OK:
            raise fg.FlashGauError(rc, "forward")

    for _ in range(warmup):
        call()
    ev = HipEvents(2)
    torch.cuda.synchronize()
    ev.hip.hipEventRecord(ctypes.c_void_p(ev.handles[0]), ctypes.c_void_p(stream))
    for _ in range(steps):
        call()
    ev.hip.hipEventRecord(ctypes.c_void_p(ev.handles[1]), ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    us = ev.ms(ev.handles[0], ev.handles[1]) * 1e3 / steps
    ev.close()
    return us


def upload(torch, dev, inp):
    """The workload's inputs as contiguous device tensors (X and the weights in the storage dtype,
    gamma and beta fp32)."""
    tdt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32

    def up(a, t=tdt):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(t).contiguous()

    return [up(inp.X), up(inp.W_u), up(inp.W_v), up(inp.W_z), up(inp.gamma, torch.float32),
            up(inp.beta, torch.float32), up(inp.W_o)]


def measure_forward(fg, torch, dev, inp, steps, warmup, settle_ms, kernel_steps, quantile_steps):
    """Times flash_gau_forward on one workload. Order: an untimed settle loop of forward calls for
    settle_ms (after host-side input generation the GPU has idled for seconds and its clocks have
    dropped), `warmup` untimed calls, then exactly `steps` calls between two device
    synchronisations (the timed region: no events, nothing else on the stream). Then two separate
    passes, outside the timed region: `kernel_steps` calls of flash_gau_forward_timed (each kernel
    launched with its own start and stop HIP events) for per-kernel durations, and `quantile_steps`
    calls each bracketed by two events for the step-time distribution. Returns the record and O."""
    B, n, d, e, s = inp.shape
    c, causal = inp.chunk, inp.causal
    dt = fg.BF16 if inp.dtype == "bf16" else fg.F32
    tens = upload(torch, dev, inp)
    nbytes = fg.workspace_size(B, n, d, e, s, c, causal, dt)
    ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
    O = torch.empty((B, n, d), dtype=tens[0].dtype, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    ptrs = tuple(t.data_ptr() for t in tens)
    nst = len(fg.STAGES)

    def step():
        rc = fg.forward_raw(*ptrs, c, causal, B, n, d, e, s, dt, O.data_ptr(), ws.data_ptr(),
                            nbytes, stream)
        if rc != fg.OK:
            raise fg.FlashGauError(rc, "flash_gau_forward")

    # settle: fixed wall-clock duration, untimed
    settle_calls = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        for _ in range(8):
            step()
        settle_calls += 8
        torch.cuda.synchronize(dev)
    settle_elapsed = (time.perf_counter() - t_settle) * 1e3
    for _ in range(warmup):
        step()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / steps

    # per-kernel durations, a pass of its own: each kernel's own start and stop events
    events = HipEvents(kernel_steps * 2 * nst)
    for k in range(kernel_steps):
        evs = events.handles[k * 2 * nst:(k + 1) * 2 * nst]
        rc = fg.forward_timed_raw(*ptrs, c, causal, B, n, d, e, s, dt, O.data_ptr(), ws.data_ptr(),
                                  nbytes, stream, evs)
        if rc != fg.OK:
            raise fg.FlashGauError(rc, "flash_gau_forward_timed")
    torch.cuda.synchronize(dev)
    stage_ms = {st: [] for st in fg.STAGES}
    for k in range(kernel_steps):
        h = events.handles[k * 2 * nst:(k + 1) * 2 * nst]
        for i, st in enumerate(fg.STAGES):
            stage_ms[st].append(events.ms(h[2 * i], h[2 * i + 1]))
    events.close()

    # step-time distribution, a pass of its own (events between steps only)
    sev = HipEvents(2 * quantile_steps)
    for k in range(quantile_steps):
        sev.hip.hipEventRecord(ctypes.c_void_p(sev.handles[2 * k]), ctypes.c_void_p(stream))
        step()
        sev.hip.hipEventRecord(ctypes.c_void_p(sev.handles[2 * k + 1]), ctypes.c_void_p(stream))
    torch.cuda.synchronize(dev)
    per_step = sorted(sev.ms(sev.handles[2 * k], sev.handles[2 * k + 1])
                      for k in range(quantile_steps))
    sev.close()

    def quantile(q):
        return per_step[min(len(per_step) - 1, int(q * (len(per_step) - 1) + 0.5))]

    esz = 2 if inp.dtype == "bf16" else 4
    ng = fg.state_groups(B, n, d, e, s, c, causal, dt)
    flops = alg_flops(B, n, d, e, s, c, causal)
    nbytes_alg = alg_bytes(B, n, d, e, s, c, causal, esz, ng)
    peak = PEAK[inp.dtype]
    stage_avg = {st: statistics.mean(v) for st, v in stage_ms.items()}
    stages = {}
    for st in fg.STAGES:
        t = stage_avg[st] / 1e3
        stages[st] = {"us": round(stage_avg[st] * 1e3, 2),
                      "tflops": round(flops[st] / t / 1e12, 2) if flops[st] and t > 0 else 0.0,
                      "gbs": round(nbytes_alg[st] / t / 1e9, 1) if t > 0 else 0.0}
    dom = max(fg.STAGES, key=lambda st: stage_avg[st])
    t_dom = stage_avg[dom] / 1e3
    if BOUND[dom] == "mfma":
        achieved, pk, unit = flops[dom] / t_dom / 1e12, peak, "TFLOP/s"
    else:
        achieved, pk, unit = nbytes_alg[dom] / t_dom / 1e9, HBM_PEAK, "GB/s"
    total_flops = sum(flops.values())
    rec = {
        "ms_per_step": round(ms_step, 4),
        "tokens_per_s": round(B * n / (ms_step / 1e3), 1),
        "frac_peak": round(total_flops / (ms_step / 1e3) / 1e12 / peak, 4),
        "peak_tflops": peak,
        "alg_gflop": round(total_flops / 1e9, 2),
        "settle_ms": round(settle_elapsed, 1),
        "settle_calls": settle_calls,
        "kernel_pass_ms": round(statistics.mean(sum(stage_ms[st][k] for st in fg.STAGES)
                                                for k in range(kernel_steps)), 4),
        "step_ms_quantiles": {"p10": round(quantile(0.1), 4), "p50": round(quantile(0.5), 4),
                              "p90": round(quantile(0.9), 4)},
        "state_branch": state_branch(B, n, c, causal, ng),
        "stages": stages,
        "dominant": {"kernel": dom, "bound": BOUND[dom], "achieved": round(achieved, 2), "peak": pk,
                     "unit": unit, "frac": round(achieved / pk, 4)},
    }
    return rec, O


def time_packed(fg, torch, dev, inp, plain_ms, steps=50, warmup=50):
    """flash_gau_forward_packed on the same workload: the weights transposed once by
    flashgau_pack_weights (as a model does once per weight set), then forward calls that skip the
    transpose. Its output must equal flash_gau_forward's bit for bit."""
    B, n, d, e, s = inp.shape
    c, causal = inp.chunk, inp.causal
    dt = fg.BF16 if inp.dtype == "bf16" else fg.F32
    X, W_u, W_v, W_z, g, b, W_o = upload(torch, dev, inp)
    packed = fg.pack_weights(W_u, W_v, W_z, W_o)
    nbytes = fg.workspace_size(B, n, d, e, s, c, causal, dt)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    O = torch.empty((B, n, d), dtype=X.dtype, device=dev)
    ref = fg.flash_gau_forward(X, W_u, W_v, W_z, g, b, W_o, c, causal, workspace=ws)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def call():
        rc = fg.forward_packed_raw(X.data_ptr(), packed.data_ptr(), packed.numel(), g.data_ptr(),
                                   b.data_ptr(), c, causal, B, n, d, e, s, dt, O.data_ptr(),
                                   ws.data_ptr(), nbytes, stream)
        if rc != fg.OK:
            raise fg.FlashGauError(rc, "flash_gau_forward_packed")

    for _ in range(warmup):
        call()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize(dev)
    ms = (time.perf_counter() - t0) * 1e3 / steps
    same = bool(torch.equal(O.view(torch.int16) if O.element_size() == 2 else O.view(torch.int32),
                            ref.view(torch.int16) if ref.element_size() == 2 else ref.view(torch.int32)))
    return {"entry": "flash_gau_forward_packed", "ms_per_step": round(ms, 4),
            "tokens_per_s": round(B * n / (ms * 1e-3), 1),
            "plain_forward_ms_per_step": plain_ms, "bitwise_equal_to_plain": same}


def oracle_sequence_error(inp, O, b):
    """max |O_gpu - O_ref| / max |O_ref| on sequence b, O_ref from the fp64 oracle."""
    import oracle
    ref = oracle.flash_forward(inp.X[b:b + 1], inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta,
                               inp.W_o, inp.chunk, inp.causal)
    got = O[b:b + 1].float().cpu().numpy().astype(np.float64)
    return float(np.abs(got - ref).max() / np.abs(ref).max())


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-ms", type=float, default=1500.0,
                    help="untimed forward calls for this long before the warm-up (clocks settle)")
    ap.add_argument("--workload", default=None, help="name in inputs.WORKLOADS")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time budget of the oracle baseline (0 disables it)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration rows (every workload of inputs.WORKLOADS)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the causal decoding measurement")
    ap.add_argument("--decode-only", action="store_true",
                    help="run only the causal decoding measurement and print its JSON object")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-pass measurement")
    ap.add_argument("--backward-only", action="store_true",
                    help="only flash_gau_backward's timing (no CPU baseline, no training pair), "
                         "one JSON line")
    ap.add_argument("--train-only", action="store_true",
                    help="only the training pair (flash_gau_forward_train, then "
                         "flash_gau_backward_saved), one JSON line")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the rotary-embedding and FLASH-Quad (chunk = n) timings")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times) and exit: the "
                         "reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.calibrate_copy_mib:
        import torch
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_mib": args.calibrate_copy_mib, "launches": 3}), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library runs the layer on one GPU and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    from efficient_transformer_attention_amd import flashgau as fg
    from efficient_transformer_attention_amd import inputs as gen

    name = args.workload or gen.HEADLINE
    B, n, d, e, s, c, causal, dtype = gen.WORKLOADS[name]
    inp = gen.workload_inputs(name, seed=0)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.backward_only:
        print(json.dumps({"workload": name, "backward": backward_measure(
            inp, dtype, torch, fg, dev, 0.0, steps=args.steps, with_saved=False)}), flush=True)
        return
    if args.train_only:
        print(json.dumps({"workload": name, "training_pair": train_measure(
            inp, dtype, torch, fg, dev, steps=args.steps)}), flush=True)
        return
    if args.decode_only:
        if not causal:
            print("--decode-only needs a causal workload", file=sys.stderr)
            sys.exit(2)
        print(json.dumps({"workload": name, "decode": decode_measure(inp, dtype, torch, fg, dev,
                                                                    min(args.cpu_seconds, 5.0))}),
              flush=True)
        return

    print(f"[bench] {name}: settle {args.settle_ms:.0f} ms, warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)
    head, O = measure_forward(fg, torch, dev, inp, args.steps, args.warmup, args.settle_ms,
                              kernel_steps=max(10, min(args.steps, 50)),
                              quantile_steps=max(50, args.steps))
    print("[bench] timed region done", file=sys.stderr, flush=True)
    props = torch.cuda.get_device_properties(dev)
    device = {"name": props.name, "compute_units": props.multi_processor_count,
              "gcn_arch": getattr(props, "gcnArchName", None),
              "max_sclk_mhz": round(getattr(props, "clock_rate", 0) / 1000.0) or None}
    dom = head["dominant"]
    roofline = dict(dom, traffic=measured_traffic(dom["kernel"], name))

    cpu = None
    max_rel_err = None
    if args.cpu_seconds > 0:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu, ref = cpu_baseline(inp, args.cpu_seconds)
        got = O[:1].float().cpu().numpy().astype(np.float64)
        max_rel_err = float(np.abs(got - ref).max() / np.abs(ref).max())
    del O

    configs = None
    if not args.no_configs:
        configs = []
        for wname, shape in gen.WORKLOADS.items():
            wB, wn, wd, we, ws_, wc, wcausal, wdtype = shape
            row = {"workload": wname, "batch": wB, "seq_len": wn, "d": wd, "e": we, "s": ws_,
                   "chunk": wc, "causal": wcausal, "dtype": wdtype}
            if wname == name:
                rec = {k: head[k] for k in ("ms_per_step", "tokens_per_s", "frac_peak", "peak_tflops",
                                            "alg_gflop", "step_ms_quantiles", "state_branch",
                                            "dominant")}
                rec["max_rel_err"] = max_rel_err
                rec["sampled_sequence"] = 0
            else:
                print(f"[bench] config {wname}", file=sys.stderr, flush=True)
                winp = gen.workload_inputs(wname, seed=0)
                full, wO = measure_forward(fg, torch, dev, winp, steps=20, warmup=10, settle_ms=300.0,
                                           kernel_steps=10, quantile_steps=10)
                rec = {k: full[k] for k in ("ms_per_step", "tokens_per_s", "frac_peak", "peak_tflops",
                                            "alg_gflop", "step_ms_quantiles", "state_branch",
                                            "dominant")}
                sb = wB - 1
                rec["max_rel_err"] = (oracle_sequence_error(winp, wO, sb)
                                      if args.cpu_seconds > 0 else None)
                rec["sampled_sequence"] = sb
                del wO
            row.update(rec)
            configs.append(row)
        torch.cuda.empty_cache()

    decode = None
    if causal and not args.no_decode:
        decode = decode_measure(inp, dtype, torch, fg, dev, min(args.cpu_seconds, 5.0))

    backward = None
    if not args.no_backward:
        print("[bench] backward pass", file=sys.stderr, flush=True)
        backward = backward_measure(inp, dtype, torch, fg, dev, min(args.cpu_seconds, 10.0))
        backward["train_step_tokens_per_s"] = round(
            B * n / ((head["ms_per_step"] + backward["ms_per_step"]) * 1e-3), 1)

    packed = None
    if not args.no_extras:
        packed = time_packed(fg, torch, dev, inp, head["ms_per_step"])

    rope = quad = None
    if not args.no_extras:
        print("[bench] rotary embedding and FLASH-Quad timings", file=sys.stderr, flush=True)
        us_rope = time_forward(fg, torch, dev, B, n, d, e, s, c, causal, dtype, rope_base=10000.0)
        us_plain = time_forward(fg, torch, dev, B, n, d, e, s, c, causal, dtype)
        rope = {"workload": name, "rope_base": 10000.0, "us_per_step": round(us_rope, 1),
                "tokens_per_s": round(B * n / (us_rope * 1e-6), 1),
                "us_per_step_without": round(us_plain, 1)}
        # the same 16384 tokens as sequences of growing length: FLASH-Quad's cost per token grows
        # with n, FLASH's does not; the crossover is where flash_speedup passes 1
        quad = []
        for qn in (512, 1024, 2048, 4096, 8192, 16384):
            qB = 16384 // qn
            us_q = time_forward(fg, torch, dev, qB, qn, d, e, s, qn, True, dtype, steps=5)
            us_f = (time_forward(fg, torch, dev, qB, qn, d, e, s, c, True, dtype, steps=5)
                    if qn > c else us_q)
            quad.append({"batch": qB, "seq_len": qn, "flash_quad_chunk_eq_n_us": round(us_q, 1),
                         f"flash_chunk_{c}_us": round(us_f, 1), "flash_speedup": round(us_q / us_f, 2)})

    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": head["settle_ms"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "seq_len": n, "d": d, "e": e, "s": s,
                   "chunk": c, "causal": causal},
        "frac_bf16_peak": head["frac_peak"] if dtype == "bf16" else None,
        "alg_gflop": head["alg_gflop"],
        "kernel_pass_ms": head["kernel_pass_ms"],
        "step_ms_quantiles": head["step_ms_quantiles"],
        "device": device,
        "roofline": roofline,
        "stages": head["stages"],
        "state_branch": head["state_branch"],
        "cpu_baseline": cpu,
        "max_rel_err_seq0": max_rel_err,
        "configs": configs,
        "decode": decode,
        "backward": backward,
        "packed_weights": packed,
        "rope": rope,
        "flash_vs_flash_quad": quad,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
