"""Benchmark of the Gated Delta Rule hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only prefill,decode,...]

A step is one gdn_prefill call over the chunked-prefill workload (B=4, H=16,
T=4096, d_k=d_v=128, bf16 q/k/v, fp32 gates and state, zero initial state),
with a workspace, i.e. its two passes: chunk_prep (every chunk's triangular
system, all chunks in parallel) and chunk_chain (the state recurrence over
chunks). ``value`` is prefill tokens/s (B*T per step). The same JSON line
carries:

* ``roofline`` of the dominant kernel (the pass with the longer average
  launch, timed with a pair of HIP events around every launch): the method's
  own bytes per step (1032 B per token-head: q, k, v, o bf16, g, beta fp32,
  plus the fp32 final states) over that kernel's average launch, against
  8 TB/s, with the matrix-core rate of the step's algorithmic flops over the
  same time. ``overhead_bytes`` counts what the two-pass design moves beyond
  them (the 96 B per token-head of bf16 T diag(beta) written by chunk_prep
  and read back by chunk_chain, and chunk_prep's second read of k, g, beta).
  ``traffic`` is the measured HBM bytes per launch from the committed counter
  summary (profiles/), or null when the kernel source has changed since.
  ``path`` gives the whole step against the method's bytes and the
  matrix-core rate against the 2.5 PFLOP/s dense bf16 peak;
* ``one_pass``: the same call without a workspace (one kernel that solves
  each chunk's system on the sequential path);
* ``decode``: one in-place step of B=256, H=32, d=128 fp32 states (512 MiB),
  GB/s of algorithmic traffic and its fraction of 8 TB/s;
* ``decode_mixer``: one fused single-token mixer step (conv against the
  3-token cache, norms, gates, state update, gated RMSNorm) at B=256, H=32,
  d=128, GB/s of algorithmic traffic against 8 TB/s;
* ``channel_gated``: one decay rate per key channel, the token-serial
  prefill at the prefill shape and one decode step at the decode shape;
* ``mixer``: prologue -> prefill -> epilogue at B=8, T=8192, H=16, d=128;
* ``varlen``: packed prefill, H=32, 8 sequences, lengths log-uniform in
  [512, 65536], non-zero initial states;
* ``seqpar``: one long sequence (B=1, H=16, T=32768) by the plain two-pass
  prefill and by the sequence-parallel prefill with 3, 4, 5, 8, 16 segments;
* ``cpu_baseline``: the fp64 CPU oracle timed on this host on the prefill
  workload (a reported baseline, not a target).

Timing: warm-up launches, then K launches bracketed by device
synchronisation and timed with HIP events recorded on the stream the kernels
run on (torch's current stream, which the binding launches on); the per-pass
figures come from an event pair around every launch (mean and median over at
least 20). Prefill
inputs and outputs alternate between two copies so that successive launches
read from HBM rather than from the 256 MB last-level cache. The first
workload (the prefill) is timed twice: from idle (its W warm-up steps, then
K timed steps) and, reported as the value, after the device has run the same
step for DEVICE_WARMUP_S seconds and then the W warm-up steps again; the
workloads after it find the device already busy.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores, TFLOP/s
METRIC = "prefill tokens/s (H=16,d=128,T=4096) + decode state GB/s vs HBM peak"
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "chunk_prefill_B4_H16_T4096_traffic.md")
CHUNK_SRC = os.path.join(ROOT, "gated_deltanet_recurrence_amd", "csrc", "prefill_split.hip")


def prefill_flops_per_token_head(dk=128, dv=128, C=64):
    """Algorithmic flops of the chunk form per token and head: the three
    state contractions W S^T, Q S^T and Delta~^T K (2 dk dv each), and the
    triangular C x C products K K^T, Q K^T, T K (C dk each) and T V, P Delta
    (C dv each), counted at half size: 6 dk dv + 3 C dk + 2 C dv."""
    return 6 * dk * dv + 3 * C * dk + 2 * C * dv


def prefill_bytes(B, T, H, dk=128, dv=128, n_states_out=None, n_states_in=0):
    tok_head = B * T * H
    per = 2 * (dk + dk + dv + dv) + 4 + 4          # q, k, v, o bf16; g, beta fp32
    states = (n_states_out if n_states_out is not None else B) * H * dv * dk * 4
    return tok_head * per + states + n_states_in * H * dv * dk * 4


# workspace per token-head: bf16 T diag(beta) per 64-token chunk (its lower
# 64 x 64 part: rows 0-31 by columns 0-31, rows 32-63 by all 64)
WS_BYTES_PER_TOKEN_HEAD = (32 * 32 + 32 * 64) * 2 // 64     # 96


def chain_bytes(B, T, H, dk=128, dv=128):
    """chunk_chain per launch as it runs: q, k, v, o bf16, g fp32, the
    workspace read back, the final states."""
    per = 2 * (dk + dk + dv + dv) + 4 + WS_BYTES_PER_TOKEN_HEAD
    return B * T * H * per + B * H * dv * dk * 4


def prep_bytes(B, T, H, dk=128):
    """chunk_solve per launch as it runs: k bf16, g and beta fp32 read, the
    workspace written."""
    return B * T * H * (2 * dk + 4 + 4 + WS_BYTES_PER_TOKEN_HEAD)


def decode_bytes(B, H, dk=128, dv=128):
    return B * H * (2 * dv * dk * 4 + 2 * (dk + dk + dv + dv) + 4 + 4)


def event_time(fn, steps, warmup):
    """Mean ms per call over `steps` calls bracketed by device synchronisation
    and one pair of HIP events (recorded on torch's current stream, the one
    the binding launches on)."""
    import torch
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps        # ms per call


DEVICE_WARMUP_S = 0.25


def device_warmup(fn, seconds=DEVICE_WARMUP_S):
    """Run `fn` (the workload's own step) for `seconds` of wall time, in
    batches of 50 calls with a synchronisation after each: from idle, the
    first ~25 ms of work run ~13% slower than the device's steady state
    (measured on the prefill workload: 0.134-0.139 ms per step after 5
    warm-up steps, 0.118 ms after 200). Returns the number of calls."""
    import torch
    t_end = time.time() + seconds
    n = 0
    while time.time() < t_end:
        for _ in range(50):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


def launch_times(fns, steps, warmup):
    """Per-launch durations (ms) of a sequence of launches: each call in
    `fns` is bracketed by its own pair of HIP events on the launch stream,
    for `steps` repetitions after `warmup` untimed ones. Returns one list of
    `steps` durations per function."""
    import torch
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        for f in fns:
            f(i)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        for j, f in enumerate(fns):
            f(i)
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    return [[ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)] for j in range(len(fns))]


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def _src_hash(path):
    """Hash of the kernel source's code: comments and blank space are dropped,
    so that an edit of the comments keeps the recorded counters valid."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, if
    the kernel source still matches the hash recorded there."""
    if not os.path.exists(PROFILE_SUMMARY):
        return None, "no counter summary"
    text = open(PROFILE_SUMMARY).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
    m_bytes = re.search(kernel + r"_hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes:
        return None, "summary lacks fields"
    if m_hash.group(1) != _src_hash(CHUNK_SRC):
        return None, "kernel changed since the counters were taken"
    return float(m_bytes.group(1)), "ok"


def bench_prefill(gdn, inputs, steps, warmup):
    import torch
    c = inputs.make_prefill()
    sets = []
    for _ in range(2):
        d = lambda t: t.cuda().contiguous()
        sets.append(dict(q=d(c.q), k=d(c.k), v=d(c.v), g=d(c.g), beta=d(c.beta),
                         o=torch.empty_like(d(c.v)),
                         fin=torch.empty((c.B, c.H, 128, 128), dtype=torch.float32,
                                         device="cuda")))

    nws = gdn.gdn_prefill_workspace_size(c.B, c.T, c.H, 128, 128, c.B, False, torch.bfloat16)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def step(i):
        s = sets[i & 1]
        gdn.gdn_prefill(s["q"], s["k"], s["v"], s["g"], s["beta"], None, s["fin"], s["o"],
                        scale=c.scale, workspace=ws)

    def step_one_pass(i):
        s = sets[i & 1]
        gdn.gdn_prefill(s["q"], s["k"], s["v"], s["g"], s["beta"], None, s["fin"], s["o"],
                        scale=c.scale, workspace=None)
    # first as the device comes from idle (the W warm-up steps only), then
    # at its steady state: the reported figure
    ms_idle = event_time(step, steps, warmup)
    n_dev_warm = device_warmup(step)
    ms = event_time(step, steps, warmup)
    ms_one = event_time(step_one_pass, max(2, steps // 4), 2)

    # each pass alone, as the steps run it: max(steps, 20) launches back to
    # back between one pair of events on the launch stream (the mean launch);
    # and the same passes with a pair of events around every launch (those
    # events leave a gap before each launch and lengthen it: reported beside)
    def prep(i):
        s = sets[i & 1]
        gdn.gdn_prefill_prepare(s["q"], s["k"], s["g"], s["beta"], ws)

    def chain(i):
        s = sets[i & 1]
        gdn.gdn_prefill_apply(s["q"], s["k"], s["v"], s["g"], ws, None, s["fin"], s["o"],
                              scale=c.scale)
    n_launch = max(steps, 20)
    prep(0)
    ms_chain = event_time(chain, n_launch, warmup)
    ms_prep = event_time(prep, n_launch, warmup)
    t_prep, t_chain = launch_times([prep, chain], n_launch, warmup)
    tokens = c.B * c.T
    return dict(ms=ms, ms_idle=ms_idle, n_dev_warm=n_dev_warm, ms_one_pass=ms_one, tokens=tokens,
                ms_prep=ms_prep, ms_chain=ms_chain,
                med_prep=_median(t_prep), med_chain=_median(t_chain), n_launch=n_launch,
                bytes=prefill_bytes(c.B, c.T, c.H), chain_bytes=chain_bytes(c.B, c.T, c.H),
                prep_bytes=prep_bytes(c.B, c.T, c.H),
                ws_bytes=2 * WS_BYTES_PER_TOKEN_HEAD * c.B * c.T * c.H,
                reread_bytes=(2 * 128 + 4 + 4) * c.B * c.T * c.H,
                flops=prefill_flops_per_token_head() * c.B * c.T * c.H, case=c)


def bench_decode(gdn, inputs, steps, warmup):
    import torch
    c = inputs.make_decode()
    st = c.s0.cuda()
    q, k, v = (x[:, 0].cuda().contiguous() for x in (c.q, c.k, c.v))
    g, beta = c.g[:, 0].cuda().contiguous(), c.beta[:, 0].cuda().contiguous()
    o = torch.empty_like(v)

    def step(i):
        gdn.gdn_decode_step(q, k, v, g, beta, st, o, scale=c.scale)
    ms = event_time(step, steps, warmup)
    nbytes = decode_bytes(c.B, c.H)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return dict(workload="decode step B=256 H=32 d_k=d_v=128, fp32 state 512 MiB in place, bf16 q/k/v",
                us_per_step=round(ms * 1e3, 2), bytes_per_step=nbytes, **{"GB/s": round(gbs, 1)},
                frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))


def decode_mixer_bytes(B, H, Hk, dk=128, dv=128, elt=2):
    """Algorithmic HBM bytes of one fused mixer step: the fp32 state read and
    written; the conv cache (3 inputs per channel) read and written; the
    token's raw q, k, v, z, a, b read and the output written; the conv
    weights and A read once."""
    C = 2 * Hk * dk + H * dv
    per_seq = 2 * H * dv * dk * 4 + 2 * 3 * C * elt + (C + H * dv) * elt + 2 * H * elt + H * dv * elt
    return B * per_seq + C * 4 * elt + H * 4


def bench_decode_mixer(gdn, inputs, steps, warmup):
    import torch
    c = inputs.make_decode_mixer()
    d = lambda t: t.cuda().contiguous()
    q, k, v, z, a, b, w, A = (d(x) for x in (c.q_raw, c.k_raw, c.v_raw, c.z, c.a, c.b,
                                               c.conv_w, c.A))
    cache, st = d(c.conv_state), d(c.state)
    out = torch.empty_like(v)

    def step(i):
        gdn.gdn_decode_mixer_step(q, k, v, w, cache, a, b, A, z, st, out=out, scale=c.scale,
                                  eps=c.eps)
    ms = event_time(step, steps, warmup)
    B, H, dv = v.shape
    nbytes = decode_mixer_bytes(B, H, q.shape[1], q.shape[2], dv)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return dict(workload="fused mixer decode step B=256 H=32 d=128 bf16: conv against a 3-token "
                         "cache + SiLU, L2-norm, gates, state update (512 MiB fp32 in place), "
                         "gated RMSNorm",
                us_per_step=round(ms * 1e3, 2), bytes_per_step=nbytes,
                **{"GB/s": round(gbs, 1)}, frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))


def bench_channel_gated(gdn, inputs, steps, warmup):
    """Per-channel decay: the prefill at the prefill workload's shape (B=4,
    H=16, T=4096, d=128, bf16) by the chunkwise two-pass path and by the
    token-serial one, and one decode step at the decode shape (B=256, H=32,
    d=128), with one log-decay per key channel."""
    import torch
    c = inputs.make_channel_gated(seed=7, B=4, T=4096, H=16, d=128, with_state=False)
    d = lambda t: t.cuda().contiguous()
    q, k, v, g, beta = (d(x) for x in (c.q, c.k, c.v, c.g, c.beta))
    fin = torch.empty((4, 16, 128, 128), dtype=torch.float32, device="cuda")
    o = torch.empty_like(v)

    ws = torch.empty(gdn.gdn_prefill_channel_workspace_size(4, 4096, 16, 128, 128, 4, False,
                                                            torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def pre(i):
        gdn.gdn_prefill_channel_gated(q, k, v, g, beta, None, fin, o, scale=c.scale, workspace=ws)

    def pre_serial(i):
        gdn.gdn_prefill_channel_gated(q, k, v, g, beta, None, fin, o, scale=c.scale,
                                      workspace=None)
    ms_pre = event_time(pre, steps, warmup)
    ms_serial = event_time(pre_serial, max(5, steps // 4), 3)
    # the method's bytes: q, k, v, o bf16, one fp32 log-decay per key channel,
    # beta, and the final states
    pre_bytes = 4 * 4096 * 16 * (4 * 128 * 2 + 128 * 4 + 4) + 4 * 16 * 128 * 128 * 4
    dc = inputs.make_decode()
    st = dc.s0.cuda()
    qd, kd, vd = (x[:, 0].cuda().contiguous() for x in (dc.q, dc.k, dc.v))
    gd = dc.g[:, 0, :, None].expand(-1, -1, 128).cuda().contiguous()
    bd = dc.beta[:, 0].cuda().contiguous()
    od = torch.empty_like(vd)

    def dec(i):
        gdn.gdn_decode_step_channel_gated(qd, kd, vd, gd, bd, st, od, scale=dc.scale)
    ms_dec = event_time(dec, steps, warmup)
    nbytes = decode_bytes(dc.B, dc.H) + dc.B * dc.H * 128 * 4 - dc.B * dc.H * 4
    gbs = nbytes / (ms_dec * 1e-3) / 1e9
    return dict(workload="per-channel decay: prefill B=4 H=16 T=4096 d=128 bf16 (chunkwise, two "
                         "passes; and token-serial); decode step B=256 H=32 d=128 (fp32 state "
                         "in place)",
                prefill_tokens_per_s=round(4 * 4096 / (ms_pre * 1e-3), 1),
                prefill_ms=round(ms_pre, 4),
                **{"prefill_GB/s": round(pre_bytes / (ms_pre * 1e-3) / 1e9, 1)},
                serial_prefill_tokens_per_s=round(4 * 4096 / (ms_serial * 1e-3), 1),
                serial_prefill_ms=round(ms_serial, 4), decode_us=round(ms_dec * 1e3, 2),
                decode_bytes=nbytes, **{"decode_GB/s": round(gbs, 1)},
                decode_frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))


def bench_seqpar(gdn, inputs, steps, warmup):
    """One long sequence (B=1, H=16, T=32768, d=128, bf16): the plain two-pass
    prefill (16 (sequence, head) pairs = 64 chain workgroups on 256 CUs)
    against the sequence-parallel prefill with 3 to 16 segments."""
    import torch
    c = inputs.make_prefill(seed=92, B=1, T=32768, H=16)
    d = lambda t: t.cuda().contiguous()
    q, k, v, g, beta = (d(x) for x in (c.q, c.k, c.v, c.g, c.beta))
    fin = torch.empty((1, 16, 128, 128), dtype=torch.float32, device="cuda")
    o = torch.empty_like(v)
    ws = torch.empty(gdn.gdn_prefill_workspace_size(1, 32768, 16, 128, 128, 1, False,
                                                    torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    ms_plain = event_time(lambda i: gdn.gdn_prefill(q, k, v, g, beta, None, fin, o,
                                                    scale=c.scale, workspace=ws),
                          max(5, steps // 4), 3)
    res = dict(workload="one sequence B=1 H=16 T=32768 d=128 bf16",
               plain_ms=round(ms_plain, 4),
               plain_tokens_per_s=round(32768 / (ms_plain * 1e-3), 1))
    for P in (3, 4, 5, 8, 16):
        wsp = torch.empty(gdn.gdn_prefill_seqpar_workspace_size(1, 32768, 16, 128, 128, 1, False,
                                                                P, torch.bfloat16),
                          dtype=torch.uint8, device="cuda")
        ms = event_time(lambda i: gdn.gdn_prefill_seqpar(q, k, v, g, beta, P, None, fin, o,
                                                         scale=c.scale, workspace=wsp),
                        max(5, steps // 4), 3)
        res[f"segments_{P}_ms"] = round(ms, 4)
        res[f"segments_{P}_tokens_per_s"] = round(32768 / (ms * 1e-3), 1)
        del wsp
    return res


def bench_mixer(gdn, inputs, steps, warmup):
    import torch
    c = inputs.make_mixer()
    d = lambda t: t.cuda().contiguous()
    raw = [d(x) for x in (c.q_raw, c.k_raw, c.v_raw, c.conv_w, c.a, c.b)]
    A, z = d(c.A), d(c.z)
    B, T, H, D = c.q_raw.shape
    outs = (torch.empty_like(raw[0]), torch.empty_like(raw[1]), torch.empty_like(raw[2]),
            torch.empty((B, T, H), dtype=torch.float32, device="cuda"),
            torch.empty((B, T, H), dtype=torch.float32, device="cuda"))
    y = torch.empty_like(raw[2])
    out = torch.empty_like(y)
    # the norm weight as a model passes it (the workload's weight is ones)
    norm_w = torch.ones(D, dtype=torch.float32, device="cuda")

    def pro(i):
        gdn.gdn_mixer_prologue(*raw, A, out=outs)

    ws = torch.empty(gdn.gdn_prefill_workspace_size(B, T, H, D, D, B, False, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def core(i):
        gdn.gdn_prefill(*outs, o=y, scale=c.scale, workspace=ws)

    def epi(i):
        gdn.gdn_mixer_epilogue(y, z, norm_w=norm_w, out=out, eps=c.eps)

    def full(i):
        pro(i); core(i); epi(i)
    # the whole step first runs for DEVICE_WARMUP_S, as for the prefill
    # value: on fresh buffers the first calls run slow (three warm-up calls
    # read 1.02 ms per step where the steady state is 0.87)
    n_dev_warm = device_warmup(full)
    ms_full = event_time(full, max(10, steps // 2), 3)
    ms_pro = event_time(pro, max(10, steps // 2), 3)
    ms_core = event_time(core, max(10, steps // 2), 3)
    ms_epi = event_time(epi, max(10, steps // 2), 3)
    pro_bytes = B * T * H * (D * 2 * 3 * 2 + 2 * 2 + 4 * 2)   # q,k,v in+out, a,b in, g,beta out
    epi_bytes = B * T * H * D * 2 * 3
    return dict(workload="token mixer B=8 T=8192 H=16 d=128 bf16: conv+SiLU, L2-norm, gates -> "
                         "chunked prefill -> gated RMSNorm",
                tokens_per_s=round(B * T / (ms_full * 1e-3), 1), ms_per_step=round(ms_full, 4),
                ms_prologue=round(ms_pro, 4), ms_prefill=round(ms_core, 4),
                ms_epilogue=round(ms_epi, 4),
                prologue_GBps=round(pro_bytes / (ms_pro * 1e-3) / 1e9, 1),
                epilogue_GBps=round(epi_bytes / (ms_epi * 1e-3) / 1e9, 1),
                device_warmup_steps=n_dev_warm)


def bench_varlen(gdn, inputs, steps, warmup):
    import torch
    c = inputs.make_varlen()
    d = lambda t: t.cuda().contiguous()
    q, k, v, g, beta, s0, cu = (d(x) for x in (c.q, c.k, c.v, c.g, c.beta, c.s0, c.cu_seqlens))
    fin = torch.empty_like(s0)
    o = torch.empty_like(v)
    N = cu.numel() - 1
    ws = torch.empty(gdn.gdn_prefill_workspace_size(1, q.shape[1], q.shape[2], 128, 128, N, True,
                                                    torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def step(i):
        gdn.gdn_prefill(q, k, v, g, beta, s0, fin, o, cu_seqlens=cu, scale=c.scale, workspace=ws)
    # a longer warm-up than the other workloads: the first of these 1.2 ms
    # calls after the buffers are allocated run ~10% slower for ~20 calls
    ms = event_time(step, max(5, steps // 4), 25)
    total = int(c.cu_seqlens[-1])
    res = dict(workload="packed prefill H=32 d=128 bf16, 8 sequences log-uniform in [512, 65536], "
                        "non-zero initial states",
               lengths=c.meta["lengths"], tokens_per_s=round(total / (ms * 1e-3), 1),
               ms_per_step=round(ms, 4),
               longest_sequence_tokens_per_s=round(max(c.meta["lengths"]) / (ms * 1e-3), 1))
    del ws
    # the same call through the sequence-parallel path, the longest sequence
    # cut into P segments (P = 1: every sequence whole)
    for P in (1, 2, 4):
        wsp = torch.empty(gdn.gdn_prefill_seqpar_workspace_size(1, q.shape[1], q.shape[2], 128,
                                                                128, N, True, P, torch.bfloat16),
                          dtype=torch.uint8, device="cuda")
        ms = event_time(lambda i: gdn.gdn_prefill_seqpar(q, k, v, g, beta, P, s0, fin, o,
                                                         cu_seqlens=cu, scale=c.scale,
                                                         workspace=wsp),
                        max(5, steps // 4), 10)
        res[f"seqpar_{P}_ms"] = round(ms, 4)
        res[f"seqpar_{P}_tokens_per_s"] = round(total / (ms * 1e-3), 1)
        del wsp
    return res


def bench_copy(steps, warmup, nbytes=1 << 30):
    """A plain device copy of known size: the calibration kernel for the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    ms = event_time(lambda i: dst.copy_(src), steps, warmup)
    return dict(bytes_read=nbytes, bytes_written=nbytes, ms=round(ms, 4),
                GBps=round(2 * nbytes / (ms * 1e-3) / 1e9, 1))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(runs=3):
    """fp64 oracle on the prefill workload's host arrays (all 4 x 16 chains of
    4096 tokens): one untimed run, then the median of `runs` timed runs. The
    oracle runs its OpenMP loop over the (sequence, head) pairs on every
    thread it is given (`cores`)."""
    import oracle
    from gated_deltanet_recurrence_amd import inputs
    c = inputs.make_prefill()
    oracle.gdn_recurrent(c.q, c.k, c.v, c.g, c.beta, None, None, c.scale)
    times = []
    for _ in range(runs):
        t = time.perf_counter()
        oracle.gdn_recurrent(c.q, c.k, c.v, c.g, c.beta, None, None, c.scale)
        times.append(time.perf_counter() - t)
    med = _median(times)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"value": round(c.B * c.T / med, 1), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "host_cpus": os.cpu_count(), "host_cpus_usable": affinity,
            "cpu_model": _cpu_model(),
            "run_seconds": [round(x, 3) for x in times],
            "sample": f"the whole prefill workload (B=4, T=4096, H=16, d=128), fp64 token "
                      f"recurrence: one untimed run, then the median of {runs} timed runs"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="prefill,decode,decode_mixer,channel,mixer,varlen,seqpar,cpu",
                    help="comma list of: prefill, decode, decode_mixer, channel, mixer, varlen, "
                         "seqpar, cpu, copy")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "heads and sequences shard across GPUs with no communication, so the per-GPU "
              "figure is the one-GPU figure", file=sys.stderr)
        sys.exit(2)
    import torch
    import gated_deltanet_recurrence_amd as gdn
    from gated_deltanet_recurrence_amd import inputs
    gdn.load()
    which = set(args.only.split(","))
    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic (seeded; q,k unit Gaussian, v N(0,1), "
                      "log(alpha) = -A softplus(N(0,1)), beta = sigmoid(N(0,1)))"}
    if "prefill" in which:
        p = bench_prefill(gdn, inputs, args.steps, args.warmup)
        sec = p["ms"] * 1e-3
        chain_dominant = p["ms_chain"] >= p["ms_prep"]
        kname = "chunk_chain_kernel" if chain_dominant else "chunk_solve_kernel"
        k_ms = p["ms_chain"] if chain_dominant else p["ms_prep"]
        k_med = p["med_chain"] if chain_dominant else p["med_prep"]
        # the method's bytes (1032 B per token-head plus the final states),
        # over the dominant kernel's average launch
        achieved = p["bytes"] / (k_ms * 1e-3) / 1e9
        k_flops = p["flops"] / (k_ms * 1e-3) / 1e12
        traffic, why = measured_traffic(kname)
        result.update({
            "value": round(p["tokens"] / sec, 1), "unit": "tokens/s",
            "ms_per_step": round(p["ms"], 5),
            "timing": {"ms_per_step_from_idle": round(p["ms_idle"], 5),
                       "tokens_per_s_from_idle": round(p["tokens"] / (p["ms_idle"] * 1e-3), 1),
                       "device_warmup_steps": p["n_dev_warm"],
                       "note": "value and ms_per_step: K steps timed after the device has run the "
                               f"same step for {DEVICE_WARMUP_S} s and then the W warm-up steps "
                               "(its steady state); from idle: the same K steps timed after the "
                               "W warm-up steps only, when the process starts"},
            "config": {"workload": "chunked prefill B=4 H=16 T=4096 d_k=d_v=128, bf16 q/k/v, "
                                   "fp32 gates and state, zero initial state, 64-token chunks",
                       "global_batch": 4, "seq_len": 4096, "heads": 16, "head_dim": 128,
                       "parallelism": "single GPU"},
            "roofline": {"kernel": kname, "bound": "hbm",
                         "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                         "traffic_note": why,
                         "algorithmic_bytes_per_launch": p["bytes"],
                         "algorithmic_bytes_note": "1032 B per token-head (q, k, v, o bf16; g, "
                                                   "beta fp32) plus the fp32 final states",
                         "overhead_bytes": p["ws_bytes"] + p["reread_bytes"],
                         "overhead_note": "workspace T diag(beta) written and read back (96 B "
                                          "each way per token-head) and k, g, beta read a "
                                          "second time by the solve pass (264 B)",
                         "mfma_tflops": round(k_flops, 2),
                         "mfma_frac_of_bf16_peak": round(k_flops / BF16_PEAK_TFLOPS, 4),
                         "avg_launch_us": round(k_ms * 1e3, 2),
                         "avg_launch_note": "launches back to back between one pair of HIP "
                                            "events on the launch stream, as in a step",
                         "launches_timed": p["n_launch"],
                         "isolated_median_launch_us": round(k_med * 1e3, 2),
                         "isolated_note": "median over per-launch event pairs; the events "
                                          "between launches lengthen each launch",
                         "other_kernel_avg_launch_us": round((p["ms_prep"] if chain_dominant
                                                              else p["ms_chain"]) * 1e3, 2),
                         "other_kernel_isolated_median_launch_us": round(
                             (p["med_prep"] if chain_dominant else p["med_chain"]) * 1e3, 2)},
            "path": {"algorithmic_bytes_per_step": p["bytes"],
                     "GB/s": round(p["bytes"] / sec / 1e9, 1),
                     "frac_of_hbm_peak": round(p["bytes"] / sec / 1e9 / HBM_PEAK_GBS, 4),
                     "mfma_algorithmic_tflops": round(p["flops"] / sec / 1e12, 2),
                     "mfma_frac_of_bf16_peak": round(p["flops"] / sec / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "bytes_moved_per_step_by_design": p["chain_bytes"] + p["prep_bytes"]},
            "one_pass": {"ms_per_step": round(p["ms_one_pass"], 5),
                         "tokens_per_s": round(p["tokens"] / (p["ms_one_pass"] * 1e-3), 1)},
        })
    else:
        result.update({"value": None, "unit": "tokens/s", "ms_per_step": None,
                       "config": {"workload": "partial run: " + args.only}})
    if "decode" in which:
        result["decode"] = bench_decode(gdn, inputs, args.steps, args.warmup)
    if "decode_mixer" in which:
        result["decode_mixer"] = bench_decode_mixer(gdn, inputs, args.steps, args.warmup)
    if "channel" in which:
        result["channel_gated"] = bench_channel_gated(gdn, inputs, args.steps, args.warmup)
    if "mixer" in which:
        result["mixer"] = bench_mixer(gdn, inputs, args.steps, args.warmup)
    if "varlen" in which:
        result["varlen"] = bench_varlen(gdn, inputs, args.steps, args.warmup)
    if "seqpar" in which:
        result["seqpar"] = bench_seqpar(gdn, inputs, args.steps, args.warmup)
    if "copy" in which:
        result["copy_calibration"] = bench_copy(args.steps, args.warmup)
    if "cpu" in which:
        result["cpu_baseline"] = cpu_baseline()
    torch.cuda.synchronize()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
