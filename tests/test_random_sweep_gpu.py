"""GPU parity over seeded random shapes: 120 cases, each through the two-pass,
one-pass and sequence-parallel chunk paths, against the fp64 oracle at the
bf16 bar ("Overwrite and Forget", section 7: the chunkwise forms must agree
with the token recurrence).

A case draws 1-6 value heads with a random divisor as query/key heads. It is
either a batch of 1-3 rows of 1-900 tokens (with or without initial states)
or 1-7 packed sequences whose lengths mix 0, 1, 2, 63, 64, 65, 127, 128 and
random ones up to 900. In half of the cases the log-decays are scaled by
0.01, so that the state carries across chunks. The sequence-parallel path
cuts the longest sequence into 1-6 segments.
"""
import random

import pytest
import torch

import oracle
import gated_deltanet_recurrence_amd as gdn
from gated_deltanet_recurrence_amd import inputs
from parity import TOL_BF16, dev, host64, o_err, o_err_packed, report, s_err

pytestmark = pytest.mark.gpu

N_CASES = 120


def _case(rng, i):
    H = rng.choice([1, 2, 3, 4, 6])
    Hk = rng.choice([d for d in range(1, H + 1) if H % d == 0])
    seed = 7000 + i
    if rng.random() < 0.5:
        lengths = [rng.choice([0, 1, 2, 63, 64, 65, 127, 128, rng.randint(1, 900)])
                   for _ in range(rng.randint(1, 7))]
        if sum(lengths) == 0:
            lengths[0] = 5
        c = inputs.make_varlen(seed=seed, H=H, lengths=lengths, Hk=Hk)
    else:
        c = inputs.make_prefill(seed=seed, B=rng.randint(1, 3), T=rng.randint(1, 900), H=H,
                                with_state=rng.random() < 0.5, Hk=Hk)
    if rng.random() < 0.5:
        c.g = (c.g * 0.01).contiguous()
    return c


def test_random_shapes_all_chunk_paths():
    rng = random.Random(20261202)
    worst = {"two_pass": 0.0, "one_pass": 0.0, "seqpar": 0.0}
    bad = []
    for i in range(N_CASES):
        c = _case(rng, i)
        H = c.H
        q, k = (oracle.expand_heads(host64(x), H) for x in (c.q, c.k))
        o_ref, s_ref = oracle.gdn_recurrent(q, k, c.v, c.g, c.beta, c.s0,
                                            cu_seqlens=c.cu_seqlens, scale=c.scale)
        cu = None if c.cu_seqlens is None else [int(x) for x in c.cu_seqlens.tolist()]
        segments = rng.randint(1, 6)
        for path in worst:
            fin = torch.empty((c.N, H, c.d_v, c.d_k), dtype=torch.float32, device="cuda:0")
            args = (dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta))
            if path == "seqpar":
                o, _ = gdn.gdn_prefill_seqpar(*args, segments, dev(c.s0), fin,
                                              cu_seqlens=dev(c.cu_seqlens), scale=c.scale)
            else:
                o, _ = gdn.gdn_prefill(*args, dev(c.s0), fin, cu_seqlens=dev(c.cu_seqlens),
                                       scale=c.scale,
                                       workspace="auto" if path == "two_pass" else None)
            torch.cuda.synchronize()
            eo = o_err_packed(o.cpu(), o_ref, cu) if cu else o_err(o.cpu(), o_ref)
            es = s_err(fin.cpu(), s_ref)
            e = max(float(eo), float(es))
            worst[path] = max(worst[path], e)
            if not e <= TOL_BF16:
                bad.append(f"case {i} {path}: o={float(eo):.3e} state={float(es):.3e} "
                           f"shape={tuple(c.q.shape)} H={H} cu={cu}")
    report(f"random sweep ({N_CASES} cases)", **worst)
    assert not bad, bad
