"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every input is seeded and synthetic (gated_deltanet_recurrence_amd.inputs);
the oracle receives exactly the values the GPU receives (bf16/fp32 upcast to
fp64). Tolerances: max over (sequence, head) slices of the inf-norm relative
error, 1e-4 for fp32 inputs and 2e-2 for bf16 inputs with an fp32 state, on
outputs and final states separately.
"""
import numpy as np
import pytest
import torch

import oracle
import gated_deltanet_recurrence_amd as gdn
from gated_deltanet_recurrence_amd import inputs
from parity import (TOL_BF16, TOL_F32, dev, host64, o_err, o_err_packed, report, s_err)

pytestmark = pytest.mark.gpu


def _tol(case):
    return TOL_F32 if case.dtype == "f32" else TOL_BF16


# gdn_prefill's two execution paths of the MFMA chunk algorithm: with a
# workspace (two passes: all chunks' triangular solves in parallel, then the
# state recurrence) and without (one pass)
PATHS = ["two_pass", "one_pass"]
WS = {"two_pass": "auto", "one_pass": None}


def run_prefill(case, entry=None, with_final=True, init=True, path="two_pass"):
    s0 = dev(case.s0) if (init and case.s0 is not None) else None
    fin = torch.empty((case.N, case.H, case.d_v, case.d_k), dtype=torch.float32,
                      device="cuda:0") if with_final else None
    extra = {} if entry is not None else {"workspace": WS[path]}
    entry = entry or gdn.gdn_prefill
    o, _ = entry(dev(case.q), dev(case.k), dev(case.v), dev(case.g), dev(case.beta), s0, fin,
                 cu_seqlens=dev(case.cu_seqlens), scale=case.scale, **extra)
    torch.cuda.synchronize()
    return o, fin


def oracle_prefill(case, init=True):
    return oracle.gdn_recurrent(case.q, case.k, case.v, case.g, case.beta,
                                case.s0 if init else None, case.cu_seqlens, case.scale)


# --- the five workloads ------------------------------------------------------

def test_tiny_fp32():
    """B=1, H=1, T=64, d=16, fp32: the fp32 path meets 1e-4."""
    c = inputs.make_tiny()
    o, fin = run_prefill(c)
    o_ref, s_ref = oracle_prefill(c)
    eo, es = o_err(o, o_ref), s_err(fin, s_ref)
    report("tiny fp32", o=eo, state=es)
    assert eo <= TOL_F32 and es <= TOL_F32


@pytest.fixture(scope="module")
def prefill_full():
    c = inputs.make_prefill()
    return c, oracle_prefill(c)


@pytest.mark.parametrize("path", PATHS)
def test_prefill_full_size(prefill_full, path):
    """B=4, H=16, T=4096, d=128, bf16, zero initial state: all 64 chains."""
    c, (o_ref, s_ref) = prefill_full
    o, fin = run_prefill(c, path=path)
    eo, es = o_err(o, o_ref), s_err(fin, s_ref)
    report(f"prefill B4 H16 T4096 {path}", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16 and eo.row <= TOL_BF16


def test_decode_full_size():
    """B=256, H=32, d=128: one in-place step of the 512 MiB fp32 state."""
    c = inputs.make_decode()
    st = dev(c.s0)
    o = gdn.gdn_decode_step(dev(c.q[:, 0]), dev(c.k[:, 0]), dev(c.v[:, 0]), dev(c.g[:, 0]),
                            dev(c.beta[:, 0]), st, scale=c.scale)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(c)
    eo, es = o_err(o[:, None], o_ref), s_err(st, s_ref)
    report("decode B256 H32", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_mixer_full_size_sampled():
    """B=8, T=8192, H=16, d=128 bf16 raw inputs through prologue -> prefill ->
    epilogue on the GPU; the oracle recomputes two batch rows x three heads
    from the raw inputs (heads never mix, so a slice is exact)."""
    c = inputs.make_mixer()
    q, k, v, g, beta = gdn.gdn_mixer_prologue(dev(c.q_raw), dev(c.k_raw), dev(c.v_raw),
                                              dev(c.conv_w), dev(c.a), dev(c.b), dev(c.A))
    y, _ = gdn.gdn_prefill(q, k, v, g, beta, scale=c.scale)
    out = gdn.gdn_mixer_epilogue(y, dev(c.z), eps=c.eps)
    torch.cuda.synchronize()
    rows, heads = [0, 7], [0, 9, 15]
    ref, mid = oracle.mixer(c.q_raw, c.k_raw, c.v_raw, c.z, c.a, c.b, c.conv_w, c.A,
                            scale=c.scale, eps=c.eps, heads=heads, rows=rows,
                            return_intermediates=True)
    sel = lambda t: t[rows][:, :, heads]
    e_out = o_err(sel(out.cpu()), ref)
    e_q = o_err(sel(q.cpu()), mid["q"])
    e_k = o_err(sel(k.cpu()), mid["k"])
    e_v = o_err(sel(v.cpu()), mid["v"])
    e_g = float(np.abs(host64(sel(g.cpu())) - mid["g"]).max() / np.abs(mid["g"]).max())
    e_b = float(np.abs(host64(sel(beta.cpu())) - mid["beta"]).max())
    e_y = o_err(sel(y.cpu()), mid["y"])
    report("mixer B8 T8192 H16", out=e_out, q=e_q, k=e_k, v=e_v, g=e_g, beta=e_b, y=e_y)
    assert max(e_q, e_k, e_v) <= TOL_BF16 and e_g <= 1e-5 and e_b <= 1e-6
    assert e_y <= TOL_BF16 and e_out <= TOL_BF16


VARLEN_HEADS = [0, 5, 17, 31]


@pytest.fixture(scope="module")
def varlen_full():
    c = inputs.make_varlen()
    ref = oracle.gdn_recurrent_heads(c.q, c.k, c.v, c.g, c.beta, VARLEN_HEADS, c.s0,
                                     c.cu_seqlens, c.scale, nthreads=0)
    return c, ref


@pytest.mark.parametrize("path", PATHS)
def test_varlen_full_size_sampled(varlen_full, path):
    """H=32, d=128, 8 packed sequences (lengths log-uniform in [512, 65536]),
    non-zero initial states: every sequence, four heads."""
    c, (outs, s_ref) = varlen_full
    o, fin = run_prefill(c, path=path)
    cu = [int(x) for x in c.cu_seqlens.tolist()]
    o_h = o.cpu()[:, :, VARLEN_HEADS]
    eo = max(o_err(o_h[:, a:b], r) for (a, b), r in zip(zip(cu[:-1], cu[1:]), outs) if b > a)
    es = s_err(fin.cpu()[:, VARLEN_HEADS], s_ref)
    report(f"varlen {path} lengths={c.meta['lengths']}", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


# --- smaller shapes: tiles, ragged tails, edge cases ------------------------

@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 130, 257])
@pytest.mark.parametrize("with_state", [False, True])
def test_prefill_ragged_bf16(T, with_state, path):
    c = inputs.make_prefill(seed=1000 + T, B=2, T=T, H=3, d=128, with_state=with_state)
    o, fin = run_prefill(c, path=path)
    o_ref, s_ref = oracle_prefill(c)
    eo, es = o_err(o, o_ref), s_err(fin, s_ref)
    report(f"prefill bf16 T={T} state={with_state} {path}", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_head_dims(d, dtype):
    c = inputs.make_prefill(seed=2000 + d, B=2, T=77, H=2, d=d, dtype=dtype, with_state=True)
    o, fin = run_prefill(c)
    o_ref, s_ref = oracle_prefill(c)
    eo, es = o_err(o, o_ref), s_err(fin, s_ref)
    report(f"prefill {dtype} d={d}", o=eo, state=es)
    tol = _tol(c)
    assert eo <= tol and es <= tol


def test_prefill_fp32_d128():
    """fp32 inputs at d=128 meet the fp32 tolerance."""
    c = inputs.make_prefill(seed=7, B=1, T=300, H=2, d=128, dtype="f32", with_state=True)
    o, fin = run_prefill(c)
    o_ref, s_ref = oracle_prefill(c)
    eo, es = o_err(o, o_ref), s_err(fin, s_ref)
    report("prefill f32 d=128", o=eo, state=es)
    assert eo <= TOL_F32 and es <= TOL_F32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_small(dtype):
    c = inputs.make_decode(seed=31, B=5, H=3, d=128, dtype=dtype)
    st = dev(c.s0)
    o = gdn.gdn_decode_step(dev(c.q[:, 0]), dev(c.k[:, 0]), dev(c.v[:, 0]), dev(c.g[:, 0]),
                            dev(c.beta[:, 0]), st, scale=c.scale)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(c)
    eo, es = o_err(o[:, None], o_ref), s_err(st, s_ref)
    report(f"decode {dtype}", o=eo, state=es)
    assert eo <= _tol(c) and es <= _tol(c)


@pytest.mark.parametrize("d", [16, 32, 64])
def test_decode_head_dims(d):
    c = inputs.make_decode(seed=40 + d, B=3, H=2, d=d, dtype="f32")
    st = dev(c.s0)
    o = gdn.gdn_decode_step(dev(c.q[:, 0]), dev(c.k[:, 0]), dev(c.v[:, 0]), dev(c.g[:, 0]),
                            dev(c.beta[:, 0]), st, scale=c.scale)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(c)
    assert o_err(o[:, None], o_ref) <= TOL_F32 and s_err(st, s_ref) <= TOL_F32


@pytest.mark.parametrize("path", PATHS)
def test_packed_with_empty_and_tiny_sequences(path):
    """Packed sequences including empty ones and ones shorter than a chunk; an
    empty sequence returns its initial state."""
    lengths = [0, 1, 64, 0, 3, 129, 70]
    c = inputs.make_varlen(seed=55, H=2, d=128, lengths=lengths)
    o, fin = run_prefill(c, path=path)
    o_ref, s_ref = oracle_prefill(c)
    cu = [int(x) for x in c.cu_seqlens.tolist()]
    eo, es = o_err_packed(o, o_ref, cu), s_err(fin, s_ref)
    report(f"packed with empties {path}", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16
    for n, L in enumerate(lengths):
        if L == 0:
            assert torch.equal(fin[n].cpu(), c.s0[n])


_AGREE_CASES = [
    ("prefill B=4 T=4096 H=16", lambda: inputs.make_prefill()),
    ("B=3 T=700 H=3 with states", lambda: inputs.make_prefill(seed=15, B=3, T=700, H=3, d=128,
                                                               with_state=True)),
    ("B=1 T=199 H=4 H_k=2", lambda: inputs.make_prefill(seed=2, B=1, T=199, H=4, d=128, Hk=2)),
    ("B=3 T=65 H=2 H_k=1 with states", lambda: inputs.make_prefill(seed=3, B=3, T=65, H=2, d=128,
                                                                    Hk=1, with_state=True)),
    ("packed 0,1,64,3,129,257 H=2", lambda: inputs.make_varlen(seed=58, H=2, d=128,
                                                                lengths=[0, 1, 64, 3, 129, 257])),
]


@pytest.mark.parametrize("name,make", _AGREE_CASES, ids=[c[0] for c in _AGREE_CASES])
def test_two_pass_and_one_pass_agree_bit_for_bit(name, make):
    """The one-pass kernel solves each chunk on two of its own waves with the
    solve pass's arithmetic and forms P^T on its output waves with the code the
    two-pass chain runs on its staging waves: the two paths' outputs and final
    states are identical bit for bit (each is held to the oracle by the tests
    above)."""
    c = make()
    o2, f2 = run_prefill(c, path="two_pass")
    o1, f1 = run_prefill(c, path="one_pass")
    same_o = torch.equal(o2.view(torch.int16), o1.view(torch.int16))
    same_s = torch.equal(f2.view(torch.int32), f1.view(torch.int32))
    print(f"[agree] {name}: outputs bit-identical {same_o}, states bit-identical {same_s}",
          flush=True)
    assert same_o and same_s


def _many_lengths(n=300, seed=57):
    rnd = np.random.default_rng(seed)
    lengths = [int(x) for x in rnd.integers(0, 150, size=n)]
    lengths[7] = 700                       # one sequence of 11 chunks among short ones
    return lengths


@pytest.mark.parametrize("path", PATHS)
def test_packed_more_sequences_than_ranked(path):
    """300 packed sequences (0 to 149 tokens, one of 700): more than the 256
    that the chain pass deals longest first, so its index-order dealing runs;
    every sequence against the oracle, empty ones keep their state."""
    lengths = _many_lengths()
    c = inputs.make_varlen(seed=56, H=2, d=128, lengths=lengths)
    o, fin = run_prefill(c, path=path)
    o_ref, s_ref = oracle_prefill(c)
    cu = [int(x) for x in c.cu_seqlens.tolist()]
    eo, es = o_err_packed(o, o_ref, cu), s_err(fin, s_ref)
    report(f"packed 300 sequences {path}", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16
    for n, L in enumerate(lengths):
        if L == 0:
            assert torch.equal(fin[n].cpu(), c.s0[n])


@pytest.mark.parametrize("segments", [1, 3])
def test_seqpar_more_sequences_than_ranked(segments):
    """The same 300 packed sequences through the sequence-parallel path: its
    plan deals jobs in index order above 256 sequences; with 3 segments the
    700-token sequence has middle segments."""
    lengths = _many_lengths()
    c = inputs.make_varlen(seed=56, H=2, d=128, lengths=lengths)
    fin = torch.empty((len(lengths), 2, 128, 128), dtype=torch.float32, device="cuda:0")
    o, _ = gdn.gdn_prefill_seqpar(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta), segments,
                                  dev(c.s0), fin, cu_seqlens=dev(c.cu_seqlens), scale=c.scale)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(c)
    cu = [int(x) for x in c.cu_seqlens.tolist()]
    eo, es = o_err_packed(o, o_ref, cu), s_err(fin, s_ref)
    report(f"seqpar packed 300 sequences segments={segments}", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("path", PATHS)
def test_zero_length_batch(path):
    """T = 0: nothing to compute; the final state is the initial state."""
    c = inputs.make_prefill(seed=3, B=2, T=0, H=2, d=128, with_state=True)
    o, fin = run_prefill(c, path=path)
    assert o.numel() == 0 and torch.equal(fin.cpu(), c.s0)


@pytest.mark.parametrize("path", PATHS)
def test_gate_special_cases(path):
    """beta = 0, alpha = 1 leaves the state unchanged; beta = 0 alone scales it."""
    c = inputs.make_prefill(seed=4, B=1, T=100, H=2, d=128, with_state=True)
    c.beta.zero_()
    c.g.zero_()
    _, fin = run_prefill(c, path=path)
    assert s_err(fin, host64(c.s0)) <= 1e-6
    c = inputs.make_prefill(seed=5, B=1, T=100, H=2, d=128, with_state=True)
    c.beta.zero_()
    c.g.mul_(0.02)                     # keep the accumulated decay well above denormals
    _, fin = run_prefill(c, path=path)
    decay = np.exp(host64(c.g)[0].sum(axis=0))            # [H]
    assert s_err(fin, host64(c.s0) * decay[None, :, None, None]) <= 1e-4


# --- execution-path consistency ---------------------------------------------

def test_split_resume():
    """prefill(T1) -> state -> prefill(T2, state) equals prefill(T1 + T2), and
    prefill followed by decode steps equals a longer prefill."""
    c = inputs.make_prefill(seed=9, B=2, T=200, H=2, d=128, with_state=True)
    o_all, f_all = run_prefill(c)
    T1 = 77
    fin1 = torch.empty_like(f_all)
    o1, _ = gdn.gdn_prefill(dev(c.q[:, :T1]), dev(c.k[:, :T1]), dev(c.v[:, :T1]),
                            dev(c.g[:, :T1]), dev(c.beta[:, :T1]), dev(c.s0), fin1, scale=c.scale)
    fin2 = torch.empty_like(f_all)
    o2, _ = gdn.gdn_prefill(dev(c.q[:, T1:196]), dev(c.k[:, T1:196]), dev(c.v[:, T1:196]),
                            dev(c.g[:, T1:196]), dev(c.beta[:, T1:196]), fin1, fin2,
                            scale=c.scale)
    st = fin2.clone()
    outs = []
    for t in range(196, 200):
        outs.append(gdn.gdn_decode_step(dev(c.q[:, t]), dev(c.k[:, t]), dev(c.v[:, t]),
                                        dev(c.g[:, t]), dev(c.beta[:, t]), st, scale=c.scale))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(c)
    o_cat = torch.cat([o1, o2, torch.stack(outs, 1)], 1)
    eo, es = o_err(o_cat, o_ref), s_err(st, s_ref)
    report("split/resume", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16
    assert o_err(o_cat, host64(o_all)) <= TOL_BF16


def test_in_place_state_continuation():
    """initial_state and final_state may be the same buffer."""
    c = inputs.make_prefill(seed=12, B=2, T=90, H=2, d=128, with_state=True)
    st = dev(c.s0)
    gdn.gdn_prefill(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta), st, st, scale=c.scale)
    torch.cuda.synchronize()
    _, s_ref = oracle_prefill(c)
    assert s_err(st, s_ref) <= TOL_BF16


def test_chunk_matches_recurrent_on_gpu():
    """The chunkwise path and the token-serial path agree ("parallel, chunkwise
    and recurrent paths must agree" - Overwrite and Forget, section 7)."""
    c = inputs.make_prefill(seed=13, B=2, T=333, H=4, d=128, with_state=True)
    o_c, f_c = run_prefill(c)
    o_r, f_r = run_prefill(c, entry=gdn.gdn_prefill_recurrent)
    assert o_err(o_c, host64(o_r)) <= TOL_BF16 and s_err(f_c, host64(f_r)) <= TOL_BF16


@pytest.mark.parametrize("path", PATHS)
def test_deterministic(path):
    c = inputs.make_prefill(seed=14, B=2, T=300, H=2, d=128, with_state=True)
    o1, f1 = run_prefill(c, path=path)
    o2, f2 = run_prefill(c, path=path)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_workspace_reuse_and_dirty_contents():
    """A caller-owned workspace full of garbage, reused by calls of different
    sizes, gives the results of a fresh one."""
    big = inputs.make_prefill(seed=16, B=2, T=500, H=3, d=128, with_state=True)
    small = inputs.make_varlen(seed=17, H=3, d=128, lengths=[5, 0, 130, 64])
    need = max(gdn.gdn_prefill_workspace_size(2, 500, 3, 128, 128, 2, False, torch.bfloat16),
               gdn.gdn_prefill_workspace_size(1, 199, 3, 128, 128, 4, True, torch.bfloat16))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda:0")   # NaN bf16 patterns
    for c in (big, small, big):
        s0 = dev(c.s0)
        fin = torch.empty_like(s0)
        o, _ = gdn.gdn_prefill(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta), s0, fin,
                               cu_seqlens=dev(c.cu_seqlens), scale=c.scale, workspace=ws)
        o_ref, f_ref = run_prefill(c, path="two_pass")
        assert torch.equal(o, o_ref) and torch.equal(fin, f_ref)


@pytest.mark.parametrize("H,d", [(2, 128), (20, 128), (3, 64)])
def test_prologue_packed_sequences(H, d):
    """The convolution history restarts at each packed sequence start, and the
    gates are right for head counts that leave a workgroup's head groups
    partly empty."""
    c = inputs.make_mixer(seed=21, B=1, T=300, H=H, d=d)
    cu = torch.tensor([0, 5, 5, 130, 300], dtype=torch.int32)
    q, k, v, g, beta = gdn.gdn_mixer_prologue(dev(c.q_raw), dev(c.k_raw), dev(c.v_raw),
                                              dev(c.conv_w), dev(c.a), dev(c.b), dev(c.A),
                                              cu_seqlens=dev(cu))
    torch.cuda.synchronize()
    _, mid = oracle.mixer(c.q_raw, c.k_raw, c.v_raw, c.z, c.a, c.b, c.conv_w, c.A,
                          scale=c.scale, cu_seqlens=cu.tolist(), return_intermediates=True)
    eq, ek, ev = o_err(q.cpu(), mid["q"]), o_err(k.cpu(), mid["k"]), o_err(v.cpu(), mid["v"])
    g_ref, b_ref = torch.as_tensor(mid["g"]), torch.as_tensor(mid["beta"])
    eg = float((g.cpu().double() - g_ref).abs().max() / g_ref.abs().max())
    eb = float((beta.cpu().double() - b_ref).abs().max() / b_ref.abs().max())
    report(f"prologue packed H={H} d={d}", q=eq, k=ek, v=ev, g=eg, beta=eb)
    assert eq <= TOL_BF16 and ek <= TOL_BF16 and ev <= TOL_BF16
    assert eg <= TOL_F32 and eb <= TOL_F32


def test_prepare_then_apply_equals_prefill():
    """gdn_prefill with a workspace is gdn_prefill_prepare then gdn_prefill_apply."""
    c = inputs.make_varlen(seed=18, H=2, d=128, lengths=[70, 0, 200, 1])
    N = c.cu_seqlens.numel() - 1
    ws = torch.empty(gdn.gdn_prefill_workspace_size(1, c.q.shape[1], 2, 128, 128, N, True,
                                                    torch.bfloat16),
                     dtype=torch.uint8, device="cuda:0")
    q, k, v, g, beta, s0, cu = (dev(x) for x in (c.q, c.k, c.v, c.g, c.beta, c.s0, c.cu_seqlens))
    gdn.gdn_prefill_prepare(q, k, g, beta, ws, cu_seqlens=cu)
    fin = torch.empty_like(s0)
    o, _ = gdn.gdn_prefill_apply(q, k, v, g, ws, s0, fin, cu_seqlens=cu, scale=c.scale)
    o_ref, f_ref = run_prefill(c, path="two_pass")
    assert torch.equal(o, o_ref) and torch.equal(fin, f_ref)


# --- grouped query/key heads (H_k < H) -----------------------------------------

@pytest.mark.parametrize("Hk", [1, 2])
@pytest.mark.parametrize("path", PATHS)
def test_prefill_grouped_heads(Hk, path):
    """H = 4 value heads reading H_k query/key heads (value head h uses key
    head h // (H / H_k)), bf16 d=128 on both chunk paths, several chunks and a
    ragged tail, non-zero initial state."""
    c = inputs.make_prefill(seed=61 + Hk, B=2, T=193, H=4, Hk=Hk, with_state=True)
    o, fin = run_prefill(c, path=path)
    o_ref, s_ref = oracle_prefill(c)
    eo, es = o_err(o, o_ref), s_err(fin, s_ref)
    report(f"grouped heads H4 Hk{Hk} {path}", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("path", PATHS)
def test_varlen_grouped_heads(path):
    """Packed sequences with grouped heads (H = 6, H_k = 3)."""
    c = inputs.make_varlen(seed=63, H=6, Hk=3, d=128, lengths=[130, 0, 64, 7, 200])
    o, fin = run_prefill(c, path=path)
    o_ref, s_ref = oracle_prefill(c)
    cu = [int(x) for x in c.cu_seqlens.tolist()]
    eo, es = o_err_packed(o, o_ref, cu), s_err(fin, s_ref)
    report(f"varlen grouped heads {path}", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 32)])
def test_prefill_recurrent_grouped_heads(dtype, d):
    """The token-serial kernel with grouped heads (fp32 1e-4, bf16 2e-2)."""
    c = inputs.make_prefill(seed=64, B=2, T=70, H=6, Hk=2, d=d, dtype=dtype, with_state=True)
    o, fin = run_prefill(c, entry=gdn.gdn_prefill_recurrent)
    o_ref, s_ref = oracle_prefill(c)
    eo, es = o_err(o, o_ref), s_err(fin, s_ref)
    report(f"recurrent grouped heads {dtype} d{d}", o=eo, state=es)
    assert eo <= _tol(c) and es <= _tol(c)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_grouped_heads(dtype):
    c = inputs.make_decode(seed=65, B=3, H=8, Hk=2, d=128, dtype=dtype)
    st = dev(c.s0)
    o = gdn.gdn_decode_step(dev(c.q[:, 0]), dev(c.k[:, 0]), dev(c.v[:, 0]), dev(c.g[:, 0]),
                            dev(c.beta[:, 0]), st, scale=c.scale)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(c)
    eo, es = o_err(o[:, None], o_ref), s_err(st, s_ref)
    report(f"decode grouped heads {dtype}", o=eo, state=es)
    assert eo <= _tol(c) and es <= _tol(c)


def test_mixer_grouped_heads():
    """Prologue -> prefill -> epilogue with H_k = 2 query/key heads and H = 4
    value heads: conv channels 2 H_k d + H d, gates per value head; the
    gated RMSNorm with a norm weight (seeded, U(0.5, 1.5) per channel)."""
    c = inputs.make_mixer(seed=66, B=2, T=150, H=4, Hk=2, d=128)
    nw = 0.5 + torch.rand(128, generator=torch.Generator().manual_seed(67))
    q, k, v, g, beta = gdn.gdn_mixer_prologue(dev(c.q_raw), dev(c.k_raw), dev(c.v_raw),
                                              dev(c.conv_w), dev(c.a), dev(c.b), dev(c.A))
    y, _ = gdn.gdn_prefill(q, k, v, g, beta, scale=c.scale)
    out = gdn.gdn_mixer_epilogue(y, dev(c.z), norm_w=dev(nw), eps=c.eps)
    torch.cuda.synchronize()
    ref, mid = oracle.mixer(c.q_raw, c.k_raw, c.v_raw, c.z, c.a, c.b, c.conv_w, c.A,
                            norm_w=nw, scale=c.scale, eps=c.eps, return_intermediates=True)
    e_out, e_y = o_err(out.cpu(), ref), o_err(y.cpu(), mid["y"])
    e_q, e_k, e_v = o_err(q.cpu(), mid["q"]), o_err(k.cpu(), mid["k"]), o_err(v.cpu(), mid["v"])
    e_g = float(np.abs(host64(g.cpu()) - mid["g"]).max() / np.abs(mid["g"]).max())
    e_b = float(np.abs(host64(beta.cpu()) - mid["beta"]).max())
    report("mixer grouped heads", out=e_out, y=e_y, q=e_q, k=e_k, v=e_v, g=e_g, beta=e_b)
    assert max(e_q, e_k, e_v) <= TOL_BF16 and e_g <= 1e-5 and e_b <= 1e-6
    assert e_y <= TOL_BF16 and e_out <= TOL_BF16


# --- the fused single-token mixer step --------------------------------------------

@pytest.mark.parametrize("dtype,H,Hk,dk,dv", [("bf16", 4, 2, 128, 128), ("f32", 3, 3, 64, 32),
                                              ("bf16", 2, 1, 32, 256), ("f32", 4, 4, 16, 16)])
def test_decode_mixer_steps_continue_the_sequence(dtype, H, Hk, dk, dv):
    """T = 7 fused steps from an empty conv cache and a zero state on the GPU
    against the oracle's mixer over the same 7 tokens (every step's output),
    the final state, and the cache, which must hold the last three raw inputs
    bit for bit."""
    B, T = 2, 7
    gen = torch.Generator().manual_seed(71)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    rnd = lambda *shape, std=1.0: (torch.randn(shape, generator=gen) * std).to(td)
    qr, kr = rnd(B, T, Hk, dk), rnd(B, T, Hk, dk)
    vr, z = rnd(B, T, H, dv), rnd(B, T, H, dv)
    a, b = rnd(B, T, H), rnd(B, T, H)
    C = 2 * Hk * dk + H * dv
    w = rnd(C, 4, std=0.5)
    A = torch.rand(H, generator=gen) * 1.5 + 0.5
    dtb = torch.randn(H, generator=gen)
    nw = torch.rand(dv, generator=gen) + 0.5
    scale = dk ** -0.5
    ref, mid = oracle.mixer(qr, kr, vr, z, a, b, w, A, dt_bias=dtb, norm_w=nw, scale=scale,
                            return_intermediates=True)
    cache = torch.zeros((B, 3, C), dtype=td, device="cuda:0")
    st = torch.zeros((B, H, dv, dk), dtype=torch.float32, device="cuda:0")
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    errs = []
    for t in range(T):
        out = gdn.gdn_decode_mixer_step(dev(qr[:, t]), dev(kr[:, t]), dev(vr[:, t]), dev(w), cache,
                                        dev(a[:, t]), dev(b[:, t]), dev(A), dev(z[:, t]), st,
                                        dt_bias=dev(dtb), norm_w=dev(nw), scale=scale)
        torch.cuda.synchronize()
        errs.append(o_err(out.cpu()[:, None], ref[:, t:t + 1]))
    es = s_err(st, mid["s_final"])
    report(f"decode mixer steps {dtype} H{H} Hk{Hk} dk{dk} dv{dv}", out=max(errs), state=es)
    assert max(errs) <= tol and es <= tol
    raw = torch.cat([qr.reshape(B, T, -1), kr.reshape(B, T, -1), vr.reshape(B, T, -1)], 2)
    assert torch.equal(cache.cpu(), raw[:, T - 3:])


def test_decode_mixer_full_size_sampled():
    """B=256, H=32, d=128 bf16 (512 MiB state, a random conv cache): one fused
    step; the oracle recomputes four sequences (all heads) from the same
    inputs."""
    c = inputs.make_decode_mixer()
    cache, st = dev(c.conv_state), dev(c.state)
    out = gdn.gdn_decode_mixer_step(dev(c.q_raw), dev(c.k_raw), dev(c.v_raw), dev(c.conv_w),
                                    cache, dev(c.a), dev(c.b), dev(c.A), dev(c.z), st,
                                    scale=c.scale, eps=c.eps)
    torch.cuda.synchronize()
    rows = [0, 1, 128, 255]
    r = lambda x: x[rows]
    o_ref, s_ref, c_ref = oracle.mixer_decode_step(r(c.q_raw), r(c.k_raw), r(c.v_raw), r(c.z),
                                                   r(c.a), r(c.b), c.conv_w, r(c.conv_state),
                                                   c.A, r(c.state), scale=c.scale, eps=c.eps)
    eo = o_err(out.cpu()[rows][:, None], o_ref[:, None])
    es = s_err(st.cpu()[rows], s_ref)
    report("decode mixer B256 H32", out=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16
    assert torch.equal(cache.cpu()[rows], torch.from_numpy(c_ref).to(cache.dtype))


# --- per-channel decay (one rate per key channel) -----------------------------------

def _oracle_channel(c, init=True):
    return oracle.gdn_recurrent_channel(c.q, c.k, c.v, c.g, c.beta, c.s0 if init else None,
                                        c.cu_seqlens, c.scale)


@pytest.mark.parametrize("dtype,d,Hk", [("bf16", 128, 4), ("bf16", 128, 2), ("f32", 64, 4),
                                        ("f32", 16, 1)])
def test_channel_gated_prefill(dtype, d, Hk):
    c = inputs.make_channel_gated(seed=81, B=2, T=150, H=4, Hk=Hk, d=d, dtype=dtype)
    o, fin = run_prefill(c, entry=gdn.gdn_prefill_channel_gated)
    o_ref, s_ref = _oracle_channel(c)
    eo, es = o_err(o, o_ref), s_err(fin, s_ref)
    report(f"channel gated prefill {dtype} d{d} Hk{Hk}", o=eo, state=es)
    assert eo <= _tol(c) and es <= _tol(c)


def test_channel_gated_packed():
    c = inputs.make_channel_gated(seed=82, H=3, d=128, lengths=[40, 0, 1, 129, 64])
    o, fin = run_prefill(c, entry=gdn.gdn_prefill_channel_gated)
    o_ref, s_ref = _oracle_channel(c)
    cu = [int(x) for x in c.cu_seqlens.tolist()]
    eo, es = o_err_packed(o, o_ref, cu), s_err(fin, s_ref)
    report("channel gated packed", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16
    assert torch.equal(fin[1].cpu(), c.s0[1])          # the empty sequence keeps its state


def test_channel_gated_equal_channels_match_the_head_gate():
    """Equal rates on every channel: the per-channel kernels give the per-head
    kernels' result (fp32, same token-serial arithmetic up to rounding)."""
    c = inputs.make_prefill(seed=83, B=2, T=100, H=3, d=64, dtype="f32", with_state=True)
    gc = c.g[..., None].expand(-1, -1, -1, 64).contiguous()
    s0 = dev(c.s0)
    f1 = torch.empty_like(s0)
    f2 = torch.empty_like(s0)
    o1, _ = gdn.gdn_prefill_recurrent(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta), s0, f1,
                                      scale=c.scale)
    o2, _ = gdn.gdn_prefill_channel_gated(dev(c.q), dev(c.k), dev(c.v), dev(gc), dev(c.beta), s0,
                                          f2, scale=c.scale)
    torch.cuda.synchronize()
    assert o_err(o2, host64(o1)) <= 1e-5 and s_err(f2, host64(f1)) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_channel_gated_decode_continues_prefill(dtype):
    """Prefill of 70 tokens then 3 decode steps, all per-channel gated, against
    the oracle over the 73 tokens."""
    c = inputs.make_channel_gated(seed=84, B=3, T=73, H=4, Hk=2, d=128, dtype=dtype)
    fin = torch.empty((3, 4, 128, 128), dtype=torch.float32, device="cuda:0")
    o1, _ = gdn.gdn_prefill_channel_gated(dev(c.q[:, :70]), dev(c.k[:, :70]), dev(c.v[:, :70]),
                                          dev(c.g[:, :70]), dev(c.beta[:, :70]), dev(c.s0), fin,
                                          scale=c.scale)
    outs = [o1.cpu()]
    for t in range(70, 73):
        o = gdn.gdn_decode_step_channel_gated(dev(c.q[:, t]), dev(c.k[:, t]), dev(c.v[:, t]),
                                              dev(c.g[:, t]), dev(c.beta[:, t]), fin, scale=c.scale)
        outs.append(o.cpu()[:, None])
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle_channel(c)
    eo, es = o_err(torch.cat(outs, 1), o_ref), s_err(fin, s_ref)
    report(f"channel gated prefill + decode {dtype}", o=eo, state=es)
    assert eo <= _tol(c) and es <= _tol(c)


# --- sequence-parallel prefill (segments of one sequence side by side) ---------------

@pytest.mark.parametrize("segments,Hk", [(1, 3), (3, 3), (4, 1), (40, 3)])
def test_seqpar_matches_oracle(segments, Hk):
    """B=2 sequences of 1000 tokens (16 chunks, a ragged tail) cut into 1, 3,
    4 or 40 segments (more segments than chunks: empty ones), non-zero initial
    states, grouped heads."""
    c = inputs.make_prefill(seed=91, B=2, T=1000, H=3, Hk=Hk, with_state=True)
    fin = torch.empty((2, 3, 128, 128), dtype=torch.float32, device="cuda:0")
    o, _ = gdn.gdn_prefill_seqpar(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta), segments,
                                  dev(c.s0), fin, scale=c.scale)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(c)
    eo, es = o_err(o, o_ref), s_err(fin, s_ref)
    report(f"seqpar segments={segments} Hk={Hk}", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_seqpar_long_sequence_sampled():
    """One sequence of 32768 tokens, H=16, 8 segments: every head against the
    oracle on the final state and on the outputs of the last 2048 tokens plus
    the first 2048 (the oracle runs the whole sequence)."""
    c = inputs.make_prefill(seed=92, B=1, T=32768, H=16)
    fin = torch.empty((1, 16, 128, 128), dtype=torch.float32, device="cuda:0")
    o, _ = gdn.gdn_prefill_seqpar(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta), 8,
                                  None, fin, scale=c.scale)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(c)
    oc = o.cpu()
    eo = max(o_err(oc[:, :2048], o_ref[:, :2048]), o_err(oc[:, -2048:], o_ref[:, -2048:]))
    es = s_err(fin, s_ref)
    report("seqpar B1 H16 T32768 segments=8", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("segments", [1, 2, 3, 5, 40])
def test_seqpar_packed_matches_oracle(segments):
    """Packed sequences of 900, 64, 1, 0, 2500, 130 and 65 tokens (ragged
    tails, an empty and a 1-token sequence), grouped heads, initial states:
    the longest (40 chunks) cut into 1, 2, 3, 5 or 40 segments and the
    others into segments of the same length."""
    c = inputs.make_varlen(seed=95, H=4, Hk=2, lengths=[900, 64, 1, 0, 2500, 130, 65])
    fin = torch.empty((7, 4, 128, 128), dtype=torch.float32, device="cuda:0")
    o, _ = gdn.gdn_prefill_seqpar(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta), segments,
                                  dev(c.s0), fin, cu_seqlens=dev(c.cu_seqlens), scale=c.scale)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(c)
    cu = [int(x) for x in c.cu_seqlens.tolist()]
    eo, es = o_err_packed(o, o_ref, cu), s_err(fin, s_ref)
    report(f"seqpar packed segments={segments}", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("segments", [2, 4])
def test_seqpar_varlen_full_size_sampled(varlen_full, segments):
    """The packed workload at full size (H=32, 8 sequences log-uniform in
    [512, 65536], non-zero initial states) through the sequence-parallel
    path: every sequence, four heads, against the oracle."""
    c, (outs, s_ref) = varlen_full
    fin = torch.empty((c.N, c.H, 128, 128), dtype=torch.float32, device="cuda:0")
    o, _ = gdn.gdn_prefill_seqpar(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta), segments,
                                  dev(c.s0), fin, cu_seqlens=dev(c.cu_seqlens), scale=c.scale)
    torch.cuda.synchronize()
    cu = [int(x) for x in c.cu_seqlens.tolist()]
    o_h = o.cpu()[:, :, VARLEN_HEADS]
    eo = max(o_err(o_h[:, a:b], r) for (a, b), r in zip(zip(cu[:-1], cu[1:]), outs) if b > a)
    es = s_err(fin.cpu()[:, VARLEN_HEADS], s_ref)
    report(f"varlen seqpar segments={segments} lengths={c.meta['lengths']}", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_seqpar_packed_zero_tokens_keeps_the_states():
    c = inputs.make_varlen(seed=96, H=2, lengths=[0, 0, 0])
    fin = torch.full((3, 2, 128, 128), 7.0, dtype=torch.float32, device="cuda:0")
    gdn.gdn_prefill_seqpar(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta), 4, dev(c.s0),
                           fin, cu_seqlens=dev(c.cu_seqlens), scale=c.scale)
    torch.cuda.synchronize()
    assert torch.equal(fin.cpu(), c.s0)


def test_seqpar_zero_tokens_keeps_the_state():
    c = inputs.make_prefill(seed=93, B=2, T=0, H=2, with_state=True)
    fin = torch.full((2, 2, 128, 128), 7.0, dtype=torch.float32, device="cuda:0")
    gdn.gdn_prefill_seqpar(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta), 4, dev(c.s0),
                           fin, scale=c.scale)
    torch.cuda.synchronize()
    assert torch.equal(fin.cpu(), c.s0)


# --- value head sizes that are not a multiple of the row blocks ----------------------

def _with_dv(c, dv):
    """The case with v (and the state's rows) cut to the first dv channels."""
    import dataclasses
    return dataclasses.replace(c, v=c.v[..., :dv].contiguous(),
                               s0=None if c.s0 is None else c.s0[:, :, :dv, :].contiguous())


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 100), ("f32", 128, 36), ("f32", 16, 7)])
def test_decode_ragged_value_rows(dtype, dk, dv):
    c = _with_dv(inputs.make_decode(seed=95, B=3, H=4, Hk=2, d=dk, dtype=dtype), dv)
    st = dev(c.s0)
    o = gdn.gdn_decode_step(dev(c.q[:, 0]), dev(c.k[:, 0]), dev(c.v[:, 0]), dev(c.g[:, 0]),
                            dev(c.beta[:, 0]), st, scale=c.scale)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(c)
    eo, es = o_err(o[:, None], o_ref), s_err(st, s_ref)
    report(f"decode d_k={dk} d_v={dv} {dtype}", o=eo, state=es)
    assert eo <= _tol(c) and es <= _tol(c)


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 100), ("f32", 64, 48), ("f32", 32, 5)])
def test_prefill_ragged_value_rows(dtype, dk, dv):
    """Token-serial path (d_v < 128 leaves the MFMA kernels) with a partial
    last row block, packed sequences and initial states."""
    c = _with_dv(inputs.make_varlen(seed=96, H=2, d=dk, dtype=dtype, lengths=[33, 0, 100]), dv)
    o, fin = run_prefill(c)
    o_ref, s_ref = oracle_prefill(c)
    cu = [int(x) for x in c.cu_seqlens.tolist()]
    eo, es = o_err_packed(o, o_ref, cu), s_err(fin, s_ref)
    report(f"prefill d_k={dk} d_v={dv} {dtype}", o=eo, state=es)
    assert eo <= _tol(c) and es <= _tol(c)


def test_channel_gated_ragged_value_rows():
    c = _with_dv(inputs.make_channel_gated(seed=97, B=2, T=70, H=2, d=64, dtype="f32"), 40)
    o, fin = run_prefill(c, entry=gdn.gdn_prefill_channel_gated)
    o_ref, s_ref = oracle.gdn_recurrent_channel(c.q, c.k, c.v, c.g, c.beta, c.s0, None, c.scale)
    assert o_err(o, o_ref) <= TOL_F32 and s_err(fin, s_ref) <= TOL_F32


# --- per-channel decay, chunkwise (two passes through the workspace) -----------------

def _channel_run(c, workspace="auto", init=True):
    s0 = dev(c.s0) if (init and c.s0 is not None) else None
    fin = torch.empty((c.N, c.H, c.d_v, c.d_k), dtype=torch.float32, device="cuda:0")
    o, _ = gdn.gdn_prefill_channel_gated(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta), s0,
                                         fin, cu_seqlens=dev(c.cu_seqlens), scale=c.scale,
                                         workspace=workspace)
    torch.cuda.synchronize()
    return o, fin


@pytest.mark.parametrize("T,init,Hk", [(1, True, 3), (63, False, 3), (64, True, 1), (130, True, 3),
                                       (257, False, 1)])
def test_channel_gated_chunk_ragged(T, init, Hk):
    """Chunkwise per-channel path: partial chunks, with and without initial
    states, grouped query/key heads."""
    c = inputs.make_channel_gated(seed=120 + T, B=2, T=T, H=3, Hk=Hk, d=128, dtype="bf16")
    o, fin = _channel_run(c, init=init)
    o_ref, s_ref = _oracle_channel(c, init=init)
    eo, es = o_err(o, o_ref), s_err(fin, s_ref)
    report(f"channel chunk T={T} init={init} Hk={Hk}", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_channel_gated_chunk_and_serial_agree():
    """The chunkwise and token-serial per-channel paths on the same inputs,
    both against the oracle."""
    c = inputs.make_channel_gated(seed=131, B=2, T=200, H=4, Hk=2, d=128, dtype="bf16")
    o_ref, s_ref = _oracle_channel(c)
    for ws in ("auto", None):
        o, fin = _channel_run(c, workspace=ws)
        eo, es = o_err(o, o_ref), s_err(fin, s_ref)
        report(f"channel {'chunk' if ws else 'serial'}", o=eo, state=es)
        assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("rate", [30.0, 200.0])
def test_channel_gated_chunk_strong_decay(rate):
    """Chunks in which a channel decays by more than e^-80 inside 16 tokens
    take the exact element-wise diagonal blocks, the others (other heads,
    other chunks of the same head) the products; against the oracle."""
    import dataclasses
    c = inputs.make_channel_gated(seed=132, B=2, T=150, H=3, d=128, dtype="bf16")
    g = c.g.clone()
    g[:, :, 0, :16] = -rate                  # head 0: 16 channels forget almost at once
    g[:, 40:60, 1, 16:32] = -rate / 3.0      # head 1: a burst in one chunk; head 2 as drawn
    c = dataclasses.replace(c, g=g)
    o, fin = _channel_run(c)
    o_ref, s_ref = _oracle_channel(c)
    eo, es = o_err(o, o_ref), s_err(fin, s_ref)
    report(f"channel chunk strong decay {rate}", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_channel_gated_chunk_packed_with_states():
    c = inputs.make_channel_gated(seed=133, H=2, d=128, lengths=[64, 0, 1, 200, 65])
    o, fin = _channel_run(c)
    o_ref, s_ref = _oracle_channel(c)
    cu = [int(x) for x in c.cu_seqlens.tolist()]
    eo, es = o_err_packed(o, o_ref, cu), s_err(fin, s_ref)
    report("channel chunk packed", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16
    assert torch.equal(fin[1].cpu(), c.s0[1])          # the empty sequence keeps its state


def test_channel_gated_chunk_full_size():
    """The per-channel workload bench.py times (B=4, T=4096, H=16, d=128),
    every output and final state against the oracle."""
    c = inputs.make_channel_gated(seed=7, B=4, T=4096, H=16, d=128, dtype="bf16", with_state=False)
    o, fin = _channel_run(c, init=False)
    o_ref, s_ref = _oracle_channel(c, init=False)
    eo, es = o_err(o, o_ref), s_err(fin, s_ref)
    report("channel chunk full size", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_channel_gated_chunk_equal_channels_match_the_head_gate():
    """Equal rates on every channel through the chunkwise per-channel path
    give the scalar-gate chunkwise path's result, and both the oracle's."""
    c = inputs.make_prefill(seed=134, B=2, T=300, H=4, d=128, dtype="bf16", with_state=True)
    gc = c.g[..., None].expand(-1, -1, -1, 128).contiguous()
    s0 = dev(c.s0)
    f1 = torch.empty_like(s0)
    f2 = torch.empty_like(s0)
    o1, _ = gdn.gdn_prefill(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta), s0, f1,
                            scale=c.scale)
    o2, _ = gdn.gdn_prefill_channel_gated(dev(c.q), dev(c.k), dev(c.v), dev(gc), dev(c.beta), s0,
                                          f2, scale=c.scale)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(c)
    e12 = o_err(o2, host64(o1))
    report("channel chunk, equal channels vs head gate", o_vs_head=e12,
           o=o_err(o2, o_ref), state=s_err(f2, s_ref))
    assert e12 <= TOL_BF16
    assert o_err(o2, o_ref) <= TOL_BF16 and s_err(f2, s_ref) <= TOL_BF16


def test_channel_gated_chunk_strong_decay_packed():
    """The exact diagonal blocks in packed sequences (partial chunks at every
    sequence end), against the oracle."""
    import dataclasses
    c = inputs.make_channel_gated(seed=135, H=2, d=128, lengths=[70, 1, 130, 0, 33])
    g = c.g.clone()
    g[:, :, 1, 64:96] = -50.0                # head 1: 32 channels forget at once
    c = dataclasses.replace(c, g=g)
    o, fin = _channel_run(c)
    o_ref, s_ref = _oracle_channel(c)
    cu = [int(x) for x in c.cu_seqlens.tolist()]
    eo, es = o_err_packed(o, o_ref, cu), s_err(fin, s_ref)
    report("channel chunk strong decay packed", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_channel_gated_chunk_near_orthogonal_query_key():
    """Short packed sequences whose queries are nearly orthogonal to the keys
    of their own 16-token block: the intra-block products q_i k_j nearly
    cancel, so the output of a one-token sequence (P_00 Delta_0, no initial
    state) is small and carries the full relative error of P_00. Against
    the oracle, per sequence and head."""
    import dataclasses
    c = inputs.make_channel_gated(seed=136, H=2, d=128, lengths=[1, 2, 1, 3, 16, 1, 17])
    q = c.q.float()
    k = c.k.float()
    kn = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-6)
    q = q - (q * kn).sum(-1, keepdim=True) * kn + 0.02 * q.norm(dim=-1, keepdim=True) * kn
    c = dataclasses.replace(c, q=q.to(c.q.dtype))
    o, fin = _channel_run(c, init=False)
    o_ref, s_ref = _oracle_channel(c, init=False)
    cu = [int(x) for x in c.cu_seqlens.tolist()]
    eo, es = o_err_packed(o, o_ref, cu), s_err(fin, s_ref)
    report("channel chunk near-orthogonal q, k", o=eo, state=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_prefill_and_decode_replay_from_a_captured_graph():
    """The two-pass prefill (caller workspace) and a decode step captured into
    one HIP graph: the library allocates nothing and clears nothing with
    memset nodes, so every replay (three, with eager work and synchronisation
    between them) gives the eager results bit for bit."""
    c = inputs.make_prefill(seed=150, B=2, T=300, H=4, d=128, dtype="bf16", with_state=True)
    q, k, v, g, b = dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta)
    s0 = dev(c.s0)
    ws = torch.empty(gdn.gdn_prefill_workspace_size(2, 300, 4, 128, 128, 2, 0, torch.bfloat16),
                     dtype=torch.uint8, device="cuda:0")
    o, fin, st = torch.empty_like(v), torch.empty_like(s0), torch.empty_like(s0)
    q1, k1, v1, g1, b1 = (x[:, -1].contiguous() for x in (q, k, v, g, b))
    o1 = torch.empty_like(v1)

    def step():
        gdn.gdn_prefill(q, k, v, g, b, s0, fin, o, scale=c.scale, workspace=ws)
        torch.add(fin, 0.0, out=st)            # the decode step updates its own copy
        gdn.gdn_decode_step(q1, k1, v1, g1, b1, st, o1, scale=c.scale)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (o, fin, st, o1)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        for x in (o, fin, st, o1):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((o, fin, st, o1), ref):
            assert torch.equal(got, want)


@pytest.mark.parametrize("seed", range(500, 512))
def test_seed_sweep_short_and_packed(seed):
    """Many small cases per seed, every chunk path against the oracle: a short
    batch (1-200 tokens, with or without initial states) and packed sequences
    of 1, 64, 0, 2, 129, 17 and 1 tokens through the two-pass, one-pass and
    per-channel chunk paths, and a sequence-parallel run with 1-12 segments."""
    import random
    rnd = random.Random(seed)
    cases = [inputs.make_prefill(seed=seed, B=2, T=rnd.randint(1, 200), H=3, d=128, dtype="bf16",
                                 with_state=rnd.random() < 0.5),
             inputs.make_varlen(seed=seed, H=3, d=128, lengths=[1, 64, 0, 2, 129, 17, 1])]
    for c in cases:
        o_ref, s_ref = oracle_prefill(c)
        cu = None if c.cu_seqlens is None else [int(x) for x in c.cu_seqlens.tolist()]
        for path in WS:
            o, fin = run_prefill(c, path=path)
            eo = o_err(o, o_ref) if cu is None else o_err_packed(o, o_ref, cu)
            assert eo <= TOL_BF16 and s_err(fin, s_ref) <= TOL_BF16, (path, cu)
    cc = inputs.make_channel_gated(seed=seed, H=2, d=128, lengths=[rnd.randint(1, 80), 1, 2, 65])
    o, fin = _channel_run(cc)
    o_ref, s_ref = _oracle_channel(cc)
    cu = [int(x) for x in cc.cu_seqlens.tolist()]
    assert o_err_packed(o, o_ref, cu) <= TOL_BF16 and s_err(fin, s_ref) <= TOL_BF16
    c = inputs.make_prefill(seed=seed, B=2, T=rnd.randint(1, 700), H=2, d=128, dtype="bf16",
                            with_state=True)
    fin = torch.empty((2, 2, 128, 128), dtype=torch.float32, device="cuda:0")
    o, _ = gdn.gdn_prefill_seqpar(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta),
                                  rnd.randint(1, 12), dev(c.s0), fin, scale=c.scale)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(c)
    assert o_err(o, o_ref) <= TOL_BF16 and s_err(fin, s_ref) <= TOL_BF16
