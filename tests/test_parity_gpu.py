"""GPU parity of the HIP forward path against the fp64 CPU oracle.

Every case runs ``kda_fwd`` through the C ABI (via the Python binding) on
seeded synthetic inputs and compares ``out`` and ``final_state`` with the
oracle on the same bf16/fp32 inputs:

    relative L2 error <= 1e-2  and  max abs error <= 3e-2

for each of ``out`` and ``final_state`` separately (max-abs alone where the
reference is all zero).  Output buffers sit between guard regions that must
come back untouched.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import gated_delta_rule_36_amd as kda
from gated_delta_rule_36_amd import synth
from kda_testutil import errors
from oracle import kda_oracle

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_ABS = 3e-2

# kda.fwd options (kernel, inverse, sigmoid) the current test selected; every
# call below goes through fwd(), which applies them.
_OPTS = {}


def fwd(*args, **kw):
    return kda.fwd(*args, **{**_OPTS, **kw})


@pytest.fixture
def options():
    """options(kernel=..., inverse=..., sigmoid=...) selects the library
    options for the rest of the test."""
    def select(**kw):
        _OPTS.clear()
        _OPTS.update(kw)
    yield select
    _OPTS.clear()
GUARD = 4096
SENTINEL = {torch.bfloat16: 0x7FC1, torch.float32: 0x7FC00001}


def _guarded(shape, dtype):
    """A tensor of `shape` inside a buffer with sentinel guard regions."""
    n = int(np.prod(shape))
    if dtype == torch.bfloat16:
        buf = torch.full((n + 2 * GUARD,), SENTINEL[dtype], dtype=torch.int16, device="cuda")
        view = buf.view(torch.bfloat16)
    else:
        buf = torch.full((n + 2 * GUARD,), SENTINEL[dtype], dtype=torch.int32, device="cuda")
        view = buf.view(torch.float32)
    return buf, view[GUARD:GUARD + n].view(*shape)


def _guards_intact(buf, dtype):
    s = SENTINEL[dtype]
    return bool((buf[:GUARD] == s).all()) and bool((buf[-GUARD:] == s).all())


def run_gpu(x: synth.KdaInputs, final_dtype=None, initial_state="inputs", out_fill=None,
            segment_chunks=None):
    """Run the library on inputs already on the GPU; returns (out, final) on
    the CPU as float64 numpy arrays (final None if not requested).
    ``segment_chunks`` selects the segmented form (kda_fwd_scan)."""
    B, T, H, _ = x.q.shape
    N = x.num_seqs
    ob, out = _guarded((B, T, H, 128), torch.bfloat16)
    if out_fill is not None:
        out.fill_(out_fill)
    init = x.initial_state if initial_state == "inputs" else initial_state
    fb = final = None
    if final_dtype is not None:
        fb, final = _guarded((N, H, 128, 128), final_dtype)
    fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, out, x.A_log, x.dt_bias, x.lower_bound,
            initial_state=init, final_state=final, cu_seqlens=x.cu_seqlens,
            segment_chunks=segment_chunks)
    torch.cuda.synchronize()
    assert _guards_intact(ob, torch.bfloat16), "write outside out"
    if fb is not None:
        assert _guards_intact(fb, final_dtype), "write outside final_state"
    o = out.double().cpu().numpy()
    f = None if final is None else final.double().cpu().numpy()
    return o, f


def oracle_of(x: synth.KdaInputs, chains=None, initial_state="inputs"):
    c = x.to("cpu")
    init = c.initial_state if initial_state == "inputs" else initial_state
    return kda_oracle(c.q, c.k, c.v, c.g, c.beta, c.scale, c.A_log, c.dt_bias, c.lower_bound,
                      initial_state=init, cu_seqlens=c.cu_seqlens, chains=chains)


def assert_close(name, got, ref):
    rel, mx = errors(got, ref)
    nref = float(np.abs(np.asarray(ref)).max()) if np.asarray(ref).size else 0.0
    print(f"[parity] {name}: rel_l2={rel:.3e} max_abs={mx:.3e} (|ref|max={nref:.3e})", flush=True)
    assert np.isfinite(np.asarray(got)).all(), f"{name}: non-finite values"
    if nref > 0:
        assert rel <= REL_L2, f"{name}: relative L2 {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS, f"{name}: max abs {mx:.3e} > {MAX_ABS}"


# Threads for the oracle: the host share of one GPU (16 cores), whatever the
# machine's affinity mask shows.
ORACLE_THREADS = min(16, len(os.sched_getaffinity(0)))


class _Err:
    """Whole-tensor error sums, accumulated one chain at a time."""

    def __init__(self):
        self.d2 = self.r2 = self.mx = self.rmax = 0.0
        self.finite = True
        self.n = 0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        self.finite &= bool(np.isfinite(got).all())
        d = got - ref
        self.d2 += float(np.sum(d * d))
        self.r2 += float(np.sum(ref * ref))
        if d.size:
            self.mx = max(self.mx, float(np.max(np.abs(d))))
            self.rmax = max(self.rmax, float(np.max(np.abs(ref))))
        self.n += d.size

    def check(self, name):
        rel = math.sqrt(self.d2 / self.r2) if self.r2 > 0 else 0.0
        print(f"[parity] {name}: rel_l2={rel:.3e} max_abs={self.mx:.3e} (|ref|max={self.rmax:.3e}, "
              f"{self.n} values)", flush=True)
        assert self.finite, f"{name}: non-finite values"
        if self.r2 > 0:
            assert rel <= REL_L2, f"{name}: relative L2 {rel:.3e} > {REL_L2}"
        assert self.mx <= MAX_ABS, f"{name}: max abs {self.mx:.3e} > {MAX_ABS}"


def check_all_chains(tag, x, out, final, batch=64):
    """Every (sequence, head) chain of ``out`` and ``final`` (GPU tensors)
    against the oracle, streamed: the oracle runs ``batch`` chains at a time
    and each chain's rows are compared with the bf16 / state values of that
    chain, accumulating the whole-tensor sums of squared differences and
    squared reference values and the largest difference.  Nothing of the
    size of the whole output is held in fp64."""
    c = x.to("cpu")
    o = out.cpu()
    f = None if final is None else final.cpu()
    B, T, H, _ = c.q.shape
    cu = None if c.cu_seqlens is None else c.cu_seqlens.numpy()
    N = x.num_seqs
    seg = [(0, T, n) for n in range(N)] if cu is None else [(int(cu[n]), int(cu[n + 1]), 0) for n in range(N)]
    chains = [(n, h) for n in range(N) for h in range(H)]
    eo, ef = _Err(), _Err()
    for i in range(0, len(chains), batch):
        part = chains[i:i + batch]
        res = kda_oracle(c.q, c.k, c.v, c.g, c.beta, c.scale, c.A_log, c.dt_bias, c.lower_bound,
                         initial_state=c.initial_state, cu_seqlens=c.cu_seqlens, chains=part,
                         threads=ORACLE_THREADS, want_final=f is not None)
        for (n, h), (ro, rf) in zip(part, res):
            t0, t1, b = seg[n]
            eo.add(o[b, t0:t1, h].double().numpy(), ro)
            if f is not None:
                ef.add(f[n, h].double().numpy(), rf)
    print(f"[parity] {tag}: {len(chains)} chains compared", flush=True)
    eo.check(f"{tag} out")
    if f is not None:
        ef.check(f"{tag} final")


def check_full(tag, x, final_dtype, segment_chunks=None):
    o, f = run_gpu(x, final_dtype, segment_chunks=segment_chunks)
    ro, rf = oracle_of(x)
    assert_close(f"{tag} out", o, ro)
    if final_dtype is not None:
        assert_close(f"{tag} final", f, rf)
    return o, f


# --------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_b1_t64_h2", "small_b2_t128_h8",
                                  "long_b1_t8192_h16_state", "decode_b64_t1_h32_state",
                                  "decode_b64_t8_h32_state", "decode_b64_t15_h32_state"])
def test_workload_parity_full(name):
    print(f"[case] workload {name}", flush=True)
    x = synth.workload(name, device="cuda")
    # the tiny and small workloads write no state; ask for one anyway here
    check_full(name, x, x.final_dtype or torch.float32)


def _run_workload(name, final_dtype):
    x = synth.workload(name, device="cuda")
    out = torch.empty_like(x.v)
    final = None
    if final_dtype is not None:
        final = torch.empty(x.num_seqs, x.q.shape[2], 128, 128, dtype=final_dtype, device="cuda")
    fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, out, x.A_log, x.dt_bias, x.lower_bound,
            initial_state=x.initial_state, final_state=final, cu_seqlens=x.cu_seqlens)
    torch.cuda.synchronize()
    return x, out, final


def test_varlen_workload_parity_all_chains():
    """Packed workload (8 sequences of 100..4000 tokens, 32 heads, bf16 states):
    all 256 chains against the oracle."""
    name = "varlen_n8_h32_bf16state"
    print(f"[case] workload {name}", flush=True)
    x, out, final = _run_workload(name, torch.bfloat16)
    check_all_chains(name, x, out, final)


def test_large_workload_parity_all_chains():
    """Large workload (B=8, T=16384, H=32, fp32 final state): all 256 chains,
    i.e. every output value and every final-state value, against the oracle."""
    name = "large_b8_t16384_h32"
    print(f"[case] workload {name}", flush=True)
    x, out, final = _run_workload(name, torch.float32)
    check_all_chains(name, x, out, final, batch=32)


# --------------------------------------------------------------------------
# edges: ragged tails, empty inputs, extreme gates, state dtypes
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", [None, "mfma"])
@pytest.mark.parametrize("T", [0, 1, 15, 16, 17, 32, 33, 48, 49, 100])
def test_chunk_edges(T, kernel, options):
    """Short calls take the recurrent kernel by default; kernel="mfma"
    keeps the chunked kernel covered on the same shapes: one to four chunks,
    full or with a tail (the pipelined kernel loads two chunks ahead and
    stops loading for the last two)."""
    if kernel:
        options(kernel=kernel)
    print(f"[case] chunk edge T={T} kernel={kernel or 'default'}", flush=True)
    x = synth.make_inputs(2, T, 3, lower_bound=-5.0, seed=T, init_dtype=torch.float32,
                          device="cuda")
    o, f = run_gpu(x, torch.float32)
    ro, rf = oracle_of(x)
    if T:
        assert_close(f"T={T} out", o, ro)
    assert_close(f"T={T} final", f, rf)


@pytest.mark.parametrize("state", [torch.bfloat16, torch.float32])
def test_varlen_edges(state):
    lens = [1, 16, 17, 0, 33, 5, 48, 2]
    print(f"[case] varlen edges {lens} state={state}", flush=True)
    x = synth.make_inputs(1, 0, 4, lower_bound=-5.0, seed=7, seq_lengths=lens,
                          init_dtype=state, device="cuda")
    check_full(f"varlen edges {state}", x, state)


@pytest.mark.parametrize("lb", [0.0, -5.0, -0.5])
def test_lower_bound_values(lb):
    print(f"[case] lower_bound={lb}", flush=True)
    x = synth.make_inputs(2, 77, 4, lower_bound=lb, seed=11, init_dtype=torch.float32,
                          device="cuda")
    check_full(f"lb={lb}", x, torch.float32)


def test_max_decay_stress():
    """g = +100 everywhere saturates the sigmoid, so every token decays by
    the full e^lb = e^-5 on every channel: the largest exponent range a chunk
    can see.  Outputs must stay finite and match."""
    print("[case] max decay stress", flush=True)
    x = synth.make_inputs(2, 96, 4, lower_bound=-5.0, seed=12, init_dtype=torch.float32,
                          device="cuda")
    x.g.fill_(100.0)
    check_full("max decay", x, torch.float32)


def test_min_decay_and_large_beta():
    """g = -100 (no decay) and beta logits of +8 (beta ~ 1): the plain,
    nearly-overwriting delta rule."""
    print("[case] min decay, large beta", flush=True)
    x = synth.make_inputs(1, 64, 2, lower_bound=-5.0, seed=13, init_dtype=torch.float32,
                          device="cuda")
    x.g.fill_(-100.0)
    x.beta.fill_(8.0)
    check_full("min decay", x, torch.float32)


def test_without_gate_params():
    print("[case] A_log/dt_bias None", flush=True)
    x = synth.make_inputs(2, 40, 2, lower_bound=-4.0, seed=14, with_gate_params=False,
                          device="cuda")
    check_full("no gate params", x, torch.bfloat16)


@pytest.mark.parametrize("init,final", [(None, torch.bfloat16), (torch.bfloat16, torch.bfloat16),
                                        (torch.float32, None), (None, None)])
def test_state_combinations(init, final):
    print(f"[case] init={init} final={final}", flush=True)
    x = synth.make_inputs(1, 50, 3, lower_bound=-5.0, seed=15, init_dtype=init, device="cuda")
    o, f = run_gpu(x, final)
    ro, rf = oracle_of(x)
    assert_close("state combo out", o, ro)
    if final is not None:
        assert_close("state combo final", f, rf)


# --------------------------------------------------------------------------
# invariants on the GPU
# --------------------------------------------------------------------------

def test_deterministic():
    x = synth.make_inputs(2, 70, 4, lower_bound=-5.0, seed=16, init_dtype=torch.float32,
                          device="cuda")
    o1, f1 = run_gpu(x, torch.float32)
    o2, f2 = run_gpu(x, torch.float32, out_fill=1.0)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_power_of_two_equivariance():
    """(out, final) is linear in (v, initial_state); scaling both by 2
    commutes with every rounding step, so the result doubles exactly."""
    x = synth.make_inputs(2, 70, 4, lower_bound=-5.0, seed=17, init_dtype=torch.float32,
                          device="cuda")
    o1, f1 = run_gpu(x, torch.float32)
    x2 = synth.KdaInputs(**{**x.__dict__, "v": x.v * 2, "initial_state": x.initial_state * 2})
    o2, f2 = run_gpu(x2, torch.float32)
    assert np.array_equal(o2, 2 * o1) and np.array_equal(f2, 2 * f1)


@pytest.mark.parametrize("split", [48, 37])
def test_split_sequence_chaining(split):
    """Two calls chained through an fp32 final_state -> initial_state equal
    one call; bit for bit when the split falls on a chunk boundary."""
    x = synth.make_inputs(1, 80, 3, lower_bound=-5.0, seed=18, init_dtype=torch.float32,
                          device="cuda")
    o, f = run_gpu(x, torch.float32)

    def part(sl):
        return synth.KdaInputs(**{**x.__dict__, "q": x.q[:, sl].contiguous(),
                                  "k": x.k[:, sl].contiguous(), "v": x.v[:, sl].contiguous(),
                                  "g": x.g[:, sl].contiguous(),
                                  "beta": x.beta[:, sl].contiguous()})
    o1, f1 = run_gpu(part(slice(0, split)), torch.float32)
    o2, f2 = run_gpu(part(slice(split, None)), torch.float32,
                     initial_state=torch.from_numpy(f1.astype(np.float32)).cuda())
    oc = np.concatenate([o1, o2], axis=1)
    if split % 16 == 0:
        assert np.array_equal(oc, o) and np.array_equal(f2, f)
    else:
        assert_close("split out", oc, o)
        assert_close("split final", f2, f)


@pytest.mark.parametrize("kernel", ["mfma", "recurrent"])
def test_packed_equals_separate_runs(kernel, options):
    """Packed sequences give exactly the results of separate calls on the
    same kernel (short separate calls would otherwise take the recurrent
    kernel, so the kernel is pinned)."""
    options(kernel=kernel)
    lens = [20, 3, 35, 16]
    x = synth.make_inputs(1, 0, 2, lower_bound=-5.0, seed=19, seq_lengths=lens,
                          init_dtype=torch.float32, device="cuda")
    o, f = run_gpu(x, torch.float32)
    cu = x.cu_seqlens.cpu().numpy()
    for n in range(len(lens)):
        sl = slice(int(cu[n]), int(cu[n + 1]))
        xn = synth.KdaInputs(**{**x.__dict__, "q": x.q[:, sl].contiguous(),
                                "k": x.k[:, sl].contiguous(), "v": x.v[:, sl].contiguous(),
                                "g": x.g[:, sl].contiguous(), "beta": x.beta[:, sl].contiguous(),
                                "initial_state": x.initial_state[n:n + 1].contiguous(),
                                "cu_seqlens": None})
        on, fn = run_gpu(xn, torch.float32)
        assert np.array_equal(on[0], o[0, sl]) and np.array_equal(fn[0], f[n])


def test_head_permutation():
    x = synth.make_inputs(2, 40, 4, lower_bound=-5.0, seed=20, init_dtype=torch.float32,
                          device="cuda")
    perm = torch.tensor([3, 1, 0, 2], device="cuda")
    xp = synth.KdaInputs(**{**x.__dict__,
                            **{n: getattr(x, n)[:, :, perm].contiguous()
                               for n in ("q", "k", "v", "g", "beta")},
                            "A_log": x.A_log[perm].contiguous(),
                            "dt_bias": x.dt_bias[perm].contiguous(),
                            "initial_state": x.initial_state[:, perm].contiguous()})
    o, f = run_gpu(x, torch.float32)
    op, fp = run_gpu(xp, torch.float32)
    pc = perm.cpu().numpy()
    assert np.array_equal(op, o[:, :, pc]) and np.array_equal(fp, f[:, pc])


def test_in_place_state():
    """initial_state and final_state may be the same buffer."""
    x = synth.make_inputs(2, 45, 3, lower_bound=-5.0, seed=21, init_dtype=torch.float32,
                          device="cuda")
    o, f = run_gpu(x, torch.float32)
    st = x.initial_state.clone()
    out = torch.empty_like(x.v)
    fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, out, x.A_log, x.dt_bias, x.lower_bound,
            initial_state=st, final_state=st)
    torch.cuda.synchronize()
    assert np.array_equal(out.double().cpu().numpy(), o)
    assert np.array_equal(st.double().cpu().numpy(), f)


def test_errors_raise_before_launch_on_gpu():
    x = synth.make_inputs(1, 16, 2, lower_bound=-5.0, seed=22, device="cuda")
    out = torch.empty_like(x.v)
    with pytest.raises(kda.KdaArgumentError):
        fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, out, x.A_log, x.dt_bias, 1.0)
    with pytest.raises(kda.KdaArgumentError):
        fwd(x.q, x.k, x.v, x.g, x.beta, math.inf, out, x.A_log, x.dt_bias, -1.0)
    with pytest.raises(ValueError):
        fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, out, x.A_log, x.dt_bias, -1.0,
                cu_seqlens=torch.tensor([0, 5, 3, 16], device="cuda"))


# --------------------------------------------------------------------------
# the segmented form (kda_fwd_scan): parallel over segments of each chain
# --------------------------------------------------------------------------

def test_scan_long_workload_parity():
    """16 chains of 512 chunks: the case the segmented form is for."""
    name = "long_b1_t8192_h16_state"
    print(f"[case] scan {name}", flush=True)
    x = synth.workload(name, device="cuda")
    seg = kda.auto_segment_chunks(x.num_seqs * x.q.shape[2], x.q.shape[1])
    assert seg == 32
    o, f = check_full(f"scan {name}", x, x.final_dtype, segment_chunks=seg)
    # and it agrees with the whole-chain form as closely as either with the oracle
    o1, f1 = run_gpu(x, x.final_dtype)
    assert_close(f"scan vs whole {name} out", o, o1)
    assert_close(f"scan vs whole {name} final", f, f1)


@pytest.mark.parametrize("T,seg", [(17, 1), (100, 1), (100, 3), (257, 2), (257, 5), (48, 1)])
def test_scan_ragged_lengths(T, seg):
    print(f"[case] scan T={T} seg={seg}", flush=True)
    x = synth.make_inputs(2, T, 3, lower_bound=-5.0, seed=100 + T + seg,
                          init_dtype=torch.float32, device="cuda")
    check_full(f"scan T={T} seg={seg}", x, torch.float32, segment_chunks=seg)


def test_scan_many_segments():
    """One chain of 8192 tokens in segments of 2 chunks: 256 segments, so the
    combine step chains 254 products on hi/lo bf16 operands; its rounding
    must not build up (final state against the oracle and the whole-chain
    kernel)."""
    print("[case] scan 1 chain x 256 segments", flush=True)
    x = synth.make_inputs(1, 8192, 1, lower_bound=-3.0, seed=37, init_dtype=torch.float32,
                          device="cuda")
    o, f = check_full("scan 256 segments", x, torch.float32, segment_chunks=2)
    o1, f1 = run_gpu(x, torch.float32)
    assert_close("scan 256 segments vs whole out", o, o1)
    assert_close("scan 256 segments vs whole final", f, f1)


def test_scan_chain_count_not_multiple_of_8():
    """10 chains of 10 segments: the combine places the 8 blocks of chains
    0-7 on one XCD each and maps chains 8-9 plainly, in one grid."""
    print("[case] scan 10 chains x 10 segments", flush=True)
    x = synth.make_inputs(2, 300, 5, lower_bound=-5.0, seed=36, init_dtype=torch.float32,
                          device="cuda")
    check_full("scan 10 chains", x, torch.float32, segment_chunks=2)


@pytest.mark.parametrize("state,seg", [(torch.bfloat16, 1), (torch.float32, 2), (torch.bfloat16, 3)])
def test_scan_varlen_edges(state, seg):
    lens = [1, 16, 17, 0, 33, 5, 48, 2, 130]
    print(f"[case] scan varlen {lens} state={state} seg={seg}", flush=True)
    x = synth.make_inputs(1, 0, 4, lower_bound=-5.0, seed=21 + seg, seq_lengths=lens,
                          init_dtype=state, device="cuda")
    check_full(f"scan varlen {state} seg={seg}", x, state, segment_chunks=seg)


def test_scan_states_absent_or_partial():
    x = synth.make_inputs(1, 200, 2, lower_bound=-3.0, seed=31, device="cuda")
    print("[case] scan no initial state", flush=True)
    check_full("scan no init", x, torch.float32, segment_chunks=2)
    print("[case] scan no final state", flush=True)
    o, f = run_gpu(x, None, segment_chunks=2)
    ro, _ = oracle_of(x)
    assert f is None
    assert_close("scan no final out", o, ro)


def test_scan_in_place_state():
    """final_state may be the initial_state buffer."""
    print("[case] scan in-place state", flush=True)
    x = synth.make_inputs(2, 150, 2, lower_bound=-5.0, seed=32, init_dtype=torch.float32,
                          device="cuda")
    ro, rf = oracle_of(x)
    st = x.initial_state.clone()
    out = torch.empty_like(x.v)
    fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, out, x.A_log, x.dt_bias, x.lower_bound,
            initial_state=st, final_state=st, segment_chunks=2)
    torch.cuda.synchronize()
    assert_close("scan in-place out", out.double().cpu().numpy(), ro)
    assert_close("scan in-place final", st.double().cpu().numpy(), rf)


@pytest.mark.parametrize("state", [torch.float32, torch.bfloat16])
def test_scan_in_place_state_many_blocks(state):
    """final_state is the initial_state buffer, with more workgroups than
    compute units in every pass (21 chains of 20 segments: 420) and a chain
    count that is not a multiple of 8, so the last segment of a chain can
    store the final state before segment 0 of that chain has read its start
    state; segment 0 must read the copy the map pass kept."""
    print(f"[case] scan in-place state, 420 blocks, {state}", flush=True)
    x = synth.make_inputs(3, 640, 7, lower_bound=-5.0, seed=38, init_dtype=state, device="cuda")
    ro, rf = oracle_of(x)
    st = x.initial_state.clone()
    out = torch.empty_like(x.v)
    fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, out, x.A_log, x.dt_bias, x.lower_bound,
            initial_state=st, final_state=st, segment_chunks=2)
    torch.cuda.synchronize()
    assert_close(f"scan in-place 420 blocks {state} out", out.double().cpu().numpy(), ro)
    assert_close(f"scan in-place 420 blocks {state} final", st.double().cpu().numpy(), rf)
    # and the same as the separate-buffer call
    o2, f2 = run_gpu(x, state, segment_chunks=2)
    assert np.array_equal(out.double().cpu().numpy(), o2)
    assert np.array_equal(st.double().cpu().numpy(), f2)


def test_scan_one_segment_is_kda_fwd():
    """A segment at least as long as every chain is the whole-chain kernel:
    bit-identical results."""
    print("[case] scan one segment", flush=True)
    x = synth.make_inputs(2, 77, 3, lower_bound=-5.0, seed=33, init_dtype=torch.bfloat16,
                          device="cuda")
    o1, f1 = run_gpu(x, torch.bfloat16)
    o2, f2 = run_gpu(x, torch.bfloat16, segment_chunks=5)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_scan_max_decay_and_no_decay():
    """The extremes of the transition matrices: every channel decaying by
    the full e^lb per token, and no decay at all (lower_bound = 0)."""
    x = synth.make_inputs(1, 160, 2, lower_bound=-5.0, seed=34, init_dtype=torch.float32,
                          device="cuda")
    x.g.fill_(100.0)
    print("[case] scan max decay", flush=True)
    check_full("scan max decay", x, torch.float32, segment_chunks=2)
    y = synth.make_inputs(1, 160, 2, lower_bound=0.0, seed=35, init_dtype=torch.float32,
                          device="cuda")
    print("[case] scan no decay", flush=True)
    check_full("scan no decay", y, torch.float32, segment_chunks=2)


# --------------------------------------------------------------------------
# the fp16 Neumann-product inverse (inverse="neumann"): an ablation of the
# pages' choice of inverse against the default fp32 forward substitution
# --------------------------------------------------------------------------

@pytest.fixture
def neumann_inverse(options):
    options(inverse="neumann", kernel="mfma")


def test_neumann_small_workload(neumann_inverse):
    print("[case] neumann small workload", flush=True)
    check_full("neumann small", synth.workload("small_b2_t128_h8", device="cuda"), torch.float32)


@pytest.mark.parametrize("T", [1, 17, 100])
def test_neumann_ragged(neumann_inverse, T):
    print(f"[case] neumann T={T}", flush=True)
    x = synth.make_inputs(2, T, 3, lower_bound=-5.0, seed=200 + T, init_dtype=torch.float32,
                          device="cuda")
    check_full(f"neumann T={T}", x, torch.float32)


def test_neumann_varlen_and_scan(neumann_inverse):
    lens = [1, 16, 17, 0, 33, 5, 48, 2, 130]
    print("[case] neumann varlen + segmented form", flush=True)
    x = synth.make_inputs(1, 0, 4, lower_bound=-5.0, seed=41, seq_lengths=lens,
                          init_dtype=torch.bfloat16, device="cuda")
    check_full("neumann varlen", x, torch.bfloat16)
    check_full("neumann varlen scan", x, torch.bfloat16, segment_chunks=2)


def test_neumann_gate_extremes(neumann_inverse):
    """No decay with beta ~ 1 gives the largest entries of T; full decay the
    smallest operands."""
    x = synth.make_inputs(1, 64, 2, lower_bound=-5.0, seed=42, init_dtype=torch.float32,
                          device="cuda")
    x.g.fill_(-100.0)
    x.beta.fill_(8.0)
    print("[case] neumann min decay, large beta", flush=True)
    check_full("neumann min decay", x, torch.float32)
    y = synth.make_inputs(2, 96, 4, lower_bound=-5.0, seed=43, init_dtype=torch.float32,
                          device="cuda")
    y.g.fill_(100.0)
    print("[case] neumann max decay", flush=True)
    check_full("neumann max decay", y, torch.float32)


def test_inverse_option(options):
    """The two inverses give different roundings, and the option applies to
    the call it is passed to (nothing is kept between calls)."""
    x = synth.make_inputs(1, 64, 2, lower_bound=-5.0, seed=44, device="cuda")
    o_sub, _ = run_gpu(x)
    options(inverse="neumann")
    o_neu, _ = run_gpu(x)
    options()
    o_sub2, _ = run_gpu(x)
    assert np.array_equal(o_sub, o_sub2)
    assert not np.array_equal(o_sub, o_neu)


# --------------------------------------------------------------------------
# the recurrent kernel (decode-shaped calls; kernel="recurrent" forces it
# for any call, which covers several 8-token passes, tails and packed input)
# --------------------------------------------------------------------------

@pytest.fixture
def recurrent_kernel(options):
    options(kernel="recurrent")


@pytest.mark.parametrize("name", ["decode_b64_t1_h32_state", "decode_b64_t8_h32_state",
                                  "decode_b64_t15_h32_state"])
def test_decode_workloads_on_the_chunked_kernel(name, options):
    """The decode workloads take the recurrent kernel by default; the chunked
    kernel must agree with the oracle on them too."""
    options(kernel="mfma")
    print(f"[case] workload {name} on the chunked kernel", flush=True)
    x = synth.workload(name, device="cuda")
    check_full(f"{name} mfma", x, x.final_dtype)


@pytest.mark.parametrize("T", [0, 1, 7, 8, 9, 16, 17, 33, 100])
def test_recurrent_lengths(recurrent_kernel, T):
    print(f"[case] recurrent T={T}", flush=True)
    x = synth.make_inputs(2, T, 3, lower_bound=-5.0, seed=300 + T, init_dtype=torch.float32,
                          device="cuda")
    o, f = run_gpu(x, torch.float32)
    ro, rf = oracle_of(x)
    if T:
        assert_close(f"recurrent T={T} out", o, ro)
    assert_close(f"recurrent T={T} final", f, rf)


@pytest.mark.parametrize("state", [torch.bfloat16, torch.float32])
def test_recurrent_varlen(recurrent_kernel, state):
    lens = [1, 16, 17, 0, 33, 5, 48, 2, 8, 9]
    print(f"[case] recurrent varlen {lens} state={state}", flush=True)
    x = synth.make_inputs(1, 0, 4, lower_bound=-5.0, seed=51, seq_lengths=lens,
                          init_dtype=state, device="cuda")
    check_full(f"recurrent varlen {state}", x, state)


@pytest.mark.parametrize("lb", [0.0, -5.0, -0.5])
def test_recurrent_lower_bound_values(recurrent_kernel, lb):
    print(f"[case] recurrent lower_bound={lb}", flush=True)
    x = synth.make_inputs(2, 15, 4, lower_bound=lb, seed=52, init_dtype=torch.float32,
                          device="cuda")
    check_full(f"recurrent lb={lb}", x, torch.float32)


def test_recurrent_gate_extremes(recurrent_kernel):
    """Full decay on every channel and token (the widest range of the
    factored state within a pass), then no decay with beta ~ 1."""
    x = synth.make_inputs(2, 40, 4, lower_bound=-5.0, seed=53, init_dtype=torch.float32,
                          device="cuda")
    x.g.fill_(100.0)
    print("[case] recurrent max decay", flush=True)
    check_full("recurrent max decay", x, torch.float32)
    y = synth.make_inputs(1, 40, 2, lower_bound=-5.0, seed=54, init_dtype=torch.float32,
                          device="cuda")
    y.g.fill_(-100.0)
    y.beta.fill_(8.0)
    print("[case] recurrent min decay, large beta", flush=True)
    check_full("recurrent min decay", y, torch.float32)


def test_recurrent_without_gate_params(recurrent_kernel):
    print("[case] recurrent A_log/dt_bias None", flush=True)
    x = synth.make_inputs(2, 12, 2, lower_bound=-4.0, seed=55, with_gate_params=False,
                          device="cuda")
    check_full("recurrent no gate params", x, torch.bfloat16)


@pytest.mark.parametrize("init,final", [(None, torch.bfloat16), (torch.bfloat16, torch.bfloat16),
                                        (torch.float32, None), (None, None),
                                        (torch.float32, torch.float32)])
def test_recurrent_state_combinations(recurrent_kernel, init, final):
    print(f"[case] recurrent init={init} final={final}", flush=True)
    x = synth.make_inputs(1, 11, 3, lower_bound=-5.0, seed=56, init_dtype=init, device="cuda")
    o, f = run_gpu(x, final)
    ro, rf = oracle_of(x)
    assert_close("recurrent state combo out", o, ro)
    if final is not None:
        assert_close("recurrent state combo final", f, rf)


def test_recurrent_in_place_state(recurrent_kernel):
    x = synth.make_inputs(3, 5, 3, lower_bound=-5.0, seed=57, init_dtype=torch.float32,
                          device="cuda")
    o, f = run_gpu(x, torch.float32)
    st = x.initial_state.clone()
    out = torch.empty_like(x.v)
    fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, out, x.A_log, x.dt_bias, x.lower_bound,
            initial_state=st, final_state=st)
    torch.cuda.synchronize()
    assert np.array_equal(out.double().cpu().numpy(), o)
    assert np.array_equal(st.double().cpu().numpy(), f)


def test_recurrent_invariants(recurrent_kernel):
    """Deterministic, and exactly linear in (v, initial_state) under scaling
    by 2 (every rounding step commutes with it)."""
    x = synth.make_inputs(2, 13, 4, lower_bound=-5.0, seed=58, init_dtype=torch.float32,
                          device="cuda")
    o1, f1 = run_gpu(x, torch.float32)
    o2, f2 = run_gpu(x, torch.float32, out_fill=1.0)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)
    x2 = synth.KdaInputs(**{**x.__dict__, "v": x.v * 2, "initial_state": x.initial_state * 2})
    o3, f3 = run_gpu(x2, torch.float32)
    assert np.array_equal(o3, 2 * o1) and np.array_equal(f3, 2 * f1)


def test_kernel_option(options):
    """A 5-token call takes the recurrent kernel unless the kernel option
    says otherwise; the two kernels round differently and agree within the
    tolerance."""
    x = synth.make_inputs(2, 5, 3, lower_bound=-5.0, seed=59, init_dtype=torch.float32,
                          device="cuda")
    o_def, f_def = run_gpu(x, torch.float32)
    options(kernel="recurrent")
    o_rec, f_rec = run_gpu(x, torch.float32)
    options(kernel="mfma")
    o_mf, f_mf = run_gpu(x, torch.float32)
    options()
    assert np.array_equal(o_def, o_rec) and np.array_equal(f_def, f_rec)
    assert not np.array_equal(f_rec, f_mf)
    assert_close("recurrent vs chunked out", o_rec, o_mf)
    assert_close("recurrent vs chunked final", f_rec, f_mf)


# --------------------------------------------------------------------------
# the tanh form of the gate's logistic function (sigmoid="tanh"): an
# ablation of the pages' choice, on whole-chain calls of the chunked kernel
# --------------------------------------------------------------------------

@pytest.fixture
def tanh_sigmoid(options):
    options(sigmoid="tanh", kernel="mfma")


def test_tanh_sigmoid_small_workload(tanh_sigmoid):
    print("[case] tanh sigmoid small workload", flush=True)
    check_full("tanh small", synth.workload("small_b2_t128_h8", device="cuda"), torch.float32)


@pytest.mark.parametrize("T", [1, 17, 100])
def test_tanh_sigmoid_ragged(tanh_sigmoid, T):
    print(f"[case] tanh sigmoid T={T}", flush=True)
    x = synth.make_inputs(2, T, 3, lower_bound=-5.0, seed=400 + T, init_dtype=torch.float32,
                          device="cuda")
    check_full(f"tanh T={T}", x, torch.float32)


def test_tanh_sigmoid_gate_extremes(tanh_sigmoid):
    """Saturated gates (g = +-100) hit the clamp of the rational tanh."""
    x = synth.make_inputs(2, 96, 4, lower_bound=-5.0, seed=401, init_dtype=torch.float32,
                          device="cuda")
    x.g.fill_(100.0)
    print("[case] tanh max decay", flush=True)
    check_full("tanh max decay", x, torch.float32)
    y = synth.make_inputs(1, 64, 2, lower_bound=-5.0, seed=402, init_dtype=torch.float32,
                          device="cuda")
    y.g.fill_(-100.0)
    y.beta.fill_(8.0)
    print("[case] tanh min decay, large beta", flush=True)
    check_full("tanh min decay", y, torch.float32)


def test_sigmoid_option(options):
    x = synth.make_inputs(1, 64, 2, lower_bound=-5.0, seed=403, device="cuda")
    o_exp, _ = run_gpu(x)
    options(sigmoid="tanh")
    o_tanh, _ = run_gpu(x)
    options()
    o_exp2, _ = run_gpu(x)
    assert np.array_equal(o_exp, o_exp2)
    assert not np.array_equal(o_exp, o_tanh)
    assert_close("tanh vs exp2 sigmoid", o_tanh, o_exp)


# --------------------------------------------------------------------------
# more chains than compute units, and the write-free degenerate case, on
# both kernels
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", ["mfma", "recurrent"])
def test_many_chains(kernel, options):
    """2048 chains (8 per compute unit) of 40 tokens: grids far larger than
    the GPU, with a ragged last chunk; every chain against the oracle."""
    options(kernel=kernel)
    print(f"[case] many chains kernel={kernel}", flush=True)
    x = synth.make_inputs(2, 40, 1024, lower_bound=-5.0, seed=500, init_dtype=torch.float32,
                          device="cuda")
    check_full(f"many chains {kernel}", x, torch.float32)


@pytest.mark.parametrize("kernel", ["mfma", "recurrent"])
def test_beta_zero_is_pure_decay(kernel, options):
    """beta logits of -100 (beta = 3.7e-44, i.e. no writes): the state only
    decays, final = diag(Gamma_L) S0 and o_t = scale (diag(Gamma_t) S0)^T q_t;
    the oracle computes the same closed form token by token."""
    options(kernel=kernel)
    print(f"[case] beta = 0 kernel={kernel}", flush=True)
    x = synth.make_inputs(2, 37, 3, lower_bound=-2.0, seed=501, init_dtype=torch.float32,
                          device="cuda")
    x.beta.fill_(-100.0)
    check_full(f"beta zero {kernel}", x, torch.float32)


# --------------------------------------------------------------------------
# the single-chunk kernel (kernel="single"): the chunked stages for calls
# of at most 16 tokens per sequence, one 4-wave workgroup per chain
# --------------------------------------------------------------------------

@pytest.fixture
def single_kernel(options):
    options(kernel="single")


@pytest.mark.parametrize("name", ["decode_b64_t1_h32_state", "decode_b64_t8_h32_state",
                                  "decode_b64_t15_h32_state"])
def test_single_decode_workloads(single_kernel, name):
    assert kda.fwd_kernel(16, kernel="single") == "single"
    print(f"[case] single-chunk kernel, workload {name}", flush=True)
    x = synth.workload(name, device="cuda")
    check_full(f"single {name}", x, x.final_dtype)


@pytest.mark.parametrize("T", [0, 1, 5, 15, 16])
def test_single_lengths(single_kernel, T):
    print(f"[case] single-chunk kernel T={T}", flush=True)
    x = synth.make_inputs(2, T, 3, lower_bound=-5.0, seed=600 + T, init_dtype=torch.float32,
                          device="cuda")
    o, f = run_gpu(x, torch.float32)
    ro, rf = oracle_of(x)
    if T:
        assert_close(f"single T={T} out", o, ro)
    assert_close(f"single T={T} final", f, rf)


@pytest.mark.parametrize("init,final", [(None, torch.bfloat16), (torch.bfloat16, torch.bfloat16),
                                        (torch.float32, None), (None, None)])
def test_single_state_combinations(single_kernel, init, final):
    print(f"[case] single-chunk kernel init={init} final={final}", flush=True)
    x = synth.make_inputs(1, 11, 3, lower_bound=-5.0, seed=610, init_dtype=init, device="cuda")
    o, f = run_gpu(x, final)
    ro, rf = oracle_of(x)
    assert_close("single state combo out", o, ro)
    if final is not None:
        assert_close("single state combo final", f, rf)


@pytest.mark.parametrize("case", ["lb0", "lb-0.5", "max_decay", "min_decay", "beta_zero",
                                  "no_gate_params", "tanh"])
def test_single_gates(case, options):
    """Gate extremes and variants on the single-chunk kernel."""
    print(f"[case] single-chunk kernel {case}", flush=True)
    lb = {"lb0": 0.0, "lb-0.5": -0.5}.get(case, -5.0)
    x = synth.make_inputs(2, 16, 4, lower_bound=lb, seed=620, init_dtype=torch.float32,
                          with_gate_params=case != "no_gate_params", device="cuda")
    if case == "max_decay":
        x.g.fill_(100.0)
    if case == "min_decay":
        x.g.fill_(-100.0)
        x.beta.fill_(8.0)
    if case == "beta_zero":
        x.beta.fill_(-100.0)
    options(kernel="single", sigmoid="tanh" if case == "tanh" else None)
    check_full(f"single {case}", x, torch.float32)


def test_single_in_place_and_invariants(single_kernel):
    x = synth.make_inputs(3, 9, 3, lower_bound=-5.0, seed=630, init_dtype=torch.float32,
                          device="cuda")
    o, f = run_gpu(x, torch.float32)
    o2, f2 = run_gpu(x, torch.float32, out_fill=1.0)
    assert np.array_equal(o, o2) and np.array_equal(f, f2)
    x2 = synth.KdaInputs(**{**x.__dict__, "v": x.v * 2, "initial_state": x.initial_state * 2})
    o3, f3 = run_gpu(x2, torch.float32)
    assert np.array_equal(o3, 2 * o) and np.array_equal(f3, 2 * f)
    st = x.initial_state.clone()
    out = torch.empty_like(x.v)
    fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, out, x.A_log, x.dt_bias, x.lower_bound,
            initial_state=st, final_state=st)
    torch.cuda.synchronize()
    assert np.array_equal(out.double().cpu().numpy(), o)
    assert np.array_equal(st.double().cpu().numpy(), f)


def test_single_many_chains(single_kernel):
    print("[case] single-chunk kernel, 2048 chains", flush=True)
    x = synth.make_inputs(2, 13, 1024, lower_bound=-5.0, seed=640, init_dtype=torch.bfloat16,
                          device="cuda")
    check_full("single many", x, torch.bfloat16)


def test_single_rejects_longer_calls(single_kernel):
    """kernel="single" takes only calls of at most 16 tokens without
    cu_seqlens; longer or packed calls are an option error, reported before
    any launch (out stays untouched)."""
    for T, varlen in ((17, False), (8, True)):
        with pytest.raises(ValueError):
            kda.fwd_kernel(T, varlen=varlen, kernel="single")
    x = synth.make_inputs(1, 40, 2, lower_bound=-5.0, seed=650, init_dtype=torch.float32,
                          device="cuda")
    out = torch.zeros_like(x.v)
    with pytest.raises(kda.KdaArgumentError):
        fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, out, x.A_log, x.dt_bias, x.lower_bound)
    torch.cuda.synchronize()
    assert not out.any()


@pytest.mark.parametrize("T,kernel", [(2, "recurrent"), (12, "single"), (17, "mfma")])
def test_max_heads(T, kernel):
    """H = 65536, the most heads the API takes: a grid of 65536 workgroups on
    each of the default kernels (chosen by T); every head against the
    oracle.  No states, so the inputs stay small."""
    assert kda.fwd_kernel(T) == kernel
    print(f"[case] max heads T={T} ({kernel})", flush=True)
    x = synth.make_inputs(1, T, 65536, lower_bound=-5.0, seed=700 + T, device="cuda")
    out = torch.empty_like(x.v)
    fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, out, x.A_log, x.dt_bias, x.lower_bound)
    torch.cuda.synchronize()
    check_all_chains(f"max heads T={T}", x, out, None, batch=8192)


def test_tensors_beyond_4gib():
    """B=8, T=2^20, H=4: every input tensor is 8 GiB, so the last batch
    row's tokens sit more than 7 GiB into it (64-bit offsets everywhere).
    The first 2048 tokens of rows 0 and 7 (all heads) against the oracle, and
    row 7 as a whole (out and final state, all 2^20 tokens) bit for bit
    against the same row run on its own from low addresses."""
    B, T, H = 8, 1 << 20, 4
    print(f"[case] beyond 4 GiB: B={B} T={T} H={H} (inputs {4 * B * T * H * 256 >> 30} GiB)", flush=True)
    x = synth.make_inputs(B, T, H, lower_bound=-5.0, seed=910, device="cuda")
    out = torch.empty_like(x.v)
    final = torch.empty(B, H, 128, 128, dtype=torch.float32, device="cuda")
    fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, out, x.A_log, x.dt_bias, x.lower_bound,
        final_state=final)
    torch.cuda.synchronize()
    n = 2048
    for row in (0, B - 1):
        sl = slice(row, row + 1)
        q, k, v, g, beta = (t[sl, :n].cpu() for t in (x.q, x.k, x.v, x.g, x.beta))
        ro, _ = kda_oracle(q, k, v, g, beta, x.scale, x.A_log.cpu(), x.dt_bias.cpu(),
                           x.lower_bound)
        assert_close(f"beyond 4 GiB row {row} out[:{n}]", out[sl, :n].double().cpu().numpy(), ro)
    row = B - 1
    y = synth.KdaInputs(**{**x.__dict__, **{t: getattr(x, t)[row:row + 1].contiguous()
                                            for t in ("q", "k", "v", "g", "beta")}})
    del x
    out1 = torch.empty_like(y.v)
    final1 = torch.empty(1, H, 128, 128, dtype=torch.float32, device="cuda")
    fwd(y.q, y.k, y.v, y.g, y.beta, y.scale, out1, y.A_log, y.dt_bias, y.lower_bound,
        final_state=final1)
    torch.cuda.synchronize()
    assert torch.equal(out1[0], out[row]), "row 7: out differs from the same row run alone"
    assert torch.equal(final1[0], final[row]), "row 7: final state differs"
    assert torch.isfinite(final).all()


# --------------------------------------------------------------------------
# HIP graph capture (serving loops replay a captured call)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,seg,kernel", [(3, None, "recurrent"), (12, None, "single"),
                                          (100, None, "mfma"), (600, 2, "segmented")])
def test_graph_capture_replays(T, seg, kernel):
    """kda.fwd captured in a HIP graph (torch.cuda.CUDAGraph) and replayed
    three times, with new inputs copied in and the outputs cleared (eager
    work) and a synchronisation between replays: every replay equals the
    eager call on the same inputs bit for bit, and the last one the oracle."""
    B, H = (4, 4) if seg is None else (1, 2)
    if seg is None:
        assert kda.fwd_kernel(T) == kernel
    print(f"[case] graph capture {kernel} B={B} T={T} H={H}", flush=True)
    x = synth.make_inputs(B, T, H, lower_bound=-5.0, seed=900 + T, init_dtype=torch.float32,
                          device="cuda")
    out, fin = torch.empty_like(x.v), torch.empty_like(x.initial_state)
    ref_out, ref_fin = torch.empty_like(out), torch.empty_like(fin)

    def call(o, f):
        fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, o, x.A_log, x.dt_bias, x.lower_bound,
                initial_state=x.initial_state, final_state=f, segment_chunks=seg)

    call(out, fin)  # outside the capture first (loads the library)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out, fin)
    for r in range(3):
        y = synth.make_inputs(B, T, H, lower_bound=-5.0, seed=910 + 10 * T + r,
                              init_dtype=torch.float32, device="cuda")
        for name in ("q", "k", "v", "g", "beta", "initial_state"):
            getattr(x, name).copy_(getattr(y, name))
        out.zero_()
        fin.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        call(ref_out, ref_fin)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(fin, ref_fin), f"replay {r} differs from the eager call"
    ro, rf = oracle_of(x)
    assert_close(f"graph {kernel} out", out.double().cpu().numpy(), ro)
    assert_close(f"graph {kernel} final", fin.double().cpu().numpy(), rf)


# --------------------------------------------------------------------------
# Seeded sweep: random shapes, packed lengths, gate bounds, state dtypes and
# the library's kernels and forms, each checked against the oracle.
# --------------------------------------------------------------------------

SWEEP_STATES = [(None, None), (None, torch.bfloat16), (None, torch.float32),
                (torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                (torch.float32, None), (torch.bfloat16, None)]


def sweep_case(i):
    """Case i of the sweep: a plain description of one call (seeded)."""
    import random
    rng = random.Random(1000 + i)
    varlen = rng.random() < 0.4
    H = rng.randint(1, 6)
    lb = rng.choice([-5.0, -3.0, -0.5, 0.0, round(rng.uniform(-5.0, 0.0), 3)])
    init, final = rng.choice(SWEEP_STATES)
    if varlen:
        lens = [rng.choice([0, 1, 15, 16, 17, rng.randint(0, 300)]) for _ in range(rng.randint(1, 4))]
        B, T = 1, sum(lens)
    else:
        lens = None
        B = rng.randint(1, 3)
        T = rng.choice([0, 1, rng.randint(2, 16), rng.randint(17, 64), rng.randint(65, 400)])
    form = rng.choice(["auto", "mfma", "recurrent", "single", "neumann", "tanh", "segmented"])
    if form == "single" and (varlen or T > 16):
        form = "auto"
    seg = rng.randint(1, 4) if form == "segmented" else None
    return dict(B=B, T=T, H=H, lens=lens, lb=lb, init=init, final=final, form=form, seg=seg,
                seed=2000 + i)


@pytest.mark.parametrize("i", range(40))
def test_seeded_sweep(i, options):
    c = sweep_case(i)
    print(f"[case] sweep {i}: {c}", flush=True)
    form = c["form"]
    if form in ("mfma", "recurrent", "single"):
        options(kernel=form)
    elif form == "neumann":
        options(inverse="neumann")
    elif form == "tanh":
        options(sigmoid="tanh")
    x = synth.make_inputs(c["B"], c["T"], c["H"], lower_bound=c["lb"], seed=c["seed"],
                          seq_lengths=c["lens"], init_dtype=c["init"], device="cuda")
    o, f = run_gpu(x, c["final"], segment_chunks=c["seg"])
    ro, rf = oracle_of(x)
    if c["T"]:
        assert_close(f"sweep {i} out", o, ro)
    if f is not None:
        assert_close(f"sweep {i} final", f, rf)
