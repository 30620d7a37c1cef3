"""Host-side checks of the C-ABI boundary and the Python binding (no GPU).

The library must load and export every entry point ``include/kda.h``
declares, and every argument error must be reported before any launch, so
these calls never reach a kernel (the pointers passed are never read).
"""
from __future__ import annotations

import ctypes
import math
import os
import re
import subprocess

import pytest
import torch

import gated_delta_rule_36_amd as kda
from gated_delta_rule_36_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIBRARY], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kda_\w+)", nm))
    assert set(declared_functions()) <= exported
    assert lib.kda_abi_version() == _lib.ABI_VERSION


def test_library_has_gfx950_code_and_no_oracle():
    data = open(_lib.LIBRARY, "rb").read()
    assert b"gfx950" in data
    assert b"kda_oracle" not in data


# --------------------------------------------------------------------------
# C-ABI argument errors (host checks only; pointers are dummies)
# --------------------------------------------------------------------------

FAKE = [ctypes.create_string_buffer(64 + 16) for _ in range(12)]
ADDR = [(ctypes.addressof(b) + 15) & ~15 for b in FAKE]  # 16-byte aligned, like allocator memory
# a whole fp32 state (H = 1) of its own, so that a state span cannot overlap the other dummies
STATE_BUF = ctypes.create_string_buffer(128 * 128 * 4 + 32)
STATE_ADDR = (ctypes.addressof(STATE_BUF) + 15) & ~15


def call(**over):
    """kda_fwd with well-formed dummy arguments, some replaced by ``over``."""
    a = dict(q=ADDR[0], k=ADDR[1], v=ADDR[2], g=ADDR[3], beta=ADDR[4], scale=0.1,
             out=ADDR[5], A_log=ADDR[6], dt_bias=ADDR[7], lower_bound=-5.0,
             init=None, init_dtype=0, final=None, final_dtype=0, cu=None, num_seqs=0,
             B=1, T=0, H=1, K=128, V=128)
    a.update(over)
    lib = _lib.load()
    args = (a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["out"], a["A_log"],
            a["dt_bias"], a["lower_bound"], a["init"], a["init_dtype"], a["final"],
            a["final_dtype"], a["cu"], a["num_seqs"], a["B"], a["T"], a["H"], a["K"], a["V"])
    if "options" in a:
        return lib.kda_fwd_ex(*args, a["options"], None)
    return lib.kda_fwd(*args, None)


# The dummy buffers are only 64 bytes, but the size checks use the declared
# shapes; with T = 0 nothing is launched even when every check passes, so the
# base call must fail only on the planted error.  Overlap checks see the
# dummies' real addresses with the declared sizes, so calls that would
# otherwise pass with T > 0 are never made.
@pytest.mark.parametrize("over,code", [
    (dict(q=None, T=1), _lib.KDA_ERR_NULL_POINTER),
    (dict(beta=None, T=1), _lib.KDA_ERR_NULL_POINTER),
    (dict(out=None, T=1), _lib.KDA_ERR_NULL_POINTER),
    (dict(init=ADDR[8], init_dtype=0), _lib.KDA_ERR_NULL_POINTER),
    (dict(K=64), _lib.KDA_ERR_HEAD_DIM),
    (dict(V=256), _lib.KDA_ERR_HEAD_DIM),
    (dict(lower_bound=0.5), _lib.KDA_ERR_LOWER_BOUND),
    (dict(lower_bound=-5.0001), _lib.KDA_ERR_LOWER_BOUND),
    (dict(lower_bound=math.nan), _lib.KDA_ERR_LOWER_BOUND),
    (dict(cu=ADDR[9], num_seqs=1, B=2), _lib.KDA_ERR_VARLEN_BATCH),
    (dict(cu=ADDR[9], num_seqs=-1), _lib.KDA_ERR_VARLEN_BATCH),
    (dict(init=ADDR[8], init_dtype=1, final=ADDR[10], final_dtype=2), _lib.KDA_ERR_STATE_DTYPE),
    (dict(init=ADDR[8], init_dtype=7), _lib.KDA_ERR_STATE_DTYPE),
    (dict(out=ADDR[0], T=1), _lib.KDA_ERR_ALIAS),
    (dict(final=ADDR[3], final_dtype=2, T=1), _lib.KDA_ERR_ALIAS),
    (dict(init=ADDR[8], init_dtype=2, final=ADDR[8] + 4, final_dtype=2), _lib.KDA_ERR_ALIAS),
    (dict(B=0), _lib.KDA_ERR_SIZE),
    (dict(H=0), _lib.KDA_ERR_SIZE),
    (dict(H=65537), _lib.KDA_ERR_SIZE),
    (dict(T=-1), _lib.KDA_ERR_SIZE),
    (dict(B=1 << 40, T=1 << 30), _lib.KDA_ERR_SIZE),
    (dict(scale=math.inf), _lib.KDA_ERR_SCALE),
    (dict(scale=math.nan), _lib.KDA_ERR_SCALE),
    (dict(q=ADDR[0] + 8), _lib.KDA_ERR_ALIGNMENT),
    (dict(g=ADDR[3] + 2), _lib.KDA_ERR_ALIGNMENT),
    (dict(out=ADDR[5] + 4), _lib.KDA_ERR_ALIGNMENT),
    (dict(beta=ADDR[4] + 1), _lib.KDA_ERR_ALIGNMENT),
    (dict(dt_bias=ADDR[7] + 2), _lib.KDA_ERR_ALIGNMENT),
    (dict(init=ADDR[8] + 8, init_dtype=1), _lib.KDA_ERR_ALIGNMENT),
    (dict(final=STATE_ADDR + 8, final_dtype=2), _lib.KDA_ERR_ALIGNMENT),
    (dict(cu=ADDR[9] + 4, num_seqs=0), _lib.KDA_ERR_ALIGNMENT),
])
def test_argument_errors_are_reported_before_launch(over, code):
    assert call(**over) == code


def test_status_strings_are_distinct():
    msgs = [_lib.status_string(c) for c in range(13)]
    assert len(set(msgs)) == 13 and msgs[0] == "ok"
    assert _lib.status_string(123) == "unknown status"


# --------------------------------------------------------------------------
# kda_fwd_scan: workspace size and its argument errors (host checks only)
# --------------------------------------------------------------------------

SLAB = 128 * 128 * 4


def test_scan_workspace_bytes():
    ws = _lib.load().kda_fwd_scan_workspace_bytes
    # 16 chains of 512 chunks in segments of 32: 16 segments, two fp32 slabs each
    assert ws(None, 0, 1, 8192, 16, 32) == 16 * 16 * 2 * SLAB
    # a partial last segment still counts, and T = 0 has one (empty) segment
    assert ws(None, 0, 2, 8192 + 1, 3, 32) == 6 * 17 * 2 * SLAB
    assert ws(None, 0, 2, 0, 3, 5) == 6 * 1 * 2 * SLAB
    # packed mode counts num_seqs chains per head; cu_seqlens is not read
    assert ws(ADDR[9], 5, 1, 100, 2, 1) == 10 * 7 * 2 * SLAB
    assert ws(None, 0, 1, 64, 1, 0) == -1
    assert ws(None, 0, 1, -1, 1, 4) == -1
    assert ws(None, 0, 1 << 40, 1 << 30, 1 << 20, 1) == -1


# separate 4 KiB dummies: with T = 1 the declared spans (256 bytes per token
# tensor) stay inside them, so only the planted overlap is seen
BIG = [ctypes.create_string_buffer((1 << 12) + 16) for _ in range(12)]
BADDR = [(ctypes.addressof(b) + 15) & ~15 for b in BIG]


def call_scan(seg=4, ws=None, ws_bytes=1 << 30, **over):
    a = dict(q=BADDR[0], k=BADDR[1], v=BADDR[2], g=BADDR[3], beta=BADDR[4], scale=0.1,
             out=BADDR[5], A_log=BADDR[6], dt_bias=BADDR[7], lower_bound=-5.0,
             init=None, init_dtype=0, final=None, final_dtype=0, cu=None, num_seqs=0,
             B=1, T=0, H=1, K=128, V=128)
    a.update(over)
    return _lib.load().kda_fwd_scan(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["out"],
                                    a["A_log"], a["dt_bias"], a["lower_bound"], a["init"],
                                    a["init_dtype"], a["final"], a["final_dtype"], a["cu"],
                                    a["num_seqs"], a["B"], a["T"], a["H"], a["K"], a["V"],
                                    seg, ws, ws_bytes, a.get("options"), None)


# Every call fails on the planted error, so nothing is launched.
@pytest.mark.parametrize("kw,code", [
    (dict(seg=0, ws=BADDR[11]), _lib.KDA_ERR_SIZE),
    (dict(seg=-3, ws=BADDR[11]), _lib.KDA_ERR_SIZE),
    (dict(ws=None), _lib.KDA_ERR_WORKSPACE),
    (dict(ws=BADDR[11], ws_bytes=2 * SLAB - 1), _lib.KDA_ERR_WORKSPACE),
    (dict(ws=BADDR[11] + 4), _lib.KDA_ERR_WORKSPACE),
    (dict(ws=BADDR[0], T=1), _lib.KDA_ERR_WORKSPACE),          # overlaps q
    (dict(ws=BADDR[5] - 64, T=1), _lib.KDA_ERR_WORKSPACE),     # overlaps out
    (dict(ws=BADDR[11], K=64), _lib.KDA_ERR_HEAD_DIM),         # kda_fwd's checks come first
    (dict(ws=BADDR[11], out=BADDR[0], T=1), _lib.KDA_ERR_ALIAS),
])
def test_scan_argument_errors_are_reported_before_launch(kw, code):
    over = {k: v for k, v in kw.items() if k not in ("seg", "ws", "ws_bytes")}
    args = {k: v for k, v in kw.items() if k in ("seg", "ws", "ws_bytes")}
    assert call_scan(**args, **over) == code


def call_static(seg=4, **over):
    a = dict(q=BADDR[0], k=BADDR[1], v=BADDR[2], g=BADDR[3], beta=BADDR[4], scale=0.1,
             out=BADDR[5], A_log=BADDR[6], dt_bias=BADDR[7], lower_bound=-5.0,
             init=None, init_dtype=0, final=None, final_dtype=0, cu=None, num_seqs=0,
             B=1, T=0, H=1, K=128, V=128)
    a.update(over)
    return _lib.load().kda_fwd_scan_static(
        a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["out"], a["A_log"], a["dt_bias"],
        a["lower_bound"], a["init"], a["init_dtype"], a["final"], a["final_dtype"], a["cu"],
        a["num_seqs"], a["B"], a["T"], a["H"], a["K"], a["V"], seg, a.get("options"), None)


def test_scan_static_host_checks():
    """kda_fwd_scan_static: the argument and option checks of kda_fwd_scan,
    and scratch beyond KDA_SCAN_STATIC_BYTES refused, all before the
    library's array is looked up or anything is enqueued."""
    tb = 1 << 44  # fake addresses 16 TiB apart, never dereferenced
    fake = {n: (i + 1) * tb for i, n in enumerate(["q", "k", "v", "g", "beta", "out", "A_log", "dt_bias"])}
    # 4 chains x 66 segments x 128 KiB = 33 MiB > 32 MiB
    assert call_static(seg=1, T=16 * 66, H=4, **fake) == _lib.KDA_ERR_WORKSPACE
    assert call_static(seg=0) == _lib.KDA_ERR_SIZE
    assert call_static(K=64) == _lib.KDA_ERR_HEAD_DIM
    assert call_static(options=_opts(sigmoid=_lib.KDA_SIGMOID_TANH)) == _lib.KDA_ERR_OPTION
    # no chain: nothing to do, no lookup
    assert call_static(cu=BADDR[9], num_seqs=0) == _lib.KDA_OK


def test_scan_combine_grid_limit():
    """With more than two segments the combine step runs 8 blocks per chain:
    more than INT32_MAX / 8 chains is a size error, reported before the
    workspace is looked at, even where chains x segments still fits."""
    tb = 1 << 44  # fake addresses 16 TiB apart, never dereferenced: no declared spans overlap
    fake = {n: (i + 1) * tb for i, n in enumerate(["q", "k", "v", "g", "beta", "out", "A_log", "dt_bias"])}
    B, H = 4097, 65536  # 268,500,992 chains: above 2^31 / 8, and x 3 segments below 2^31
    assert call_scan(seg=1, ws=None, T=48, B=B, H=H, **fake) == _lib.KDA_ERR_SIZE
    # one segment per chain: no combine step, so the missing workspace is the error
    assert call_scan(seg=16, ws=None, T=48, B=B, H=H, **fake) == _lib.KDA_ERR_WORKSPACE


def test_auto_segment_chunks_policy():
    auto = kda.auto_segment_chunks
    assert auto(16, 8192) == 32          # 16 chains x 16 segments of 32 chunks
    assert auto(1, 100000) == 25         # one chain: about 256 segments
    assert auto(128, 1 << 20) is None    # enough chains already
    assert auto(256, 16384) is None
    assert auto(4, 200) is None          # too short to cut
    assert auto(0, 1000) is None


def _opts(kernel=0, inverse=0, sigmoid=0, reserved=0):
    return ctypes.byref(_lib.Options(kernel, inverse, sigmoid, reserved))


def test_kernel_choice():
    """Decode-shaped calls (no cu_seqlens, at most 16 tokens) take the
    recurrent kernel up to 8 tokens and the single-chunk kernel beyond,
    everything else the pipelined chunked one; the options force a kernel,
    and restrict the automatic choice to the kernels that implement a
    non-default inverse or sigmoid.  No environment variable is read."""
    choice = kda.fwd_kernel
    assert [choice(t) for t in (0, 1, 8)] == ["recurrent"] * 3
    assert [choice(t) for t in (9, 15, 16)] == ["single"] * 3
    assert [choice(t) for t in (17, 64, 16384)] == ["mfma"] * 3
    assert choice(1, varlen=True) == choice(16, varlen=True) == "mfma"
    for forced in ("mfma", "recurrent"):
        assert choice(1, kernel=forced) == choice(10000, kernel=forced) == \
            choice(5, varlen=True, kernel=forced) == forced
    assert choice(0, kernel="single") == choice(16, kernel="single") == "single"
    for bad in (dict(T=17), dict(T=5, varlen=True)):
        with pytest.raises(ValueError):
            choice(kernel="single", **bad)
    # the Neumann inverse exists in the chunked kernel only
    assert choice(1, inverse="neumann") == choice(16, inverse="neumann") == "mfma"
    with pytest.raises(ValueError):
        choice(1, kernel="recurrent", inverse="neumann")
    with pytest.raises(ValueError):
        choice(12, kernel="single", inverse="neumann")
    # the tanh-form sigmoid: single-chunk kernel for decode-shaped calls, else chunked
    assert choice(3, sigmoid="tanh") == choice(16, sigmoid="tanh") == "single"
    assert choice(17, sigmoid="tanh") == choice(3, varlen=True, sigmoid="tanh") == "mfma"
    with pytest.raises(ValueError):
        choice(3, kernel="recurrent", sigmoid="tanh")
    with pytest.raises(ValueError):
        choice(100, inverse="neumann", sigmoid="tanh")
    with pytest.raises(ValueError):
        choice(100, kernel="simt")


def test_kernel_choice_ignores_the_environment(monkeypatch):
    monkeypatch.setenv("KDA_KERNEL", "mfma")
    monkeypatch.setenv("KDA_INVERSE", "neumann")
    monkeypatch.setenv("KDA_SIGMOID", "tanh")
    assert kda.fwd_kernel(1) == "recurrent" and kda.fwd_kernel(12) == "single"


def test_kda_fwd_kernel_c_abi():
    f = _lib.load().kda_fwd_kernel
    assert f(5, 0, None) == b"recurrent" and f(5, 1, None) == b"mfma"
    assert f(5, 0, _opts(kernel=_lib.KDA_KERNEL_SINGLE)) == b"single"
    assert f(5, 0, _opts(kernel=9)) is None
    assert f(5, 0, _opts(inverse=2)) is None
    assert f(5, 0, _opts(sigmoid=-1)) is None
    assert f(5, 0, _opts(reserved=1)) is None


@pytest.mark.parametrize("opts", [dict(kernel=4), dict(inverse=7), dict(sigmoid=2), dict(reserved=3),
                                  dict(kernel=_lib.KDA_KERNEL_RECURRENT, inverse=_lib.KDA_INVERSE_NEUMANN),
                                  dict(kernel=_lib.KDA_KERNEL_SINGLE, inverse=_lib.KDA_INVERSE_NEUMANN),
                                  dict(inverse=_lib.KDA_INVERSE_NEUMANN, sigmoid=_lib.KDA_SIGMOID_TANH)])
def test_option_errors_are_reported_before_launch(opts):
    assert call(options=_opts(**opts)) == _lib.KDA_ERR_OPTION
    # and the argument checks still come first
    assert call(options=_opts(**opts), K=64) == _lib.KDA_ERR_HEAD_DIM


def test_default_options_equal_kda_fwd():
    # packed mode with no sequence: every check passes and nothing is launched
    none = dict(cu=ADDR[9], num_seqs=0)
    assert call(options=None, **none) == call(options=_opts(), **none) == call(**none) == _lib.KDA_OK


def test_scan_option_errors():
    ws = dict(ws=BADDR[11])
    for o in (dict(kernel=_lib.KDA_KERNEL_RECURRENT), dict(kernel=_lib.KDA_KERNEL_SINGLE),
              dict(sigmoid=_lib.KDA_SIGMOID_TANH), dict(reserved=1), dict(inverse=5)):
        assert call_scan(**ws, options=_opts(**o)) == _lib.KDA_ERR_OPTION, o
    for o in (dict(kernel=_lib.KDA_KERNEL_CHUNKED), dict(inverse=_lib.KDA_INVERSE_NEUMANN), dict()):
        # packed mode with no sequence: valid options pass, nothing is launched
        assert call_scan(**ws, cu=BADDR[9], num_seqs=0, options=_opts(**o)) == _lib.KDA_OK, o


def test_binding_rejects_unknown_option_names():
    with pytest.raises(ValueError, match="kernel"):
        kda.fwd_kernel(5, kernel="simt")
    with pytest.raises(ValueError, match="sigmoid"):
        kda.fwd_kernel(5, sigmoid="logistic")


def test_empty_token_tensors_may_be_null():
    """With T = 0 the token tensors are empty (torch gives them a NULL data
    pointer), which is accepted; packed mode with no sequence launches
    nothing, so this stays a host-only call."""
    assert call(q=None, k=None, v=None, g=None, beta=None, out=None, cu=ADDR[9],
                num_seqs=0) == _lib.KDA_OK


def test_zero_sequences_is_a_no_op():
    # packed mode with N = 0 has no chain: OK without a launch
    assert call(cu=ADDR[9], num_seqs=0) == _lib.KDA_OK


# --------------------------------------------------------------------------
# Python binding checks (raised before the library is called)
# --------------------------------------------------------------------------

def _cpu_args(**over):
    B, T, H = 1, 4, 2
    a = dict(q=torch.zeros(B, T, H, 128, dtype=torch.bfloat16),
             k=torch.zeros(B, T, H, 128, dtype=torch.bfloat16),
             v=torch.zeros(B, T, H, 128, dtype=torch.bfloat16),
             g=torch.zeros(B, T, H, 128, dtype=torch.bfloat16),
             beta=torch.zeros(B, T, H, dtype=torch.bfloat16), scale=0.1,
             out=torch.zeros(B, T, H, 128, dtype=torch.bfloat16),
             A_log=torch.zeros(H), dt_bias=torch.zeros(H, 128), lower_bound=-5.0)
    a.update(over)
    return a


def test_binding_rejects_wrong_dtype():
    with pytest.raises(TypeError):
        kda.fwd(**_cpu_args(q=torch.zeros(1, 4, 2, 128)))
    with pytest.raises(TypeError):
        kda.fwd(**_cpu_args(beta=torch.zeros(1, 4, 2)))


def test_binding_rejects_host_tensors():
    with pytest.raises(ValueError, match="GPU"):
        kda.fwd(**_cpu_args())


def test_binding_rejects_non_tensors():
    with pytest.raises(TypeError):
        kda.fwd(**_cpu_args(q=[1, 2, 3]))


def test_rational_tanh_constants_match_their_fit():
    """The kernel's rational-tanh coefficients are the ones fit_tanh.py
    produces, and their fp32 evaluation stays within 5e-7 of tanh."""
    import re
    import numpy as np
    from gated_delta_rule_36_amd import fit_tanh
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "gated_delta_rule_36_amd", "csrc", "kda_chunk_mfma.hip")).read()
    consts = {m.group(1): float(m.group(2)) for m in re.finditer(r"kTanh([PQ]\d) = ([0-9.e+-]+)f", src)}
    p, q = fit_tanh.fit()
    for i in range(1, 5):
        assert np.float32(consts[f"P{i}"]) == p[i] and np.float32(consts[f"Q{i}"]) == q[i]
    assert p[0] == 1.0 and q[0] == 1.0
    ys = np.linspace(-20, 20, 100001)
    assert float(np.abs(fit_tanh.tanh32(ys, p, q) - np.tanh(ys)).max()) < 5e-7
