"""The C ABI on the host: the library loads without a GPU, exports every
function include/kda.h declares, and its synchronous validation paths return
the documented status before any device work (no compute call is made)."""
import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_110_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "kda.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\S.*?\b(kda_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        kda.build()
    return kda.library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) >= {"kda_fwd", "kda_fwd_workspace_size", "kda_status_string"}
    dyn = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert hasattr(lib, n), n
        assert re.search(r"\bT %s$" % n, dyn, flags=re.M), n


def test_status_strings(lib):
    for s in range(9):
        assert lib.kda_status_string(s)
    assert lib.kda_status_string(99) == b"unknown status"


def _desc(**kw):
    d = kda.KdaDesc(1, 64, 2, 128, 128, 1, 2, 2, None, 0, None)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def _call(lib, d, lb=-5.0, scale=0.1, null=(), align=None, cu=None):
    ptrs = {n: ctypes.c_void_p(FAKE) for n in ("q", "k", "v", "g", "beta", "A_log", "dt_bias", "out")}
    for n in null:
        ptrs[n] = None
    if align:
        ptrs[align] = ctypes.c_void_p(FAKE + 2)
    return lib.kda_fwd(ptrs["q"], ptrs["k"], ptrs["v"], ptrs["g"], ptrs["beta"], scale, ptrs["A_log"],
                       ptrs["dt_bias"], lb, None, None, cu, ptrs["out"], ctypes.byref(d), None)


def test_validation_errors(lib):
    ws = kda.workspace_size(1, 64, 2)
    ok_ws = dict(workspace=ctypes.c_void_p(0x100000), workspace_bytes=0)  # too small on purpose
    assert _call(lib, _desc(K=64)) == 3
    assert _call(lib, _desc(V=256)) == 3
    assert _call(lib, _desc(B=0)) == 2
    assert _call(lib, _desc(H=0)) == 2
    assert _call(lib, _desc(T=-1)) == 2
    assert _call(lib, _desc(num_seqs=3)) == 2                 # unpacked: num_seqs must equal B
    assert _call(lib, _desc(B=2, num_seqs=2), cu=ctypes.c_void_p(FAKE)) == 2  # packed needs B == 1
    assert _call(lib, _desc(), lb=-5.5) == 4
    assert _call(lib, _desc(), lb=0.25) == 4
    assert _call(lib, _desc(), lb=float("nan")) == 4
    assert _call(lib, _desc(), scale=float("inf")) == 4
    for n in ("q", "k", "v", "g", "beta", "out", "A_log", "dt_bias"):
        assert _call(lib, _desc(), null=(n,)) == 1, n
    for n in ("q", "k", "v", "g", "out", "dt_bias"):
        assert _call(lib, _desc(), align=n) == 6, n
    d = _desc(**ok_ws)
    assert _call(lib, d) == 7
    d = _desc(workspace=ctypes.c_void_p(0x100010), workspace_bytes=ws)  # not 256-aligned
    assert _call(lib, d) == 6
    assert _call(lib, _desc(save_states=-1)) == 4
    assert _call(lib, _desc(save_states=2)) == 4
    # the saved states need a larger workspace
    d = _desc(B=2, num_seqs=2, save_states=1, workspace=ctypes.c_void_p(0x100000),
              workspace_bytes=kda.workspace_size(2, 64, 2))
    assert _call(lib, d) == 7
    # bad state dtype
    d = _desc(final_state_dtype=7)
    assert lib.kda_fwd(*([ctypes.c_void_p(FAKE)] * 5), 0.1, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), -5.0,
                       None, ctypes.c_void_p(FAKE), None, ctypes.c_void_p(FAKE), ctypes.byref(d), None) == 5


def test_workspace_size_monotone(lib):
    prev = 0
    for T in (0, 1, 64, 65, 1000, 8192):
        s = kda.workspace_size(1, T, 4)
        assert s >= prev and s % 256 == 0
        prev = s
    assert kda.workspace_size(1, 8192, 32, num_seqs=10) > kda.workspace_size(1, 8192, 32)
    assert kda.workspace_size(2, 64, 2, num_seqs=3) == 0          # invalid shapes -> 0
    # about 72.5 KiB per (64-token chunk, head)
    per = (kda.workspace_size(4, 64 * 100, 8) - kda.workspace_size(4, 64 * 50, 8)) / (4 * 50 * 8)
    assert abs(per - 72.5 * 1024) < 512
    # and 64 KiB more for the saved fp32 states
    assert kda.workspace_size(4, 64 * 100, 8, save_states=True) - kda.workspace_size(4, 64 * 100, 8) == \
        4 * 100 * 8 * 65536


def test_chain_segments_rule(lib):
    # automatic: split only when the B*H chains (8 workgroups each) leave most CUs idle (at
    # least 3 segments); the larger of one round of segment workgroups over the 256 CUs with
    # at least 32 chunks per segment, and two rounds with at least 64 chunks per segment
    assert kda.chain_segments_for(1, 8192, 32) == 1
    assert kda.chain_segments_for(1, 131072, 32) == 1           # two rounds: 2 segments, too few
    assert kda.chain_segments_for(1, 131072, 24) == 1
    assert kda.chain_segments_for(1, 131072, 20) == 3           # two rounds
    assert kda.chain_segments_for(1, 131072, 16) == 4
    assert kda.chain_segments_for(1, 131072, 12) == 5
    assert kda.chain_segments_for(1, 131072, 10) == 6
    assert kda.chain_segments_for(1, 131072, 8) == 8
    assert kda.chain_segments_for(1, 131072, 4) == 16
    assert kda.chain_segments_for(1, 131072, 2) == 32
    assert kda.chain_segments_for(1, 131072, 1) == 32           # one round: 64 chunks per segment
    assert kda.chain_segments_for(2, 131072, 1) == 32
    assert kda.chain_segments_for(1, 65536, 4) == 16
    assert kda.chain_segments_for(1, 16384, 4) == 8             # one round: two would need 64 chunks
    assert kda.chain_segments_for(1, 8192, 4) == 4              # 128 chunks: at most 4 segments
    assert kda.chain_segments_for(1, 4096, 4) == 1              # 64 chunks: 2 segments only
    assert kda.chain_segments_for(1, 1024, 1) == 1
    # forced: equal segments of ceil(chunks / n) chunks, at most one per chunk
    assert kda.chain_segments_for(1, 64 * 40 + 17, 2, 4) == 4   # 41 chunks: 11, 11, 11, 8
    assert kda.chain_segments_for(1, 64 * 10, 2, 3) == 3        # 4, 4, 2
    assert kda.chain_segments_for(1, 64 * 9, 2, 4) == 3         # 3, 3, 3
    assert kda.chain_segments_for(1, 64 * 5 + 1, 2, 100) == 6
    assert kda.chain_segments_for(1, 8192, 4, 1) == 1
    assert kda.chain_segments_for(1, 0, 4, 4) == 1
    assert kda.chain_segments_for(1, 8192, 4, -1) == -1
    # errors: a negative count; a split asked for together with cu_seqlens
    assert _call(lib, _desc(chain_segments=-2)) == 4
    assert _call(lib, _desc(launch_piece=-1)) == 4              # negative launch cap
    assert _call(lib, _desc(chain_segments=2), cu=ctypes.c_void_p(FAKE)) == 3
    # 192 KiB of workspace per (batch row, segment, head): two maps and the entering state,
    # fp32 128 x 128 each (B = 2: only the unpacked layout counts)
    extra = kda.workspace_size(2, 64 * 40, 2, chain_segments=4) - kda.workspace_size(2, 64 * 40, 2, chain_segments=1)
    assert 2 * 4 * 2 * 192 * 1024 <= extra <= 2 * 4 * 2 * 192 * 1024 + 1024


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kda.fwd(x, x, x, x, torch.zeros((1, 64, 2), dtype=torch.bfloat16), 0.1, None,
                torch.zeros(2), torch.zeros(2, 128), -5.0)


def _call_decode(lib, d, lb=-5.0, scale=0.1, null=(), align=None, h0=None, ht=None):
    ptrs = {n: ctypes.c_void_p(FAKE) for n in ("q", "k", "v", "g", "beta", "A_log", "dt_bias", "out")}
    for n in null:
        ptrs[n] = None
    if align:
        ptrs[align] = ctypes.c_void_p(FAKE + 2)
    return lib.kda_decode(ptrs["q"], ptrs["k"], ptrs["v"], ptrs["g"], ptrs["beta"], scale, ptrs["A_log"],
                          ptrs["dt_bias"], lb, h0, ht, ptrs["out"], ctypes.byref(d), None)


def test_decode_validation_errors(lib):
    one = dict(T=1, B=3, num_seqs=3)
    assert _call_decode(lib, _desc(**dict(one, T=2))) == 2          # one token per sequence
    assert _call_decode(lib, _desc(**dict(one, num_seqs=2))) == 2
    assert _call_decode(lib, _desc(**dict(one, B=0, num_seqs=0))) == 2
    assert _call_decode(lib, _desc(**dict(one, K=64))) == 3
    assert _call_decode(lib, _desc(**one), lb=-6.0) == 4
    assert _call_decode(lib, _desc(**one), scale=float("nan")) == 4
    for n in ("q", "k", "v", "g", "beta", "out", "A_log", "dt_bias"):
        assert _call_decode(lib, _desc(**one), null=(n,)) == 1, n
    for n in ("q", "k", "v", "g", "out", "dt_bias"):
        assert _call_decode(lib, _desc(**one), align=n) == 6, n
    assert _call_decode(lib, _desc(**dict(one, initial_state_dtype=9)), h0=ctypes.c_void_p(FAKE)) == 5
    assert _call_decode(lib, _desc(**one), ht=ctypes.c_void_p(FAKE + 4)) == 6


def test_python_decode_rejects_bad_shapes():
    import torch
    x = torch.zeros((2, 2, 3, 128), dtype=torch.bfloat16)   # two tokens: not a decode step
    with pytest.raises(ValueError):
        kda.decode(x, x, x, x, torch.zeros((2, 2, 3), dtype=torch.bfloat16), 0.1, None,
                   torch.zeros(3), torch.zeros(3, 128), -5.0)


def test_python_status_errors():
    # argument statuses are ValueErrors (and KdaErrors); a HIP launch error is a RuntimeError only
    lib = kda.library()
    with pytest.raises(ValueError) as e:
        kda._raise_status(lib, 4)
    assert isinstance(e.value, kda.KdaArgumentError) and e.value.status == 4
    with pytest.raises(kda.KdaError) as e:
        kda._raise_status(lib, kda.KDA_ERR_HIP)
    assert not isinstance(e.value, ValueError) and isinstance(e.value, RuntimeError)


def test_noalloc_validation_and_limit(lib):
    # kda_fwd_noalloc validates exactly like kda_fwd, and refuses a call whose workspace
    # would exceed its static scratch before touching the device (no GPU needed here)
    lib.kda_fwd_noalloc.restype = ctypes.c_int
    lib.kda_fwd_noalloc_max_workspace.restype = ctypes.c_size_t
    cap = lib.kda_fwd_noalloc_max_workspace()
    assert cap == 128 << 20

    def call(d, lb=-5.0):
        ptrs = [ctypes.c_void_p(FAKE)] * 5
        return lib.kda_fwd_noalloc(*ptrs, ctypes.c_float(0.1), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                                   ctypes.c_float(lb), None, None, None, ctypes.c_void_p(FAKE), ctypes.byref(d),
                                   None)
    assert call(_desc(K=64)) == 3
    assert call(_desc(), lb=0.5) == 4
    assert call(_desc(launch_piece=-1)) == 4
    assert call(_desc(save_states=1)) == 4     # later calls reuse the scratch: nothing to keep
    big = _desc(T=8192, H=32)  # 4096 (chunk, head) pairs: about 290 MiB of workspace
    assert kda.workspace_size(1, 8192, 32) > cap
    assert call(big) == 9
    assert lib.kda_status_string(9).startswith(b"workspace need exceeds the static scratch")


def _call_bwd(lib, d, lb=-5.0, scale=0.1, null=(), align=None, cu=None):
    names = ("q", "k", "v", "g", "beta", "A_log", "dt_bias", "d_out", "dq", "dk", "dv", "dg", "dbeta",
             "dA_log", "ddt_bias")
    ptrs = {n: ctypes.c_void_p(FAKE) for n in names}
    for n in null:
        ptrs[n] = None
    if align:
        ptrs[align] = ctypes.c_void_p(FAKE + 2)
    return lib.kda_bwd(ptrs["q"], ptrs["k"], ptrs["v"], ptrs["g"], ptrs["beta"], scale, ptrs["A_log"],
                       ptrs["dt_bias"], lb, None, cu, ptrs["d_out"], None, ptrs["dq"], ptrs["dk"], ptrs["dv"],
                       ptrs["dg"], ptrs["dbeta"], None, ptrs["dA_log"], ptrs["ddt_bias"], ctypes.byref(d), None)


def test_bwd_validation_errors(lib):
    # the backward checks its arguments like the forward, before any device work
    assert _call_bwd(lib, _desc(K=64)) == 3
    assert _call_bwd(lib, _desc(B=0)) == 2
    assert _call_bwd(lib, _desc(B=2, num_seqs=2), cu=ctypes.c_void_p(FAKE)) == 2
    assert _call_bwd(lib, _desc(chain_segments=2), cu=ctypes.c_void_p(FAKE)) == 3   # packed: never split
    assert _call_bwd(lib, _desc(chain_segments=-1)) == 4
    assert _call_bwd(lib, _desc(launch_piece=-1)) == 4
    assert _call_bwd(lib, _desc(), lb=-6.0) == 4
    assert _call_bwd(lib, _desc(), scale=float("nan")) == 4
    for n in ("q", "k", "v", "g", "beta", "d_out", "dq", "dk", "dv", "dg", "dbeta", "A_log", "dt_bias",
              "dA_log", "ddt_bias"):
        assert _call_bwd(lib, _desc(), null=(n,)) == 1, n
    for n in ("q", "d_out", "dq", "dk", "dv", "dg", "dt_bias"):
        assert _call_bwd(lib, _desc(), align=n) == 6, n
    d = _desc(workspace=ctypes.c_void_p(0x100000), workspace_bytes=1024)
    assert _call_bwd(lib, d) == 7
    d = _desc(forward_workspace=ctypes.c_void_p(0x100010))  # not 256-aligned
    assert _call_bwd(lib, d) == 6
    assert _call_bwd(lib, _desc(save_states=2)) == 4
    d = _desc(initial_state_dtype=9)
    assert lib.kda_bwd(*([ctypes.c_void_p(FAKE)] * 5), 0.1, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), -5.0,
                       ctypes.c_void_p(FAKE), None, ctypes.c_void_p(FAKE), None,
                       *([ctypes.c_void_p(FAKE)] * 5), None, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                       ctypes.byref(d), None) == 5


def test_bwd_workspace_size(lib):
    # the forward's 72.5 KiB per (chunk, head) plus 2 x 64 KiB of states, 32 KiB of dUt,
    # 32 KiB of cumulative log-decay, 2 x 16 KiB of the Gram and its inverse, 768 B of row scalars,
    # 516 B of parameter partials and 57856 B of the reverse chain's fp16 operands (the recomputed
    # forward produces the states only, no output; the normalised rows are recomputed, not stored)
    per = (kda.bwd_workspace_size(4, 64 * 100, 8) - kda.bwd_workspace_size(4, 64 * 50, 8)) / (4 * 50 * 8)
    expect = 72.5 * 1024 + 2 * 65536 + 32768 + 32768 + 2 * 16384 + 3 * 256 + 516 + 57856
    assert abs(per - expect) < 1024
    assert kda.bwd_workspace_size(1, 0, 4) > 0 or kda.bwd_workspace_size(1, 0, 4) == 0
    assert kda.bwd_workspace_size(2, 64, 2, num_seqs=3) == 0
    # split chains: the forward's segment table and three fp32 maps per (segment, head) on top
    # (the reverse chains reuse them)
    # (B = 2: the packed layout, which B = 1 also covers, plays no part)
    unsplit = kda.bwd_workspace_size(2, 64 * 64, 2, chain_segments=1)
    split = kda.bwd_workspace_size(2, 64 * 64, 2, chain_segments=4)
    assert split - unsplit == kda.workspace_size(2, 64 * 64, 2, chain_segments=4) - \
        kda.workspace_size(2, 64 * 64, 2, chain_segments=1)
    assert split - unsplit >= 3 * 2 * 4 * 2 * 65536
    assert kda.bwd_workspace_size(2, 64 * 64, 2) == kda.bwd_workspace_size(
        2, 64 * 64, 2, chain_segments=kda.chain_segments_for(2, 64 * 64, 2))
    d = _desc(chain_segments=-1)
    assert lib.kda_bwd_workspace_size(ctypes.byref(d)) == 0
