"""The C-ABI library loads, exports every entry point include/gsa.h declares,
and rejects bad arguments on the host before anything is enqueued (no GPU
needed: every call here fails validation first)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gsa.h")


@pytest.fixture(scope="module")
def gsa():
    import slot_memory_sequence_amd as m
    return m


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(gsa_\w+|gla_\w+)\s*\(", text)
    return sorted(set(names))


def test_header_symbols_exported(gsa):
    names = _declared()
    assert {"gsa_fwd", "gla_fwd", "gsa_decode_step", "gsa_abi_version"} <= set(names)
    for n in names:
        assert hasattr(gsa.lib, n), "missing export: " + n
    assert gsa.lib.gsa_abi_version() == 5


def test_status_strings(gsa):
    for s in range(0, 9):
        assert gsa.status_string(s) and gsa.status_string(s) != "unknown status"
    assert gsa.status_string(99) == "unknown status"


def test_supported_sets(gsa):
    assert gsa.gsa_fwd_supported(128, 128, 64, 64, 1)
    assert gsa.gsa_fwd_supported(64, 64, 32, 64, 0)
    assert not gsa.gsa_fwd_supported(128, 128, 64, 32, 1)   # only C = 64 compiled
    assert not gsa.gsa_fwd_supported(128, 64, 64, 64, 1)
    assert not gsa.gsa_fwd_supported(128, 128, 64, 64, 7)
    assert gsa.gla_fwd_supported(128, 128, 64, 1)
    assert gsa.gsa_decode_supported(128, 128, 64, 1)
    assert not gsa.gsa_decode_supported(96, 128, 64, 1)
    # 128 slots: bf16 forward (two slot groups) and decode; not float32 at d 128
    assert gsa.gsa_fwd_supported(128, 128, 128, 64, 1) and gsa.gsa_fwd_supported(64, 64, 128, 64, 1)
    assert not gsa.gsa_fwd_supported(128, 128, 128, 64, 0)
    assert gsa.gsa_decode_supported(128, 128, 128, 1) and gsa.gsa_decode_supported(128, 128, 128, 0)


def test_workspace_query(gsa):
    # one segment per unit needs no workspace
    assert gsa.gsa_fwd_workspace_bytes(1, 1, 64, 128, 128, 64, 64, 1, 0) == 0
    nb = gsa.gsa_fwd_workspace_bytes(8, 4, 2048, 128, 128, 64, 64, 1, 4)
    P = 2048 // 64 // 4
    state = 32 * P * 64 * 256 * 4
    assert nb == ((state + 255) // 256) * 256 + 32 * P * 64 * 4
    assert gsa.gsa_fwd_workspace_bytes(-1, 4, 16, 128, 128, 64, 64, 1, 0) == (1 << 64) - 1
    # m = 128 in bf16: 64 slot-group units (default split: 4 segments of 8
    # chunks each), then the groups' output rows [B*H*T][2][dv] bf16 and
    # log-sum-exps [B*H*T][2] fp32, each 256-byte aligned
    a256 = lambda x: (x + 255) // 256 * 256
    rows, P2 = 32 * 2048, 4
    maps = a256(64 * P2 * 64 * 256 * 4) + 64 * P2 * 64 * 4
    assert gsa.gsa_fwd_workspace_bytes(8, 4, 2048, 128, 128, 128, 64, 1, 0) == \
        a256(a256(maps) + rows * 2 * 128 * 2) + rows * 2 * 4
    # one chunk: no segment maps, the group rows only
    assert gsa.gsa_fwd_workspace_bytes(1, 1, 64, 128, 128, 128, 64, 1, 0) == a256(64 * 2 * 128 * 2) + 64 * 2 * 4
    assert gsa.gla_fwd_workspace_bytes(8, 16, 4096, 128, 128, 64, 1, 0) > 0
    # bf16 GLA: 64 units, 2 output segments, each split into 4 state-map
    # sub-segments -> max(P, (P-1)*4) = 4 slots per unit; fp32 keeps P = 2
    a256 = lambda x: (x + 255) // 256 * 256
    assert gsa.gla_fwd_workspace_bytes(8, 8, 640, 64, 64, 64, 1, 5) == \
        a256(64 * 4 * 64 * 64 * 4) + 64 * 4 * 64 * 4
    assert gsa.gla_fwd_workspace_bytes(8, 8, 640, 64, 64, 64, 0, 5) == \
        a256(64 * 2 * 64 * 64 * 4) + 64 * 2 * 64 * 4


FAKE = 0x10000  # never dereferenced: every call below fails validation


def _gsa_call(gsa, **over):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, g=FAKE + 0x300000, k0=None, v0=None,
             o=FAKE + 0x400000, kf=None, vf=None, B=1, H=1, T=64, dk=128, dv=128, m=64, C=64,
             tau=8.0, dtype=1, ws=None, wsb=0, cps=0)
    a.update(over)
    P = ctypes.c_void_p
    return gsa.lib.gsa_fwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["k0"]), P(a["v0"]),
                           P(a["o"]), P(a["kf"]), P(a["vf"]), a["B"], a["H"], a["T"], a["dk"],
                           a["dv"], a["m"], a["C"], a["tau"], a["dtype"], P(a["ws"]), a["wsb"],
                           a["cps"], None)


def test_gsa_fwd_validation(gsa):
    assert _gsa_call(gsa, B=-1) == 2
    assert _gsa_call(gsa, tau=0.0) == 2
    assert _gsa_call(gsa, tau=float("nan")) == 2
    assert _gsa_call(gsa, dtype=3) == 2
    assert _gsa_call(gsa, C=32) == 4
    assert _gsa_call(gsa, m=48) == 4
    assert _gsa_call(gsa, dk=64) == 4
    assert _gsa_call(gsa, q=None) == 1
    assert _gsa_call(gsa, o=None) == 1
    assert _gsa_call(gsa, g=FAKE + 0x300008) == 3
    assert _gsa_call(gsa, o=FAKE + 0x20) == 7            # output overlaps q
    assert _gsa_call(gsa, kf=FAKE + 0x500000, vf=FAKE + 0x500000) == 7
    # long sequence on one unit needs a workspace
    assert _gsa_call(gsa, T=4096, cps=1) == 5
    assert _gsa_call(gsa, T=4096, cps=1, ws=FAKE + 0x10000000, wsb=16) == 5
    assert _gsa_call(gsa, B=70000) == 4
    # 128 slots run as two groups of 64, each group a unit of the grid: at most
    # 32767 (batch, head) pairs (the next step at the limit is the workspace check)
    far = dict(k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30), o=FAKE + (4 << 30))
    assert _gsa_call(gsa, B=32768, m=128, **far) == 4
    assert _gsa_call(gsa, B=32767, m=128, **far) == 5


def test_gla_and_decode_validation(gsa):
    P = ctypes.c_void_p
    f = gsa.lib.gla_fwd
    base = [P(FAKE), P(FAKE + 0x100000), P(FAKE + 0x200000), P(FAKE + 0x300000), P(None),
            P(FAKE + 0x400000), P(None)]
    assert f(*base, 1, 1, 64, 128, 128, 64, 0.0, 1, None, 0, 0, None) == 2
    assert f(*base, 1, 1, 64, 128, 96, 64, 16.0, 1, None, 0, 0, None) == 4
    bad = list(base)
    bad[5] = P(FAKE + 0x100010)   # o overlaps k
    assert f(*bad, 1, 1, 64, 128, 128, 64, 16.0, 1, None, 0, 0, None) == 7
    d = gsa.lib.gsa_decode_step
    args = [P(FAKE), P(FAKE + 0x1000), P(FAKE + 0x2000), P(FAKE + 0x3000), P(FAKE + 0x100000),
            P(FAKE + 0x200000), P(FAKE + 0x4000)]
    assert d(*args, 1, 1, 128, 128, 64, -1.0, 1, None) == 2
    args2 = list(args)
    args2[5] = P(FAKE + 0x100100)  # v_state overlaps k_state
    assert d(*args2, 1, 1, 128, 128, 64, 8.0, 1, None) == 7
    args3 = list(args)
    args3[4] = None
    assert d(*args3, 1, 1, 128, 128, 64, 8.0, 1, None) == 1


def test_nonlinearity_validation(gsa):
    """The _ex entry points reject a code outside gsa_slot_nonlinearity with
    GSA_ERR_SHAPE before looking at anything else, and take every listed code
    as far as the (failing) pointer checks."""
    P = ctypes.c_void_p
    f = gsa.lib.gsa_fwd_ex
    args = [P(FAKE), P(FAKE + 0x100000), P(FAKE + 0x200000), P(FAKE + 0x300000), P(None),
            P(None), P(FAKE + 0x400000), P(None), P(None), 1, 1, 64, 128, 128, 64, 64, 8.0, 1,
            None, 0, 0]
    for bad in (-1, 5, 99):
        assert f(*args, bad, None, None) == 2
    unaligned = list(args)
    unaligned[3] = P(FAKE + 0x300008)
    for code in gsa.NONLINEARITIES.values():
        assert f(*unaligned, code, None, None) == 3
    d = gsa.lib.gsa_decode_step_ex
    dargs = [P(FAKE), P(FAKE + 0x1000), P(FAKE + 0x2000), P(FAKE + 0x3000), P(FAKE + 0x100000),
             P(FAKE + 0x200000), P(FAKE + 0x4000), 1, 1, 128, 128, 64, 8.0, 1]
    assert d(*dargs, 5, None, None) == 2
    assert d(*dargs, -1, None, None) == 2
    dbad = list(dargs)
    dbad[4] = None
    for code in gsa.NONLINEARITIES.values():
        assert d(*dbad, code, None, None) == 1
    with pytest.raises(ValueError):
        gsa._nl("tanh")


def test_varlen_validation(gsa):
    """The packed variable-length forward checks its host offsets before
    anything is enqueued."""
    P = ctypes.c_void_p
    f = gsa.lib.gsa_fwd_varlen

    def call(cu, n=None, H=2, dtype=1, q=FAKE, dk=128, m=64):
        arr = (ctypes.c_int * len(cu))(*cu)
        n = len(cu) - 1 if n is None else n
        return f(P(q), P(FAKE + 0x1000000), P(FAKE + 0x2000000), P(FAKE + 0x3000000),
                 ctypes.cast(arr, P), n, H, None, None, P(FAKE + 0x4000000), None, None, dk, dk,
                 m, 64, 8.0, dtype, None, 0, 0, None, None)

    assert call([1, 5]) == 2                       # cu[0] != 0
    assert call([0, 70, 60]) == 2                  # decreasing
    assert call([0, 5], n=-1) == 2
    assert call([0] * 258, H=300) == 4             # a group of 256 x 300 units exceeds the grid
    assert f(P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, 1, 2, None, None, P(FAKE), None, None,
             128, 128, 64, 64, 8.0, 1, None, 0, 0, None, None) == 2   # no offsets
    assert call([0, 5, 9], dtype=0) == 4           # bf16 only
    assert call([0, 5, 9], m=128) == 4             # 128 slots: dense batches only
    cu = (ctypes.c_int * 3)(0, 5, 9)
    assert gsa.lib.gsa_bwd_varlen(P(FAKE), P(FAKE + 0x1000000), P(FAKE + 0x2000000), P(FAKE + 0x3000000),
                                  P(FAKE + 0x4000000), ctypes.cast(cu, P), 2, 2, None, None, None, None,
                                  P(FAKE + 0x5000000), P(FAKE + 0x6000000), P(FAKE + 0x7000000),
                                  P(FAKE + 0x8000000), None, None, 128, 128, 128, 8.0, 1, P(FAKE + 0x9000000),
                                  1 << 40, None, None) == 4
    assert call([0, 5, 9], dk=96) == 4
    assert call([0, 5, 9], q=FAKE + 8) == 3
    assert call([0, 5, 9], q=None) == 1
    ws = gsa.gsa_fwd_varlen_workspace_bytes
    # equal lengths split exactly like the dense batch
    assert ws([0, 2048, 4096, 6144, 8192], 8, 128, 128, 64) == \
        gsa.gsa_fwd_workspace_bytes(4, 8, 2048, 128, 128, 64, 64, 1, 0)
    assert ws([0, 64] + [64] * 0, 1, 128, 128, 64) == 0
    assert ws([0, 5, 3], 2, 128, 128, 64) == (1 << 64) - 1
    # more than 256 sequences: the workspace of one group of 256
    many = [64 * i for i in range(601)]
    assert ws(many, 2, 128, 128, 64, chunks_per_segment=0) == 0          # one chunk each: P = 1
    long_ = [0] + [64 * 40 * (i + 1) for i in range(600)]
    assert ws(long_, 2, 128, 128, 64, chunks_per_segment=20) == \
        gsa.gsa_fwd_varlen_workspace_bytes(long_[:257], 2, 128, 128, 64, chunks_per_segment=20)
    with pytest.raises(ValueError):
        ws([], 2, 128, 128, 64)


def test_measure_validation(gsa):
    """The calibration entry points reject bad arguments on the host."""
    P = ctypes.c_void_p
    c = gsa.lib.gsa_measure_hbm
    assert c(None, P(FAKE), 64, 0, None, None) == 1
    assert c(P(FAKE), None, 64, 1, None, None) == 1
    assert c(P(FAKE), P(FAKE + 0x10000), 64, 2, None, None) == 2
    assert c(P(FAKE), P(FAKE + 0x10000), 0, 0, None, None) == 2
    assert c(P(FAKE), P(FAKE + 0x10000), 24, 0, None, None) == 2
    assert c(P(FAKE + 4), P(FAKE + 0x10000), 64, 0, None, None) == 3
    assert c(P(FAKE), P(FAKE + 32), 64, 0, None, None) == 7
    f = gsa.lib.gsa_measure_mfma_bf16
    assert f(None, 1024, 10, None, None, None) == 1
    assert f(P(FAKE), 1024, 0, None, None, None) == 2
    assert f(P(FAKE), 1023, 10, None, None, None) == 5
    assert f(P(FAKE + 4), 1024, 10, None, None, None) == 3


def test_gla_decode_validation(gsa):
    P = ctypes.c_void_p
    d = gsa.lib.gla_decode_step
    args = [P(FAKE), P(FAKE + 0x1000), P(FAKE + 0x2000), P(FAKE + 0x3000), P(FAKE + 0x100000),
            P(FAKE + 0x4000)]
    assert d(*args, 1, 1, 128, 128, 16.0, 1, 2, None, None) == 2       # bad gate code
    assert d(*args, 1, 1, 128, 128, -1.0, 1, 0, None, None) == 2       # bad tau with logits
    assert d(*args, 1, 1, 96, 96, 16.0, 1, 0, None, None) == 4
    bad = list(args)
    bad[4] = P(FAKE + 0x1010)                                          # state overlaps k
    assert d(*bad, 1, 1, 128, 128, 16.0, 1, 0, None, None) == 7
    bad = list(args)
    bad[5] = None
    assert d(*bad, 1, 1, 128, 128, -1.0, 1, 1, None, None) == 1       # tau unused with log-decays
    assert gsa.lib.gla_decode_supported(128, 128, 1) == 1
    assert gsa.lib.gla_decode_supported(64, 128, 1) == 0


def test_package_has_no_cpu_fallback():
    """The product package never imports, loads or calls the oracle."""
    pkg = os.path.join(ROOT, "slot_memory_sequence_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                for bad in ("import oracle", "from oracle", "liboracle", "oracle_gsa", "oracle_gla"):
                    assert bad not in text, (f, bad)


def test_bwd_validation(gsa):
    """gsa_bwd: shape, support, null, alignment, aliasing and workspace checks."""
    f = gsa.lib.gsa_bwd
    P = ctypes.c_void_p
    ws = FAKE + 0x10000000
    need = gsa.gsa_bwd_workspace_bytes(1, 1, 64, 128, 128, 64, 1)  # the bf16 path's need
    assert gsa.gsa_bwd_workspace_bytes(1, 1, 64, 128, 128, 64, 1, "relu") == \
        gsa.gsa_bwd_workspace_bytes(1, 1, 64, 128, 128, 64, 0)  # ReLU: the token walks
    assert 0 < need <= gsa.gsa_bwd_workspace_bytes(1, 1, 64, 128, 128, 64)  # <= enough for either
    assert gsa.gsa_bwd_workspace_bytes(1, 1, 0, 128, 128, 64) == 0       # T = 0: nothing kept
    assert gsa.gsa_bwd_workspace_bytes(-1, 1, 64, 128, 128, 64) == 0
    # the bf16 path at the training shape (B8 H4 T2048 d128 m64): segment
    # start states and reverse maps (8 segments of 4 chunks per unit, fp32),
    # the final state per unit, and bf16 s, dz, h per token
    U, nseg = 32, 8
    a256 = lambda x: (x + 255) // 256 * 256
    big = 2 * a256(U * nseg * 64 * 256 * 4) + 2 * a256(U * nseg * 64 * 4) + a256(U * 64 * 256 * 4) + \
        3 * a256(U * 2048 * 64 * 2)
    assert gsa.gsa_bwd_workspace_bytes(8, 4, 2048, 128, 128, 64, 1) == big < 64 * 10 ** 6
    assert gsa.gsa_bwd_supported(128, 128, 64, 1) and gsa.gsa_bwd_supported(64, 64, 32, 0)
    assert not gsa.gsa_bwd_supported(96, 96, 64, 1) and not gsa.gsa_bwd_supported(128, 128, 48, 1)
    # 128 slots (bf16 only): two groups of 64 as 64 group units (4 segments of
    # 8 chunks), then the groups' statistics [rows][2][2], the merged
    # log-sum-exp and delta [rows], and fp32 partial dq, dk, dv [rows][2][128]
    assert gsa.gsa_bwd_supported(128, 128, 128, 1) and gsa.gsa_bwd_supported(64, 64, 128, 1)
    assert not gsa.gsa_bwd_supported(128, 128, 128, 0)
    U2, nseg2, rows = 64, 4, 32 * 2048
    own = 2 * a256(U2 * nseg2 * 64 * 256 * 4) + 2 * a256(U2 * nseg2 * 64 * 4) + a256(U2 * 64 * 256 * 4) + \
        3 * a256(U2 * 2048 * 64 * 2)
    grp = a256(rows * 16) + 2 * a256(rows * 4) + 3 * a256(rows * 2 * 128 * 4)
    assert gsa.gsa_bwd_workspace_bytes(8, 4, 2048, 128, 128, 128, 1) == a256(own) + grp

    def call(**kw):
        a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, g=FAKE + 0x300000,
                 do=FAKE + 0x400000, k0=None, v0=None, dkf=None, dvf=None, dq=FAKE + 0x500000,
                 dk=FAKE + 0x600000, dv=FAKE + 0x700000, dg=FAKE + 0x800000, dk0=None, dv0=None,
                 B=1, H=1, T=64, d_k=128, d_v=128, m=64, tau=8.0, dtype=1, ws=ws, wsb=need)
        a.update(kw)
        return f(P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["do"]), P(a["k0"]), P(a["v0"]),
                 P(a["dkf"]), P(a["dvf"]), P(a["dq"]), P(a["dk"]), P(a["dv"]), P(a["dg"]),
                 P(a["dk0"]), P(a["dv0"]), a["B"], a["H"], a["T"], a["d_k"], a["d_v"], a["m"],
                 a["tau"], a["dtype"], P(a["ws"]), a["wsb"], None, None)

    assert call(tau=0.0) == 2 and call(tau=float("inf")) == 2 and call(T=-1) == 2
    assert call(dtype=5) == 2
    assert call(d_k=96, d_v=96) == 4
    assert call(m=128, dtype=0) == 4                    # 128 slots: bf16 only
    assert call(B=65536) == 4
    far = {n: FAKE + (i << 30) for i, n in enumerate(("k", "v", "g", "do", "dq", "dk", "dv", "dg"), 1)}
    assert call(B=32768, m=128, ws=FAKE + (9 << 30), **far) == 4   # two slot groups per (batch, head)
    assert call(B=32767, m=128, ws=FAKE + (9 << 30), **far) == 5   # within the grid: the workspace check
    assert call(T=65535 * 64 + 1) == 4                  # more chunks than the grid takes
    assert call(B=0) == 0                               # nothing to do
    assert call(q=None) == 1 and call(do=None) == 1 and call(dg=None) == 1
    assert call(dq=FAKE + 0x500008) == 3
    assert call(dq=FAKE + 0x20) == 7                    # d_q overlaps q
    assert call(dk=FAKE + 0x500000) == 7                # d_k overlaps d_q
    assert call(dk0=FAKE + 0x10) == 7                   # d_k0 overlaps q
    assert call(ws=FAKE + 0x400000) == 7                # workspace overlaps d_o
    assert call(wsb=need - 16) == 5 and call(ws=None) == 5


def test_bwd_ex_nonlinearity_validation(gsa):
    f = gsa.lib.gsa_bwd_ex
    P = ctypes.c_void_p
    need = gsa.gsa_bwd_workspace_bytes(1, 1, 64, 128, 128, 64)
    args = [P(FAKE), P(FAKE + 0x100000), P(FAKE + 0x200000), P(FAKE + 0x300000), P(FAKE + 0x400000),
            None, None, None, None, P(FAKE + 0x500000), P(FAKE + 0x600000), P(FAKE + 0x700000),
            P(FAKE + 0x800000), None, None, 1, 1, 64, 128, 128, 64, 8.0, 1,
            P(FAKE + 0x10000000), need]
    assert f(*args, 5, None, None) == 2 and f(*args, -1, None, None) == 2
    bad = list(args)
    bad[9] = P(FAKE + 0x10)             # d_q overlaps q: the codes 0..4 pass the shape check
    for code in range(5):
        assert f(*bad, code, None, None) == 7


def test_bwd_varlen_validation(gsa):
    """Every call here fails validation on the host (nothing is launched)."""
    f = gsa.lib.gsa_bwd_varlen
    P = ctypes.c_void_p

    def call(cu, n=None, H=2, dtype=1, dq=FAKE + 0x5000000, dk=128, ws=FAKE + 0x40000000, wsb=None):
        arr = (ctypes.c_int * len(cu))(*cu)
        n = len(cu) - 1 if n is None else n
        if wsb is None:
            wsb = gsa.lib.gsa_bwd_varlen_workspace_bytes(ctypes.cast(arr, P), n, H, dk, dk, 64)
        return f(P(FAKE), P(FAKE + 0x1000000), P(FAKE + 0x2000000), P(FAKE + 0x3000000),
                 P(FAKE + 0x4000000), ctypes.cast(arr, P), n, H, None, None, None, None,
                 P(dq), P(FAKE + 0x6000000), P(FAKE + 0x7000000), P(FAKE + 0x8000000),
                 None, None, dk, dk, 64, 8.0, dtype, P(ws), wsb, None, None)

    assert call([0, 5, 3]) == 2                       # decreasing offsets
    assert call([1, 5]) == 2                          # cu[0] != 0
    assert call([0, 5], dtype=9) == 2
    assert call([0, 5], dk=96) == 4
    assert call([0, 70, 200], dq=FAKE + 0x10) == 7    # d_q overlaps q
    assert call([0, 70, 200], wsb=16) == 5
    arr = (ctypes.c_int * 3)(0, 70, 200)
    assert gsa.lib.gsa_bwd_varlen_workspace_bytes(ctypes.cast(arr, P), 2, 2, 128, 128, 64) > 0
    assert gsa.lib.gsa_bwd_varlen_workspace_bytes(None, 2, 2, 128, 128, 64) == 0


def test_noalloc_rejects_before_touching_the_device(gsa):
    """gsa_fwd_noalloc refuses problems whose scratch exceeds its fixed array
    (GSA_ERR_SCRATCH_LIMIT) and invalid sizes (GSA_ERR_SHAPE) on the host,
    before it looks up a device or enqueues anything -- so these calls run
    without a GPU."""
    P = ctypes.c_void_p
    f = gsa.lib.gsa_fwd_noalloc
    cap = gsa.lib.gsa_fwd_noalloc_scratch_bytes()
    assert cap == 32 << 20
    args = [P(FAKE), P(FAKE + 0x100000), P(FAKE + 0x200000), P(FAKE + 0x300000), P(None), P(None),
            P(FAKE + 0x400000), P(None), P(None)]
    # 64 units x 16384 tokens, one chunk per segment: 64 * 256 maps of 64 KB
    B, H, T = 16, 4, 16384
    need = gsa.gsa_fwd_workspace_bytes(B, H, T, 128, 128, 64, 64, 1, 1)
    assert need > cap
    assert f(*args, B, H, T, 128, 128, 64, 64, 8.0, 1, 1, 0, None, None) == 8
    assert gsa.status_string(8) != "unknown status"
    assert f(*args, -1, H, T, 128, 128, 64, 64, 8.0, 1, 0, 0, None, None) == 2


def test_train_pair_validation(gsa):
    """gsa_fwd_train / gsa_bwd_train: sizes, support and reject paths (every
    call below fails validation before anything is enqueued)."""
    P = ctypes.c_void_p
    a256 = lambda x: (x + 255) // 256 * 256
    # the backward's split at B8 H4 T2048: 8 segments of 4 chunks per unit
    assert gsa.gsa_train_states_bytes(8, 4, 2048, 128, 128, 64) == 32 * 8 * 64 * 256 * 4
    # 128 slots: 64 group units, 4 segments of 8 chunks, the same bytes per segment and slot
    assert gsa.gsa_train_states_bytes(8, 4, 2048, 128, 128, 128) == 64 * 4 * 64 * 256 * 4
    assert gsa.gsa_train_states_bytes(8, 4, 2048, 128, 128, 64, 0) == 0      # float32: not compiled
    assert gsa.gsa_train_states_bytes(8, 4, 0, 128, 128, 64) == 0
    assert gsa.gsa_train_states_bytes(-1, 4, 64, 128, 128, 64) == (1 << 64) - 1
    # workspace of the training forward: the decay products only (m = 64)
    assert gsa.lib.gsa_fwd_train_workspace_bytes(8, 4, 2048, 128, 128, 64, 1) == 32 * 8 * 64 * 4
    assert gsa.lib.gsa_fwd_train_workspace_bytes(8, 4, 2048, 128, 128, 128, 1) == \
        a256(a256(64 * 4 * 64 * 4) + 32 * 2048 * 2 * 128 * 2) + 32 * 2048 * 2 * 4

    need = gsa.gsa_train_states_bytes(1, 1, 256, 128, 128, 64)
    wsf = gsa.lib.gsa_fwd_train_workspace_bytes(1, 1, 256, 128, 128, 64, 1)

    def fwd(**kw):
        a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, g=FAKE + 0x300000, o=FAKE + 0x400000,
                 ws=FAKE + 0x500000, wsb=wsf, st=FAKE + 0x600000, stb=need, nl=0, dtype=1, m=64)
        a.update(kw)
        return gsa.lib.gsa_fwd_train(P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), None, None, P(a["o"]), None,
                                     None, 1, 1, 256, 128, 128, a["m"], 8.0, a["dtype"], P(a["ws"]), a["wsb"],
                                     P(a["st"]), a["stb"], a["nl"], None, None)

    assert fwd(nl=3) == 4                      # ReLU: the backward keeps its token walks
    assert fwd(dtype=0) == 4                   # float32
    assert fwd(st=None) == 1                   # states buffer missing
    assert fwd(stb=need - 4) == 5              # states buffer too small
    assert fwd(st=FAKE + 0x400000) == 7        # states over the output
    assert fwd(st=FAKE + 0x600004) == 3        # misaligned states
    assert fwd(wsb=wsf - 4) == 5

    def bwd(**kw):
        a = dict(st=FAKE + 0x900000, stb=need, nl=0, dq=FAKE + 0x500000, ws=FAKE + 0xa00000)
        a.update(kw)
        return gsa.lib.gsa_bwd_train(P(FAKE), P(FAKE + 0x100000), P(FAKE + 0x200000), P(FAKE + 0x300000),
                                     P(FAKE + 0x400000), None, None, None, None, P(a["dq"]),
                                     P(FAKE + 0x600000), P(FAKE + 0x700000), P(FAKE + 0x800000), None, None,
                                     1, 1, 256, 128, 128, 64, 8.0, 1, P(a["ws"]), 1 << 30, P(a["st"]),
                                     a["stb"], a["nl"], None, None)

    assert bwd(nl=3) == 4
    assert bwd(st=None) == 1
    assert bwd(stb=need - 4) == 5
    assert bwd(dq=FAKE + 0x900000) == 7        # an output over the states
