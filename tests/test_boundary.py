"""CPU tests of the C-ABI boundary: the library loads, exports every function
include/linattn.h declares, sizes workspaces, and rejects bad arguments with
the documented status before any device work (these calls never reach the
GPU, so they run without one)."""
import ctypes
import os
import subprocess

import pytest

import linear_attention_transformers_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(la.LIB_PATH):
        from linear_attention_transformers_amd import build
        build.build()
    return la.load_library()


def test_exports_every_declared_symbol(lib):
    names = la.header_functions()
    assert {"la_fwd", "la_bwd", "la_workspace_bytes", "la_status_string"} <= set(names)
    nm = subprocess.run(["nm", "-D", "--defined-only", la.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = {line.split()[-1] for line in nm.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    for st in range(4):
        assert lib.la_status_string(st).startswith(b"LA_")
    assert lib.la_status_string(99) == b"unknown status"


def _fwd(lib, **over):
    p = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: validation fails first
    kw = dict(q=p, k=p, v=p, out=p, B=1, H=2, H_kv=2, N=16, D=32, dtype=la.LA_BF16, causal=1,
              phi=0, eps=1e-6, cw=None, sw=None, ws=p, ws_bytes=1 << 40, stream=None)
    kw.update(over)
    return lib.la_fwd(kw["q"], kw["k"], kw["v"], kw["out"], kw["B"], kw["H"], kw["H_kv"],
                      kw["N"], kw["D"], kw["dtype"], kw["causal"], kw["phi"], kw["eps"], kw["cw"],
                      kw["sw"], kw["ws"], kw["ws_bytes"], kw["stream"])


def _bwd(lib, **over):
    p = ctypes.c_void_p(1 << 20)
    kw = dict(q=p, k=p, v=p, g=p, dq=p, dk=p, dv=p, B=1, H=2, H_kv=2, N=16, D=32,
              dtype=la.LA_F32, causal=0, phi=1, eps=1e-6, cw=None, sw=None, ws=p,
              ws_bytes=1 << 40, stream=None)
    kw.update(over)
    return lib.la_bwd(kw["q"], kw["k"], kw["v"], kw["g"], kw["dq"], kw["dk"], kw["dv"], kw["B"],
                      kw["H"], kw["H_kv"], kw["N"], kw["D"], kw["dtype"], kw["causal"], kw["phi"],
                      kw["eps"], kw["cw"], kw["sw"], kw["ws"], kw["ws_bytes"], kw["stream"])


FP = ctypes.cast(ctypes.c_void_p(1 << 20), ctypes.POINTER(ctypes.c_float))
BAD = [
    ("null q", dict(q=None), la.LA_ERR_INVALID),
    ("zero B", dict(B=0), la.LA_ERR_INVALID),
    ("negative N", dict(N=-3), la.LA_ERR_INVALID),
    ("H not multiple of H_kv", dict(H=3, H_kv=2), la.LA_ERR_INVALID),
    ("zero H_kv", dict(H_kv=0), la.LA_ERR_INVALID),
    ("unknown dtype", dict(dtype=7), la.LA_ERR_INVALID),
    ("unknown phi", dict(phi=3), la.LA_ERR_INVALID),
    ("negative eps", dict(eps=-1.0), la.LA_ERR_INVALID),
    ("nan eps", dict(eps=float("nan")), la.LA_ERR_INVALID),
    ("cos without sin", dict(cw=FP), la.LA_ERR_INVALID),
    ("sin without cos", dict(sw=FP), la.LA_ERR_INVALID),
    ("misaligned q", dict(q=ctypes.c_void_p((1 << 20) + 2)), la.LA_ERR_INVALID),
    ("workspace too small", dict(ws_bytes=8), la.LA_ERR_INVALID),
    ("null workspace", dict(ws=None), la.LA_ERR_INVALID),
    ("D = 48", dict(D=48), la.LA_ERR_UNSUPPORTED),
    ("D = 256", dict(D=256), la.LA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("name,over,status", BAD, ids=[b[0] for b in BAD])
def test_forward_rejects(lib, name, over, status):
    assert _fwd(lib, **over) == status
    assert lib.la_last_error() != b""


@pytest.mark.parametrize("name,over,status", BAD, ids=[b[0] for b in BAD])
def test_backward_rejects(lib, name, over, status):
    over = {("g" if k == "out" else k): v for k, v in over.items()}
    assert _bwd(lib, **over) == status


def test_backward_rejects_null_gradient(lib):
    assert _bwd(lib, g=None) == la.LA_ERR_INVALID
    assert _bwd(lib, dk=None) == la.LA_ERR_INVALID


def test_workspace_sizes(lib):
    for op in (la.LA_OP_FWD, la.LA_OP_BWD):
        for causal in (0, 1):
            for cos in (0, 1):
                n = lib.la_workspace_bytes(op, 2, 4, 2, 1000, 64, la.LA_BF16, causal, cos)
                assert n > 0 and n % 256 == 0
    # backward needs more than forward; cos/sin doubles the state
    f = lib.la_workspace_bytes(la.LA_OP_FWD, 1, 4, 4, 4096, 128, 1, 1, 0)
    b = lib.la_workspace_bytes(la.LA_OP_BWD, 1, 4, 4, 4096, 128, 1, 1, 0)
    c = lib.la_workspace_bytes(la.LA_OP_FWD, 1, 4, 4, 4096, 128, 1, 1, 1)
    assert b > f and c > f
    # rejected arguments size to zero
    assert lib.la_workspace_bytes(la.LA_OP_FWD, 1, 3, 2, 16, 32, 1, 1, 0) == 0
    assert lib.la_workspace_bytes(la.LA_OP_FWD, 1, 2, 2, 16, 48, 1, 1, 0) == 0
    assert lib.la_workspace_bytes(5, 1, 2, 2, 16, 32, 1, 1, 0) == 0
    # explicit segment length: more segments, more workspace
    a = lib.la_workspace_bytes_ex(la.LA_OP_FWD, 1, 2, 2, 4096, 64, 1, 1, 0, 64)
    z = lib.la_workspace_bytes_ex(la.LA_OP_FWD, 1, 2, 2, 4096, 64, 1, 1, 0, 4096)
    assert a > z > 0


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 2, 8, 32)
    with pytest.raises(ValueError):
        la.fwd(q, q, q)
    with pytest.raises(ValueError):
        la.bwd(q, q, q, q)
    assert not la.is_supported(q, q, q)


def test_product_never_imports_oracle():
    """The library and its binding share no code with the CPU oracle."""
    pkg = os.path.join(ROOT, "linear_attention_transformers_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read().lower()
                assert "oracle" not in text, f


# ---------------------------------------------------------------------------
# la_gqa_expand / la_gqa_reduce (include/la_gqa.h): every rejection happens in
# validation, before any device work
# ---------------------------------------------------------------------------
def _gqa(lib, fn, **over):
    p = ctypes.c_void_p(1 << 20)
    kw = dict(a=p, b=p, ao=ctypes.c_void_p(1 << 21), bo=ctypes.c_void_p(1 << 22), B=1, H_kv=2, H=8,
              N=16, D=64, dtype=la.LA_BF16, stream=None)
    kw.update(over)
    f = lib.la_gqa_expand if fn == "expand" else lib.la_gqa_reduce
    return f(kw["a"], kw["b"], kw["ao"], kw["bo"], kw["B"], kw["H_kv"], kw["H"], kw["N"], kw["D"],
             kw["dtype"], kw["stream"])


@pytest.mark.parametrize("fn", ["expand", "reduce"])
@pytest.mark.parametrize("over,status", [
    (dict(B=0), 1), (dict(H_kv=0), 1), (dict(H=0), 1), (dict(N=0), 1), (dict(D=-1), 1),
    (dict(H=7), 1),                      # not a multiple of H_kv
    (dict(dtype=5), 1),
    (dict(a=None), 1), (dict(ao=None), 1),
    (dict(b=None), 1), (dict(bo=None), 1),   # exactly one of the v pair
    (dict(a=ctypes.c_void_p((1 << 20) + 1)), 1),                     # bf16 needs 2-byte alignment
    (dict(dtype=la.LA_F32, bo=ctypes.c_void_p((1 << 22) + 2)), 1),   # f32 needs 4-byte alignment
    (dict(B=65536, H_kv=1, H=1), 2),     # one grid row per KV slab
])
def test_gqa_rejects(lib, fn, over, status):
    assert _gqa(lib, fn, **over) == status
    assert lib.la_last_error()


def test_gqa_python_rejects_bad_heads():
    torch = pytest.importorskip("torch")
    from linear_attention_transformers_amd import gqa
    k = torch.zeros(1, 2, 4, 8)
    with pytest.raises(ValueError):
        gqa.fwd(k, k, 2, 5)
    # equal head counts: the inputs come back untouched, as on the gqa page
    a, b = gqa.fwd(k, k, 2, 2)
    assert a is k and b is k
    assert not gqa.is_supported(k, k, 2, 4)   # CPU tensors


# ---------------------------------------------------------------------------
# la_lowrank_* (include/la_lowrank.h): validation before any device work
# ---------------------------------------------------------------------------
def test_lowrank_workspace_bytes(lib):
    f = lib.la_lowrank_workspace_bytes
    assert f(la.LA_OP_FWD, 37, 64, 16, 32, la.LA_BF16) >= 37 * 16 * 2
    assert f(la.LA_OP_BWD, 37, 64, 16, 32, la.LA_BF16) > f(la.LA_OP_FWD, 37, 64, 16, 32, la.LA_BF16)
    for bad in [(la.LA_OP_FWD, 0, 64, 16, 32, la.LA_BF16), (la.LA_OP_FWD, 8, 60, 16, 32, la.LA_BF16),
                (la.LA_OP_FWD, 8, 64, 4, 32, la.LA_BF16), (la.LA_OP_FWD, 8, 64, 16, 32, la.LA_F32),
                (7, 8, 64, 16, 32, la.LA_BF16)]:
        assert f(*bad) == 0


def _lr(lib, fn, **over):
    p = ctypes.c_void_p(1 << 20)
    kw = dict(x=p, U=p, V=p, b=None, y=ctypes.c_void_p(1 << 21), g=p, gx=ctypes.c_void_p(1 << 22),
              gU=ctypes.c_void_p(1 << 23), gV=ctypes.c_void_p(1 << 24), gb=None, M=37, n_in=64, rank=16,
              n_out=32, dtype=la.LA_BF16, ws=ctypes.c_void_p(1 << 25), ws_bytes=1 << 40, stream=None)
    kw.update(over)
    if fn == "fwd":
        return lib.la_lowrank_fwd(kw["x"], kw["U"], kw["V"], kw["b"], kw["y"], kw["M"], kw["n_in"], kw["rank"],
                                  kw["n_out"], kw["dtype"], kw["ws"], kw["ws_bytes"], kw["stream"])
    return lib.la_lowrank_bwd(kw["x"], kw["U"], kw["V"], kw["g"], kw["gx"], kw["gU"], kw["gV"], kw["gb"],
                              kw["M"], kw["n_in"], kw["rank"], kw["n_out"], kw["dtype"], kw["ws"],
                              kw["ws_bytes"], kw["stream"])


@pytest.mark.parametrize("fn", ["fwd", "bwd"])
@pytest.mark.parametrize("over,status", [
    (dict(M=0), 1), (dict(n_in=60), 1), (dict(rank=0), 1), (dict(n_out=12), 1),
    (dict(dtype=la.LA_F32), 2), (dict(dtype=9), 1),
    (dict(x=None), 1), (dict(U=None), 1), (dict(V=None), 1),
    (dict(x=ctypes.c_void_p((1 << 20) + 8)), 1),        # not 16-byte aligned
    (dict(ws=None), 1), (dict(ws=ctypes.c_void_p((1 << 25) + 16)), 1), (dict(ws_bytes=16), 1),
])
def test_lowrank_rejects(lib, fn, over, status):
    assert _lr(lib, fn, **over) == status
    assert lib.la_last_error()


def test_lowrank_rejects_missing_outputs(lib):
    assert _lr(lib, "fwd", y=None) == 1
    for k in ("g", "gx", "gU", "gV"):
        assert _lr(lib, "bwd", **{k: None}) == 1
    assert _lr(lib, "bwd", gb=ctypes.c_void_p((1 << 26) + 2)) == 1   # misaligned optional output
