"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol the header declares, validates its arguments before touching the device,
and sizes its partial buffers as the memory table of the method prescribes."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from triangular_attention_amd import _lib
    return _lib.load()


def _header_symbols():
    txt = open(os.path.join(ROOT, "include", "tri_attn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(tri_attn_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol(lib):
    from triangular_attention_amd import _lib
    syms = _header_symbols()
    assert set(syms) == set(_lib.EXPORTS)
    for s in syms:
        assert hasattr(lib, s), s
    assert lib.tri_attn_version().decode().count(".") == 2


def test_status_strings(lib):
    for code in range(7):
        assert lib.tri_attn_status_string(code)
    assert lib.tri_attn_status_string(99) == b"unknown status"


def _dims(**kw):
    from triangular_attention_amd import _lib
    base = dict(B=1, N_o=8, H=2, N=8, D=32, scale=0.125)
    base.update(kw)
    return _lib.Dims(base["B"], base["N_o"], base["H"], base["N"], base["D"], base["scale"])


P = ctypes.c_void_p(0x100000)       # aligned, never dereferenced on the host
MIS = ctypes.c_void_p(0x100008)     # 8-byte aligned only


def _fwd(lib, d, **ptrs):
    a = dict(q=P, k=P, v=P, bias=P, mask=None, o=P, o_res=None, lse=P)
    a.update(ptrs)
    return lib.tri_attn_fwd(None if d is None else ctypes.byref(d), a["q"], a["k"], a["v"], a["bias"],
                            a["mask"], a["o"], a["o_res"], a["lse"], None)


def test_validation_errors_before_launch(lib):
    assert _fwd(lib, None) == 1
    assert _fwd(lib, _dims(D=128)) == 3
    assert _fwd(lib, _dims(D=8)) == 3
    assert _fwd(lib, _dims(N=0)) == 2
    assert _fwd(lib, _dims(N=32768, N_o=1)) == 2     # 4*N*N must fit in 32 bits
    assert _fwd(lib, _dims(B=0)) == 2
    assert _fwd(lib, _dims(scale=float("nan"))) == 2
    assert _fwd(lib, _dims(scale=float("inf"))) == 2
    # -lse / scale must stay finite in FP32: zero and tiny scales are rejected, 2^-64 is accepted
    assert _fwd(lib, _dims(scale=0.0)) == 2
    assert _fwd(lib, _dims(scale=-0.0)) == 2
    assert _fwd(lib, _dims(scale=1e-30)) == 2
    assert lib.tri_attn_workspace(ctypes.byref(_dims(scale=2.0 ** -64)), None, None, None, None, None, None) == 0
    assert lib.tri_attn_workspace(ctypes.byref(_dims(scale=-0.5)), None, None, None, None, None, None) == 0
    # huge dimensions are rejected before any product of them is formed (no int64 overflow)
    for big in (2 ** 62, 2 ** 40, 65536):
        assert _fwd(lib, _dims(B=big)) == 2
        assert _fwd(lib, _dims(N_o=big)) == 2
        assert _fwd(lib, _dims(H=big)) == 2
    assert _fwd(lib, _dims(N=2 ** 62)) == 2
    assert _fwd(lib, _dims(B=300, N_o=300)) == 2             # B * N_o past the grid limit
    assert _fwd(lib, _dims(B=1, N_o=4096, H=4096, N=4096)) == 2   # rows past the 32-bit index limit
    assert _fwd(lib, _dims(), q=None) == 1
    assert _fwd(lib, _dims(), lse=None) == 1
    assert _fwd(lib, _dims(), k=MIS) == 4
    assert _fwd(lib, _dims(), mask=MIS) == 4
    assert _fwd(lib, _dims(), o_res=MIS) == 4
    d = _dims()
    assert lib.tri_attn_bwd_delta(ctypes.byref(d), P, None, None, P, None) == 1
    assert lib.tri_attn_bwd_delta(ctypes.byref(d), P, MIS, P, P, None) == 4
    assert lib.tri_attn_bwd(ctypes.byref(d), P, P, P, P, None, P, P, P, P, P, P, None, None) == 1
    assert lib.tri_attn_bwd(ctypes.byref(d), P, P, P, P, None, P, P, P, P, P, MIS, P, None) == 4
    assert lib.tri_attn_bwd(ctypes.byref(_dims(D=48)), P, P, P, P, None, P, P, P, P, P, P, P, None) == 3
    assert lib.tri_attn_reduce_dq(ctypes.byref(d), None, P, None) == 1
    assert lib.tri_attn_reduce_dq(ctypes.byref(d), P, MIS, None) == 4
    assert lib.tri_attn_reduce_dbias(ctypes.byref(d), P, None, None) == 1
    assert lib.tri_attn_reduce_dbias(ctypes.byref(_dims(H=0)), P, P, None) == 2
    # the bf16-partial variant validates like the FP32 calls
    assert lib.tri_attn_bwd_bf16p(ctypes.byref(d), P, P, P, P, None, P, P, P, P, P, P, None, None) == 1
    assert lib.tri_attn_bwd_bf16p(ctypes.byref(d), P, P, P, P, None, P, P, P, P, P, MIS, P, None) == 4
    assert lib.tri_attn_bwd_bf16p(ctypes.byref(_dims(D=128)), P, P, P, P, None, P, P, P, P, P, P, P, None) == 3
    assert lib.tri_attn_reduce_dq_bf16p(ctypes.byref(d), None, P, None) == 1
    assert lib.tri_attn_reduce_dq_bf16p(ctypes.byref(d), MIS, P, None) == 4
    assert lib.tri_attn_reduce_dbias_bf16p(ctypes.byref(_dims(N=0)), P, P, None) == 2


def test_python_binding_raises(lib):
    from triangular_attention_amd import _lib
    with pytest.raises(_lib.TriAttnError):
        _lib.check("tri_attn_fwd", _fwd(lib, _dims(D=128)))


def _golden_table2():
    rows = []
    for line in open(os.path.join(ROOT, "tests", "golden", "table2_alloc_mib.txt")):
        if line.strip() and not line.startswith("#"):
            rows.append([int(x) for x in line.split()])
    return rows


def test_workspace_matches_memory_table():
    """Partial sizes follow the closed forms behind the memory table (Table 2): J_K = N / key
    tile dQ partials and L = N_o / G dbias partials.  The table uses key tile 64, G = 4 and
    BF16 partials; this library uses FP32 partials and its own key tile, so the check is
    that the table's numbers come out of the same formulas, and that our workspace equals
    those formulas at our tile sizes."""
    from triangular_attention_amd import api
    mib = float(2 ** 20)

    def w_q(N, tau_k, bytes_):       # dQ partials: (N / tau_k) Q-sized tensors
        return -(-N // tau_k) * N * 4 * N * 32 * bytes_ / mib

    def w_bias(N, G, bytes_):        # dbias partials: N_o / G bias-sized tensors
        return -(-N // G) * 4 * N * N * bytes_ / mib

    for N, WQ, Wb_all, Wb_res, WE, WdS in _golden_table2():
        assert w_q(N, 64, 2) == WQ and w_bias(N, 4, 2) == Wb_all
        assert N * 4 * N * 32 * 2 / mib == WE                     # residual E, one bf16 Q-sized tensor
        assert N * 4 * N * N * 4 / mib == WdS                     # dense dS, never stored
        assert Wb_res <= Wb_all
        d = _dims(B=1, N_o=N, H=4, N=N, D=32)
        ws = api.workspace(d)
        tk, G = ws["key_tile"], ws["outer_group"]
        assert ws["j_k"] == -(-N // tk) and ws["l"] == -(-N // G)
        assert ws["dq_partial_elems"] * 4 / mib == w_q(N, tk, 4)
        assert ws["dbias_partial_elems"] * 4 / mib == w_bias(N, G, 4)


def test_workspace_ragged():
    """Partial counts of the single-pass key-tile kernel for ragged shapes.  The outer group is
    4 slices except on the direct-load path with D = 16 (N even), where the smaller accumulators
    leave room for 6, and 2 slices for D = 64, whose accumulators are twice as large.  For
    D = 64, and D = 16 up to N = 640, the default backward is that kernel, so both queries
    agree."""
    from triangular_attention_amd import api
    for (N_o, N, D, G) in ((10, 65, 16, 4), (10, 64, 16, 6), (10, 66, 16, 6), (10, 64, 32, 4), (13, 200, 16, 6),
                           (13, 201, 32, 4), (13, 200, 64, 2), (13, 201, 64, 2)):
        d = _dims(B=2, N_o=N_o, H=3, N=N, D=D)
        ws = api.workspace(d, single_pass=True)
        jk, L = -(-N // ws["key_tile"]), -(-N_o // G)
        assert ws["outer_group"] == G and ws["key_tile"] == 128
        assert ws["j_k"] == jk and ws["l"] == L
        assert ws["dq_partial_elems"] == jk * 2 * N_o * 3 * N * D
        assert ws["dbias_partial_elems"] == L * 2 * 3 * N * N
        if D != 32:     # N <= 640: D = 16 runs the single-pass kernel too
            assert api.workspace(d) == ws


@pytest.mark.parametrize("B,N_o,H,N,kr,J", [(1, 768, 4, 768, 384, 2), (1, 384, 4, 384, 384, 1),
                                            (1, 1024, 4, 1024, 384, 3), (2, 5, 2, 100, 128, 1),
                                            (1, 3, 1, 300, 384, 1), (1, 2, 1, 500, 256, 2),
                                            (1, 2, 1, 800, 384, 3), (1, 1, 1, 1, 128, 1),
                                            (1, 70, 1, 40, 128, 1), (1, 9, 3, 2000, 384, 6)])
def test_workspace_two_kernel_plan(B, N_o, H, N, kr, J):
    """D = 32 (and D = 16 past N = 640): the query-tile kernel's plan.  J = ceil(N / 384) key ranges of the smallest range
    (128, 256 or 384 keys) that covers N / J, one FP32 dQ partial per range and one FP32 dbias
    partial per outer group, at most 64 groups of equal size (the last one ragged)."""
    from triangular_attention_amd import api
    for D in ((16, 32) if N > 640 else (32,)):
        ws = api.workspace(_dims(B=B, N_o=N_o, H=H, N=N, D=D))
        assert ws["key_tile"] == kr and ws["j_k"] == J and J * kr >= N
        gs, L = ws["outer_group"], ws["l"]
        assert 1 <= L <= min(64, N_o) and L == -(-N_o // gs) and (L - 1) * gs < N_o
        assert ws["dq_partial_elems"] == J * B * N_o * H * N * D
        assert ws["dbias_partial_elems"] == L * B * H * N * N


# --------------------------------------------------------------------------- block ABI


def _block_header_symbols():
    txt = open(os.path.join(ROOT, "include", "tri_attn_block.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(tri_block_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_block_symbol(lib):
    from triangular_attention_amd import _lib
    syms = _block_header_symbols()
    assert set(syms) == set(_lib.BLOCK_EXPORTS)
    for s in syms:
        assert hasattr(lib, s), s


def _bdims(**kw):
    from triangular_attention_amd import _lib
    base = dict(B=1, N=8, C_z=128, H=4, D=32, ending=0, eps=1e-5)
    base.update(kw)
    return _lib.BlockDims(base["B"], base["N"], base["C_z"], base["H"], base["D"], base["ending"], base["eps"])


def _ln_proj(lib, d, **ptrs):
    names = ("z", "gamma", "beta", "w_qkvg", "w_b", "q", "k", "v", "g", "bias", "ln_stats")
    a = {n: P for n in names}
    a.update(ptrs)
    return lib.tri_block_ln_proj(None if d is None else ctypes.byref(d), *[a[n] for n in names], None)


def test_block_validation_errors_before_launch(lib):
    assert _ln_proj(lib, None) == 1
    assert _ln_proj(lib, _bdims(C_z=64)) == 3
    assert _ln_proj(lib, _bdims(H=2, D=32)) == 3          # H * D != 128
    assert _ln_proj(lib, _bdims(H=2, D=64)) == 3          # D not 16 or 32
    assert _ln_proj(lib, _bdims(N=0)) == 2
    assert _ln_proj(lib, _bdims(eps=0.0)) == 2
    assert _ln_proj(lib, _bdims(eps=float("nan"))) == 2
    assert _ln_proj(lib, _bdims(ending=2)) == 2
    assert _ln_proj(lib, _bdims(N=3000)) == 2             # pair tensor past 2^31 bytes
    assert _ln_proj(lib, _bdims(B=2 ** 62)) == 2          # no int64 overflow in the size check
    assert _ln_proj(lib, _bdims(B=2 ** 40, N=32767)) == 2
    assert _ln_proj(lib, _bdims(), z=None) == 1
    assert _ln_proj(lib, _bdims(), bias=MIS) == 4
    d = _bdims(H=8, D=16, ending=1)
    assert lib.tri_block_gate_out(ctypes.byref(d), P, P, P, None, None) == 1
    assert lib.tri_block_gate_out_bwd(ctypes.byref(d), P, P, P, P, P, P, MIS, None) == 4
    assert lib.tri_block_proj_bwd_dz(ctypes.byref(d), *([P] * 11), None, None) == 1
    assert lib.tri_block_proj_bwd_dw(ctypes.byref(d), *([P] * 9), MIS, None) == 4
    assert lib.tri_block_reduce_wgrad(ctypes.byref(d), *([P] * 7), None, None) == 1


@pytest.mark.parametrize("B,N", [(1, 8), (1, 100), (2, 181), (1, 768)])
def test_block_workspace_counts(lib, B, N):
    """Partial buffers = workgroups of the fixed persistent grids (at most 256, 128 tile groups
    for the weight gradients): pairs in tiles of 128 (output projection) and 64 (projections)."""
    d = _bdims(B=B, N=N)
    vals = [ctypes.c_int64() for _ in range(3)]
    assert lib.tri_block_workspace(ctypes.byref(d), *[ctypes.byref(v) for v in vals]) == 0
    pairs = B * N * N
    assert vals[0].value == min(-(-pairs // 128), 256)
    assert vals[1].value == min(-(-pairs // 64), 128)
    assert vals[2].value == min(-(-pairs // 64), 256)


# --------------------------------------------------------------------------- triangle multiplication ABI


def test_library_exports_every_trimul_symbol(lib):
    from triangular_attention_amd import _lib
    txt = open(os.path.join(ROOT, "include", "tri_mul.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    syms = sorted(set(re.findall(r"\b(tri_mul_[a-z0-9_]+)\s*\(", txt)))
    assert set(syms) == set(_lib.TRIMUL_EXPORTS)
    for s in syms:
        assert hasattr(lib, s), s


def _mdims(**kw):
    from triangular_attention_amd import _lib
    base = dict(B=1, N=16, C_z=128, c=128, incoming=0, eps=1e-5)
    base.update(kw)
    return _lib.MulDims(base["B"], base["N"], base["C_z"], base["c"], base["incoming"], base["eps"])


def test_trimul_validation_errors_before_launch(lib):
    f = lambda d, **p: lib.tri_mul_in_fwd(None if d is None else ctypes.byref(d),
                                          *[p.get(n, P) for n in ("z", "g1", "b1", "w", "a", "b", "g", "s")], None)
    assert f(None) == 1
    assert f(_mdims(c=32)) == 3
    assert f(_mdims(C_z=64)) == 3
    assert f(_mdims(N=12)) == 2            # N % 8 != 0
    assert f(_mdims(N=0)) == 2
    assert f(_mdims(eps=-1.0)) == 2
    assert f(_mdims(incoming=3)) == 2
    assert f(_mdims(N=1456, c=128)) == 2   # dproj past 2^31 bytes
    assert f(_mdims(B=2 ** 62)) == 2       # no int64 overflow in the size check
    assert f(_mdims(B=2 ** 40, N=32760)) == 2
    assert f(_mdims(), z=None) == 1
    assert f(_mdims(), a=MIS) == 4
    d = _mdims(c=64, incoming=1)
    assert lib.tri_mul_contract(ctypes.byref(d), P, P, None, None) == 1
    assert lib.tri_mul_contract_bwd(ctypes.byref(d), P, P, P, P, MIS, None) == 4
    assert lib.tri_mul_out_bwd(ctypes.byref(d), *([P] * 10), None, None) == 1
    assert lib.tri_mul_in_bwd_dw(ctypes.byref(d), *([P] * 6), MIS, None) == 4
    assert lib.tri_mul_reduce_wgrad(ctypes.byref(d), *([P] * 9), None, None) == 1


@pytest.mark.parametrize("B,N,c", [(1, 8, 64), (1, 136, 128), (2, 384, 64), (1, 768, 128)])
def test_trimul_workspace_counts(lib, B, N, c):
    """Partial buffers = workgroups of the fixed persistent grids: tiles of 64 (output backward) and
    32 (input dZ) pairs capped at 256, tile groups of 64 pairs capped at 8 * floor(256 / (8 * rows / 128))
    for the input weight gradient (rows = 4c + 128), and two wave halves per workgroup for the output
    normalisation when c = 64."""
    d = _mdims(B=B, N=N, c=c)
    vals = [ctypes.c_int64() for _ in range(4)]
    assert lib.tri_mul_workspace(ctypes.byref(d), *[ctypes.byref(v) for v in vals]) == 0
    pairs = B * N * N
    splits = (4 * c + 128) // 128
    assert vals[0].value == min(-(-pairs // 64), 8 * (512 // (8 * splits)))
    assert vals[1].value == min(-(-pairs // 64), 256)
    assert vals[2].value == min(-(-pairs // 32), 256)
    assert vals[3].value == vals[1].value * (128 // c)


# --------------------------------------------------------------------------- chunked backward


def _chunked(lib, d, ws=P, nbytes=1 << 40, **ptrs):
    names = ("q", "k", "v", "bias", "mask", "d_o", "lse", "delta", "dq", "dk", "dv", "dbias")
    a = {n: P for n in names}
    a["mask"] = None
    a.update(ptrs)
    return lib.tri_attn_bwd_chunked(None if d is None else ctypes.byref(d), *[a[n] for n in names], ws, nbytes, None)


def test_chunked_validation_errors_before_launch(lib):
    d = _dims(N_o=10, N=100)
    assert _chunked(lib, None) == 1
    assert _chunked(lib, d, ws=None) == 1
    assert _chunked(lib, d, dbias=None) == 1
    assert _chunked(lib, d, ws=MIS) == 4
    assert _chunked(lib, d, dq=MIS) == 4
    assert _chunked(lib, _dims(D=48)) == 3
    assert _chunked(lib, _dims(scale=0.0)) == 2
    need = ctypes.c_int64()
    assert lib.tri_attn_bwd_chunked_workspace(ctypes.byref(d), 1, ctypes.byref(need), None) == 0
    assert _chunked(lib, d, nbytes=need.value - 1) == 6        # not even one outer group fits
    assert _chunked(lib, d, nbytes=0) == 6
    assert lib.tri_attn_bwd_chunked_workspace(ctypes.byref(d), 0, ctypes.byref(need), None) == 2


@pytest.mark.parametrize("B,N_o,H,N,D", [(1, 768, 4, 768, 32), (2, 13, 3, 100, 16), (1, 9, 2, 67, 64),
                                         (3, 5, 1, 33, 32)])
def test_chunked_workspace_sizes(lib, B, N_o, H, N, D):
    """Bytes of one chunk of C outer groups: dQ partials J_K * B * min(C * G, N_o) * H * N * D, dbias
    partials C * B * H * N * N and, when there is more than one chunk, the running dbias sum
    B * H * N * N, all FP32 and each rounded up to 256 bytes; C is clamped to 1..L."""
    from triangular_attention_amd import api
    d = _dims(B=B, N_o=N_o, H=H, N=N, D=D)
    ws = api.workspace(d, single_pass=True)
    G, L, jk = ws["outer_group"], ws["l"], ws["j_k"]
    up = lambda x: -(-x // 256) * 256
    for C in (1, 2, 3, L - 1, L, L + 5):
        if C < 1:
            continue
        Cc = min(C, L)
        chunks = -(-L // Cc)
        want = up(4 * jk * B * min(Cc * G, N_o) * H * N * D) + up(4 * Cc * B * H * N * N) + \
            (up(4 * B * H * N * N) if chunks > 1 else 0)
        got = api.chunked_workspace(d, C)
        assert got == {"bytes": want, "groups_per_chunk": Cc}, (C, got, want)


def test_noalloc_validation_before_any_device_access(lib):
    """The allocation-free backward checks its arguments, and that one outer group's buffers fit
    its scratch array, before it looks the array up on the device."""
    names = ("q", "k", "v", "bias", "mask", "d_o", "lse", "delta", "dq", "dk", "dv", "dbias")

    def call(d, **ptrs):
        a = {n: P for n in names}
        a["mask"] = None
        a.update(ptrs)
        return lib.tri_attn_bwd_chunked_noalloc(None if d is None else ctypes.byref(d), *[a[n] for n in names], None)

    assert lib.tri_attn_noalloc_scratch_bytes() == 128 * 2 ** 20
    assert call(None) == 1
    assert call(_dims(), dq=None) == 1
    assert call(_dims(), dbias=MIS) == 4
    assert call(_dims(D=48)) == 3
    # N = 4096, H = 4: the FP32 running dbias sum alone is 256 MiB, past the 128 MiB scratch
    assert call(_dims(N_o=64, H=4, N=4096)) == 6
    # one outer group at N = 1536, H = 4, D = 32 still fits (37.7 MB dQ + 37.7 MB dbias + 37.7 MB sum)
    need = ctypes.c_int64()
    assert lib.tri_attn_bwd_chunked_workspace(ctypes.byref(_dims(N_o=1536, H=4, N=1536)), 1, ctypes.byref(need),
                                              None) == 0
    assert need.value <= lib.tri_attn_noalloc_scratch_bytes()
