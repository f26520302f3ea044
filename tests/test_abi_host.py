"""Host-side checks of the C ABI (CPU only: no kernel is ever launched here).

The library must load, export every function include/fp8rl.h declares, and reject invalid
arguments with the documented status before making any HIP call.
"""

import ctypes
import os
import re

import pytest

from fp8_blockwise_quantization_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8rl.h")

OK, ENULL, ESHAPE, EALIGN, EDTYPE, EWS, EHIP, EARG, ESCRATCH = range(9)
A = 1 << 20  # a fake, 16-byte aligned "device address": never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8rl_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    # FP8RL_TEST_LIBRARY: run these checks against another build of the same sources (the
    # address-sanitized host build of tests/test_abi_asan.py)
    other = os.environ.get("FP8RL_TEST_LIBRARY")
    if other:
        return _lib.declare(ctypes.CDLL(other))
    return _lib.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) == 23
    for n in names:
        assert hasattr(L, n), n
    assert sorted(_lib.EXPORTED) == names


def test_scale_format_and_accum_validation(L):
    # unknown scale format / accumulation mode: rejected before anything else
    assert L.fp8rl_quant_weight_blk128_ex(A, 128, 128, 128, A, 128, A, 2, None) == EARG
    assert L.fp8rl_quant_weight_blk128_ex(A, 128, 128, 128, A, 128, A, -1, None) == EARG
    assert L.fp8rl_quant_weight_blk128_ex(A, 0, 128, 128, A, 128, A, 1, None) == OK
    assert L.fp8rl_quant_weight_blk128_ex(A + 2, 128, 128, 128, A, 128, A, 1, None) == EALIGN
    assert L.fp8rl_quant_act_tok128_ex(A, 4, 128, 128, A, 128, A, 7, None) == EARG
    assert L.fp8rl_quant_act_tok128_ex(A, 0, 128, 128, A, 128, A, 1, None) == OK
    assert L.fp8rl_quant_act_tok128_ex(None, 4, 128, 128, A, 128, A, 1, None) == ENULL
    assert L.fp8rl_quant_weight_blk128_batched_ex(None, 0, 1, None) == OK
    assert L.fp8rl_quant_weight_blk128_batched_ex(None, 1, 1, None) == ENULL
    assert L.fp8rl_quant_weight_blk128_batched_ex(None, 1, 3, None) == EARG
    g = L.fp8rl_gemm_w8a8_blockscaled
    assert g(A, A, A, A, 64, 256, 256, A, 0, 256, 4, None, 0, None) == EARG
    assert g(A, A, A, A, 64, 256, 256, A, 0, 256, -1, None, 0, None) == EARG
    assert g(A, A, A, A, 0, 256, 256, A, 0, 256, 2, None, 0, None) == OK
    # FP8 and MX slice sums are refused with float32 output (y_dtype 1), on every GEMM entry
    # point, before any HIP call; F16 and AUTO are not refused by that check
    for acc in (0, 2):
        assert g(A, A, A, A, 64, 256, 256, A, 1, 256, acc, None, 0, None) == EARG
        assert L.fp8rl_gemm_w8a8_rowscaled(A, A, A, A, 64, 256, 256, A, 1, 256, acc, None, 0,
                                           None) == EARG
        assert L.fp8rl_grouped_gemm_w8a8(A, A, A, A, A, 2, 64, 256, 256, A, 1, acc, None, 0,
                                         None) == EARG
        assert L.fp8rl_gemm_w8a8_fused_act_quant(A, 256, A, A, 64, 256, 256, A, 1, 256, acc, 1,
                                                 None, 0, None) == EARG
    # accepted combinations reach the later checks (here: the missing workspace of a split-K
    # decode shape)
    need = L.fp8rl_workspace_bytes(0, 200, 1024, 4096, 0)
    assert need > 0
    for acc, out in ((3, 0), (3, 1), (1, 1), (0, 0), (2, 0)):
        assert g(A, A, A, A, 200, 1024, 4096, A, out, 1024, acc, None, 0, None) == EWS


def test_status_strings_and_version(L):
    for s in range(9):
        assert L.fp8rl_status_string(s)
    assert L.fp8rl_status_string(99) == b"unknown status"
    assert L.fp8rl_version() >= 100


def test_quant_weight_validation(L):
    f = L.fp8rl_quant_weight_blk128
    assert f(A, 0, 128, 128, A, 128, A, None) == OK  # nothing to do
    assert f(A, 128, 0, 128, A, 128, A, None) == OK
    assert f(None, 128, 128, 128, A, 128, A, None) == ENULL
    assert f(A, 128, 128, 128, A, 128, None, None) == ENULL
    assert f(A, -1, 128, 128, A, 128, A, None) == ESHAPE
    assert f(A, 100, 128, 128, A, 128, A, None) == ESHAPE
    assert f(A, 128, 130, 130, A, 130, A, None) == ESHAPE
    assert f(A, 128, 128, 64, A, 128, A, None) == ESHAPE  # ld < K
    assert f(A + 2, 128, 128, 128, A, 128, A, None) == EALIGN
    assert f(A, 128, 128, 132, A, 128, A, None) == EALIGN  # 264-byte pitch
    assert f(A, 128, 128, 128, A, 136, A, None) == EALIGN
    assert f(A, 128, 128, 128, A, 128, A + 2, None) == EALIGN


def test_quant_weight_batched_validation(L):
    f = L.fp8rl_quant_weight_blk128_batched
    D = _lib.WeightDesc
    ok = D(A, A, A, 128, 256, 256, 256)
    arr = (D * 3)(ok, D(A, A, A, 0, 256, 256, 256), D(A, A, A + 2, 128, 256, 256, 256))
    assert f(arr, 0, None) == OK
    assert f(None, 2, None) == ENULL
    assert f(arr, -1, None) == EARG
    assert f(arr, 3, None) == EALIGN  # the third descriptor fails: nothing is launched
    bad = (D * 2)(ok, D(A, A, A, 100, 256, 256, 256))
    assert f(bad, 2, None) == ESHAPE
    assert f((D * 1)(D(A, None, A, 128, 128, 128, 128)), 1, None) == ENULL


def test_quant_act_validation(L):
    f = L.fp8rl_quant_act_tok128
    assert f(None, 0, 128, 128, None, 128, None, None) == OK  # M == 0
    assert f(None, 4, 128, 128, A, 128, A, None) == ENULL
    assert f(A, 4, 100, 128, A, 128, A, None) == ESHAPE
    assert f(A, -4, 128, 128, A, 128, A, None) == ESHAPE
    assert f(A, 4, 128, 128, A + 8, 128, A, None) == EALIGN


def test_per_tensor_validation(L):
    a = L.fp8rl_amax_bf16
    assert a(None, 0, 16, 16, None, None) == OK  # nothing to do
    assert a(None, 4, 16, 16, A, None) == ENULL
    assert a(A, 4, 16, 16, None, None) == ENULL
    assert a(A, 4, 12, 16, A, None) == ESHAPE  # cols % 8
    assert a(A, 4, 16, 8, A, None) == ESHAPE   # ld < cols
    assert a(A, 1 << 28, 128, 128, A, None) == ESHAPE  # 2^32 chunks
    assert a(A + 8, 4, 16, 16, A, None) == EALIGN
    assert a(A, 4, 16, 20, A, None) == EALIGN
    assert a(A, 4, 16, 16, A + 2, None) == EALIGN
    D = _lib.TensorDesc
    b = L.fp8rl_amax_bf16_batched
    arr = (D * 2)(D(A, A, 4, 16, 16), D(A, A + 1, 4, 16, 16))
    assert b(arr, 0, None) == OK
    assert b(None, 1, None) == ENULL
    assert b(arr, -1, None) == EARG
    assert b(arr, 2, None) == EALIGN  # the second descriptor fails: nothing is launched
    assert b((D * 1)(D(None, None, 0, 16, 16)), 1, None) == OK
    sc = L.fp8rl_scale_from_amax
    assert sc(None, 0, None, None) == OK
    assert sc(None, 3, A, None) == ENULL
    assert sc(A, -1, A, None) == ESHAPE
    assert sc(A, 3, A + 2, None) == EALIGN
    q = L.fp8rl_quant_bf16_per_tensor
    assert q(None, 0, 16, 16, None, None, 0, 16, None, None) == OK
    assert q(A, 4, 16, 16, None, A, 4, 16, None, None) == ENULL
    assert q(A, 4, 16, 16, A, None, 4, 16, None, None) == ENULL
    assert q(A, 4, 16, 16, A, A, 3, 16, None, None) == ESHAPE  # rows > out rows without slots
    assert q(A, 4, 16, 16, A, A, 4, 8, None, None) == ESHAPE   # ld_out < cols
    assert q(A, 4, 16, 16, A, A, -1, 16, A, None) == ESHAPE
    assert q(A, 4, 16, 16, A, A + 4, 4, 16, None, None) == EALIGN
    assert q(A, 4, 16, 16, A, A, 4, 20, None, None) == EALIGN
    assert q(A, 4, 16, 16, A, A, 4, 16, A + 4, None) == EALIGN
    assert q(A, 4, 16, 16, A + 2, A, 4, 16, None, None) == EALIGN
    Q = _lib.QuantDesc
    qb = L.fp8rl_quant_bf16_per_tensor_batched
    good = Q(A, A, A, None, 4, 16, 16, 4, 16)
    assert qb(None, 0, None) == OK
    assert qb(None, 2, None) == ENULL
    assert qb((Q * 1)(good), -1, None) == EARG
    assert qb((Q * 2)(good, Q(A, A, A, None, 5, 16, 16, 4, 16)), 2, None) == ESHAPE
    assert qb((Q * 2)(good, Q(A, None, A, None, 4, 16, 16, 4, 16)), 2, None) == ENULL
    assert qb((Q * 2)(good, Q(A, A, A, A + 2, 4, 16, 16, 4, 16)), 2, None) == EALIGN
    assert qb((Q * 1)(Q(None, None, None, None, 0, 16, 16, 0, 16)), 1, None) == OK


def test_backward_validation(L):
    w = L.fp8rl_quant_weight_blk128_t
    assert w(A, 0, 128, 128, None, 0, None, A, 0, A, 0, None) == OK
    assert w(A, 128, 256, 256, A, 256, None, A, 128, A, 0, None) == ENULL  # wq without sw
    assert w(A, 128, 256, 256, None, 0, None, None, 128, A, 0, None) == ENULL
    assert w(A, 128, 256, 256, None, 0, None, A, 64, A, 0, None) == ESHAPE  # ld_wqt < N
    assert w(A, 100, 256, 256, None, 0, None, A, 128, A, 0, None) == ESHAPE
    assert w(A, 128, 256, 256, None, 0, None, A + 8, 128, A, 0, None) == EALIGN
    assert w(A, 128, 256, 256, None, 0, None, A, 128, A, 5, None) == EARG
    c = L.fp8rl_quant_act_colwise128
    assert c(A, 0, 128, 128, None, 0, None, A, 0, A, 0, None) == OK
    assert c(A, 100, 128, 128, None, 0, None, A, 128, A, 0, None) == ESHAPE  # M % 128
    assert c(A, 128, 128, 128, A, 128, None, A, 128, A, 0, None) == ENULL
    assert c(A, 128, 128, 128, None, 0, None, A, 64, A, 0, None) == ESHAPE
    assert c(A, 128, 128, 128, None, 0, None, A, 128, A + 2, 0, None) == EALIGN
    assert c(A, 128, 128, 128, None, 0, None, A, 128, A, 9, None) == EARG
    g = L.fp8rl_gemm_w8a8_rowscaled
    assert g(A, A, A, A, 0, 256, 256, A, 0, 256, 0, None, 0, None) == OK
    assert g(A, A, A, A, 64, 256, 200, A, 0, 256, 0, None, 0, None) == ESHAPE
    assert g(A, A, A, None, 64, 256, 256, A, 0, 256, 0, None, 0, None) == ENULL
    assert g(A, A, A, A, 64, 256, 256, A, 0, 256, 4, None, 0, None) == EARG
    # row-scaled B never takes the decode path: its small-M plan has its own workspace rule
    ws_row = L.fp8rl_workspace_bytes(2, 64, 4096, 4096, 0)
    ws_blk = L.fp8rl_workspace_bytes(0, 64, 4096, 4096, 0)
    assert ws_row != ws_blk
    assert g(A, A, A, A, 64, 4096, 4096, A, 0, 4096, 0, A, ws_row - 1, None) == EWS


def test_encode_validation(L):
    f = L.fp8rl_encode_e4m3_f32
    assert f(None, 0, None, None) == OK
    assert f(None, 4, A, None) == ENULL
    assert f(A + 4, 4, A, None) == EALIGN
    assert f(A, -1, A, None) == ESHAPE


def test_gemm_validation(L):
    f = L.fp8rl_gemm_w8a8_blockscaled
    args = lambda **k: dict(dict(xq=A, sa=A, wq=A, sw=A, M=64, N=256, K=256, y=A, dt=0, ldy=256,
                                 acc=0, ws=A, wsb=1 << 30), **k)

    def call(**k):
        a = args(**k)
        return f(a["xq"], a["sa"], a["wq"], a["sw"], a["M"], a["N"], a["K"], a["y"], a["dt"],
                 a["ldy"], a["acc"], a["ws"], a["wsb"], None)

    assert call(M=0, xq=None) == OK
    assert call(xq=None) == ENULL
    assert call(y=None) == ENULL
    assert call(N=200) == ESHAPE
    assert call(K=192) == ESHAPE
    assert call(M=-1) == ESHAPE
    assert call(ldy=128) == ESHAPE
    assert call(dt=5) == EDTYPE
    assert call(acc=4) == EARG  # (2 is FP8RL_ACCUM_MX, 3 FP8RL_ACCUM_AUTO)
    assert call(acc=-1) == EARG
    assert call(xq=A + 1) == EALIGN
    assert call(ldy=260) == EALIGN  # 520-byte bf16 pitch
    assert L.fp8rl_workspace_bytes(0, 4, 256, 4096, 0) == 0  # up to 4 rows: none
    need = L.fp8rl_workspace_bytes(0, 200, 256, 4096, 0)
    assert need > 0  # a mid-M problem uses split-K partials
    assert call(M=200, K=4096, wsb=need - 1) == EWS
    assert call(M=200, K=4096, ws=None) == EWS


def test_fused_act_gemm_validation(L):
    f = L.fp8rl_gemm_w8a8_fused_act_quant
    args = lambda **k: dict(dict(x=A, ldx=4096, wq=A, sw=A, M=64, N=256, K=4096, y=A, dt=0,
                                 ldy=256, acc=0, sf=0, ws=A, wsb=1 << 30), **k)

    def call(**k):
        a = args(**k)
        return f(a["x"], a["ldx"], a["wq"], a["sw"], a["M"], a["N"], a["K"], a["y"], a["dt"],
                 a["ldy"], a["acc"], a["sf"], a["ws"], a["wsb"], None)

    assert call(M=0, x=None) == OK
    assert call(x=None) == ENULL
    assert call(sw=None) == ENULL
    assert call(N=200) == ESHAPE
    assert call(ldx=4000) == ESHAPE  # pitch below K
    assert call(dt=2) == EDTYPE
    assert call(acc=4) == EARG
    assert call(sf=2) == EARG
    assert call(acc=2, sf=0) == EARG  # matrix-core scaling needs power-of-two scales
    assert call(x=A + 2) == EALIGN
    assert call(ldx=4100) == EALIGN  # 8200-byte bf16 pitch
    need = L.fp8rl_workspace_bytes(3, 64, 256, 4096, 0)
    assert need > 0  # above 4 rows the codes and scales are staged in the workspace
    assert call(wsb=need - 1) == EWS
    assert call(ws=None) == EWS
    assert call(M=65, wsb=L.fp8rl_workspace_bytes(3, 65, 256, 4096, 0) - 1) == EWS
    assert call(K=384, ldx=384, wsb=L.fp8rl_workspace_bytes(3, 64, 256, 384, 0) - 1) == EWS


def test_grouped_gemm_validation(L):
    f = L.fp8rl_grouped_gemm_w8a8
    base = [A, A, A, A, A, 4, 1000, 256, 256, A, 0, 0, None, 0, None]
    assert f(*base[:6], 0, *base[7:]) == OK  # M_total == 0
    b = list(base)
    b[5] = 0
    assert f(*b) == EARG
    b = list(base)
    b[4] = None
    assert f(*b) == ENULL
    b = list(base)
    b[7] = 300
    assert f(*b) == ESHAPE
    b = list(base)
    b[4] = A + 2
    assert f(*b) == EALIGN
    b = list(base)
    b[10] = 3
    assert f(*b) == EDTYPE
    b = list(base)
    b[11] = 5
    assert f(*b) == EARG


def test_grouped_fused_act_validation(L):
    f = L.fp8rl_grouped_gemm_w8a8_fused_act_quant
    # the Qwen3-30B-A3B gate/up shape: 4096 tokens, top-8 (32768 grouped rows), 128 experts
    args = lambda **k: dict(dict(x=A, ldx=2048, src=4096, ids=A, wq=A, sw=A, off=A, E=128,
                                 M=32768, N=1536, K=2048, y=A, dt=0, acc=3, sf=0, ws=A,
                                 wsb=1 << 30), **k)

    def call(**k):
        a = args(**k)
        return f(a["x"], a["ldx"], a["src"], a["ids"], a["wq"], a["sw"], a["off"], a["E"],
                 a["M"], a["N"], a["K"], a["y"], a["dt"], a["acc"], a["sf"], a["ws"], a["wsb"],
                 None)

    assert call(M=0, x=None, ids=None) == OK  # nothing to do
    assert call(E=0) == EARG
    assert call(E=1025) == EARG
    for k in ("x", "wq", "sw", "off", "y"):
        assert call(**{k: None}) == ENULL, k
    assert call(N=200) == ESHAPE
    assert call(K=2000, ldx=2048) == ESHAPE
    assert call(ldx=1920) == ESHAPE  # pitch below K
    assert call(src=0) == ESHAPE  # a gather needs at least one source row
    assert call(ids=None) == ESHAPE  # no gather: x must hold the M_total grouped rows
    assert call(src=(1 << 32) // 2048, M=32768) == ESHAPE  # source offsets beyond 32 bits
    assert call(src=(1 << 30) // 16, ids=A, wsb=1 << 62) == ESHAPE  # quantizer grid limit
    assert call(dt=2) == EDTYPE
    assert call(acc=4) == EARG
    assert call(dt=1, acc=0) == EARG  # FP8 slice sums with float32 output
    assert call(sf=2) == EARG
    assert call(acc=2, sf=0) == EARG  # matrix-core scaling needs power-of-two scales
    assert call(x=A + 2) == EALIGN
    assert call(ldx=2052) == EALIGN  # 4104-byte bf16 pitch
    assert call(ids=A + 2) == EALIGN
    assert call(off=A + 2) == EALIGN
    need = L.fp8rl_workspace_bytes(4, 32768, 1536, 2048, 128)
    assert call(wsb=need - 1) == EWS
    assert call(ws=None) == EWS
    assert call(ws=A + 8, wsb=need) == EALIGN
    # the workspace is sized for max(src_rows, M_total) rows
    assert call(src=40000, ids=A, wsb=need) == EWS
    assert call(src=32768, ids=None, M=32768, wsb=need - 1) == EWS


def test_workspace_query_is_pure_host(L):
    hdr = _lib.WORKSPACE_HEADER_BYTES
    assert hdr == 4096  # FP8RL_WORKSPACE_HEADER_BYTES
    # the blockscaled GEMM up to 4 rows splits K only inside each workgroup (no workspace); the
    # decode GEMM above that (up to 64 rows) splits K over workgroups: above 32 rows with at least
    # 192 tiles of 128 columns, 128-column tiles and no split; otherwise 64-column tiles and K
    # split S ways: up to 256 tiles S the largest power of two with tiles * 2S <= 256 and ranges
    # of >= 4 slices, past 256 tiles S = 1 (2 at <= 32 rows with >= 8 slices), S = 1 past 1024
    # tiles; workspace = header + [tiles][S] partial tiles of 64 columns x padded rows (32 or 64)
    def dec(M, N, K):
        kb = K // 128
        if M > 32 and N // 128 >= 192:
            return 0
        tiles, S = N // 64, 1
        if tiles <= 256:
            while tiles * 2 * S <= 256 and kb // (2 * S) >= 4:
                S *= 2
        elif M <= 32 and kb >= 8:
            S = 2
        if tiles > 1024:
            S = 1
        per = -(-kb // S)
        S = -(-kb // per)
        bm = 32 if M <= 32 else 64
        return hdr + tiles * S * 64 * bm * 4 if S > 1 else 0
    def a256(n):
        return (n + 255) // 256 * 256

    # the GEMM on bf16 activations (op 3): one kernel and no workspace up to 4 rows; above, the
    # blockscaled GEMM's workspace (its counter header reserved even when it splits nothing),
    # then the staged codes and their scales, each part 256-byte aligned
    def fused(M, N, K):
        if M <= 4:
            return 0
        return (max(a256(L.fp8rl_workspace_bytes(0, M, N, K, 0)), hdr) + a256(M * K)
                + M * (K // 128) * 4)
    for shape in [(64, 4096, 4096), (20, 1024, 12288), (64, 6144, 4096), (17, 6144, 4096),
                  (32, 24576, 4096), (48, 4096, 384 * 3), (5, 4096, 4096), (16, 2048, 4096)]:
        assert L.fp8rl_workspace_bytes(0, *shape, 0) == dec(*shape) > 0, shape
    for shape in [(64, 4096, 4096), (20, 1024, 12288), (64, 12288, 4096), (1, 256, 2048),
                  (4, 4096, 4096), (5, 4096, 4096), (16, 4096, 4096), (17, 4096, 4096),
                  (65, 256, 4096), (64, 4096, 384),
                  (300, 768, 2048), (8192, 4096, 4096)]:
        assert L.fp8rl_workspace_bytes(3, *shape, 0) == fused(*shape), shape
    assert L.fp8rl_workspace_bytes(3, 64, 4096, 4096, 0) == (hdr + 64 * 4 * 64 * 64 * 4
                                                             + 64 * 4096 + 64 * 32 * 4)
    assert L.fp8rl_workspace_bytes(3, 8192, 4096, 4096, 0) == hdr + 8192 * 4096 + 8192 * 32 * 4
    assert L.fp8rl_workspace_bytes(3, 1, 256, 2048, 0) == 0
    assert L.fp8rl_workspace_bytes(0, 64, 4096, 512, 0) == 0  # 4 slices: one range
    assert L.fp8rl_workspace_bytes(0, 64, 4096, 1024, 0) == hdr + 64 * 2 * 64 * 64 * 4
    assert L.fp8rl_workspace_bytes(0, 32, 131072, 2048, 0) == 0  # more tiles than counters
    assert L.fp8rl_workspace_bytes(0, 64, 24576, 4096, 0) == 0  # 128-column tiles, K unsplit
    assert L.fp8rl_workspace_bytes(0, 64, 12288, 4096, 0) == 0  # 192 tiles: two K halves each
    assert L.fp8rl_workspace_bytes(0, 32, 24576, 4096, 0) == hdr + 384 * 2 * 64 * 32 * 4
    assert L.fp8rl_workspace_bytes(0, 0, 256, 256, 0) == 0
    assert L.fp8rl_workspace_bytes(0, 8192, 4096, 4096, 0) == 0  # large M: no split
    assert L.fp8rl_workspace_bytes(1, 32768, 1536, 2048, 128) == 0
    assert L.fp8rl_workspace_bytes(7, 64, 256, 256, 0) == 0
    # the grouped GEMM on bf16 activations (op 4), for M rows: the counter header (left alone),
    # then the codes and scales of M rows, each 256-byte aligned; twice that area past
    # K = 32768, where the gathered codes are copied out for the register-staged tiles
    def grouped_fused(M, N, K):
        area = a256(M * K) + a256(M * (K // 128) * 4)
        return hdr + (1 if K <= 32768 else 2) * area
    for shape in [(32768, 1536, 2048), (32768, 2048, 768), (1, 256, 128), (1000, 256, 32768),
                  (1000, 256, 32896), (77, 384, 640)]:
        assert L.fp8rl_workspace_bytes(4, *shape, 128) == grouped_fused(*shape), shape
    assert L.fp8rl_workspace_bytes(4, 32768, 1536, 2048, 128) == 4096 + 32768 * 2048 + 32768 * 64
    assert L.fp8rl_workspace_bytes(4, 0, 1536, 2048, 128) == 0


def test_python_binding_rejects_host_tensors():
    import torch

    w = torch.zeros((128, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        _lib.fp8rl_quant_weight_blk128(w)


def test_binding_size_checks():
    """The bindings compare every tensor the C call reads or writes by pointer alone with the size
    the call will assume (a smaller tensor would be accessed past its end)."""
    import torch

    t = torch.zeros((4, 256))
    _lib._sizes(y=(t, (4, 256)), s=(t, 1024), none=(None, 7))
    with pytest.raises(ValueError):
        _lib._sizes(y=(t, (3, 256)))
    with pytest.raises(ValueError):
        _lib._sizes(y=(t, (4, 384)))
    with pytest.raises(ValueError):
        _lib._sizes(s=(t, 1023))


def test_noalloc_gemm_validation(L):
    """The no-allocation GEMM validates like the workspace form and refuses, before any HIP call,
    a shape whose scratch need exceeds the static buffer."""
    g = L.fp8rl_gemm_w8a8_blockscaled_noalloc
    scratch = 32 << 20
    assert g(A, A, A, A, 0, 256, 256, A, 0, 256, 3, None) == OK
    assert g(None, A, A, A, 64, 256, 256, A, 0, 256, 3, None) == ENULL
    assert g(A, A, A, A, 64, 256, 200, A, 0, 256, 3, None) == ESHAPE
    assert g(A, A, A, A, 64, 256, 256, A, 5, 256, 3, None) == EDTYPE
    assert g(A, A, A, A, 64, 256, 256, A, 1, 256, 0, None) == EARG  # FP8 slices, float32 out
    assert g(A, A, A, A, 64, 256, 256, A + 2, 0, 256, 3, None) == EALIGN
    # a split-K shape (K beyond the DMA-fed tiles) whose partials need more than the scratch holds
    M, N, K = 1024, 1152, 65536
    need = L.fp8rl_workspace_bytes(0, M, N, K, 0)
    assert need > scratch, need
    assert g(A, A, A, A, M, N, K, A, 0, N, 3, None) == ESCRATCH
    # the decode shapes of the workloads fit
    for m, n, k in ((64, 24576, 4096), (64, 6144, 4096), (64, 4096, 12288), (64, 28672, 4096)):
        assert L.fp8rl_workspace_bytes(0, m, n, k, 0) <= scratch
