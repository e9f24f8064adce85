"""The C ABI library: it loads without a GPU, exports every symbol that
include/awq.h declares, and rejects bad arguments on the host before any
launch (so none of these calls touches device memory)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq.h")

abi = pytest.importorskip("weight_only_int4_stats_amd._abi")


def _lib():
    if not os.path.exists(abi.LIB_PATH):
        pytest.fail("libawq_gfx950.so is not built (python -m weight_only_int4_stats_amd.build)")
    return abi.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(awq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_calls_and_helpers():
    names = declared_functions()
    for n in ("awq_act_stats", "awq_search_scales", "awq_search_scales_ex", "awq_quantize_pack", "awq_w4a16_gemm",
              "awq_fold_scales", "awq_quantize_codes", "awq_salient_channels", "awq_workspace_bytes",
              "awq_status_str", "awq_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in abi.SIGNATURES, f"binding lacks {name}"


def test_status_strings_and_version():
    lib = _lib()
    assert lib.awq_abi_version() == 6
    for code in range(8):
        assert lib.awq_status_str(code).decode()
    assert lib.awq_status_str(0).decode() == "ok"


def test_workspace_sizes():
    lib = _lib()
    assert lib.awq_workspace_bytes(abi.AWQ_OP_ACT_STATS, 0, 0, 4096, 65536, 0) >= 4096 * 8
    assert lib.awq_workspace_bytes(abi.AWQ_OP_QUANTIZE, 0, 11008, 4096, 0, 0) == 0
    n = lib.awq_workspace_bytes(abi.AWQ_OP_SEARCH, 0, 11008, 4096, 65536, 20)
    assert n >= 11008 * 4096 * 2 + 20 * 4096 * 4
    assert lib.awq_workspace_bytes(abi.AWQ_OP_SEARCH, 0, -1, 4096, 64, 20) == 0


def test_small_batch_product_workspace():
    """17..64 tokens: fp16 activations, row and weight-row exponents, and fp32
    partial sums only where the layer is split over K (256 compute units when
    no device is visible): layers with more 16-row tiles than compute units
    are never split; smaller ones only when the activations exceed 256 KB."""
    lib = _lib()

    def a(n):
        return (n + 255) // 256 * 256

    def expect(M, N, K, S):
        return a(2 * M * K) + a(4 * M) + a(4 * N) + (a(4 * S * M * N) if S > 1 else 0)

    for M, N, K, S in ((32, 4096, 4096, 1),      # 256 KB of activations: whole, one tile per block
                       (32, 11008, 4096, 1),     # 688 tiles: whole rounds of balanced row blocks
                       (17, 57344, 8192, 1),
                       (32, 4096, 11008, 4),     # 688 KB: 64-row blocks over 4 slices
                       (48, 4096, 4096, 2),      # 384 KB: 32-row blocks over 2 slices
                       (64, 777, 8192, 8),       # 25 blocks of 32 rows, 8 slices of 8 units
                       (40, 65, 128, 1)):        # a single unit: no slices
        assert lib.awq_workspace_bytes(abi.AWQ_OP_GEMM, M, N, K, 0, 0) == expect(M, N, K, S), (M, N, K)


# fake device addresses: validation must fail before anything dereferences them
A = ctypes.c_void_p(0x10000)       # 16-byte aligned
A2 = ctypes.c_void_p(0x20000)
A3 = ctypes.c_void_p(0x30000)
BAD = ctypes.c_void_p(0x10002)     # misaligned
NULL = None
E = abi


def test_act_stats_validation():
    lib = _lib()
    f = lib.awq_act_stats
    ws_ok = 1 << 20
    assert f(NULL, E.AWQ_F16, 64, 512, 512, A2, A3, ws_ok, NULL) == 1
    assert f(A, E.AWQ_F16, 64, 512, 512, NULL, A3, ws_ok, NULL) == 1
    assert f(A, E.AWQ_F32, 64, 512, 512, A2, A3, ws_ok, NULL) == 3
    assert f(A, E.AWQ_F16, 0, 512, 512, A2, A3, ws_ok, NULL) == 2        # empty calibration
    assert f(A, E.AWQ_F16, 64, 512, 500, A2, A3, ws_ok, NULL) == 2       # ld < K
    assert f(A, E.AWQ_F16, 64, 500, 504, A2, A3, ws_ok, NULL) == 4       # K % 8
    assert f(BAD, E.AWQ_F16, 64, 512, 512, A2, A3, ws_ok, NULL) == 4
    assert f(A, E.AWQ_F16, 64, 512, 512, A2, NULL, ws_ok, NULL) == 6
    assert f(A, E.AWQ_F16, 64, 512, 512, A2, A3, 16, NULL) == 6


def test_search_validation():
    lib = _lib()
    f = lib.awq_search_scales_ex
    ws = 1 << 40

    def call(**kw):
        a = dict(w=A, dt=E.AWQ_F16, N=512, K=512, x=A2, T=64, ldx=512, m=A3, al=A3, na=20, g=128,
                 bits=4, sym=0, kept=NULL, s=A2, inv=NULL, loss=NULL, best=NULL, ws=A3, wsb=ws)
        a.update(kw)
        return f(a["w"], a["dt"], a["N"], a["K"], a["x"], a["T"], a["ldx"], a["m"], a["al"], a["na"],
                 a["g"], a["bits"], a["sym"], a["kept"], a["s"], a["inv"], a["loss"], a["best"], a["ws"],
                 a["wsb"], NULL)

    assert call(w=NULL) == 1
    assert call(s=NULL) == 1
    assert call(dt=E.AWQ_F32) == 3
    assert call(g=32) == 5
    assert call(g=512) == 5
    assert call(bits=1) == 5
    assert call(bits=9) == 5
    assert call(bits=8, sym=1) == 5          # 2^8 + 1 symmetric levels do not fit a byte
    assert call(sym=2) == 5
    assert call(g=256, K=384, ldx=384) == 2  # K % group
    assert call(g=64, K=576, ldx=576) == 2   # K % 128
    assert call(na=0) == 5
    assert call(na=65) == 5
    assert call(K=500, ldx=504) == 2
    assert call(T=0) == 2
    assert call(N=0) == 2
    assert call(ldx=256) == 2
    assert call(w=BAD) == 4
    assert call(kept=ctypes.c_void_p(0x20008)) == 4   # the mask is read 8 channels at a time
    assert call(ws=NULL) == 6
    assert call(wsb=1024) == 6


def test_plain_search_validation():
    """awq_search_scales (the 4-bit asymmetric grid, no mask) validates the
    same way as the variant entry point."""
    lib = _lib()
    f = lib.awq_search_scales

    def call(**kw):
        a = dict(w=A, dt=E.AWQ_F16, N=512, K=512, x=A2, T=64, ldx=512, m=A3, al=A3, na=20, g=128,
                 s=A2, inv=NULL, loss=NULL, best=NULL, ws=A3, wsb=1 << 40)
        a.update(kw)
        return f(a["w"], a["dt"], a["N"], a["K"], a["x"], a["T"], a["ldx"], a["m"], a["al"], a["na"],
                 a["g"], a["s"], a["inv"], a["loss"], a["best"], a["ws"], a["wsb"], NULL)

    assert call(x=NULL) == 1
    assert call(dt=E.AWQ_F32) == 3
    assert call(K=500, ldx=504) == 2
    assert call(g=96) == 5
    assert call(na=65) == 5
    assert call(x=BAD) == 4
    assert call(wsb=1024) == 6


def _prototypes():
    """name -> (return type, [parameter types]) of every function in awq.h,
    whitespace normalised, parameter names dropped."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for ret, name, params in re.findall(r"([A-Za-z_][\w\s\*]*?)\s*\b(awq_[a-z0-9_]+)\s*\(([^;{]*?)\)\s*;",
                                        text):
        types = []
        for prm in params.split(","):
            prm = " ".join(prm.split())
            if prm in ("", "void"):
                continue
            m = re.match(r"(.*?)([A-Za-z_]\w*)$", prm)
            types.append(m.group(1).replace(" *", "*").strip())
        out[name] = (" ".join(ret.split()).replace(" *", "*"), types)
    return out


# The boundary contract: the four calls and two helpers, their argument types
# in order.  A stream is a hipStream_t, which this header (free of HIP
# headers) passes as void*: the same pointer in the calling convention.
CONTRACT = {
    "awq_act_stats": ("awq_status", ["const void*", "awq_dtype", "int64_t", "int64_t", "int64_t",
                                     "float*", "void*", "size_t", "void*"]),
    "awq_search_scales": ("awq_status", ["const void*", "awq_dtype", "int64_t", "int64_t",
                                         "const void*", "int64_t", "int64_t", "const float*",
                                         "const double*", "int", "int", "float*", "float*",
                                         "double*", "int32_t*", "void*", "size_t", "void*"]),
    "awq_quantize_pack": ("awq_status", ["const void*", "awq_dtype", "int64_t", "int64_t",
                                         "const float*", "int", "int32_t*", "uint16_t*", "uint8_t*",
                                         "float*", "void*"]),
    "awq_w4a16_gemm": ("awq_status", ["const void*", "awq_dtype", "int64_t", "int64_t", "int64_t",
                                      "const int32_t*", "const uint16_t*", "const uint8_t*",
                                      "int64_t", "int", "const float*", "void*", "awq_dtype",
                                      "int64_t", "void*", "size_t", "void*"]),
    "awq_workspace_bytes": ("size_t", ["awq_op", "int64_t", "int64_t", "int64_t", "int64_t", "int"]),
    "awq_status_str": ("const char*", ["awq_status"]),
}


def test_header_prototypes_match_the_contract():
    protos = _prototypes()
    for name, want in CONTRACT.items():
        assert protos.get(name) == want, (name, protos.get(name), want)


def test_binding_argument_counts_match_the_header():
    for name, (_, types) in _prototypes().items():
        assert len(abi.SIGNATURES[name][1]) == len(types), name


def _direct_search_ws(N, K, T, n_alpha):
    """Bytes of the direct-form search workspace for bf16 tokens (the larger
    layout): candidate scales and reciprocals, then for the candidates scored
    per launch (as many as fit 64 MiB of error rows, at least one) their row
    exponents and error rows, the losses, their tile partials, the tokens
    rounded to fp16 and their exponents, each piece rounded up to 256 bytes."""
    up = lambda b: (b + 255) // 256 * 256  # noqa: E731
    tiles = -(-N // 256) * -(-T // 256)
    nc = max(1, min(n_alpha, (64 << 20) // (N * K * 2)))
    return (2 * up(n_alpha * K * 4) + up(nc * N * 4) + up(nc * N * K * 2) + up(n_alpha * 8) +
            up(nc * tiles * 8) + up(T * K * 2) + up(T * 4))


def test_gram_form_token_limit():
    """Past 2^23 padded tokens the Gram form's 32-bit row offsets would wrap:
    the search then takes the direct form, whose workspace the library
    reports; just below the limit it still takes the Gram form."""
    lib = _lib()
    N, K = 256, 256
    for T in ((1 << 23), (1 << 23) + 1000):
        assert lib.awq_workspace_bytes(abi.AWQ_OP_SEARCH, 0, N, K, T, 20) == _direct_search_ws(N, K, T, 20)
    T = (1 << 23) - 256
    assert lib.awq_workspace_bytes(abi.AWQ_OP_SEARCH, 0, N, K, T, 20) != _direct_search_ws(N, K, T, 20)


def test_quantize_validation():
    lib = _lib()
    f = lib.awq_quantize_pack
    assert f(A, E.AWQ_F16, 0, 512, NULL, 128, NULL, NULL, NULL, NULL, NULL) == 0   # N = 0: no-op
    assert f(NULL, E.AWQ_F16, 4, 512, NULL, 128, A2, A3, A3, NULL, NULL) == 1
    assert f(A, E.AWQ_F16, 4, 512, NULL, 128, A2, NULL, A3, NULL, NULL) == 1
    assert f(A, E.AWQ_F32, 4, 512, NULL, 128, A2, A3, A3, NULL, NULL) == 3
    assert f(A, E.AWQ_F16, 4, 500, NULL, 128, A2, A3, A3, NULL, NULL) == 2
    assert f(A, E.AWQ_F16, -1, 512, NULL, 128, A2, A3, A3, NULL, NULL) == 2
    assert f(A, E.AWQ_F16, 4, 512, NULL, 96, A2, A3, A3, NULL, NULL) == 5
    assert f(A, E.AWQ_F16, 4, 384, NULL, 256, A2, A3, A3, NULL, NULL) == 2
    assert f(BAD, E.AWQ_F16, 4, 512, NULL, 128, A2, A3, A3, NULL, NULL) == 4
    assert f(A, E.AWQ_F16, 4, 512, BAD, 128, A2, A3, A3, NULL, NULL) == 4


def test_quantize_codes_validation():
    lib = _lib()
    f = lib.awq_quantize_codes

    def call(**kw):
        a = dict(w=A, dt=E.AWQ_F16, N=4, K=512, s=NULL, g=128, bits=3, sym=0, q=A2, sc=A3, z=A3)
        a.update(kw)
        return f(a["w"], a["dt"], a["N"], a["K"], a["s"], a["g"], a["bits"], a["sym"], a["q"], a["sc"],
                 a["z"], NULL)

    assert call(N=0, w=NULL, q=NULL) == 0        # no-op
    assert call(w=NULL) == 1
    assert call(z=NULL) == 1
    assert call(dt=E.AWQ_F32) == 3
    assert call(K=448) == 2
    assert call(N=-1) == 2
    assert call(g=96) == 5
    assert call(bits=1) == 5
    assert call(bits=8, sym=1) == 5
    assert call(bits=9) == 5
    assert call(q=ctypes.c_void_p(0x20008)) == 4  # codes 16-byte aligned
    assert call(w=BAD) == 4
    assert call(s=BAD) == 4


def test_salient_validation():
    lib = _lib()
    f = lib.awq_salient_channels
    assert f(NULL, 512, 5, A2, NULL) == 1
    assert f(A, 512, 5, NULL, NULL) == 1
    assert f(A, 0, 0, A2, NULL) == 2
    assert f(A, 512, -1, A2, NULL) == 2
    assert f(A, 512, 513, A2, NULL) == 2
    assert f(ctypes.c_void_p(0x10002), 512, 5, A2, NULL) == 4
    assert f(A, 1 << 20, 5, A2, NULL) == 5


def test_gemm_validation():
    lib = _lib()
    f = lib.awq_w4a16_gemm

    def call(**kw):
        a = dict(x=A, xdt=E.AWQ_F16, M=1, K=4096, ldx=4096, q=A2, sc=A3, z=A3, N=11008, g=128,
                 r=NULL, y=A2, ydt=E.AWQ_F16, ldy=11008)
        a.update(kw)
        return f(a["x"], a["xdt"], a["M"], a["K"], a["ldx"], a["q"], a["sc"], a["z"], a["N"], a["g"],
                 a["r"], a["y"], a["ydt"], a["ldy"], NULL, 0, NULL)

    assert call(M=0, x=NULL) == 0          # empty input: no-op
    assert call(N=0, ldy=0, q=NULL) == 0
    assert call(x=NULL) == 1
    assert call(y=NULL) == 1
    assert call(xdt=E.AWQ_F32) == 3
    assert call(ydt=7) == 3
    assert call(K=4000, ldx=4000) == 2
    assert call(ldy=100) == 2
    assert call(M=-1) == 2
    assert call(g=32) == 5
    assert call(g=256, K=4224, ldx=4224) == 2   # K % group
    assert call(x=BAD) == 4
    assert call(ldx=4100) == 4
    assert call(r=BAD) == 4


def test_fold_validation():
    lib = _lib()
    E = abi
    f = lib.awq_fold_scales
    NULL = None
    A = ctypes.c_void_p(1 << 20)          # never dereferenced: every case fails on the host
    S = ctypes.c_void_p(1 << 21)
    assert f(A, 7, 4, 8, 8, S, 1, NULL) == 3                 # dtype
    assert f(A, E.AWQ_F16, 4, 8, 7, S, 1, NULL) == 2         # ld < cols
    assert f(A, E.AWQ_F16, -1, 8, 8, S, 1, NULL) == 2        # negative rows
    assert f(A, E.AWQ_F16, 4, 8, 8, S, 2, NULL) == 2         # axis
    assert f(NULL, E.AWQ_F16, 4, 8, 8, S, 1, NULL) == 1
    assert f(A, E.AWQ_F16, 4, 8, 8, NULL, 0, NULL) == 1
    assert f(ctypes.c_void_p((1 << 20) + 1), E.AWQ_F16, 4, 8, 8, S, 1, NULL) == 4   # odd address
    assert f(ctypes.c_void_p((1 << 20) + 2), E.AWQ_F32, 4, 8, 8, S, 1, NULL) == 4
    assert f(NULL, E.AWQ_F16, 0, 8, 8, NULL, 1, NULL) == 0   # empty: no-op



def test_gemm_noalloc_validation():
    """awq_w4a16_gemm_noalloc rejects bad arguments on the host, and sizes
    whose scratch exceeds the library's array, before any launch."""
    lib = _lib()
    f = lib.awq_w4a16_gemm_noalloc

    def call(**kw):
        a = dict(x=A, xdt=E.AWQ_F16, M=1, K=4096, ldx=4096, q=A2, sc=A3, z=A3, N=11008, g=128,
                 r=NULL, y=A2, ydt=E.AWQ_F16, ldy=11008)
        a.update(kw)
        return f(a["x"], a["xdt"], a["M"], a["K"], a["ldx"], a["q"], a["sc"], a["z"], a["N"], a["g"],
                 a["r"], a["y"], a["ydt"], a["ldy"], NULL)

    assert call(M=0, x=NULL) == 0
    assert call(x=NULL) == 1
    assert call(xdt=E.AWQ_F32) == 3
    assert call(K=4000, ldx=4000) == 2
    assert call(g=32) == 5
    assert call(x=BAD) == 4
    # 2048 tokens, 28672 -> 8192, groups of 64: about 147 MB of scratch
    assert call(M=2048, K=28672, ldx=28672, N=8192, ldy=8192, g=64, xdt=E.AWQ_BF16) == 5
    assert abi.AWQ_NOALLOC_SCRATCH_BYTES == 128 << 20


def test_read_stream_validation():
    """awq_read_stream (the streaming-read diagnostic) rejects bad arguments on
    the host before any launch."""
    lib = _lib()
    f = lib.awq_read_stream
    assert f(NULL, 1024, 256, 4, A, NULL) == 1
    assert f(A, 1024, 256, 4, NULL, NULL) == 1
    assert f(A, 0, 256, 4, A, NULL) == 2
    assert f(A, 1000, 256, 4, A, NULL) == 2
    assert f(A, 1024, 0, 4, A, NULL) == 2
    assert f(A, 1024, 65536, 4, A, NULL) == 2
    assert f(A, 1024, 256, 3, A, NULL) == 5
    assert f(BAD, 1024, 256, 4, A, NULL) == 4

