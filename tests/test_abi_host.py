"""Host-side checks of the C ABI (no GPU needed).

The library loads, exports every function declared in include/mxfp4.h, and
refuses bad arguments before touching the GPU (every check runs on the host
ahead of any HIP call), in the manner of the pages' entry points ("cortiq-
engine 0.8.40, src/gpu_wgpu/mxfp4.rs", matmat: b == 0, rows == 0,
cols % 32 != 0, wrong dtype/shape are refused).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp4.h")
LIB = os.path.join(ROOT, "gemm_mxfp4_dequant_amd", "libmxfp4.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmxfp4.so not built")


def declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|int64_t|size_t|char)\s*\*?\s*(\w+)\s*\(", src,
                       flags=re.M)
    return names


@pytest.fixture(scope="module")
def m():
    from gemm_mxfp4_dequant_amd import mxfp4
    mxfp4.lib()
    return mxfp4


def test_exports_every_declared_symbol(m):
    names = declared_functions()
    assert len(names) == 21, names
    L = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(L, n), n


def test_exports_every_symbol_of_every_header(m):
    """Every header under include/ (the boundary and the measurement helper)
    declares only functions the library exports."""
    L = ctypes.CDLL(LIB)
    inc = os.path.join(ROOT, "include")
    seen = 0
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            for n in declared_functions(os.path.join(inc, h)):
                assert hasattr(L, n), (h, n)
                seen += 1
    assert seen >= 14


def test_probe_refusals(m):
    f = ctypes.CDLL(LIB).mxfp4_probe_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p]
    assert f(None, 1024, 8, FAKE, None) == -1
    assert f(FAKE, 1000, 8, FAKE, None) == -1     # not a multiple of 16
    assert f(FAKE, 1024, 5, FAKE, None) == -1     # loads per thread
    assert f(FAKE + 8, 1024, 8, FAKE, None) == -1  # alignment
    assert f(FAKE, 1024, 8, None, None) == -1


def test_no_undefined_library_symbols():
    """Every kernel the library launches is defined in it: a kernel template
    whose host stub the compiler dropped shows up here as an undefined mx::
    symbol, long before a GPU run would fail to load the library."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "-C", "--undefined-only", LIB], capture_output=True,
                         text=True, check=True).stdout
    bad = [l for l in out.splitlines() if "mx::" in l]
    assert not bad, bad


def test_nbytes(m):
    assert m.mxfp4_nbytes(2304, 5120) == 2304 * 5120 * 17 // 32
    assert m.mxfp4_nbytes(1, 32) == 17
    assert m.mxfp4_nbytes(4, 48) == -1
    assert m.mxfp4_nbytes(-1, 32) == -1


FAKE = 0x100000  # 16-byte aligned, never dereferenced: calls below are refused first


def status(fn, *args):
    return fn(*args)


@pytest.mark.parametrize("rows,cols,b,xdt,ydt,expect", [
    (0, 64, 1, 0, 0, -1),        # rows == 0
    (16, 48, 1, 0, 0, -1),       # cols % 32
    (16, 0, 1, 0, 0, -1),
    (16, 64, 0, 0, 0, -1),       # b == 0
    (16, 64, 1, 2, 0, -1),       # bad x dtype
    (16, 64, 1, 0, 7, -1),       # bad y dtype
    (16, 1 << 15, 1, 0, 0, -1),  # cols above the cap
    ((1 << 24) + 1, 32, 1, 0, 0, -1),  # rows above the cap
    (246724, 16384, 1, 0, 0, -1),      # tensor bytes above the cap (246723 rows fit)
    (16, 64, (1 << 20) + 1, 0, 0, -1),  # tokens above the cap
])
def test_gemm_refusals(m, rows, cols, b, xdt, ydt, expect):
    L = m.lib()
    assert L.mxfp4_gemm(FAKE, rows, cols, FAKE, xdt, b, FAKE, ydt, None) == expect
    assert m.mxfp4_last_error() != ""


def test_alignment_and_null(m):
    L = m.lib()
    assert L.mxfp4_gemm(FAKE + 4, 16, 64, FAKE, 0, 1, FAKE, 0, None) == m.MXFP4_EALIGN
    assert L.mxfp4_gemm(None, 16, 64, FAKE, 0, 1, FAKE, 0, None) == m.MXFP4_EINVAL
    assert L.mxfp4_gemm(FAKE, 16, 64, FAKE + 8, 0, 1, FAKE, 0, None) == m.MXFP4_EALIGN
    assert L.mxfp4_matvec(FAKE, 16, 64, None, FAKE, None) == m.MXFP4_EINVAL
    assert L.mxfp4_dequant(FAKE, 16, 64, FAKE, 3, None) == m.MXFP4_EINVAL
    assert L.mxfp4_dequant(FAKE, 16, 40, FAKE, 0, None) == m.MXFP4_EINVAL
    assert "cols" in m.mxfp4_last_error()


def test_moe_refusals(m):
    L = m.lib()
    ws = m.moe_experts_mxfp4_workspace_size(8, 6, 64, 4096, 2048, 0)
    assert ws > 8 * 6 * 4096 * 4
    assert m.moe_experts_mxfp4_workspace_size(8, 6, 64, 4096, 2000, 0) == 0
    args = dict(E=64, H=4096, I=2048, T=8, K=6)

    def call(E=64, H=4096, I=2048, T=8, K=6, ws_bytes=ws, xdt=0, odt=1, wsp=FAKE, ids=FAKE):
        return L.moe_experts_mxfp4(FAKE, FAKE, FAKE, E, H, I, FAKE, xdt, T, ids, FAKE, K, FAKE,
                                   odt, wsp, ws_bytes, None)

    assert call(K=65) == m.MXFP4_EINVAL           # top_k > n_experts
    assert call(E=0) == m.MXFP4_EINVAL
    assert call(T=0) == m.MXFP4_EINVAL            # empty
    assert call(I=2000) == m.MXFP4_EINVAL         # inter % 32
    assert call(ws_bytes=ws - 1) == m.MXFP4_EWORKSPACE
    assert call(wsp=FAKE + 4) == m.MXFP4_EALIGN
    assert call(ids=FAKE + 2) == m.MXFP4_EALIGN
    assert call(xdt=5) == m.MXFP4_EINVAL
    assert args


def test_moe_a8_refusals(m):
    """The FP4 x FP8 expert bank sizes its own workspace (the plain bank's
    with h in fp32, plus the MXFP8 codes and scales of x and h), needs hidden
    and inter in multiples of 512, and refuses like the plain bank before
    any launch."""
    L = m.lib()
    T, K, E, H, I = 512, 8, 256, 7168, 2048
    ws = m.moe_experts_mxfp4_a8_workspace_size(T, K, E, H, I)
    base = m.moe_experts_mxfp4_workspace_size(T, K, E, H, I, 0)
    assert ws >= base + T * H + T * H // 32 + T * K * I + T * K * I // 32
    assert m.moe_experts_mxfp4_a8_workspace_size(T, K, E, 7168 - 32, I) == 0
    assert m.moe_experts_mxfp4_a8_workspace_size(T, K, E, H, 2048 + 256) == 0
    assert m.moe_experts_mxfp4_a8_workspace_size(0, K, E, H, I) == 0

    def call(E=E, H=H, I=I, K=K, ws_bytes=ws, wsp=FAKE, xdt=1):
        return L.moe_experts_mxfp4_a8(FAKE, FAKE, FAKE, E, H, I, FAKE, xdt, T, FAKE, FAKE, K,
                                      FAKE, 1, wsp, ws_bytes, None)

    assert call(H=7168 - 32) == m.MXFP4_EINVAL      # hidden % 512
    assert "512" in m.mxfp4_last_error()
    assert call(I=2048 + 256) == m.MXFP4_EINVAL     # inter % 512
    assert call(ws_bytes=ws - 1) == m.MXFP4_EWORKSPACE
    assert call(wsp=FAKE + 4) == m.MXFP4_EALIGN
    assert call(K=257) == m.MXFP4_EINVAL
    assert call(xdt=7) == m.MXFP4_EINVAL


def test_v41_refusals(m):
    """The V4.1 bank refuses a negative or non-finite limit, has_shared
    outside {0, 1}, and a workspace sized without the shared expert's slot."""
    L = m.lib()
    ws0 = m.moe_experts_mxfp4_v41_workspace_size(16, 8, 256, 1024, 512, 0)
    ws1 = m.moe_experts_mxfp4_v41_workspace_size(16, 8, 256, 1024, 512, 1)
    assert ws1 > ws0 > 0
    assert m.moe_experts_mxfp4_v41_workspace_size(16, 8, 256, 1024, 512, 2) == 0

    def call(lim=10.0, shared=1, ws_bytes=ws1, K=8, E=256):
        return L.moe_experts_mxfp4_v41(FAKE, FAKE, FAKE, E, 1024, 512, FAKE, 16, FAKE, FAKE, K,
                                       lim, shared, FAKE, FAKE, ws_bytes, None)

    assert call(lim=-1.0) == m.MXFP4_EINVAL
    assert call(lim=float("nan")) == m.MXFP4_EINVAL
    assert call(lim=float("inf")) == m.MXFP4_EINVAL
    assert call(shared=2) == m.MXFP4_EINVAL
    assert call(ws_bytes=ws0) == m.MXFP4_EWORKSPACE   # no room for the shared slot
    assert call(K=257) == m.MXFP4_EINVAL
    assert call(K=32, E=256) == m.MXFP4_EINVAL         # 32 routed + 1 shared > 32 slots
    r = L.moe_experts_mxfp4_v41_stages(FAKE, FAKE, FAKE, 256, 1024, 512, FAKE, 16, FAKE, FAKE, 8,
                                       10.0, 1, None, FAKE, ws1, None, None, None)
    assert r == m.MXFP4_EINVAL                          # nothing requested


def test_router_refusals(m):
    """The router refuses top_k above n_experts or 32, n_experts outside
    [1, 1024], no tokens, and unaligned pointers, before any launch."""
    L = m.lib()

    def call(T=8, E=64, K=6, logits=FAKE, ids=FAKE, w=FAKE):
        return L.moe_route_topk(logits, T, E, K, ids, w, None)

    assert call(K=65) == m.MXFP4_EINVAL
    assert "top_k" in m.mxfp4_last_error()
    assert call(K=33, E=64) == m.MXFP4_EINVAL
    assert call(K=0) == m.MXFP4_EINVAL
    assert call(E=1025, K=8) == m.MXFP4_EINVAL
    assert call(E=0, K=1) == m.MXFP4_EINVAL
    assert call(T=0) == m.MXFP4_EINVAL
    assert call(logits=None) == m.MXFP4_EINVAL
    assert call(ids=FAKE + 2) == m.MXFP4_EALIGN


def test_v41_slot_cap(m):
    """V4.1: top_k + has_shared slots per token, at most MXFP4_MAX_TOP_K."""
    L = m.lib()
    assert m.moe_experts_mxfp4_v41_workspace_size(4, 31, 40, 512, 256, True) > 0
    assert m.moe_experts_mxfp4_v41_workspace_size(4, 32, 40, 512, 256, False) > 0
    assert m.moe_experts_mxfp4_v41_workspace_size(4, 32, 40, 512, 256, True) == 0
    ws = m.moe_experts_mxfp4_v41_workspace_size(4, 31, 40, 512, 256, True)
    r = L.moe_experts_mxfp4_v41(FAKE, FAKE, FAKE, 40, 512, 256, FAKE, 4, FAKE, FAKE, 32, 0.0, 1,
                                FAKE, FAKE, ws * 2, None)
    assert r == m.MXFP4_EINVAL
    assert "top_k" in m.mxfp4_last_error()


def test_stage_refusals(m):
    L = m.lib()
    ws = m.moe_experts_mxfp4_workspace_size(4, 2, 8, 512, 256, 0)
    r = L.moe_experts_mxfp4_stages(FAKE, FAKE, FAKE, 8, 512, 256, FAKE, 0, 4, FAKE, FAKE, 2,
                                   None, 1, FAKE, ws, None, None, None)
    assert r == m.MXFP4_EINVAL  # nothing requested
    r = L.moe_experts_mxfp4_stages(FAKE, FAKE, FAKE, 8, 512, 256, FAKE, 0, 4, FAKE, FAKE, 2,
                                   FAKE, 1, FAKE, ws, FAKE, FAKE, None)
    assert r == m.MXFP4_EINVAL  # h_in and h_out together


def test_group_refusals(m):
    L = m.lib()
    assert L.moe_route_group(FAKE, 4, 2, 0, FAKE, FAKE, FAKE, None) == m.MXFP4_EINVAL
    assert L.moe_route_group(FAKE, 4, 0, 8, FAKE, FAKE, FAKE, None) == m.MXFP4_EINVAL
    assert L.moe_route_group(FAKE + 1, 4, 2, 8, FAKE, FAKE, FAKE, None) == m.MXFP4_EALIGN


def test_noalloc_refusals_before_any_launch():
    """The allocation-free expert bank refuses, on the host and before any
    HIP call, sizes whose scratch exceeds its static array, and the usual
    bad arguments."""
    L = ctypes.CDLL(LIB)
    f = L.moe_experts_mxfp4_noalloc
    f.restype = ctypes.c_int
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    f.argtypes = [P, P, P, I64, I64, I64, P, I, I64, P, P, I64, P, I, P]
    err = L.mxfp4_last_error
    err.restype = ctypes.c_char_p
    # the 512-token prefill layer: 134 MB of scratch
    assert f(FAKE, FAKE, FAKE, 256, 7168, 2048, FAKE, 1, 512, FAKE, FAKE, 8, FAKE, 1, None) == -3
    assert b"static scratch" in err()
    assert f(FAKE, FAKE, FAKE, 0, 4096, 2048, FAKE, 0, 8, FAKE, FAKE, 6, FAKE, 1, None) == -1
    assert f(FAKE, FAKE, FAKE, 64, 4096, 2048, FAKE, 0, 8, FAKE, FAKE, 6, None, 1, None) == -1
    assert f(FAKE, FAKE, FAKE, 64, 4096, 2048, FAKE + 4, 0, 8, FAKE, FAKE, 6, FAKE, 1,
             None) == -2
