"""GPU parity of mxfp4_matvec / mxfp4_gemm against the fp64 oracle.

Pass rule: |y - y_oracle| <= 1e-4 * sum|w*x| + 1e-30 per output.  Shapes:
the five measured workloads (every output at full size),
the pages' adversarial shapes (300 x 2304, 70000 x 64, 5 x 5120), ragged
rows and columns, bf16 activations and outputs.  Invariants: a batch equals
its tokens' matvecs bit for bit (b in 2, 8, 9, 19 as in the pages' device
test), permuting tokens permutes outputs bit for bit, reruns are bitwise
equal, NaN scales give NaN rows, writes stay inside y.
"""
import numpy as np
import pytest
import torch

from gemm_mxfp4_dequant_amd import inputs
from tests.helpers import assert_within, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    from gemm_mxfp4_dequant_amd import mxfp4
    mxfp4.lib()
    return mxfp4


def run(m, w, rows, cols, x, y_dtype=torch.float32):
    xd = dev(x)
    y = m.mxfp4_gemm(dev(w), rows, cols, xd, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return host(y)


def check(m, orc, rows, cols, b, seed, lo=118, hi=132, xdt="f32", what=""):
    w, x = inputs.gemm_case(seed, rows, cols, b, lo, hi, xdt)
    y = run(m, w, rows, cols, x)
    want, mag = orc.gemm(w, rows, cols, x)
    return assert_within(y, want, mag, what=what or f"{rows}x{cols} b={b}")


def test_workload1_matvec(m, orc):
    w, x = inputs.workload_case(1)
    xd = dev(x[0])
    y = host(m.mxfp4_matvec(dev(w), 256, 512, xd))
    want, mag = orc.gemm(w, 256, 512, x)
    assert_within(y, want[0], mag[0], what="256x512 matvec")


@pytest.mark.parametrize("b", [1, 8])
def test_workload2_full(m, orc, b):
    check(m, orc, 4096, 4096, b, 2)


@pytest.fixture(scope="module")
def workload3():
    """14336 x 4096 with 32 tokens, and the oracle's every output for them
    (the smaller batches are the first b tokens: each output row depends on
    its own token only)."""
    import oracle
    rows, cols = 14336, 4096
    w, x = inputs.gemm_case(3, rows, cols, 32)
    want, mag = oracle.gemm(w, rows, cols, x)
    return w, x, want, mag


@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 32])
def test_workload3_every_row(m, workload3, b):
    """14336 x 4096 at b = 1, 2, 4, 8 (skinny kernels) and 16, 32 (tiled):
    every output of every token against the oracle."""
    rows, cols = 14336, 4096
    w, x, want, mag = workload3
    y = run(m, w, rows, cols, x[:b])
    assert_within(y, want[:b], mag[:b], what=f"14336x4096 b={b}")


@pytest.mark.parametrize("rows,cols", [(300, 2304), (70000, 64), (5, 5120), (1, 32), (17, 96),
                                       (64, 512), (65, 1024), (129, 7168), (33, 2048)])
@pytest.mark.parametrize("b", [1, 3, 8, 9])
def test_shapes(m, orc, rows, cols, b):
    check(m, orc, rows, cols, b, rows + cols + b)


@pytest.mark.parametrize("b", [1, 7, 16, 17, 40])
def test_bf16_activations(m, orc, b):
    check(m, orc, 200, 2048, b, 50 + b, xdt="bf16")
    check(m, orc, 70, 4096, b, 60 + b, xdt="bf16")


def test_bf16_output(m, orc):
    rows, cols, b = 96, 1024, 5
    w, x = inputs.gemm_case(7, rows, cols, b)
    y = run(m, w, rows, cols, x, torch.bfloat16)
    want, mag = orc.gemm(w, rows, cols, x)
    yf = (y.astype(np.uint32) << 16).view(np.float32)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-38))) - 7)
    assert_within(yf, want, mag, extra=ulp, what="bf16 out")


def test_wide_scale_range(m, orc):
    """Scales across most of E8M0 (outputs span many binades; the rule is
    relative to each output's own magnitude sum)."""
    check(m, orc, 128, 1024, 4, 11, lo=60, hi=190)


@pytest.mark.parametrize("b,xdt", [(9, "f32"), (23, "f32"), (40, "f32"), (17, "bf16"),
                                   (40, "bf16"), (64, "bf16")])
def test_tiled_shapes(m, orc, b, xdt):
    """Enough row blocks for the tiled kernel (12300 rows, a ragged last
    block), 1 to 4 column tiles in use, bf16 activations and fp32 ones
    (split into hi / lo rows once per K step)."""
    check(m, orc, 12300, 1024, b, 700 + b, xdt=xdt)


def test_many_row_blocks_per_workgroup(m, orc):
    """Tall, narrow weights with 40 tokens: enough workgroups that each one
    walks several row blocks (ragged last block)."""
    check(m, orc, 65553, 512, 40, 31)


@pytest.mark.parametrize("b", [1, 3])
def test_row_walk_odd_block_count(m, orc, b):
    """65552 rows = 4097 blocks of 16, walked two per workgroup: the last
    workgroup has a single block (the walk's prefetch and double-buffered
    reduction end early)."""
    check(m, orc, 65552, 512, b, 60 + b)


@pytest.mark.parametrize("rows,cols", [(300, 2304), (5, 5120), (128, 4096), (64, 7168),
                                       (14336, 4096), (200, 1024), (65553, 512)])
def test_batch_equals_matvec_bitwise(m, rows, cols):
    """Every token of a batch equals its own matvec bit for bit, for one and
    several token chunks, with and without row-block walking, and every launch
    shape: all kernels sum in one canonical order."""
    w, x = inputs.gemm_case(rows + cols, rows, cols, 40)
    wd = dev(w)
    for b in (2, 8, 9, 19, 40):
        xb = dev(x[:b])
        yb = host(m.mxfp4_gemm(wd, rows, cols, xb))
        for t in range(b):
            y1 = host(m.mxfp4_matvec(wd, rows, cols, dev(x[t])))
            assert np.array_equal(y1.view(np.uint32), yb[t].view(np.uint32)), (b, t)


@pytest.mark.parametrize("rows,cols", [(256, 4096), (96, 2048), (12300, 1024)])
def test_bf16_batch_equals_single_bitwise(m, rows, cols):
    w, x = inputs.gemm_case(rows + 7, rows, cols, 70, x_dtype="bf16")
    wd = dev(w)
    xd = dev(x)
    y1 = [host(m.mxfp4_gemm(wd, rows, cols, xd[t:t + 1])) for t in range(70)]
    for b in (3, 16, 17, 70):
        yb = host(m.mxfp4_gemm(wd, rows, cols, xd[:b]))
        for t in range(b):
            assert np.array_equal(y1[t][0].view(np.uint32), yb[t].view(np.uint32)), (b, t)


def test_permuted_tokens_permute_outputs(m):
    rows, cols, b = 256, 4096, 8
    w, x = inputs.gemm_case(21, rows, cols, b)
    perm = np.random.default_rng(0).permutation(b)
    y = run(m, w, rows, cols, x)
    yp = run(m, w, rows, cols, x[perm])
    assert np.array_equal(yp.view(np.uint32), y[perm].view(np.uint32))


def test_rerun_bitwise(m):
    rows, cols, b = 14336, 4096, 8
    w, x = inputs.gemm_case(22, rows, cols, b)
    wd, xd = dev(w), dev(x)
    y1 = host(m.mxfp4_gemm(wd, rows, cols, xd))
    y2 = host(m.mxfp4_gemm(wd, rows, cols, xd))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_nan_scale_gives_nan_row(m, orc):
    rows, cols = 40, 1024
    w, x = inputs.gemm_case(23, rows, cols, 2)
    w = w.copy()
    w[rows * cols // 2 + 17 * (cols // 32) + 5] = 255  # row 17, group 5
    y = run(m, w, rows, cols, x)
    want, mag = orc.gemm(w, rows, cols, x)
    assert np.all(np.isnan(y[:, 17]))
    assert_within(y, want, mag, what="nan row")


def test_guard_band(m):
    rows, cols, b = 70, 512, 3
    w, x = inputs.gemm_case(24, rows, cols, b)
    buf = torch.full((b * rows + 64,), 777.0, device="cuda")
    y = buf[32:32 + b * rows].view(b, rows)
    m.mxfp4_gemm(dev(w), rows, cols, dev(x), y=y)
    hb = host(buf)
    assert np.all(hb[:32] == 777.0) and np.all(hb[-32:] == 777.0)
    assert not np.any(hb[32:-32] == 777.0)


@pytest.mark.parametrize("rows,cols,b", [(64, 1024, 4), (12300, 512, 9)])
def test_huge_and_infinite_activations(m, orc, rows, cols, b):
    """fp32 activations beyond the bf16 range, up to the fp32 maximum (a
    nearest-even bf16 of these would be infinite; the library's hi / lo
    split truncates hi, so the products stay finite and within the
    tolerance), and the documented behaviour of an infinite activation:
    every output of its token is NaN.  Skinny kernel (64 rows) and tiled
    kernel (12300 rows, b = 9)."""
    w, x = inputs.gemm_case(25 + b, rows, cols, b, 118, 122)
    x = x.copy()
    x[0, 3] = np.float32(3.4e38)         # nearest bf16 overflows
    x[0, 400] = np.float32(-3.4028235e38)  # fp32 maximum
    x[1, 10] = np.float32(3.3e38)         # within the bf16 range
    x[1, 11] = np.float32(3.3961514e38)   # exactly the bf16 overflow threshold
    x[2, 5] = np.inf
    x[3, 300] = -np.inf
    y = run(m, w, rows, cols, x)
    fin_tok = [t for t in range(b) if np.all(np.isfinite(x[t]))]
    want, mag = orc.gemm(w, rows, cols, x[fin_tok])
    assert np.all(np.isfinite(want[:2]))
    assert_within(y[fin_tok], want, mag, what="huge finite activations")
    assert np.all(np.isnan(y[2])) and np.all(np.isnan(y[3])), "infinite activation"


def rows_subtensor(w, rows, cols, sel):
    """The stored tensor of the rows ``sel`` of a rows x cols tensor (each
    plane's rows taken in the same order)."""
    cb = rows * cols // 2
    codes = w[:cb].reshape(rows, cols // 2)[sel]
    scales = w[cb:cb + rows * (cols // 32)].reshape(rows, cols // 32)[sel]
    return np.concatenate([codes.ravel(), scales.ravel()])


@pytest.mark.parametrize("rows,cols,b", [(1 << 24, 32, 1), (1 << 24, 32, 8),
                                         (246723, 16384, 1), (246723, 16384, 8)])
def test_maximum_sizes(m, orc, rows, cols, b):
    """The largest accepted tensors: MXFP4_MAX_ROWS rows at the narrowest
    width, and MXFP4_MAX_COLS columns at the largest row count whose tensor
    fits MXFP4_MAX_TENSOR_BYTES (246723 x 16384: 2,147,476,992 bytes; one
    more row is refused).  Every token of the first and last rows, the
    16-row tile and chunk boundaries and 200 seeded random rows against the
    oracle on a tensor of just those rows."""
    assert m.mxfp4_nbytes(rows, cols) <= 1 << 31
    w, x = inputs.gemm_case(880 + b + cols, rows, cols, b)
    y = run(m, w, rows, cols, x)
    rng = np.random.default_rng(rows + b)
    sel = np.unique(np.concatenate([[0, 1, 15, 16, 17, 63, 64, rows // 2, rows - 17, rows - 16,
                                     rows - 2, rows - 1], rng.integers(0, rows, 200)]))
    want, mag = orc.gemm(rows_subtensor(w, rows, cols, sel), len(sel), cols, x)
    assert_within(y[:, sel], want, mag, what=f"{rows}x{cols} b={b}, {len(sel)} rows")


def onehot_weights(rows, cols):
    """Row r holds +1 (E2M1 code 2 under scale 2^0) in column r % cols and
    zeros elsewhere (codes low nibble first)."""
    codes = np.zeros((rows, cols), np.uint8)
    codes[np.arange(rows), np.arange(rows) % cols] = 2
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = np.full((rows, cols // 32), 127, np.uint8)
    return np.concatenate([packed.ravel(), scales.ravel()])


@pytest.mark.parametrize("rows,cols,b", [(64, 64, 1), (300, 96, 5), (512, 512, 8),
                                         (4096, 1024, 3), (24576, 512, 32), (14336, 4096, 16)])
def test_activation_split_bitwise(m, rows, cols, b):
    """One-hot weights make every output a single fp32 activation carried
    through the kernels' split: hi = x truncated to bf16, lo = the nearest
    bf16 to x - hi (exact in fp32), y = hi + lo (exact in fp32), so
    |y - x| < 2^-15 |x|.  Checked bit for bit on the generic (96 columns),
    split-K (GEMV and GEMM) and tiled (b = 16, 32) kernels, with activations
    of every binade from 2^-100 to 2^100 and low mantissa bits all ones."""
    rng = np.random.default_rng(rows + b)
    x = (rng.standard_normal((b, cols)) * np.exp2(rng.integers(-100, 100, (b, cols)))).astype(
        np.float32)
    # every 7th activation: low 16 mantissa bits all ones (the split's
    # largest error), random sign, top mantissa bits and normal exponent
    n = x[:, ::7].size
    bits = ((rng.integers(0, 2, n, dtype=np.uint32) << np.uint32(31))
            | (rng.integers(27, 227, n, dtype=np.uint32) << np.uint32(23))
            | (rng.integers(0, 128, n, dtype=np.uint32) << np.uint32(16)) | np.uint32(0xFFFF))
    x[:, ::7] = bits.view(np.float32).reshape(x[:, ::7].shape)
    xb = x.view(np.uint32)
    hi = (xb & np.uint32(0xFFFF0000)).view(np.float32)
    rest = (x - hi).astype(np.float32)
    lo = torch.from_numpy(rest).to(torch.bfloat16).to(torch.float32).numpy()
    want = (hi + lo).astype(np.float32)
    assert np.all(np.abs(want - x) < np.ldexp(np.abs(x), -15))
    y = run(m, onehot_weights(rows, cols), rows, cols, x)
    exp = want[:, np.arange(rows) % cols]
    assert np.array_equal(y.view(np.uint32), exp.view(np.uint32)), \
        int(np.count_nonzero(y.view(np.uint32) != exp.view(np.uint32)))
