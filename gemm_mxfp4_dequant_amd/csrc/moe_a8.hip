// Routed expert bank on the block-scaled FP4 x FP8 product: the opt-in
// path for dense prefill experts, with the activations quantized to MXFP8
// (E4M3 elements, one E8M0 scale per 32: the OCP MX family that
// "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs" names in its module doc) and
// the expert products on v_mfma_scale_f32_16x16x128_f8f6f4, which takes the
// weights as stored.  What is computed is the expert bank of
// "cortiq-engine 0.8.77, src/qtensor/moe_fast.rs" (gate_up_block,
// down_block) with x and h quantized before their products.
//
// One kernel serves gate/up (two matrices, SwiGLU epilogue, h in fp32) and
// down (y in fp32), for work items of up to 64 tokens of one expert:
//  * a workgroup of 8 waves owns 128 rows of every matrix of the mode (a
//    16-row tile per wave and matrix) and the item's tokens in 4 tiles of 16;
//  * codes: a pair of 128-column steps per load, each tile's 16 rows as two
//    1 KB loads of 8 rows x 128 contiguous bytes (whole cache lines) into
//    per-wave pair buffers chosen by pair parity, the pair's 16-byte piece p
//    of row r at position p ^ ((r / 2) & 7) so that the sixteen lanes reading
//    one A fragment hit distinct banks; a pair goes out two steps before its
//    first step;
//  * activations: a ring of four LDS stages, one per step, each holding the
//    step's 64 tokens x 128 E4M3 bytes (chunk k of token t at position
//    k ^ (t & 7)), gathered by direct global -> LDS loads three steps ahead;
//  * scales: with a unit's first step one load per wave brings the unit's
//    16 scale bytes of its rows in each matrix (lanes 16 m .. 16 m + 15) and
//    of one token tile's tokens (the remaining lanes); the waves copy them to
//    registers at that step;
//  * every wave issues the same loads at the same place of each unit, so a
//    constant vmcnt per place says "this step's operands have landed", then
//    one barrier per step.
// Each accumulator takes the steps in ascending order.
#include "device.h"
#include "launch.h"

namespace mx {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int MA_NW = 8; // waves; 16-row tiles of every matrix
constexpr int MA_NC = 4; // token tiles of 16

template <int N> struct MaTag {
    static constexpr int value = N;
};

template <int MODE>
__global__ __launch_bounds__(MA_NW * 64) void moe_a8_kernel(MoeA8Args a)
{
    constexpr int NMAT = MODE == MODE_GATEUP ? 2 : 1;
    constexpr int NW = MA_NW, NC = MA_NC;
    constexpr int SLAB = NC * 16 * 128; // one step's 64 tokens x 128 E4M3 bytes
    static_assert(SLAB == NW * 1024, "one slab load per wave and step");
    static_assert(NMAT + 1 <= 4, "one scale load per wave covers the matrices and a token tile");

    // one variable per buffer: loads into one and reads of another are then
    // known not to alias, and the compiler adds no waits of its own
    __shared__ __align__(16) uint8_t st0[SLAB], st1[SLAB], st2[SLAB], st3[SLAB];
    __shared__ __align__(16) uint8_t pb0[NW * NMAT * 2048], pb1[NW * NMAT * 2048];
    __shared__ __align__(16) uint8_t scs[NW * 1024];
    auto stage = [&] __device__(auto tag) -> uint8_t * {
        constexpr int k = decltype(tag)::value;
        if constexpr (k == 0)
            return st0;
        else if constexpr (k == 1)
            return st1;
        else if constexpr (k == 2)
            return st2;
        else
            return st3;
    };
    auto pairbuf = [&] __device__(auto tag) -> uint8_t * {
        if constexpr (decltype(tag)::value == 0)
            return pb0;
        else
            return pb1;
    };

    const int C = a.cols, R = a.rows;
    const int gpr = C / 32;
    const int nunits = C / 512;
    const int nsteps = nunits * 4;
    const int npairs = nsteps / 2;
    // work item and row block: dispatch order, row blocks fastest (an
    // item's blocks run together); the grid is sized by an upper bound on
    // the items and the surplus, dispatched last, exits
    const int nrb = (R + NW * 16 - 1) / (NW * 16);
    if ((int)blockIdx.x >= *a.n_work * nrb)
        return;
    const int sub = (int)blockIdx.x / nrb;
    const int row0 = ((int)blockIdx.x % nrb) * (NW * 16);
    const int4 wk = reinterpret_cast<const int4 *>(a.work)[sub];
    const int expert = wk.x, slot0 = wk.y, ntok = wk.z;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, ls = lane >> 4;
    const int64_t code_bytes = (int64_t)R * (C / 2);
    const uint8_t *Am[NMAT];
    Am[0] = a.w0 + (int64_t)expert * a.expert_stride;
    if constexpr (NMAT == 2)
        Am[1] = a.w1 + (int64_t)expert * a.expert_stride;
    // activation row of item token t (tokens past the item read its last:
    // never stored, and an MFMA output column depends on its own token only)
    auto xrow = [&] __device__(int t) -> int64_t {
        const int tc = min(t, ntok - 1);
        return MODE == MODE_GATEUP ? (int64_t)a.token_of_slot[slot0 + tc] : (int64_t)(slot0 + tc);
    };

    // ---- per-lane load sources (rows past the end read row R - 1: never
    // stored, and an MFMA output row depends on its own A row only)
    const uint8_t *csrc[NMAT][2];
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int lr = 8 * i + (lane >> 3);
            const int r = min(row0 + wave * 16 + lr, R - 1);
            csrc[mt][i] = Am[mt] + (int64_t)r * (C / 2) + ((lane & 7) ^ ((lr >> 1) & 7)) * 16;
        }
    // slab: this lane's 16-byte position of the step's slab
    const int pos = wave * 64 + lane, tt = pos >> 3;
    const uint8_t *xsrc = a.xq + xrow(tt) * C + ((pos & 7) ^ (tt & 7)) * 16;
    // scales: lanes with ls < NMAT take row li of matrix ls, the others
    // token li of token tile wave % NC
    const uint8_t *ssrc;
    if (ls < NMAT) {
        const int r = min(row0 + wave * 16 + li, R - 1);
        ssrc = (NMAT == 2 && ls == 1 ? Am[NMAT - 1] : Am[0]) + code_bytes + (int64_t)r * gpr;
    } else {
        ssrc = a.xs + xrow((wave % NC) * 16 + li) * gpr;
    }

    // the codes of pair q (clamped to the last pair, whose data is then not
    // read) into the buffer of its parity
    auto issue_codes = [&] __device__(auto pbt, int q) {
        uint8_t *P = pairbuf(pbt);
        const int qc = min(q, npairs - 1);
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                lds_dma16(csrc[mt][i] + (int64_t)qc * 128, P + (wave * NMAT + mt) * 2048 + i * 1024);
    };
    // step s's slab, and with a unit's first step the unit's scales
    auto issue = [&] __device__(auto tag, int s) {
        lds_dma16(xsrc + (int64_t)s * 128, stage(tag) + wave * 1024);
        if constexpr (decltype(tag)::value == 0)
            lds_dma16(ssrc + (s / 4) * 16, scs + wave * 1024);
    };

    f32x4 acc[NMAT][NC];
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
        for (int c = 0; c < NC; ++c)
            acc[mt][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // prologue: the loads above have landed; pair 0's codes and steps 0..2
    wait_vmcnt<0>();
    issue_codes(MaTag<0>{}, 0);
    issue(MaTag<0>{}, 0);
    issue(MaTag<1>{}, min(1, nsteps - 1));
    issue(MaTag<2>{}, min(2, nsteps - 1));

    u32x4 usa[NMAT], usb[NC]; // the unit's scale bytes: word j = step j, byte ls = group ls
    for (int un = 0; un < nunits; ++un) {
        auto step = [&] __device__(auto jt) {
            constexpr int j = decltype(jt)::value;
            const int s = un * 4 + j;
            // this step's slab (and at place 0 the unit's scales) and its
            // pair's codes have landed for every wave.  Issued per step: at
            // places 0 and 2 the next pair's codes (2 NMAT loads), then a
            // slab three steps ahead (1), plus the next unit's scales at
            // place 1 (1).  Loads issued after the last one this step needs:
            constexpr int AHEAD = j == 0   ? 2
                                  : j == 1 ? 2 * NMAT + 2
                                  : j == 2 ? 3
                                           : 2 * NMAT + 3;
            wait_vmcnt<AHEAD>();
            wait_lgkm0();
            raw_barrier();
            if constexpr (j % 2 == 0)
                issue_codes(MaTag<(j / 2 + 1) % 2>{}, s / 2 + 1);
            issue(MaTag<(j + 3) % 4>{}, min(s + 3, nsteps - 1));
            if constexpr (j == 0) { // this unit's scales, before they are refilled
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt)
                    usa[mt] = *reinterpret_cast<const u32x4 *>(scs + wave * 1024 +
                                                               (mt * 16 + li) * 16);
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    usb[c] = *reinterpret_cast<const u32x4 *>(scs + c * 1024 +
                                                              (NMAT * 16 + li) * 16);
            }
            // A: row li, group ls of the step = piece 4 (j % 2) + ls of the
            // pair's 128 bytes of the row
            const uint8_t *PB = pairbuf(MaTag<(j / 2) % 2>{});
            const int kp = 4 * (j % 2) + ls;
            const int aoff = (li >> 3) * 1024 + ((li & 7) * 8 + (kp ^ ((li >> 1) & 7))) * 16;
            i32x8 A[NMAT];
            int sa[NMAT];
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt) {
                const u32x4 av =
                    *reinterpret_cast<const u32x4 *>(PB + (wave * NMAT + mt) * 2048 + aoff);
                A[mt] = i32x8{(int)av[0], (int)av[1], (int)av[2], (int)av[3], 0, 0, 0, 0};
                sa[mt] = (int)((usa[mt][j] >> (8 * ls)) & 0xFFu); // row li, group ls
            }
            const uint8_t *S = stage(MaTag<j>{});
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int t = c * 16 + li;
                const uint8_t *row = S + t * 128;
                const u32x4 lo = *reinterpret_cast<const u32x4 *>(row + ((ls ^ (t & 7)) * 16));
                const u32x4 hi =
                    *reinterpret_cast<const u32x4 *>(row + (((4 + ls) ^ (t & 7)) * 16));
                const i32x8 B = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                const int sb = (int)((usb[c][j] >> (8 * ls)) & 0xFFu); // token t, block ls
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt)
                    acc[mt][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        A[mt], B, acc[mt][c], 4 /* A: FP4 E2M1 */, 0 /* B: FP8 E4M3 */, 0,
                        sa[mt], 0, sb);
            }
        };
        step(MaTag<0>{});
        step(MaTag<1>{});
        step(MaTag<2>{});
        step(MaTag<3>{});
    }
    // the last steps' (clamped, unused) loads land before the workgroup ends
    wait_vmcnt<0>();

    // D: lane (li, ls) holds rows 4 ls .. 4 ls + 3 of token column li
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int tok = c * 16 + li;
        if (tok >= ntok)
            continue;
        const int64_t orow = (int64_t)(slot0 + tok) * R;
        const int rbase = row0 + wave * 16 + 4 * ls;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rbase + i;
            if (r >= R)
                continue;
            float v = acc[0][c][i];
            if constexpr (MODE == MODE_GATEUP)
                v = silu(v) * acc[NMAT - 1][c][i];
            a.y[orow + r] = v;
        }
    }
}

} // namespace

int moe_a8_rows_per_wg() { return MA_NW * 16; }
int moe_a8_tokens() { return MA_NC * 16; }

hipError_t moe_a8_launch(int mode, const MoeA8Args &a, hipStream_t stream)
{
    const int64_t nrb = (a.rows + moe_a8_rows_per_wg() - 1) / moe_a8_rows_per_wg();
    const dim3 grid((unsigned)(nrb * a.max_work)), block(MA_NW * 64);
    if (mode == MODE_GATEUP)
        hipLaunchKernelGGL(moe_a8_kernel<MODE_GATEUP>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(moe_a8_kernel<MODE_DOWN>, grid, block, 0, stream, a);
    return hipGetLastError();
}

} // namespace mx
