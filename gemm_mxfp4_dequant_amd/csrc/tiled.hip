// MXFP4 x tens of activation rows: the tiled schedule of the same product,
// for work items that carry many tokens (hot experts of a prefill bank,
// GEMMs with more tokens than one skinny chunk).  The arithmetic is the
// skinny kernel's (exact bf16 decode of each weight by
// v_cvt_scalef32_pk_bf16_fp4, fp32 activations split into bf16 hi + lo
// columns, v_mfma_f32_16x16x32_bf16, fp32 accumulate, the library's
// canonical summation order), so every token's result is bit-identical to
// its own matvec.  What differs is the schedule:
//
//  * A workgroup of NW waves owns NW * RT * 16 output rows and up to 16 * NC
//    MFMA columns (16 * NC bf16 tokens, or 8 * NC fp32 tokens as hi/lo
//    pairs).  Each wave owns RT row tiles of every matrix of the mode (gate
//    and up tiles of the same rows sit in one wave, so SwiGLU needs no
//    exchange) and runs the whole K loop.
//  * K is streamed in 128-column steps.  The activations of a step pass
//    through registers into a double-buffered LDS slab, shared by all
//    waves; every decoded weight serves NC column tiles and every
//    activation fragment read from LDS serves RT * NMAT row tiles.
//  * The code words, scale bytes and activations of step s + 4 are loaded
//    together during step s.
//    Loads of one distance complete in issue order, so waiting for step
//    s + 1's activations never drains the weight loads behind them.  All
//    loads are unconditional (indices clamped), which keeps the wait counts
//    static.
//  * Work items come from the same grouping as the skinny kernel
//    ("rlx-cpu 0.2.17, src/gguf_matmul.rs", grouped_moe_sort_plan): an
//    expert's rows are streamed once per item of up to 16 * NC tokens
//    ("cortiq-engine 0.8.77, src/qtensor/moe_fast.rs": gate_up_block and
//    down_block stream an expert's rows once for all of its tokens).
#include <atomic>

#include "device.h"
#include "launch.h"

namespace mx {

namespace {

constexpr int TKS = 128;        // columns per K step
constexpr int TP = 4;           // steps loaded ahead (= steps per 512-column unit)
constexpr int TBROW = TKS + 8;  // LDS operand row stride (bf16): lanes of a row tile
                                // start 272 bytes apart -> distinct banks

template <int N> struct IntTag {
    static constexpr int value = N;
};

template <int MODE>
__device__ __forceinline__ int64_t t_token_row(const SkinnyArgs &a, int slot0, int t)
{
    if (MODE == MODE_GATEUP)
        return a.token_of_slot[slot0 + t];
    return slot0 + t;
}

} // namespace

template <int NW, int RT, int NC, bool XBF, int MODE>
__global__ __launch_bounds__(NW * 64) void tiled_kernel(SkinnyArgs a)
{
    constexpr int NT = NW * 64;
    constexpr int NMAT = (MODE == MODE_GATEUP) ? 2 : 1;
    constexpr int MT = NMAT * RT;               // A tiles per wave
    constexpr int RB = NW * RT * 16;            // output rows per workgroup
    constexpr int NCOL = 16 * NC;               // MFMA columns
    constexpr int TPD = XBF ? NCOL : NCOL / 2;  // tokens per work item
    constexpr int UNITS = TPD * (TKS / 8);      // 8-element pieces per step
    constexpr int UPT = UNITS / NT;             // pieces per thread per step
    static_assert(UNITS % NT == 0, "activation pieces must divide evenly");

    __shared__ __align__(16) __bf16 Bs[2][NCOL][TBROW];

    const int C = a.cols;
    const int R = a.rows;
    const int gpr = C / 32;
    const int nsteps = C / TKS; // a multiple of 4 (cols % 512 == 0)
    const int nunits = nsteps / 4;

    // ---- work item (XCD-grouped logical id, item fastest)
    const int lid = xcd_logical(blockIdx.x, gridDim.x);
    const int sub = lid % a.nch;
    const int row0 = (lid / a.nch) * RB;
    int ntok, slot0, expert = 0;
    if (MODE == MODE_GEMM) {
        slot0 = sub * TPD;
        ntok = min(TPD, a.b - slot0);
    } else {
        if (sub >= *a.n_work)
            return;
        const int4 wk = reinterpret_cast<const int4 *>(a.work)[sub];
        expert = wk.x;
        slot0 = wk.y;
        ntok = wk.z;
    }
    const int nct = XBF ? (ntok + 15) / 16 : (ntok + 7) / 8; // column tiles in use

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, ls = lane >> 4;
    const int64_t code_bytes = (int64_t)R * (C / 2);

    // A rows of this lane: tile mt = mat * RT + rt; rows past the end read
    // row R-1 (never stored; MFMA output rows depend on their own A row only).
    // Offsets are 32-bit from the tensor base (a tensor is < 2^31 bytes).
    const uint8_t *Am[NMAT];
    uint32_t aoff[MT], soff[MT];
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat) {
        Am[mat] = (mat ? a.w1 : a.w0) + (int64_t)expert * a.expert_stride;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int r = min(row0 + (wave * RT + rt) * 16 + li, R - 1);
            aoff[mat * RT + rt] = (uint32_t)r * (uint32_t)(C / 2) + ls * 16;
            soff[mat * RT + rt] = (uint32_t)code_bytes + (uint32_t)r * (uint32_t)gpr;
        }
    }

    // Activation pieces of this thread: piece q is token t = u / 16, columns
    // 8 * (u % 16) .. +8 of each step.  Tokens past the item's end re-read its
    // last token (their columns are never stored; MFMA columns do not mix).
    int64_t xoff[UPT];
#pragma unroll
    for (int q = 0; q < UPT; ++q) {
        const int u = tid + q * NT;
        const int t = u / (TKS / 8);
        xoff[q] = t_token_row<MODE>(a, slot0, min(t, ntok - 1)) * C + (u % (TKS / 8)) * 8;
    }

    u32x4 xr[TP][UPT][XBF ? 1 : 2]; // activation ring (bf16 words / raw fp32)
    u32x4 cw[TP][MT];               // code ring
    uint32_t sw[TP][MT];            // scale ring: the 4 scale bytes of a step

    auto load_act = [&](int slot, int s) {
#pragma unroll
        for (int q = 0; q < UPT; ++q) {
            if constexpr (XBF) {
                xr[slot][q][0] = *reinterpret_cast<const u32x4 *>(
                    reinterpret_cast<const uint16_t *>(a.x) + xoff[q] + s * TKS);
            } else {
                const float *p = reinterpret_cast<const float *>(a.x) + xoff[q] + s * TKS;
                xr[slot][q][0] = *reinterpret_cast<const u32x4 *>(p);
                xr[slot][q][1] = *reinterpret_cast<const u32x4 *>(p + 4);
            }
        }
    };
    auto load_codes = [&](int slot, int s) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint8_t *A = Am[mt / RT];
            cw[slot][mt] = *reinterpret_cast<const u32x4 *>(A + aoff[mt] + s * (TKS / 2));
            sw[slot][mt] = *reinterpret_cast<const uint32_t *>(A + soff[mt] + s * 4);
        }
    };
    auto store_act = [&](int buf, int slot) {
#pragma unroll
        for (int q = 0; q < UPT; ++q) {
            const int u = tid + q * NT;
            const int t = u / (TKS / 8), seg = u % (TKS / 8);
            if constexpr (XBF) {
                *reinterpret_cast<u32x4 *>(&Bs[buf][t][seg * 8]) = xr[slot][q][0];
            } else {
                float v[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] = __uint_as_float(xr[slot][q][0][i]);
                    v[4 + i] = __uint_as_float(xr[slot][q][1][i]);
                }
                bf16x8 hi, lo;
                split_bf16x8(v, hi, lo);
                const int rowhi = (t / 8) * 16 + (t % 8);
                *reinterpret_cast<bf16x8 *>(&Bs[buf][rowhi][seg * 8]) = hi;
                *reinterpret_cast<bf16x8 *>(&Bs[buf][rowhi + 8][seg * 8]) = lo;
            }
        }
    };

    // ---- prologue: steps 0..3, slab 0 -> LDS.  All four steps are waited
    // for here (step 0 needs its loads anyway), so the loop is entered with
    // no loads in flight and the compiler counts the loop's own loads
    // exactly; otherwise the prologue's load order, merged at the loop head,
    // makes it wait for every load at the top of each 512-column unit.
#pragma unroll
    for (int p = 0; p < TP; ++p) {
        load_act(p, p);
        load_codes(p, p);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0)
    store_act(0, 0);
    __syncthreads();

    // acc: the current 512-column unit, its 16 MFMA steps in k order; tot:
    // the units so far, summed in ascending order
    f32x4 acc[MT][NC], tot[MT][NC];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            acc[mt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
            tot[mt][c] = acc[mt][c];
        }

    // The K loop, specialised on the column tiles in use (NCU <= NC) so that
    // its body has no branches.
    auto k_loop = [&](auto ncu_tag) {
        constexpr int NCU = decltype(ncu_tag)::value;
        for (int un = 0; un < nunits; ++un) {
#pragma unroll
            for (int j = 0; j < TP; ++j) {
                const int s = un * TP + j;
                // Keep each step's instructions inside its step: hoisting a
                // later step's scale extraction to the top of the loop would
                // wait for loads issued at the end of the previous iteration.
                __builtin_amdgcn_sched_barrier(0);
                // ---- step s: decode + MFMA from slab j & 1 and code slot j
                float scf[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    scf[mt] = e8m0_operand_of(sw[j][mt], ls);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    bf16x8 bv[NCU];
#pragma unroll
                    for (int c = 0; c < NCU; ++c)
                        bv[c] = *reinterpret_cast<const bf16x8 *>(
                            &Bs[j & 1][c * 16 + li][ls * 32 + m * 8]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const bf16x8 av = decode8_bf16(cw[j][mt][m], scf[mt]);
#pragma unroll
                        for (int c = 0; c < NCU; ++c)
                            acc[mt][c] = mfma16x16x32(av, bv[c], acc[mt][c]);
                    }
                }
                // ---- loads of step s + 4 (the last step re-loaded past the end)
                const int sl = min(s + TP, nsteps - 1);
                load_act(j, sl);
                load_codes(j, sl);
                // ---- step s + 1's activations -> the other slab
                store_act((j + 1) & 1, (j + 1) % TP);
                __syncthreads();
            }
            // ---- end of a 512-column unit
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int c = 0; c < NCU; ++c) {
                    tot[mt][c] = un == 0 ? acc[mt][c] : tot[mt][c] + acc[mt][c];
                    acc[mt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        }
    };
    if (NC >= 4 && nct >= 4)
        k_loop(IntTag<NC >= 4 ? 4 : 1>{});
    else if (NC >= 3 && nct == 3)
        k_loop(IntTag<NC >= 3 ? 3 : 1>{});
    else if (nct >= 2)
        k_loop(IntTag<2>{});
    else
        k_loop(IntTag<1>{});

    // ---- outputs
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (c >= nct)
                continue;
            f32x4 g = tot[rt][c];
            f32x4 u = g;
            if (MODE == MODE_GATEUP)
                u = tot[RT + rt][c];
            if (!XBF) { // hi column li + lo column li + 8
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    g[i] += dpp_row_ror8(g[i]);
                    if (MODE == MODE_GATEUP)
                        u[i] += dpp_row_ror8(u[i]);
                }
            }
            const int tok = XBF ? c * 16 + li : c * 8 + li;
            const bool ok = XBF ? tok < ntok : (li < 8 && tok < ntok);
            if (!ok)
                continue;
            const int rbase = row0 + (wave * RT + rt) * 16 + 4 * ls;
            const int64_t orow = slot0 + tok;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rbase + i;
                if (r >= R)
                    continue;
                float v = g[i];
                if (MODE == MODE_GATEUP)
                    v = silu(g[i]) * u[i];
                if (MODE != MODE_DOWN && a.y_bf16)
                    reinterpret_cast<uint16_t *>(a.y)[orow * R + r] = f32_to_bf16_bits(v);
                else
                    reinterpret_cast<float *>(a.y)[orow * R + r] = v;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

namespace {

typedef void (*TiledFn)(SkinnyArgs);

struct TEntry {
    int mode, xbf, nw, nc;
    TiledFn fn;
};

#define MX_T(MODE, XBF, NW, NC) {MODE, XBF, NW, NC, tiled_kernel<NW, 1, NC, (bool)XBF, MODE>}
#define MX_TM(MODE) \
    MX_T(MODE, 0, 8, 4), MX_T(MODE, 1, 8, 4), MX_T(MODE, 0, 4, 4), MX_T(MODE, 1, 4, 4), \
        MX_T(MODE, 0, 4, 2), MX_T(MODE, 1, 4, 2), MX_T(MODE, 1, 8, 2)

const TEntry kTiled[] = {MX_TM(MODE_GEMM), MX_TM(MODE_GATEUP), MX_TM(MODE_DOWN)};

const TEntry *tfind(int mode, bool xbf, int nw, int nc)
{
    for (const TEntry &e : kTiled)
        if (e.mode == mode && e.xbf == (int)xbf && e.nw == nw && e.nc == nc)
            return &e;
    return nullptr;
}

} // namespace

bool tiled_supported(int cols) { return cols % 512 == 0; }

int tiled_tokens(bool xbf, int nc) { return xbf ? 16 * nc : 8 * nc; }

int tiled_rows_per_wg(int nw) { return nw * 16; }

hipError_t tiled_launch(int mode, bool xbf, int nw, int nc, const SkinnyArgs &a,
                        hipStream_t stream)
{
    const TEntry *e = tfind(mode, xbf, nw, nc);
    if (!e)
        return hipErrorInvalidValue;
    const int64_t nrb = (a.rows + tiled_rows_per_wg(nw) - 1) / tiled_rows_per_wg(nw);
    hipLaunchKernelGGL(e->fn, dim3((unsigned)(nrb * a.nch)), dim3(nw * 64), 0, stream, a);
    return hipGetLastError();
}

} // namespace mx
