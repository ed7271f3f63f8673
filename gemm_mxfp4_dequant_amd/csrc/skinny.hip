// Fused MXFP4 dequantize-and-multiply against a few activation rows, for
// gfx950 matrix cores.
//
// What is computed: y[t][r] = sum_c W[r][c] * x[t][c] for a handful of
// tokens t ("cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs": mxfp4_mv /
// mxfp4_mm and matmat), and inside the expert bank the gate/up + SwiGLU and
// down products of one expert's routed tokens ("cortiq-engine 0.8.77,
// src/qtensor/moe_fast.rs": gate_up_block, down_block).
//
// How (MI355X design, not the pages' workgroup-per-row shader):
//  * A workgroup owns a block of output rows and all of K.  Its waves split
//    the rows: each wave owns 16 rows (one MFMA tile) and streams them with
//    128-bit loads, a lane loading one whole 32-column group (16 bytes) of
//    one row per load step.  All of a wave's K blocks are in flight at once
//    (or a ring of PF blocks for long rows), so every lane keeps several KB
//    of HBM traffic outstanding.
//  * The E8M0 scales of the workgroup's rows are staged in LDS with
//    coalesced 16-byte loads, once per workgroup.
//  * The activations of the (up to TPC) tokens are staged in LDS once per
//    workgroup as bf16 MFMA operands.  fp32 activations are split exactly
//    into hi = bf16(x) and lo = bf16(x - hi) (|x - hi - lo| <= 2^-16 |x|)
//    and occupy two MFMA columns each; bf16 activations occupy one.
//  * Each group is decoded once per workgroup by v_cvt_scalef32_pk_bf16_fp4
//    straight into the MFMA A operand (exact: E2M1 times a power of two is a
//    bf16), and fed to v_mfma_f32_16x16x32_bf16, which does the K reduction
//    of the dot products (the pages' LDS reduction tree is not needed).
//    MFMA step (L, m) pairs lane slice s with group 4L+s, elements 8m..8m+7;
//    a dot product is order-free, so this k-order follows the 128-bit load.
//  * The hi and lo columns of a token are summed with one DPP row rotate.
//  * Each token's column is computed by the same instructions whatever the
//    other columns hold, so a batch equals its tokens' matvecs bit for bit.
#include <atomic>

#include "device.h"
#include "launch.h"

namespace mx {

namespace {

constexpr int KB = 512;       // columns per K block
constexpr int LPB = KB / 128; // 128-column load steps per block
constexpr int BPAD = 8;       // bf16 padding per LDS operand row (bank spread)

struct TileMap {
    int ntok;     // valid token columns of this workgroup
    int slot0;    // first token (GEMM) / first slot (MoE)
    int row0;     // first output row
    int expert;   // MoE expert (0 for GEMM)
};

// Work item of this workgroup; returns false if it has none (MoE grids are
// sized by an upper bound).
template <int MODE, int TPC>
__device__ __forceinline__ bool tile_map(const SkinnyArgs &a, int rows_wg, TileMap &m)
{
    // Flattened grid, item/chunk fastest: consecutive workgroups share row
    // blocks, so a row block's weights are reused from L2 across chunks.
    const int sub = blockIdx.x % a.nch;
    m.row0 = (blockIdx.x / a.nch) * rows_wg;
    if (MODE == MODE_GEMM) {
        const int t0 = sub * TPC;
        m.ntok = min(TPC, a.b - t0);
        m.slot0 = t0;
        m.expert = 0;
        return true;
    }
    const int item = sub;
    if (item >= *a.n_work)
        return false;
    const int4 wk = reinterpret_cast<const int4 *>(a.work)[item];
    m.expert = wk.x;
    m.slot0 = wk.y;
    m.ntok = wk.z;
    return true;
}

// Activation row of token column t.
template <int MODE>
__device__ __forceinline__ int64_t token_row(const SkinnyArgs &a, int slot0, int t)
{
    if (MODE == MODE_GATEUP)
        return a.token_of_slot[slot0 + t];
    return slot0 + t;
}

// LDS row of the B operand read by lane column j (hi rows 0..ntok-1, lo
// rows ntok..2ntok-1 for fp32; rows 0..ntok-1 for bf16), or -1 for a zero
// column.
template <bool XBF>
__device__ __forceinline__ int b_row(int j, int ntok)
{
    if (XBF)
        return j < ntok ? j : -1;
    if (j < 8)
        return j < ntok ? j : -1;
    return (j - 8) < ntok ? ntok + (j - 8) : -1;
}

// Epilogue: the wave's 16x16 accumulator tile -> outputs.
// acc[i] = D[4*ls + i][li].  For fp32 inputs the lo column li+8 is folded
// into column li.
template <int MODE, bool XBF>
__device__ __forceinline__ void epilogue(const SkinnyArgs &a, const TileMap &tm, f32x4 acc,
                                         int mat, int tile, int lane, float *xch)
{
    const int li = lane & 15, ls = lane >> 4;
    if (!XBF) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[i] += dpp_row_ror8(acc[i]);
    }
    const bool col_ok = XBF ? (li < tm.ntok) : (li < 8 && li < tm.ntok);
    const int R = a.rows;
    const int rbase = tm.row0 + tile * 16 + 4 * ls;

    if (MODE == MODE_GATEUP) {
        // up waves hand their tile to the gate waves through LDS
        if (mat == 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xch[(tile * 64 + lane) * 4 + i] = acc[i];
        }
        __syncthreads();
        if (mat == 1 || !col_ok)
            return;
        const int64_t slot = tm.slot0 + li;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rbase + i;
            if (r >= R)
                continue;
            const float u = xch[(tile * 64 + lane) * 4 + i];
            const float h = silu(acc[i]) * u;
            if (a.y_bf16)
                reinterpret_cast<uint16_t *>(a.y)[slot * R + r] = f32_to_bf16_bits(h);
            else
                reinterpret_cast<float *>(a.y)[slot * R + r] = h;
        }
        return;
    }
    if (!col_ok)
        return;
    const int64_t orow = tm.slot0 + li; // token (GEMM) or slot (DOWN)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = rbase + i;
        if (r >= R)
            continue;
        if (MODE == MODE_GEMM && a.y_bf16)
            reinterpret_cast<uint16_t *>(a.y)[orow * R + r] = f32_to_bf16_bits(acc[i]);
        else
            reinterpret_cast<float *>(a.y)[orow * R + r] = acc[i];
    }
}

} // namespace

// Static-K kernel: cols == NKB * 512.
template <int NW, int NKB, int PF, int TPC, bool XBF, int MODE>
__global__ __launch_bounds__(NW * 64) void skinny_static(SkinnyArgs a)
{
    constexpr int NT = NW * 64;
    constexpr int COLS = NKB * KB;
    constexpr int GPR = COLS / 32;
    constexpr int NMAT = (MODE == MODE_GATEUP) ? 2 : 1;
    constexpr int TILES = (MODE == MODE_GATEUP) ? NW / 2 : NW;
    constexpr int ROWS_WG = TILES * 16;
    constexpr int NBC = XBF ? TPC : 2 * TPC;
    constexpr int BSTRIDE = COLS + BPAD;
    constexpr int SSTRIDE = GPR + 16;
    constexpr int SEGS = COLS / 8;                   // 8-element segments per row
    constexpr int SPT = (SEGS + NT - 1) / NT;        // segments per thread per token
    constexpr int SCHUNK = GPR / 16;                 // 16-byte scale chunks per row
    constexpr int SUNITS = NMAT * ROWS_WG * SCHUNK;
    constexpr int SUPT = (SUNITS + NT - 1) / NT;
    static_assert(PF >= 1 && PF <= NKB, "ring depth");

    extern __shared__ __align__(16) uint8_t smem[];
    __bf16 *Bs = reinterpret_cast<__bf16 *>(smem);
    uint8_t *Ss = smem + NBC * BSTRIDE * 2;
    float *xch = reinterpret_cast<float *>(Ss + NMAT * ROWS_WG * SSTRIDE);

    TileMap tm;
    if (!tile_map<MODE, TPC>(a, ROWS_WG, tm))
        return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, ls = lane >> 4;
    const int R = a.rows;
    const uint8_t *A0 = a.w0 + (int64_t)tm.expert * a.expert_stride;
    const uint8_t *A1 = (MODE == MODE_GATEUP) ? a.w1 + (int64_t)tm.expert * a.expert_stride : A0;
    const int64_t code_bytes = (int64_t)R * (COLS / 2);

    // ---- 1. issue activation and scale loads (older than the weight loads,
    //         so waiting for them does not wait for HBM)
    float xv[TPC][SPT][8];
#pragma unroll
    for (int t = 0; t < TPC; ++t) {
        if (t < tm.ntok) {
            const float *xr = nullptr;
            const uint16_t *xb = nullptr;
            const int64_t row = token_row<MODE>(a, tm.slot0, t);
            if (XBF)
                xb = reinterpret_cast<const uint16_t *>(a.x) + row * COLS;
            else
                xr = reinterpret_cast<const float *>(a.x) + row * COLS;
#pragma unroll
            for (int q = 0; q < SPT; ++q) {
                const int seg = tid + q * NT;
                if (SEGS % NT == 0 || seg < SEGS) {
                    if (XBF) {
                        const u32x4 v = *reinterpret_cast<const u32x4 *>(xb + seg * 8);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            xv[t][q][i] = __uint_as_float(v[i]);
                    } else {
                        const f32x4 v0 = *reinterpret_cast<const f32x4 *>(xr + seg * 8);
                        const f32x4 v1 = *reinterpret_cast<const f32x4 *>(xr + seg * 8 + 4);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            xv[t][q][i] = v0[i];
                            xv[t][q][4 + i] = v1[i];
                        }
                    }
                }
            }
        }
    }
    u32x4 sv[SUPT];
#pragma unroll
    for (int q = 0; q < SUPT; ++q) {
        const int u = tid + q * NT;
        sv[q] = u32x4{0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu};
        if (SUNITS % NT == 0 || u < SUNITS) {
            const int mat = u / (ROWS_WG * SCHUNK);
            const int rr = (u / SCHUNK) % ROWS_WG;
            const int ch = u % SCHUNK;
            const int r = tm.row0 + rr;
            if (r < R) {
                const uint8_t *base = (mat ? A1 : A0) + code_bytes + (int64_t)r * GPR + ch * 16;
                sv[q] = *reinterpret_cast<const u32x4 *>(base);
            }
        }
    }

    // ---- 2. issue this wave's weight stream (ring of PF blocks)
    const int mat = (MODE == MODE_GATEUP) ? wave / TILES : 0;
    const int tile = (MODE == MODE_GATEUP) ? wave % TILES : wave;
    const int r = tm.row0 + tile * 16 + li;
    const bool rvalid = r < R;
    const uint8_t *arow = (mat ? A1 : A0) + (int64_t)(rvalid ? r : 0) * (COLS / 2) + ls * 16;
    u32x4 ring[PF][LPB];
#pragma unroll
    for (int p = 0; p < PF; ++p)
#pragma unroll
        for (int L = 0; L < LPB; ++L)
            ring[p][L] = rvalid ? *reinterpret_cast<const u32x4 *>(arow + p * 256 + L * 64)
                                : u32x4{0, 0, 0, 0};

    // ---- 3. activations -> LDS operands; scales -> LDS
#pragma unroll
    for (int t = 0; t < TPC; ++t) {
        if (t < tm.ntok) {
#pragma unroll
            for (int q = 0; q < SPT; ++q) {
                const int seg = tid + q * NT;
                if (SEGS % NT == 0 || seg < SEGS) {
                    if (XBF) {
                        u32x4 v;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            v[i] = __float_as_uint(xv[t][q][i]);
                        *reinterpret_cast<u32x4 *>(Bs + t * BSTRIDE + seg * 8) = v;
                    } else {
                        bf16x8 hi, lo;
                        split_bf16x8(xv[t][q], hi, lo);
                        *reinterpret_cast<bf16x8 *>(Bs + t * BSTRIDE + seg * 8) = hi;
                        *reinterpret_cast<bf16x8 *>(Bs + (tm.ntok + t) * BSTRIDE + seg * 8) = lo;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < SUPT; ++q) {
        const int u = tid + q * NT;
        if (SUNITS % NT == 0 || u < SUNITS) {
            const int rr = u / SCHUNK; // mat * ROWS_WG + row
            const int ch = u % SCHUNK;
            *reinterpret_cast<u32x4 *>(Ss + rr * SSTRIDE + ch * 16) = sv[q];
        }
    }
    __syncthreads();

    // ---- 4. decode + MFMA over K
    const int brow = b_row<XBF>(li, tm.ntok);
    const __bf16 *bb = Bs + (brow < 0 ? 0 : brow) * BSTRIDE + ls * 32;
    const uint8_t *srow = Ss + (mat * ROWS_WG + tile * 16 + li) * SSTRIDE;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const bf16x8 zero8 = {};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        const int slot = kb % PF;
        const u32x4 sc = *reinterpret_cast<const u32x4 *>(srow + kb * 16);
#pragma unroll
        for (int L = 0; L < LPB; ++L) {
            const float scf = e8m0_operand_of(sc[L], ls);
            const u32x4 cw = ring[slot][L];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const bf16x8 av = decode8_bf16(cw[m], scf);
                const bf16x8 bv = brow >= 0
                    ? *reinterpret_cast<const bf16x8 *>(bb + kb * KB + L * 128 + m * 8)
                    : zero8;
                acc = mfma16x16x32(av, bv, acc);
            }
        }
        if (kb + PF < NKB) {
#pragma unroll
            for (int L = 0; L < LPB; ++L)
                ring[slot][L] = rvalid
                    ? *reinterpret_cast<const u32x4 *>(arow + (kb + PF) * 256 + L * 64)
                    : u32x4{0, 0, 0, 0};
        }
    }

    epilogue<MODE, XBF>(a, tm, acc, mat, tile, lane, xch);
}

// Generic kernel: any cols % 32 == 0 (K steps of 128 columns, guarded).
template <int NW, int TPC, bool XBF, int MODE>
__global__ __launch_bounds__(NW * 64) void skinny_generic(SkinnyArgs a)
{
    constexpr int NT = NW * 64;
    constexpr int NMAT = (MODE == MODE_GATEUP) ? 2 : 1;
    constexpr int TILES = (MODE == MODE_GATEUP) ? NW / 2 : NW;
    constexpr int ROWS_WG = TILES * 16;

    extern __shared__ __align__(16) uint8_t smem[];
    const int C = a.cols;
    const int gpr = C / 32;
    const int cpad = (C + 127) / 128 * 128;
    const int bstride = cpad + BPAD;
    const int sstride = (gpr + 15) / 16 * 16 + 16;
    const int nbc = XBF ? TPC : 2 * TPC;
    __bf16 *Bs = reinterpret_cast<__bf16 *>(smem);
    uint8_t *Ss = smem + (size_t)nbc * bstride * 2;
    float *xch = reinterpret_cast<float *>(Ss + NMAT * ROWS_WG * sstride);

    TileMap tm;
    if (!tile_map<MODE, TPC>(a, ROWS_WG, tm))
        return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, ls = lane >> 4;
    const int R = a.rows;
    const uint8_t *A0 = a.w0 + (int64_t)tm.expert * a.expert_stride;
    const uint8_t *A1 = (MODE == MODE_GATEUP) ? a.w1 + (int64_t)tm.expert * a.expert_stride : A0;
    const int64_t code_bytes = (int64_t)R * (C / 2);

    // activations -> LDS (zero beyond C up to cpad)
    const int segs = cpad / 8;
    for (int t = 0; t < tm.ntok; ++t) {
        const int64_t row = token_row<MODE>(a, tm.slot0, t);
        for (int seg = tid; seg < segs; seg += NT) {
            float v[8];
            const int c = seg * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float xvv = 0.f;
                if (c + i < C) {
                    if (XBF)
                        xvv = bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(a.x)[row * C + c + i]);
                    else
                        xvv = reinterpret_cast<const float *>(a.x)[row * C + c + i];
                }
                v[i] = xvv;
            }
            if (XBF) {
                bf16x8 h;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    h[i] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(v[i]) >> 16));
                *reinterpret_cast<bf16x8 *>(Bs + t * bstride + c) = h;
            } else {
                bf16x8 hi, lo;
                split_bf16x8(v, hi, lo);
                *reinterpret_cast<bf16x8 *>(Bs + t * bstride + c) = hi;
                *reinterpret_cast<bf16x8 *>(Bs + (tm.ntok + t) * bstride + c) = lo;
            }
        }
    }
    // scales -> LDS, byte by byte
    for (int u = tid; u < NMAT * ROWS_WG * gpr; u += NT) {
        const int m = u / (ROWS_WG * gpr);
        const int rr = (u / gpr) % ROWS_WG;
        const int g = u % gpr;
        const int r = tm.row0 + rr;
        uint8_t k = 127;
        if (r < R)
            k = ((m ? A1 : A0) + code_bytes)[(int64_t)r * gpr + g];
        Ss[(m * ROWS_WG + rr) * sstride + g] = k;
    }
    __syncthreads();

    const int mat = (MODE == MODE_GATEUP) ? wave / TILES : 0;
    const int tile = (MODE == MODE_GATEUP) ? wave % TILES : wave;
    const int r = tm.row0 + tile * 16 + li;
    const bool rvalid = r < R;
    const uint8_t *arow = (mat ? A1 : A0) + (int64_t)(rvalid ? r : 0) * (C / 2);
    const uint8_t *srow = Ss + (mat * ROWS_WG + tile * 16 + li) * sstride;
    const int brow = b_row<XBF>(li, tm.ntok);
    const __bf16 *bb = Bs + (brow < 0 ? 0 : brow) * bstride + ls * 32;
    const bf16x8 zero8 = {};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int nsteps = cpad / 128;
    for (int st = 0; st < nsteps; ++st) {
        const int g = st * 4 + ls;
        u32x4 cw = {0, 0, 0, 0};
        uint32_t k = 127;
        if (rvalid && g < gpr) {
            cw = *reinterpret_cast<const u32x4 *>(arow + (int64_t)g * 16);
            k = srow[g];
        }
        const float scf = e8m0_operand(k);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const bf16x8 av = decode8_bf16(cw[m], scf);
            const bf16x8 bv = brow >= 0 ? *reinterpret_cast<const bf16x8 *>(bb + st * 128 + m * 8)
                                        : zero8;
            acc = mfma16x16x32(av, bv, acc);
        }
    }
    epilogue<MODE, XBF>(a, tm, acc, mat, tile, lane, xch);
}

// ---------------------------------------------------------------------------
// Host side: instantiation table and launch
// ---------------------------------------------------------------------------

namespace {

constexpr int NW_GEMM = 4;

size_t lds_static(int nkb, int tpc, bool xbf, int mode)
{
    const int cols = nkb * KB;
    const int nmat = mode == MODE_GATEUP ? 2 : 1;
    const int tiles = mode == MODE_GATEUP ? NW_GEMM / 2 : NW_GEMM;
    const int nbc = xbf ? tpc : 2 * tpc;
    size_t b = (size_t)nbc * (cols + BPAD) * 2;
    b += (size_t)nmat * tiles * 16 * (cols / 32 + 16);
    if (mode == MODE_GATEUP)
        b += (size_t)tiles * 64 * 4 * 4;
    return b;
}

size_t lds_generic(int cols, int tpc, bool xbf, int mode)
{
    const int nmat = mode == MODE_GATEUP ? 2 : 1;
    const int tiles = mode == MODE_GATEUP ? NW_GEMM / 2 : NW_GEMM;
    const int nbc = xbf ? tpc : 2 * tpc;
    const int cpad = (cols + 127) / 128 * 128;
    const int gpr = cols / 32;
    size_t b = (size_t)nbc * (cpad + BPAD) * 2;
    b += (size_t)nmat * tiles * 16 * ((gpr + 15) / 16 * 16 + 16);
    if (mode == MODE_GATEUP)
        b += (size_t)tiles * 64 * 4 * 4;
    return b;
}

typedef void (*KernelFn)(SkinnyArgs);

struct Entry {
    int mode, xbf, nkb, tpc; // nkb 0 = generic
    KernelFn fn;
};

#define MX_S(MODE, XBF, NKB, PF, TPC) \
    {MODE, XBF, NKB, TPC, skinny_static<NW_GEMM, NKB, PF, TPC, (bool)XBF, MODE>}
#define MX_G(MODE, XBF, TPC) {MODE, XBF, 0, TPC, skinny_generic<NW_GEMM, TPC, (bool)XBF, MODE>}

#define MX_FP32_SET(MODE, NKB, PF) \
    MX_S(MODE, 0, NKB, PF, 1), MX_S(MODE, 0, NKB, PF, 2), MX_S(MODE, 0, NKB, PF, 4), \
    MX_S(MODE, 0, NKB, PF, 8)
#define MX_BF16_SET(MODE, NKB, PF) \
    MX_S(MODE, 1, NKB, PF, 2), MX_S(MODE, 1, NKB, PF, 4), MX_S(MODE, 1, NKB, PF, 8), \
    MX_S(MODE, 1, NKB, PF, 16)
#define MX_GEN_SET(MODE) \
    MX_G(MODE, 0, 1), MX_G(MODE, 0, 2), MX_G(MODE, 0, 4), MX_G(MODE, 0, 8), MX_G(MODE, 1, 2), \
    MX_G(MODE, 1, 4), MX_G(MODE, 1, 8), MX_G(MODE, 1, 16)

const Entry kTable[] = {
    MX_FP32_SET(MODE_GEMM, 1, 1), MX_FP32_SET(MODE_GEMM, 4, 4), MX_FP32_SET(MODE_GEMM, 8, 8),
    MX_BF16_SET(MODE_GEMM, 1, 1), MX_BF16_SET(MODE_GEMM, 4, 4), MX_BF16_SET(MODE_GEMM, 8, 8),
    MX_FP32_SET(MODE_GATEUP, 8, 8), MX_FP32_SET(MODE_GATEUP, 4, 4),
    MX_BF16_SET(MODE_GATEUP, 8, 8), MX_S(MODE_GATEUP, 1, 14, 7, 2),
    MX_S(MODE_GATEUP, 1, 14, 7, 4), MX_S(MODE_GATEUP, 1, 14, 7, 8),
    MX_FP32_SET(MODE_DOWN, 4, 4), MX_FP32_SET(MODE_DOWN, 8, 8), MX_BF16_SET(MODE_DOWN, 4, 4),
    MX_GEN_SET(MODE_GEMM), MX_GEN_SET(MODE_GATEUP), MX_GEN_SET(MODE_DOWN),
};

const Entry *find(int mode, int xbf, int nkb, int tpc)
{
    for (const Entry &e : kTable)
        if (e.mode == mode && e.xbf == xbf && e.nkb == nkb && e.tpc == tpc)
            return &e;
    return nullptr;
}

} // namespace

int skinny_rows_per_wg(int mode) { return mode == MODE_GATEUP ? NW_GEMM / 2 * 16 : NW_GEMM * 16; }

int skinny_pick_tpc(int mode, bool xbf, int cols, int want)
{
    static const int f32_opts[] = {1, 2, 4, 8};
    static const int b16_opts[] = {2, 4, 8, 16};
    const int *opts = xbf ? b16_opts : f32_opts;
    int best = 0;
    for (int i = 0; i < 4; ++i) {
        const int t = opts[i];
        const bool fits = (cols % KB == 0 ? lds_static(cols / KB, t, xbf, mode)
                                          : lds_generic(cols, t, xbf, mode)) <= 160 * 1024;
        if (!fits)
            break;
        best = t;
        if (t >= want)
            break;
    }
    return best;
}

size_t skinny_lds_bytes(int mode, bool xbf, int cols, int tpc)
{
    const int nkb = cols % KB == 0 ? cols / KB : 0;
    if (nkb && find(mode, xbf, nkb, tpc))
        return lds_static(nkb, tpc, xbf, mode);
    return lds_generic(cols, tpc, xbf, mode);
}

hipError_t skinny_launch(int mode, bool xbf, int tpc, const SkinnyArgs &a, dim3 grid,
                         hipStream_t stream)
{
    const int nkb = a.cols % KB == 0 ? a.cols / KB : 0;
    const Entry *e = nkb ? find(mode, xbf, nkb, tpc) : nullptr;
    size_t lds;
    if (e) {
        lds = lds_static(nkb, tpc, xbf, mode);
    } else {
        e = find(mode, xbf, 0, tpc);
        lds = lds_generic(a.cols, tpc, xbf, mode);
    }
    if (!e)
        return hipErrorInvalidValue;
    // Opt in to more than 64 KB of LDS once per kernel (the largest request
    // a kernel ever makes is its 160 KB bound), so that later launches,
    // including ones under graph capture, make no attribute calls.
    static std::atomic<uint8_t> opted[sizeof(kTable) / sizeof(kTable[0])];
    std::atomic<uint8_t> &flag = opted[e - kTable];
    if (lds > 64 * 1024 && !flag.load(std::memory_order_acquire)) {
        hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void *>(e->fn),
                                            hipFuncAttributeMaxDynamicSharedMemorySize,
                                            160 * 1024);
        if (st != hipSuccess)
            return st;
        flag.store(1, std::memory_order_release);
    }
    hipLaunchKernelGGL(e->fn, grid, dim3(NW_GEMM * 64), lds, stream, a);
    return hipGetLastError();
}

} // namespace mx
