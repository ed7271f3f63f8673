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
//  * A workgroup owns NR tiles of 16 output rows (per matrix) and all of K,
//    for one or several row blocks (consecutive in the plain GEMM, evenly
//    spaced in the expert bank; the tokens stay in LDS while it walks the
//    blocks; the next block's weights are in flight while the current one
//    computes).  Its waves form a grid: row tile x K slab.  A wave streams its 16 rows
//    over one slab of KW columns with 128-bit loads, a lane loading one
//    whole 32-column group (16 bytes) of one row per load step; all of a
//    wave's loads are issued before it waits for any of them.
//  * The E8M0 scales of the workgroup's rows are staged in LDS with
//    coalesced 16-byte loads, once per workgroup (expert bank), or loaded
//    by each lane with its codes (plain GEMM).
//  * The activations of the (up to TPC) tokens are staged in LDS once per
//    workgroup as bf16 MFMA operands.  fp32 activations are split into
//    hi = x truncated to bf16 and lo = bf16(x - hi) (|x - hi - lo| < 2^-15 |x|)
//    and occupy two MFMA columns each; bf16 activations occupy one.
//  * Each group is decoded once per workgroup by v_cvt_scalef32_pk_bf16_fp4
//    straight into the MFMA A operand (exact: E2M1 times a power of two is a
//    bf16) and fed to v_mfma_f32_16x16x32_bf16, which does the K reduction
//    of the dot products (the pages' LDS reduction tree is not needed).
//    MFMA step (L, m) pairs lane slice s with group 4L+s, elements 8m..8m+7;
//    a dot product is order-free, so this k-order follows the 128-bit load.
//  * Summation order (the same in every kernel of this library, whatever
//    the launch shape): K is cut into 512-column units; within a unit one
//    accumulator takes the unit's 16 MFMA steps in k order (MFMA accumulation
//    into its own destination issues back to back), and the unit partials
//    are summed in ascending order (through LDS across waves).  The hi and
//    lo columns of a token are then added with one DPP row rotate.
//  * Each token's column is computed by the same instructions whatever the
//    other columns hold, so every token's result equals its own matvec bit
//    for bit, for any batch size and launch shape.
#include <algorithm>
#include <atomic>
#include <climits>
#include <mutex>

#include "device.h"
#include "launch.h"

namespace mx {

namespace {

constexpr int BPAD = 8; // bf16 padding per LDS operand row (bank spread)

struct TileMap {
    int ntok;   // valid token columns of this workgroup
    int slot0;  // first token (GEMM) / first slot (MoE)
    int row0;   // first output row
    int expert; // MoE expert (0 for GEMM)
    // GATEUP: token row and routing pair of each token column (global
    // tables, or this workgroup's own when the kernel groups the routing)
    const int *rowmap;
    const int *pairmap;
};

// Work item `sub` of this workgroup; false if it has none (MoE grids are
// sized by an upper bound).
template <int MODE, int TPC>
__device__ __forceinline__ bool item_map(const SkinnyArgs &a, int sub, TileMap &m)
{
    m.row0 = 0;
    if (MODE == MODE_GEMM) {
        const int t0 = sub * TPC;
        m.ntok = min(TPC, a.b - t0);
        m.slot0 = t0;
        m.expert = 0;
        return true;
    }
    if (sub >= *a.n_work)
        return false;
    const int4 wk = reinterpret_cast<const int4 *>(a.work)[sub];
    m.expert = wk.x;
    m.slot0 = wk.y;
    m.ntok = wk.z;
    m.rowmap = a.token_of_slot + wk.y;
    m.pairmap = a.pair_of_slot + wk.y;
    return true;
}

constexpr int FG_KEYBITS = 11;     // keys: expert ids 0..1024, and a dropped pair
constexpr int FG_DROPPED = 2047;   // key of a dropped pair (above every expert id)
// LDS of the in-kernel grouping: n_work, expert, slot0, ntok, then the
// token rows and pairs of up to 16 token columns, then a 64-entry scan
constexpr int FG_WORDS = 4 + 32 + 64;

// Routing grouped inside the gate/up kernel (one wave, at most 64 pairs):
// the counting sort of the grouping kernels ("rlx-cpu 0.2.17,
// src/gguf_matmul.rs", grouped_moe_sort_plan) by wave ballots: experts
// ascending, pairs in order within an expert, so slots, work items and
// tables equal the grouping kernel's.  Writes this workgroup's item (of the
// workgroup grid the items share, as in the split-K kernel) to fz; writer:
// also the tables the down and combine kernels read.
__device__ void fused_group(const SkinnyArgs &a, int tpc, int lid, int grid, bool writer, int *fz)
{
    const int lane = threadIdx.x & 63;
    const int P = (a.fuse_group >> 1) & 127;
    const int K = (a.fuse_group >> 8) & 63;
    const int E = (a.fuse_group >> 14) & 2047;
    int e = -1;
    if (lane < P) {
        e = a.token_of_slot[lane]; // the routing ids
        if (e < 0 || e >= E)
            e = -1;
    }
    const bool valid = e >= 0;
    const int key = valid ? e : FG_DROPPED;
    // lanes with a smaller key (lt) and with the same key (eq), among valid
    uint64_t lt = 0, eq = __ballot(valid);
#pragma unroll
    for (int b = FG_KEYBITS - 1; b >= 0; --b) {
        const int bit = (key >> b) & 1;
        const uint64_t ones = __ballot(bit);
        if (bit) {
            lt |= eq & ~ones;
            eq &= ones;
        } else {
            eq &= ~ones;
        }
    }
    const int rank = __popcll(eq & ((1ull << lane) - 1));
    const int start = __popcll(lt); // first slot of this expert
    const int slot = valid ? start + rank : -1;
    const int cnt = __popcll(eq);
    const bool leader = valid && rank == 0;
    const int nit = leader ? (cnt + tpc - 1) / tpc : 0;
    // items before each expert: exclusive scan of the items in slot order
    int *scan = fz + 36;
    scan[lane] = 0;
    if (leader)
        scan[start] = nit;
    __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0): this wave's LDS stores
    const int v = scan[lane];
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d)
            incl += o;
    }
    const int n_work = __shfl(incl, 63, 64);
    const int ibase = __shfl(incl - v, start & 63, 64); // for leaders
    // this workgroup's item
    const int nrbg = min(a.nrb, max(1, grid / max(1, n_work)));
    const int sub = lid / nrbg;
    const uint64_t mine = __ballot(leader && sub >= ibase && sub < ibase + nit);
    int ex = -1, slot0 = 0, ntok = 0;
    if (mine) {
        const int L = __ffsll((long long)mine) - 1;
        const int c = sub - __shfl(ibase, L, 64);
        ex = __shfl(e, L, 64);
        slot0 = __shfl(start, L, 64) + c * tpc;
        ntok = min(tpc, __shfl(cnt, L, 64) - c * tpc);
    }
    if (valid && slot >= slot0 && slot < slot0 + ntok) {
        fz[4 + slot - slot0] = lane / K;       // token row
        fz[4 + 16 + slot - slot0] = lane;      // routing pair
    }
    if (lane == 0) {
        fz[0] = n_work;
        fz[1] = ex;
        fz[2] = slot0;
        fz[3] = ntok;
    }
    if (writer) {
        if (lane < P)
            const_cast<int *>(a.pair_of_slot)[lane] = slot; // slot_of_pair
        if (leader)
            for (int c = 0; c < nit; ++c)
                reinterpret_cast<int4 *>(const_cast<int *>(a.work))[ibase + c] =
                    int4{e, start + c * tpc, min(tpc, cnt - c * tpc), 0};
        if (lane == 0)
            *const_cast<int *>(a.n_work) = n_work;
    }
}

// Generic kernel: flattened logical grid, item / chunk fastest, laid out so
// that the chunks / work items of one row block run on one XCD: a row
// block's weights are read from HBM once and re-read from that XCD's L2.
template <int MODE, int TPC>
__device__ __forceinline__ bool tile_map(const SkinnyArgs &a, int rows_wg, TileMap &m)
{
    const int lid = xcd_logical(blockIdx.x, gridDim.x);
    if (!item_map<MODE, TPC>(a, lid % a.nch, m))
        return false;
    m.row0 = (lid / a.nch) * rows_wg;
    return true;
}

// Activation row of token column t.
template <int MODE>
__device__ __forceinline__ int64_t token_row(const TileMap &tm, int t)
{
    if (MODE == MODE_GATEUP)
        return tm.rowmap[t];
    return tm.slot0 + t;
}

// LDS operand row read by lane column j: hi rows 0..ntok-1 and lo rows
// ntok..2ntok-1 for fp32, rows 0..ntok-1 for bf16.  A column without a
// token reads row 0: its MFMA column is never stored, and MFMA columns do
// not mix.
template <bool XBF>
__device__ __forceinline__ int b_row(int j, int ntok)
{
    if (XBF)
        return j < ntok ? j : 0;
    if (j < 8)
        return j < ntok ? j : 0;
    return (j - 8) < ntok ? ntok + (j - 8) : 0;
}

// Load the 8 activation elements of unit (t, seg) into v (bf16: 4 words).
template <int MODE, bool XBF>
__device__ __forceinline__ void load_unit(const SkinnyArgs &a, const TileMap &tm, int t, int seg,
                                          int C, float *v)
{
    const int64_t row = token_row<MODE>(tm, t);
    if (XBF) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(
            reinterpret_cast<const uint16_t *>(a.x) + row * C + seg * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = __uint_as_float(w[i]);
    } else {
        const float *xr = reinterpret_cast<const float *>(a.x) + row * C + seg * 8;
        const f32x4 v0 = *reinterpret_cast<const f32x4 *>(xr);
        const f32x4 v1 = *reinterpret_cast<const f32x4 *>(xr + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = v0[i];
            v[4 + i] = v1[i];
        }
    }
}

// Write unit (t, seg) to the LDS operand rows (fp32: split into hi and lo).
template <bool XBF>
__device__ __forceinline__ void store_unit(__bf16 *Bs, int bstride, int ntok, int t, int seg,
                                           const float *v)
{
    if (XBF) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = __float_as_uint(v[i]);
        *reinterpret_cast<u32x4 *>(Bs + t * bstride + seg * 8) = w;
    } else {
        bf16x8 hi, lo;
        split_bf16x8(v, hi, lo);
        *reinterpret_cast<bf16x8 *>(Bs + t * bstride + seg * 8) = hi;
        *reinterpret_cast<bf16x8 *>(Bs + (ntok + t) * bstride + seg * 8) = lo;
    }
}

// Row 4 ls + c of the final tile -> outputs: g = D[4 ls + c][li] of the
// (gate) tile, u the up tile (GATEUP only); the same arithmetic as
// store_tile for one accumulator component.
template <int MODE, bool XBF>
__device__ __forceinline__ void store_row(const SkinnyArgs &a, const TileMap &tm, float g, float u,
                                          int tile, int lane, int c, float pw)
{
    const int li = lane & 15, ls = lane >> 4;
    if (!XBF) {
        g += dpp_row_ror8(g);
        if (MODE == MODE_GATEUP)
            u += dpp_row_ror8(u);
    }
    const bool col_ok = XBF ? (li < tm.ntok) : (li < 8 && li < tm.ntok);
    const int r = tm.row0 + tile * 16 + 4 * ls + c;
    if (!col_ok || r >= a.rows)
        return;
    const int64_t orow = tm.slot0 + li; // token (GEMM) or slot (MoE)
    float v = g;
    if (MODE == MODE_GATEUP)
        v = a.v41 ? swiglu_v41(g, u, pw, a.lim) : silu(g) * u;
    if (MODE != MODE_DOWN && a.y_bf16)
        reinterpret_cast<uint16_t *>(a.y)[orow * a.rows + r] = f32_to_bf16_bits(v);
    else
        reinterpret_cast<float *>(a.y)[orow * a.rows + r] = v;
}

// Final tile -> outputs.  g[i] = D[4*ls + i][li] of the (gate) tile, u the
// up tile (GATEUP only).  For fp32 inputs the lo column li+8 is folded into
// column li first.
template <int MODE, bool XBF>
__device__ __forceinline__ void store_tile(const SkinnyArgs &a, const TileMap &tm, f32x4 g,
                                           f32x4 u, int tile, int lane)
{
    const int li = lane & 15, ls = lane >> 4;
    if (!XBF) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            g[i] += dpp_row_ror8(g[i]);
            if (MODE == MODE_GATEUP)
                u[i] += dpp_row_ror8(u[i]);
        }
    }
    const bool col_ok = XBF ? (li < tm.ntok) : (li < 8 && li < tm.ntok);
    if (!col_ok)
        return;
    const int R = a.rows;
    const int rbase = tm.row0 + tile * 16 + 4 * ls;
    const int64_t orow = tm.slot0 + li; // token (GEMM) or slot (MoE)
    const float pw = (MODE == MODE_GATEUP && a.v41) ? a.pair_w[tm.pairmap[li]] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = rbase + i;
        if (r >= R)
            continue;
        float v = g[i];
        if (MODE == MODE_GATEUP)
            v = a.v41 ? swiglu_v41(g[i], u[i], pw, a.lim) : silu(g[i]) * u[i];
        if (MODE != MODE_DOWN && a.y_bf16)
            reinterpret_cast<uint16_t *>(a.y)[orow * R + r] = f32_to_bf16_bits(v);
        else
            reinterpret_cast<float *>(a.y)[orow * R + r] = v;
    }
}

} // namespace

// Split-K kernel: cols % KW == 0.  blockDim = nwr * (cols / KW) * 64.  PT:
// the banks are per-expert pointer tables.
template <int KW, int TPC, bool XBF, int MODE, int MAXW, bool PT>
__global__ __launch_bounds__(MAXW * 64) void skinny_splitk(SkinnyArgs a)
{
    constexpr int LS = KW / 128; // load steps per wave
    constexpr int NBC = XBF ? TPC : 2 * TPC;
    // activation units (8 elements) per thread issued up front: enough for
    // one row tile per matrix (units <= TPC * cols / 8, threads >= cols / KW * 64)
    constexpr int UMAX = TPC * KW / 512 < 1 ? 1 : (TPC * KW / 512 > 8 ? 8 : TPC * KW / 512);
    constexpr int NMAT = (MODE == MODE_GATEUP) ? 2 : 1;
    const int C = a.cols;
    const int gpr = C / 32;
    const int nwk = C / KW;
    const int NT = blockDim.x;
    const int nwr = NT / 64 / nwk;
    const int NR = nwr / NMAT;
    const int rows_wg = NR * 16;
    const int bstride = C + BPAD;
    const int sstride = gpr + 16;

    extern __shared__ __align__(16) uint8_t smem[];
    __bf16 *Bs = reinterpret_cast<__bf16 *>(smem);
    const int nun = C / 512; // 512-column units
    // With one row block per workgroup the reduction reuses the operand rows;
    // a workgroup that walks several row blocks keeps the operands and
    // double-buffers the reduction region and the scales by block parity
    // (block j's partials in buffer j % 2, block j + 1's scales stored into
    // the other scale buffer before block j's reduction barrier), so each
    // block needs one barrier: the waves go on to the next block while the
    // reducing wave sums and stores (measured: 64-expert decode layer
    // 114.4 -> 111.9 us per layer).
    const int opbytes = (NBC * bstride * 2 + 15) & ~15;
    const int redbytes = nwr * nun * 1024;
    // (a.rbw = -1: one row block per workgroup, with reduction buffers of
    // its own all the same, which saves the barrier that protects the
    // operands from the overlaid reduction)
    const int rbw = a.rbw < 0 ? -a.rbw : a.rbw;
    const bool own_red = a.rbw != 1;
    const int ssbytes = (NMAT * rows_wg * sstride + 15) & ~15;
    const int bbytes = own_red ? opbytes + 2 * redbytes : max(opbytes, redbytes);
    f32x4 *red0 = reinterpret_cast<f32x4 *>(smem + (own_red ? opbytes : 0));
    uint8_t *Ss0 = smem + ((bbytes + 15) & ~15);

    // Work item and row blocks.  GEMM: XCD-grouped logical id, token chunks
    // fastest, so the chunks of a row block share its weights in one XCD's
    // L2; a.rbw consecutive row blocks per workgroup.  Expert bank: plain
    // dispatch order, row blocks fastest, each workgroup walking its item's
    // row blocks nrbg apart, so the workgroups resident at any moment read a
    // few experts' matrices front to back in adjacent blocks (measured,
    // 64-expert decode layer: 110.6 us with items fastest, 102.7 with row
    // blocks fastest, 102.0 with the strided walk; XCD-grouped ids over the
    // real items 106.0).  Down: an upper-bound grid of nrbg = nrb / a.rbw
    // workgroups per item; the surplus is dispatched last and exits.
    // Gate/up: a grid of about one round of resident workgroups (at least
    // one per item bound) that the n_work real items share on the device,
    // nrbg = grid / n_work each, so that no last round of a few long
    // workgroups is left (measured: gate/up 64.8 -> 63.1 us; the shorter
    // down workgroups were slower so, 29.4 -> 32.8 us).
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lid = MODE == MODE_GEMM ? xcd_logical(blockIdx.x, gridDim.x) : (int)blockIdx.x;
    TileMap tm;
    int nrbg;
    __shared__ int fz[FG_WORDS];
    if (MODE == MODE_GATEUP && a.fuse_group) {
        // the routing grouped here (no grouping kernel before this one):
        // one wave ranks the pairs, the workgroup reads its item from LDS
        if (wave == 0)
            fused_group(a, TPC, lid, (int)gridDim.x, blockIdx.x == 0, fz);
        __syncthreads();
        if (fz[3] <= 0)
            return;
        nrbg = min(a.nrb, max(1, (int)gridDim.x / max(1, fz[0])));
        tm.row0 = 0;
        tm.expert = fz[1];
        tm.slot0 = fz[2];
        tm.ntok = fz[3];
        tm.rowmap = fz + 4;
        tm.pairmap = fz + 4 + 16;
    } else {
        nrbg = MODE == MODE_GEMM   ? 1
               : MODE == MODE_DOWN ? (a.nrb + rbw - 1) / rbw
                                   : min(a.nrb, max(1, (int)gridDim.x / max(1, *a.n_work)));
        if (!item_map<MODE, TPC>(a, MODE == MODE_GEMM ? lid % a.nch : lid / nrbg, tm))
            return;
    }
    const int rstride = MODE == MODE_GEMM ? 1 : nrbg;
    const int rb_first = MODE == MODE_GEMM ? (lid / a.nch) * rbw : lid % nrbg;
    // (a gate/up workgroup without reduction buffers of its own runs in a
    // grid with a workgroup per row block and takes one block)
    const int rb_end = MODE == MODE_GEMM   ? min(a.nrb, rb_first + rbw)
                       : MODE == MODE_DOWN ? min(a.nrb, rb_first + rbw * rstride)
                       : a.rbw == 1        ? min(a.nrb, rb_first + 1)
                                           : a.nrb;

    const int wr = wave / nwk, wk = wave % nwk;
    const int mat = wr / NR, tile = wr % NR;
    const int li = lane & 15, ls = lane >> 4;
    const int R = a.rows;
    // V4.1 route weight of this lane's token column, read once here rather
    // than through two dependent loads in every row block's epilogue
    float opw = 0.0f;
    if (MODE == MODE_GATEUP && a.v41 && (XBF ? li : (li & 7)) < tm.ntok)
        opw = a.pair_w[tm.pairmap[XBF ? li : (li & 7)]];
    const uint8_t *A0 =
        MODE == MODE_GEMM ? a.w0 : expert_base<PT>(a.w0, tm.expert, a.expert_stride);
    const uint8_t *A1 =
        (MODE == MODE_GATEUP) ? expert_base<PT>(a.w1, tm.expert, a.expert_stride) : A0;
    const int64_t code_bytes = (int64_t)R * (C / 2);

    // ---- 1.-2. activation, scale and weight loads.  The activations and
    // scales go first so that staging them does not wait for HBM (measured:
    // starting the weight stream first in the expert gate/up, whose
    // activation rows sit behind one more dependent load, made the 64-expert
    // decode layer 6 % slower).
    const int segs = C / 8;
    const int units = tm.ntok * segs;
    float xv[UMAX][8];
    auto load_acts = [&]() {
#pragma unroll
        for (int q = 0; q < UMAX; ++q) {
            const int u = tid + q * NT;
            if (u < units) {
                const int t = u / segs;
                load_unit<MODE, XBF>(a, tm, t, u - t * segs, C, xv[q]);
            }
        }
    };
    auto arow_of = [&](int row0) {
        const int r = min(row0 + tile * 16 + li, R - 1);
        return (mat ? A1 : A0) + (int64_t)r * (C / 2) + wk * (KW / 2) + ls * 16;
    };
    u32x4 cw[LS];
    auto load_codes = [&]() {
        const uint8_t *arow = arow_of(rb_first * rows_wg);
#pragma unroll
        for (int L = 0; L < LS; ++L)
            cw[L] = *reinterpret_cast<const u32x4 *>(arow + L * 64);
    };
    load_acts();
    // scale chunk of this thread: one 16-byte chunk per thread per row block
    // (threads past the chunk count re-read the last chunk and do not store)
    const int sch = gpr / 16;                // 16-byte scale chunks per row
    const int sunits = NMAT * rows_wg * sch; // <= NT
    const int su = min(tid, sunits - 1);
    const int sm = su / (rows_wg * sch);
    const int srr = su / sch; // m * rows_wg + row
    const int sc16 = su % sch;
    auto load_scales = [&](int row0) {
        // rows past the end read row R-1: their outputs are never stored,
        // and an MFMA output row depends on its own A row only
        const int r = min(row0 + srr - sm * rows_wg, R - 1);
        return *reinterpret_cast<const u32x4 *>((sm ? A1 : A0) + code_bytes + (int64_t)r * gpr +
                                                 sc16 * 16);
    };
    // plain GEMM: each lane loads its own row's 16 (KW = 512) or 32 scale
    // bytes of the slab with its codes, so the first barrier does not wait
    // for HBM (measured -1 % on the 4096 x 4096 and 14336 x 4096 GEMVs; the
    // expert gate/up, with two matrices and 1024-column slabs, keeps the
    // workgroup's one coalesced LDS staging: +1.6 % per lane)
    constexpr bool DS = MODE == MODE_GEMM;
    constexpr int SUPW = KW / 512;
    auto load_sd = [&](int row0, u32x4 *dstv) {
        const int r = min(row0 + tile * 16 + li, R - 1);
        const uint8_t *sp = (mat ? A1 : A0) + code_bytes + (int64_t)r * gpr + wk * (KW / 32);
#pragma unroll
        for (int q = 0; q < SUPW; ++q)
            dstv[q] = *reinterpret_cast<const u32x4 *>(sp + 16 * q);
    };
    u32x4 sv = {0u, 0u, 0u, 0u}, sd[SUPW], sdn[SUPW];
    if constexpr (DS)
        load_sd(rb_first * rows_wg, sd);
    else
        sv = load_scales(rb_first * rows_wg);
    load_codes();

    // ---- 3. activations and scales -> LDS
#pragma unroll
    for (int q = 0; q < UMAX; ++q) {
        const int u = tid + q * NT;
        if (u < units) {
            const int t = u / segs;
            store_unit<XBF>(Bs, bstride, tm.ntok, t, u - t * segs, xv[q]);
        }
    }
    for (int u = tid + UMAX * NT; u < units; u += NT) { // beyond the up-front batch
        float v[8];
        const int t = u / segs;
        load_unit<MODE, XBF>(a, tm, t, u - t * segs, C, v);
        store_unit<XBF>(Bs, bstride, tm.ntok, t, u - t * segs, v);
    }
    if (!DS && tid < sunits)
        *reinterpret_cast<u32x4 *>(Ss0 + srr * sstride + sc16 * 16) = sv;
    __syncthreads();

    const __bf16 *bb = Bs + b_row<XBF>(li, tm.ntok) * bstride + wk * KW + ls * 32;
    const int srow_off = (mat * rows_wg + tile * 16 + li) * sstride + wk * (KW / 32);
    constexpr int UPW = KW / 512; // 512-column units per wave
    for (int rb = rb_first; rb < rb_end; rb += rstride) {
        tm.row0 = rb * rows_wg;
        const bool more = rb + rstride < rb_end;
        const int par = ((rb - rb_first) / rstride) & 1;
        const uint8_t *srow = Ss0 + par * ssbytes + srow_off;
        f32x4 *red = red0 + par * (redbytes / 16);
        // next row block: scales, then weights (younger than everything this
        // block waits for).  The expert bank issues the next block's weight
        // loads after this block's MFMA work, into the registers it has just
        // consumed, so they fly during the reduction and store: 16 fewer
        // VGPRs (decode gate/up 118 -> 104, down 110 -> 94; measured 64-expert
        // decode layer 117.0 -> 114.3 us).  The plain GEMM, which walks
        // several row blocks only at very large row counts, keeps the
        // separate prefetch registers (the 4096 x 4096 matvec was 0.7 %
        // slower with the late loads).
        constexpr bool LATE = MODE != MODE_GEMM;
        u32x4 cwn[LATE ? 1 : LS];
        auto load_next_codes = [&](u32x4 *dst) {
            const uint8_t *arow = arow_of(tm.row0 + rstride * rows_wg);
#pragma unroll
            for (int L = 0; L < LS; ++L)
                dst[L] = *reinterpret_cast<const u32x4 *>(arow + L * 64);
        };
        if (more) {
            if constexpr (DS)
                load_sd(tm.row0 + rstride * rows_wg, sdn);
            else
                sv = load_scales(tm.row0 + rstride * rows_wg);
            if constexpr (!LATE)
                load_next_codes(cwn);
        }

        // ---- 4. decode + MFMA over this wave's slab
        f32x4 part[UPW];
#pragma unroll
        for (int un = 0; un < UPW; ++un) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            // Plain GEMV (one token, 512-column slabs, 76 VGPRs otherwise):
            // the unit's 16 operand fragments are read from LDS together and
            // waited for once, so the MFMA steps do not each wait for an LDS
            // round trip (the compiler otherwise issues each read about one
            // MFMA ahead).  Measured, 4096 x 4096 b = 1: 4.74 -> 4.58 us,
            // same bits; at b = 8 (1 % slower) and with 1024-column slabs
            // (168 VGPRs, one workgroup per CU: 14336 x 4096 b = 1 3 %
            // slower) it is not used.
            constexpr bool BPRE = MODE == MODE_GEMM && MAXW <= 8 && TPC == 1 && KW == 512;
            bf16x8 bu[BPRE ? 4 : 1][4];
            if constexpr (BPRE) {
#pragma unroll
                for (int l = 0; l < 4; ++l)
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        bu[l][m] =
                            *reinterpret_cast<const bf16x8 *>(bb + (un * 4 + l) * 128 + m * 8);
#pragma unroll
                for (int l = 0; l < 4; ++l)
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        asm volatile("" : "+v"(bu[l][m]));
            }
#pragma unroll
            for (int L = un * 4; L < un * 4 + 4; ++L) {
                const float scf =
                    DS ? e8m0_operand_of(sd[L / 4][L % 4], ls)
                       : e8m0_operand_of(*reinterpret_cast<const uint32_t *>(srow + 4 * L), ls);
                bf16x8 bv[4];
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    bv[m] = BPRE ? bu[BPRE ? L - un * 4 : 0][m]
                                 : *reinterpret_cast<const bf16x8 *>(bb + L * 128 + m * 8);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const bf16x8 av = decode8_bf16(cw[L][m], scf);
                    acc = mfma16x16x32(av, bv[m], acc);
                }
            }
            part[un] = acc;
        }

        if constexpr (LATE) {
            if (more)
                load_next_codes(cw);
        }

        // ---- 5. sum the units in order, then store
        if (!own_red)
            __syncthreads(); // every wave is done with the operands red overlays
#pragma unroll
        for (int un = 0; un < UPW; ++un)
            red[(wr * nun + wk * UPW + un) * 64 + lane] = part[un];
        // the next block's scales, into the buffer no wave reads in this block
        if (!DS && more && tid < sunits)
            *reinterpret_cast<u32x4 *>(Ss0 + (par ^ 1) * ssbytes + srr * sstride + sc16 * 16) = sv;
        __syncthreads();
        // The tile's epilogue (unit sums, hi + lo fold, activation, store)
        // is split over up to four of its waves by accumulator component c
        // (output rows 4 ls + c), so that no single wave trails the others
        // into the next block's barrier.
        {
            const int q = mat * nwk + wk; // this wave's rank among the tile's waves
            const int nred = min(4, NMAT * nwk);
            if (q < nred) {
                const float *rf = reinterpret_cast<const float *>(red);
                for (int c = q; c < 4; c += nred) {
                    float g = rf[((tile * nun) * 64 + lane) * 4 + c];
                    for (int k = 1; k < nun; ++k)
                        g += rf[((tile * nun + k) * 64 + lane) * 4 + c];
                    float u = g;
                    if (MODE == MODE_GATEUP) {
                        const int wu = NR + tile;
                        u = rf[((wu * nun) * 64 + lane) * 4 + c];
                        for (int k = 1; k < nun; ++k)
                            u += rf[((wu * nun + k) * 64 + lane) * 4 + c];
                    }
                    store_row<MODE, XBF>(a, tm, g, u, tile, lane, c, opw);
                }
            }
        }
        if (!more)
            break;
#pragma unroll
        for (int q = 0; q < SUPW; ++q)
            sd[q] = sdn[q];
        if constexpr (!LATE) {
#pragma unroll
            for (int L = 0; L < LS; ++L)
                cw[L] = cwn[L];
        }
        // no barrier here: the next block writes the other reduction buffer
        // and reads the scales stored before this block's barrier; this
        // block's buffers are reused two blocks on, after the next block's
        // barrier, which the reducing wave reaches only once it is done
    }
}

// Generic kernel: any cols % 32 == 0 (K steps of 128 columns, guarded, one
// wave per row tile).  Used for column counts the split-K kernel does not
// take.
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
    const uint8_t *A0 = MODE == MODE_GEMM
                            ? a.w0
                            : expert_base_rt(a.w0, a.ptr_table, tm.expert, a.expert_stride);
    const uint8_t *A1 = (MODE == MODE_GATEUP)
                            ? expert_base_rt(a.w1, a.ptr_table, tm.expert, a.expert_stride)
                            : A0;
    const int64_t code_bytes = (int64_t)R * (C / 2);

    // activations -> LDS (zero beyond C up to cpad)
    const int segs = cpad / 8;
    for (int t = 0; t < tm.ntok; ++t) {
        const int64_t row = token_row<MODE>(tm, t);
        for (int seg = tid; seg < segs; seg += NT) {
            float v[8];
            const int c = seg * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float xvv = 0.f;
                if (c + i < C) {
                    if (XBF)
                        xvv = bf16_bits_to_f32(
                            reinterpret_cast<const uint16_t *>(a.x)[row * C + c + i]);
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
        const int r = min(tm.row0 + rr, R - 1);
        Ss[(m * ROWS_WG + rr) * sstride + g] = ((m ? A1 : A0) + code_bytes)[(int64_t)r * gpr + g];
    }
    __syncthreads();

    const int mat = (MODE == MODE_GATEUP) ? wave / TILES : 0;
    const int tile = (MODE == MODE_GATEUP) ? wave % TILES : wave;
    const int r = min(tm.row0 + tile * 16 + li, R - 1);
    const uint8_t *arow = (mat ? A1 : A0) + (int64_t)r * (C / 2);
    const uint8_t *srow = Ss + (mat * ROWS_WG + tile * 16 + li) * sstride;
    const __bf16 *bb = Bs + b_row<XBF>(li, tm.ntok) * bstride + ls * 32;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc = zero4, uacc = zero4;
    const int nsteps = cpad / 128;
    for (int st = 0; st < nsteps; ++st) {
        const int g = st * 4 + ls;
        u32x4 cw = {0, 0, 0, 0};
        uint32_t k = 127;
        if (g < gpr) {
            cw = *reinterpret_cast<const u32x4 *>(arow + (int64_t)g * 16);
            k = srow[g];
        }
        const float scf = e8m0_operand(k);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(bb + st * 128 + m * 8);
            uacc = mfma16x16x32(decode8_bf16(cw[m], scf), bv, uacc);
        }
        if ((st & 3) == 3 || st + 1 == nsteps) { // end of a 512-column unit
            acc = st < 4 ? uacc : acc + uacc;
            uacc = zero4;
        }
    }
    if (MODE == MODE_GATEUP) {
        // up waves hand their tile to the gate waves through LDS
        if (mat == 1)
            reinterpret_cast<f32x4 *>(xch)[tile * 64 + lane] = acc;
        __syncthreads();
        if (mat == 1)
            return;
        store_tile<MODE, XBF>(a, tm, acc, reinterpret_cast<f32x4 *>(xch)[tile * 64 + lane], tile,
                              lane);
        return;
    }
    store_tile<MODE, XBF>(a, tm, acc, acc, tile, lane);
}

// ---------------------------------------------------------------------------
// Host side: instantiation table, launch shape and launch
// ---------------------------------------------------------------------------

namespace {

constexpr int NW_GENERIC = 4;
// Dynamic LDS per workgroup: the CU's 160 KB less 512 bytes for the static
// LDS of the gate/up kernels that group the routing themselves (400 bytes),
// so that one opt-in value fits every kernel of the table.
constexpr int LDS_MAX = 160 * 1024 - 512;
static_assert(FG_WORDS * 4 <= 512, "static LDS of the in-kernel grouping");
// Row blocks per split-K workgroup: at most RB_MAX, and only while the grid
// keeps RB_MIN_WGS workgroups (4 per CU; 8 before the reduction was
// double-buffered: 64-expert decode layer 112.2 -> 111.3 us with 4).
constexpr int RB_MAX = 16;
constexpr int RB_MIN_WGS = 1024;

typedef void (*KernelFn)(SkinnyArgs);

struct Entry {
    int mode, xbf, kw, tpc, maxw, pt; // kw 0 = generic (either kind of bank)
    KernelFn fn;
};

#define MX_K(MODE, XBF, KW, TPC, MAXW, PT) \
    {MODE, XBF, KW, TPC, MAXW, PT, skinny_splitk<KW, TPC, (bool)XBF, MODE, MAXW, (bool)PT>}
#define MX_KW(MODE, XBF, KW, TPC, PT) \
    MX_K(MODE, XBF, KW, TPC, 8, PT), MX_K(MODE, XBF, KW, TPC, 16, PT)
#define MX_F32(MODE, KW, PT) \
    MX_KW(MODE, 0, KW, 1, PT), MX_KW(MODE, 0, KW, 2, PT), MX_KW(MODE, 0, KW, 4, PT), \
        MX_KW(MODE, 0, KW, 8, PT)
#define MX_B16(MODE, KW, PT) \
    MX_KW(MODE, 1, KW, 2, PT), MX_KW(MODE, 1, KW, 4, PT), MX_KW(MODE, 1, KW, 8, PT), \
        MX_KW(MODE, 1, KW, 16, PT)
#define MX_G(MODE, XBF, TPC) \
    {MODE, XBF, 0, TPC, NW_GENERIC, 0, skinny_generic<NW_GENERIC, TPC, (bool)XBF, MODE>}
#define MX_GEN(MODE) \
    MX_G(MODE, 0, 1), MX_G(MODE, 0, 2), MX_G(MODE, 0, 4), MX_G(MODE, 0, 8), MX_G(MODE, 1, 2), \
        MX_G(MODE, 1, 4), MX_G(MODE, 1, 8), MX_G(MODE, 1, 16)
#define MX_SPLITK(MODE, PT) \
    MX_F32(MODE, 512, PT), MX_F32(MODE, 1024, PT), MX_B16(MODE, 512, PT), MX_B16(MODE, 1024, PT)
#define MX_MODE(MODE) MX_SPLITK(MODE, 0), MX_GEN(MODE)
// expert-bank modes also over per-expert pointer tables
#define MX_MODE_BANK(MODE) MX_SPLITK(MODE, 0), MX_SPLITK(MODE, 1), MX_GEN(MODE)

const Entry kTable[] = {MX_MODE(MODE_GEMM), MX_MODE_BANK(MODE_GATEUP), MX_MODE_BANK(MODE_DOWN)};
constexpr int kTableSize = sizeof(kTable) / sizeof(kTable[0]);

const Entry *find(int mode, bool xbf, int kw, int tpc, int maxw, bool pt = false)
{
    for (const Entry &e : kTable)
        if (e.mode == mode && e.xbf == (int)xbf && e.kw == kw && e.tpc == tpc &&
            (kw == 0 || (e.maxw == maxw && e.pt == (int)pt)))
            return &e;
    return nullptr;
}

int nmat(int mode) { return mode == MODE_GATEUP ? 2 : 1; }

size_t lds_splitk(int mode, bool xbf, int cols, int kw, int tpc, int nr, int rbw)
{
    const int nbc = xbf ? tpc : 2 * tpc;
    const int nwr = nr * nmat(mode);
    const size_t opbytes = ((size_t)nbc * (cols + BPAD) * 2 + 15) & ~(size_t)15;
    const size_t redbytes = (size_t)nwr * (cols / 512) * 1024;
    const size_t ssbytes = (size_t)nwr * 16 * (cols / 32 + 16);
    (void)kw;
    if (rbw > 1) // reduction and scale regions double-buffered
        return ((opbytes + 2 * redbytes + 15) & ~(size_t)15) + 2 * ((ssbytes + 15) & ~(size_t)15);
    const size_t bbytes = std::max(opbytes, redbytes);
    return ((bbytes + 15) & ~(size_t)15) + ssbytes;
}

size_t lds_generic(int mode, bool xbf, int cols, int tpc)
{
    const int tiles = mode == MODE_GATEUP ? NW_GENERIC / 2 : NW_GENERIC;
    const int nbc = xbf ? tpc : 2 * tpc;
    const int cpad = (cols + 127) / 128 * 128;
    const int gpr = cols / 32;
    size_t b = (size_t)nbc * (cpad + BPAD) * 2;
    b += (size_t)nmat(mode) * tiles * 16 * ((gpr + 15) / 16 * 16 + 16);
    if (mode == MODE_GATEUP)
        b += (size_t)tiles * 64 * 16;
    return b;
}

// K slab width for the split-K kernel (0: use the generic kernel).
int pick_kw(int mode, int cols)
{
    for (int kw : {512, 1024})
        if (cols % kw == 0 && (cols / kw) * nmat(mode) <= 16)
            return kw;
    return 0;
}

} // namespace

int skinny_pick_tpc(int mode, bool xbf, int cols, int want)
{
    static const int f32_opts[] = {1, 2, 4, 8};
    static const int b16_opts[] = {2, 4, 8, 16};
    const int *opts = xbf ? b16_opts : f32_opts;
    const int kw = pick_kw(mode, cols);
    int best = 0;
    for (int i = 0; i < 4; ++i) {
        const int t = opts[i];
        const size_t lds =
            kw ? lds_splitk(mode, xbf, cols, kw, t, 1, 1) : lds_generic(mode, xbf, cols, t);
        if (lds > (size_t)LDS_MAX)
            break;
        best = t;
        if (t >= want)
            break;
    }
    return best;
}

namespace {

// Compute units of the current device (cached per device).
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0)
        return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
        n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Workgroups of this kernel that fit on one CU (registers, LDS, waves), as
// the runtime computes it; cached per (kernel, threads, LDS).
int wgs_per_cu(const Entry *e, int threads, size_t lds)
{
    struct Key {
        const Entry *e;
        int threads;
        size_t lds;
        int n;
    };
    static std::mutex mu;
    static Key cache[128];
    static int used = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].e == e && cache[i].threads == threads && cache[i].lds == lds)
            return cache[i].n;
    int n = 0;
    // (a failed query leaves no error behind for the next launch check)
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute(reinterpret_cast<const void *>(e->fn),
                            hipFuncAttributeMaxDynamicSharedMemorySize, LDS_MAX) != hipSuccess)
        (void)hipGetLastError();
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(e->fn),
                                                     threads, lds) != hipSuccess ||
        n < 1) {
        (void)hipGetLastError();
        n = 1;
    }
    if (used < 128)
        cache[used++] = Key{e, threads, lds, n};
    return n;
}

} // namespace

SkinnyShape skinny_shape(int mode, bool xbf, int rows, int cols, int tpc, int64_t items)
{
    SkinnyShape s = {};
    s.kw = pick_kw(mode, cols);
    s.tpc = tpc;
    s.rbw = 1;
    if (!s.kw) {
        s.nr = mode == MODE_GATEUP ? NW_GENERIC / 2 : NW_GENERIC;
        s.threads = NW_GENERIC * 64;
        s.lds = lds_generic(mode, xbf, cols, tpc);
        s.rows_per_wg = s.nr * 16;
        return s;
    }
    // Candidates: slab width x row tiles.  Measured preference order on
    // MI355X (cold 8.9 MB and 31 MB weights, b = 1..8): fewest rounds of
    // co-resident workgroups; then at least 256 workgroups (one per CU);
    // then 8-wave workgroups; then the fewest workgroups.
    bool found = false;
    int64_t bk0 = 0, bk1 = 0, bk2 = 0, bk3 = 0;
    for (int kw : {512, 1024}) {
        if (cols % kw != 0)
            continue;
        const int nwk = cols / kw;
        for (int nr = 1; nr <= 4; nr *= 2) {
            const int waves = nr * nmat(mode) * nwk;
            if (waves > 16)
                break;
            const size_t lds = lds_splitk(mode, xbf, cols, kw, tpc, nr, 1);
            if (lds > (size_t)LDS_MAX)
                break;
            const Entry *e = find(mode, xbf, kw, tpc, waves <= 8 ? 8 : 16);
            if (!e)
                continue;
            const int per_cu = wgs_per_cu(e, waves * 64, lds);
            const int64_t wgs = (int64_t)((rows + nr * 16 - 1) / (nr * 16)) * items;
            const int64_t k0 = (wgs + 256LL * per_cu - 1) / (256LL * per_cu);
            const int64_t k1 = wgs < 256 ? 1 : 0;
            const int64_t k2 = waves > 8 ? waves - 8 : 8 - waves;
            const int64_t k3 = wgs < 256 ? -wgs : wgs;
            if (!found || k0 < bk0 || (k0 == bk0 && (k1 < bk1 || (k1 == bk1 &&
                (k2 < bk2 || (k2 == bk2 && k3 < bk3)))))) {
                found = true;
                bk0 = k0, bk1 = k1, bk2 = k2, bk3 = k3;
                s.kw = kw;
                s.nr = nr;
                s.threads = waves * 64;
                s.lds = lds;
            }
        }
    }
    if (!found) { // no split-K shape fits: the generic kernel
        s.kw = 0;
        s.nr = mode == MODE_GATEUP ? NW_GENERIC / 2 : NW_GENERIC;
        s.threads = NW_GENERIC * 64;
        s.lds = lds_generic(mode, xbf, cols, tpc);
    }
    s.rows_per_wg = s.nr * 16;
    s.persist_wgs = 0;
    if (s.kw && mode == MODE_GATEUP) {
        // Expert bank: a grid of about one round of resident workgroups,
        // shared by the items on the device (reduction and scale buffers of
        // their own, so that a workgroup walks row blocks with one barrier
        // each).
        const Entry *e = find(mode, xbf, s.kw, tpc, s.threads <= 512 ? 8 : 16);
        const size_t lds2 = lds_splitk(mode, xbf, cols, s.kw, tpc, s.nr, 2);
        const int64_t nrb = (rows + s.rows_per_wg - 1) / s.rows_per_wg;
        if (e && nrb > 1 && lds2 <= (size_t)LDS_MAX) {
            s.rbw = 2;
            s.lds = lds2;
        }
        const int per_cu = e ? wgs_per_cu(e, s.threads, s.lds) : 1;
        s.persist_wgs = s.rbw > 1 ? std::max<int64_t>((int64_t)device_cus() * per_cu, items)
                                  : nrb * items;
    } else if (s.kw) {
        // Walk several row blocks per workgroup while the grid stays above
        // RB_MIN_WGS workgroups and the workgroups per CU do not drop (the
        // walking kernel needs its own reduction region): the tokens are
        // staged once per workgroup, so this divides the activation reads by
        // rbw.  Measured: -6% on the 64-expert decode gate/up, -38% on the
        // 256-expert prefill; a lower occupancy cost more than it saved.
        const int64_t nrb = (rows + s.rows_per_wg - 1) / s.rows_per_wg;
        const Entry *e = find(mode, xbf, s.kw, tpc, s.threads <= 512 ? 8 : 16);
        const int per_cu = e ? wgs_per_cu(e, s.threads, s.lds) : 0;
        while (e && s.rbw < RB_MAX &&
               ((nrb + 2 * s.rbw - 1) / (2 * s.rbw)) * items >= RB_MIN_WGS) {
            const size_t lds = lds_splitk(mode, xbf, cols, s.kw, tpc, s.nr, 2 * s.rbw);
            if (lds > (size_t)LDS_MAX || wgs_per_cu(e, s.threads, lds) < per_cu)
                break;
            s.rbw *= 2;
            s.lds = lds;
        }
        // one block per workgroup: reduction buffers of its own when they
        // cost no occupancy (one barrier per block instead of two)
        if (e && s.rbw == 1) {
            const size_t lds = lds_splitk(mode, xbf, cols, s.kw, tpc, s.nr, 2);
            if (lds <= (size_t)LDS_MAX && wgs_per_cu(e, s.threads, lds) >= per_cu) {
                s.rbw = -1;
                s.lds = lds;
            }
        }
    }
    return s;
}

int64_t skinny_blocks(const SkinnyShape &s, int rows, int nch)
{
    const int64_t nrb = (rows + s.rows_per_wg - 1) / s.rows_per_wg;
    if (s.persist_wgs > 0) // expert bank: the items share the grid on the device
        return std::min(s.persist_wgs, nrb * nch);
    const int rbw = s.rbw < 0 ? -s.rbw : s.rbw;
    return (nrb + rbw - 1) / rbw * nch;
}

hipError_t skinny_launch(int mode, bool xbf, const SkinnyShape &s, SkinnyArgs a,
                         hipStream_t stream)
{
    a.nrb = (a.rows + s.rows_per_wg - 1) / s.rows_per_wg;
    a.rbw = s.kw ? s.rbw : 1;
    const unsigned blocks = (unsigned)skinny_blocks(s, a.rows, a.nch);
    const int waves = s.threads / 64;
    const Entry *e = find(mode, xbf, s.kw, s.tpc, waves <= 8 ? 8 : 16, a.ptr_table != 0);
    if (!e)
        return hipErrorInvalidValue;
    // Opt in to more than 64 KB of LDS once per kernel, so that later
    // launches (including ones under graph capture) make no attribute calls.
    static std::atomic<uint8_t> opted[kTableSize];
    std::atomic<uint8_t> &flag = opted[e - kTable];
    if (s.lds > 64 * 1024 && !flag.load(std::memory_order_acquire)) {
        hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void *>(e->fn),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, LDS_MAX);
        if (st != hipSuccess)
            return st;
        flag.store(1, std::memory_order_release);
    }
    hipLaunchKernelGGL(e->fn, dim3(blocks), dim3(s.threads), s.lds, stream, a);
    return hipGetLastError();
}

} // namespace mx
