// MXFP4 x tens of activation rows: the tiled schedule of the same product,
// for work items that carry many tokens (hot experts of a prefill bank,
// GEMMs with more tokens than one skinny chunk).  The arithmetic is the
// skinny kernel's (exact bf16 decode of each weight by
// v_cvt_scalef32_pk_bf16_fp4, fp32 activations split into bf16 hi + lo
// columns, v_mfma_f32_16x16x32_bf16, fp32 accumulate, the library's
// canonical summation order), so every token's result is bit-identical to
// its own matvec.  What differs is the schedule:
//
//  * A workgroup of NW waves owns NW * RT * 16 output rows of every matrix
//    of the mode, RT row tiles per wave (gate and up rows of one wave are the
//    same rows, so SwiGLU needs no exchange) and up to 16 * NC MFMA columns (16 * NC bf16
//    tokens, or 8 * NC fp32 tokens as hi/lo pairs), and runs the whole K
//    loop in 128-column steps.
//  * Operands stream through a ring of four LDS stages filled by direct
//    global -> LDS loads (global_load_lds_dwordx4 / _dword): per step, each
//    wave loads its own 16 rows' code bytes (1 KB per matrix) and scale
//    bytes, and a share of the step's activation slab (only the tokens the
//    item has column tiles for), which all waves read.  Three steps are in
//    flight while one is computed, with no registers held for them.
//  * Every wave issues the same number of loads per stage, and the loop has
//    no other vector memory operations, so "stage s has landed" is one
//    constant vmcnt wait, followed by one workgroup barrier per step (which
//    also frees the stage loaded next).
//  * The activation slab is stored XOR-swizzled (16-byte chunk k of token t
//    at position k ^ (t & 15)), so the 16 lanes reading one MFMA fragment
//    hit distinct banks.
//  * fp32 tokens: once a step's slab has landed, the workgroup splits it
//    into bf16 hi / lo rows (hi of token 8c + i in MFMA column i of tile c,
//    lo in column 8 + i), once per step rather than once per wave and
//    fragment, behind one more barrier; the MFMA then reads these rows the
//    way it reads bf16 tokens.
//  * The expert bank's down product walks two row blocks per workgroup:
//    the stage ring runs on into the second block (the item's slab again,
//    the weight rows one block further), and each block's outputs go out
//    as a fixed number of stores per wave (rows and tokens past the end
//    clamped to the last ones, whose values those lanes hold too), so the
//    waits stay constants: the first two steps after a block's stores count
//    them as well.  The blocks are written out one after the other rather
//    than looped over, so that every path reaching a wait issued the same
//    loads and stores before it and the compiler adds no waits of its own.
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

constexpr int TKS = 128; // columns per K step
// Row blocks per workgroup in the expert bank's down product: the ring of
// LDS stages runs on from one block into the next (same item, same token
// rows, the weight rows RB further on), so a workgroup's start-up loads are
// paid once per two blocks (measured, 256-expert prefill layer: 1389 ->
// 1369 us median; three and four blocks per workgroup lost to the longer
// last round: +12 / +17 us against two)
constexpr int WALK_DOWN = 2;
constexpr int TNS = 4;   // LDS stages (= steps per 512-column unit)

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

template <int NW, int RT, int NC, bool XBF, int MODE, bool PT>
__global__ __launch_bounds__(NW * 64) void tiled_kernel(SkinnyArgs a)
{
    constexpr int NMAT = (MODE == MODE_GATEUP) ? 2 : 1;
    constexpr int MT = NMAT * RT;               // A tiles per wave: tile mt = mat * RT + rt
    static_assert(MT <= 4, "one 16-byte scale load per wave covers at most 4 tiles");
    constexpr int ES = XBF ? 2 : 4;             // activation element bytes
    constexpr int NCOL = 16 * NC;               // MFMA columns
    constexpr int TPD = XBF ? NCOL : NCOL / 2;  // tokens per work item
    constexpr int RB = NW * RT * 16;            // output rows per workgroup
    constexpr int ROWB = TKS * ES;              // bytes of one token per step
    constexpr int ACT_BYTES = TPD * ROWB;       // activation slab per step (at most)
    // Codes: expert bank, two steps per load into pair buffers (whole cache
    // lines, see below); plain GEMM, one step per load with the step's
    // stage (its grids hold about one workgroup per CU, where the pairs'
    // shorter lead showed: 14336 x 4096 b = 16 / 32 fp32 17.6 / 20.5 ->
    // 18.4 / 21.2 us, bf16 b = 64 19.3 -> 20.4 us)
    constexpr bool PAIRS = MODE != MODE_GEMM;
    // stage layout: [codes [NW][MT][1 KB] without pairs] | slab
    constexpr int ACT_OFF = PAIRS ? 0 : NW * MT * 1024;
    constexpr int STAGE = ACT_OFF + ACT_BYTES;
    constexpr int PBB = PAIRS ? NW * MT * 2048 : 16;

    // one variable per stage and per code buffer: loads into one and reads
    // of another are then known not to alias, and the compiler adds no waits
    // of its own
    __shared__ __align__(16) uint8_t st0[STAGE], st1[STAGE], st2[STAGE], st3[STAGE];
    // codes of a pair of steps (256 columns) by pair parity: [NW][MT][2][1 KB],
    // 1 KB i of a tile holding rows 8i .. 8i + 7 x 128 bytes (see below)
    __shared__ __align__(16) uint8_t pb0[PBB], pb1[PBB];
    // scale bytes of one 512-column unit: [NW][64 lanes][16 B], loaded with
    // stage 0 (the unit's first step) and read into registers at that step
    __shared__ __align__(16) uint8_t scs[NW * 1024];
    // fp32 tokens: the current step's slab as bf16 hi / lo rows, 16 * NC rows
    // of 128 columns, 16-byte chunk p of row r at position p ^ (r & 15)
    __shared__ __align__(16) uint8_t cvb[XBF ? 16 : NC * 16 * 256];
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

    const int C = a.cols;
    const int R = a.rows;
    const int gpr = C / 32;
    const int nsteps = C / TKS; // a multiple of 4 (cols % 512 == 0)
    const int nunits = nsteps / 4;

    // ---- work item.  GEMM: XCD-grouped logical id, token chunks fastest, so
    // the chunks of a row block share its weights in one XCD's L2.  Expert
    // bank: plain dispatch order, row blocks fastest over the n_work real
    // items (the grid is sized by an upper bound; the surplus workgroups,
    // dispatched last, exit), so the resident workgroups stream adjacent
    // blocks of a few experts' matrices (measured, 256-expert prefill layer:
    // 1563 us with XCD-grouped ids, 1528 us in dispatch order).  The down
    // product's workgroups each take WALK consecutive row blocks of their
    // item (nblk: fewer at the matrix's end).
    constexpr int WALK = MODE == MODE_DOWN ? WALK_DOWN : 1;
    static_assert(WALK >= 1 && WALK <= 4, "row blocks per workgroup");
    int sub, row0, nblk = 1;
    if (MODE == MODE_GEMM) {
        const int lid = xcd_logical(blockIdx.x, gridDim.x);
        sub = lid % a.nch;
        row0 = (lid / a.nch) * RB;
    } else {
        const int nrb = (R + RB - 1) / RB;
        const int nrbw = (nrb + WALK - 1) / WALK;
        const int real = *a.n_work * nrbw;
        if ((int)blockIdx.x >= real)
            return;
        const int lid = blockIdx.x;
        sub = lid / nrbw;
        row0 = (lid % nrbw) * WALK * RB;
        nblk = min(WALK, nrb - (lid % nrbw) * WALK);
    }
    int ntok, slot0, expert = 0;
    if (MODE == MODE_GEMM) {
        slot0 = sub * TPD;
        ntok = min(TPD, a.b - slot0);
    } else {
        const int4 wk = reinterpret_cast<const int4 *>(a.work)[sub];
        expert = wk.x;
        slot0 = wk.y;
        ntok = wk.z;
    }
    const int nct = XBF ? (ntok + 15) / 16 : (ntok + 7) / 8; // column tiles in use

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, ls = lane >> 4;
    const int64_t code_bytes = (int64_t)R * (C / 2);
    const uint8_t *Am[NMAT];
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat)
        Am[mat] = MODE == MODE_GEMM ? a.w0
                                    : expert_base<PT>(mat ? a.w1 : a.w0, expert, a.expert_stride);

    // ---- per-lane load sources (rows past the end read row R-1: never
    // stored, and MFMA output rows depend on their own A row only)
    auto lrow = [&] __device__(int rt) { return min(row0 + (wave * RT + rt) * 16 + li, R - 1); };
    // codes, two steps (128 bytes of a row: whole cache lines) per load:
    // load i of a tile takes rows 8i .. 8i + 7, lane L row 8i + L / 8 and the
    // 16-byte piece (L & 7) ^ ((row / 2) & 7) of the pair's 128 bytes, so
    // that the sixteen lanes reading one A fragment (rows 0..15, one piece)
    // spread over the banks.  Measured against 16 rows x 64 B per load and
    // step: 256-expert prefill layer 1546 -> 1403 us in a timing copy.
    // Without pairs, lane (li, ls) loads group ls of step s of row li.
    const uint8_t *csrc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if constexpr (PAIRS) {
                const int lr = 8 * i + (lane >> 3);
                const int r = min(row0 + (wave * RT + mt % RT) * 16 + lr, R - 1);
                csrc[mt][i] =
                    Am[mt / RT] + (int64_t)r * (C / 2) + ((lane & 7) ^ ((lr >> 1) & 7)) * 16;
            } else {
                csrc[mt][i] = Am[mt / RT] + (int64_t)lrow(mt % RT) * (C / 2) + ls * 16;
            }
        }
    // scales: lane (li, ls) loads the 16 scale bytes of a unit for row li of
    // tile ls % MT (lanes of a repeated tile load the same bytes)
    const int smt = ls % MT;
    const uint8_t *ssrc = Am[smt / RT] + code_bytes + (int64_t)lrow(smt % RT) * gpr;
    // a walking workgroup's later blocks: the same lanes, RB rows further
    auto code_src_blk = [&] __device__(int bk, int mt, int i) -> const uint8_t * {
        const int lr = 8 * i + (lane >> 3);
        const int r = min(row0 + bk * RB + (wave * RT + mt % RT) * 16 + lr, R - 1);
        return Am[mt / RT] + (int64_t)r * (C / 2) + ((lane & 7) ^ ((lr >> 1) & 7)) * 16;
    };
    auto scale_src_blk = [&] __device__(int bk) -> const uint8_t * {
        const int r = min(row0 + bk * RB + (wave * RT + smt % RT) * 16 + li, R - 1);
        return Am[smt / RT] + code_bytes + (int64_t)r * gpr;
    };
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
    // its body has no branches and the slab loads cover only the tokens it
    // reads: 16 bf16 / 8 fp32 tokens for one tile (4-byte loads), 32 / 16 for
    // two, the whole item for more (16-byte loads).  Every wave issues the
    // same number of loads per step either way.
    auto k_loop = [&] __device__(auto ncu_tag) {
        constexpr int NCU = decltype(ncu_tag)::value;
        constexpr int TT = XBF ? 16 : 8; // tokens per column tile
        constexpr int TMIN = NW * 1024 / ROWB;        // one 16-byte load per wave
        constexpr int TN0 = NCU <= 2 ? NCU * TT : TPD;
        constexpr int TN = TN0 < TMIN ? TMIN : TN0;   // tokens loaded per step
        constexpr int SB = TN * ROWB;                 // slab bytes loaded per step
        constexpr int AIN = SB / (NW * 1024);         // slab loads per wave per step
        static_assert(SB % (NW * 1024) == 0 && AIN >= 1 && TN <= TPD, "slab loads");

        // slab: load i of this wave fills bytes [(wave * AIN + i) KB, +1 KB)
        // of the slab; the 16 bytes at slab offset o belong to token
        // t = o / ROWB, 16-byte position p, i.e. chunk k = p ^ (t & 15)
        const uint8_t *xsrc[AIN];
#pragma unroll
        for (int i = 0; i < AIN; ++i) {
            const int o = (wave * AIN + i) * 1024 + lane * 16;
            const int t = o / ROWB, p = (o % ROWB) / 16;
            const int k = p ^ (t & 15);
            const int64_t row = t_token_row<MODE>(a, slot0, min(t, ntok - 1));
            xsrc[i] = reinterpret_cast<const uint8_t *>(a.x) + (row * C) * ES + k * 16;
        }
        // the codes of pair q (steps 2q, 2q + 1; clamped to the last pair,
        // whose data is then not read) into the buffer of its parity
        const int npb = nsteps / 2; // pairs per block
        auto issue_codes = [&] __device__(auto pbt, int q) {
            uint8_t *P = pairbuf(pbt);
            const int qc = min(q, nblk * npb - 1);
            const int bk = WALK == 1 ? 0 : qc / npb, qb = qc - bk * npb;
            // (a later block: the same lanes' rows RB further on, so one
            // address step per block unless the rows clamp at the end)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    lds_dma16((WALK == 1 ? csrc[mt][i] : code_src_blk(bk, mt, i)) + qb * TKS,
                              P + (wave * MT + mt) * 2048 + i * 1024);
        };
        // step s's slab (and its codes without pairs; with a unit's first
        // step the unit's scales)
        auto issue = [&] __device__(auto tag, int g) {
            // g: the walk's step (block g / nsteps, step g % nsteps of it)
            const int bk = WALK == 1 ? 0 : g / nsteps;
            const int s = g - bk * nsteps;
            uint8_t *S = stage(tag);
            if constexpr (!PAIRS) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    lds_dma16(csrc[mt][0] + s * (TKS / 2), S + (wave * MT + mt) * 1024);
            }
#pragma unroll
            for (int i = 0; i < AIN; ++i)
                lds_dma16(xsrc[i] + s * ROWB, S + ACT_OFF + (wave * AIN + i) * 1024);
            if constexpr (decltype(tag)::value == 0) // a unit's first step: its scales
                lds_dma16((WALK == 1 ? ssrc : scale_src_blk(bk)) + (s / 4) * 16, scs + wave * 1024);
        };
        const int gsteps = nblk * nsteps; // the walk's steps

        // prologue: the token gathers above have landed; pair 0's codes and
        // steps 0..2 in flight
        wait_vmcnt<0>();
        if constexpr (PAIRS)
            issue_codes(IntTag<0>{}, 0);
        issue(IntTag<0>{}, 0);
        issue(IntTag<1>{}, min(1, gsteps - 1));
        issue(IntTag<2>{}, min(2, gsteps - 1));

        u32x4 usc[MT]; // scale bytes of the current unit: word j = step j
        // unit un of the walk; AFTER_STORE: a later block's first unit, whose
        // steps 0 and 1 wait behind the previous block's output stores too
        auto unit = [&] __device__(int un, auto ast) {
            constexpr bool after_store = decltype(ast)::value != 0;
            auto step = [&] __device__(auto jt) {
                constexpr int j = decltype(jt)::value;
                const int s = un * TNS + j; // the walk's step
                // stage j (step s) and the codes of this step's pair have
                // landed for every wave; stage j - 1 (step s - 1) is free, and
                // at an even step so is the other pair buffer.  Issued at
                // each step: at places 0 and 2 the next pair's codes (2 MT
                // loads), then step s + 3's slab (AIN), plus the unit's
                // scales at place 1; a pair's codes go out two steps before
                // its first step, a slab three.  Loads issued after the last
                // one this step needs:
                // (without pairs: two steps' worth, MT + AIN each, plus the
                // scale load of the stage-0 step when it is one of them)
                constexpr int AHEAD = !PAIRS   ? 2 * (MT + AIN) + (j >= 2 ? 1 : 0)
                                      : j == 0 ? 2 * AIN
                                      : j == 1 ? 2 * MT + 2 * AIN
                                      : j == 2 ? 2 * AIN + 1
                                               : 2 * MT + 2 * AIN + 1;
                // (this wave's LDS reads of the previous step, which was
                // stage j - 1, the one refilled below, are done before the
                // barrier: the barrier itself orders no memory)
                constexpr int S_ST = WALK > 1 ? RT * NCU * 4 : 0; // stores per block
                if constexpr (j < 2 && after_store)
                    wait_vmcnt<AHEAD + S_ST>();
                else
                    wait_vmcnt<AHEAD>();
                wait_lgkm0();
                raw_barrier();
                if constexpr (PAIRS && j % 2 == 0)
                    issue_codes(IntTag<(j / 2 + 1) % 2>{}, s / 2 + 1);
                issue(IntTag<(j + 3) % TNS>{}, min(s + 3, gsteps - 1));

                const uint8_t *S = stage(IntTag<j>{});
                if constexpr (!XBF) {
                    // split the slab's first 8 * NCU tokens (token t, chunk k
                    // of four columns) into rows 16 (t / 8) + t % 8 (hi) and
                    // + 8 (lo)
                    constexpr int CCH = NCU * 8 * 32;
#pragma unroll
                    for (int i0 = 0; i0 < CCH; i0 += NW * 64) {
                        const int i = i0 + tid;
                        if (CCH % (NW * 64) == 0 || i < CCH) {
                            const int t = i >> 5, k = i & 31;
                            const f32x4 v = *reinterpret_cast<const f32x4 *>(
                                S + ACT_OFF + t * ROWB + (k ^ (t & 15)) * 16);
                            u32x2 hi, lo;
                            split_bf16x4(v, hi, lo);
                            const int rh = (t >> 3) * 16 + (t & 7), rl = rh + 8;
                            const int p = k >> 1, o = (k & 1) * 8;
                            *reinterpret_cast<u32x2 *>(cvb + rh * 256 + (p ^ (rh & 15)) * 16 + o) =
                                hi;
                            *reinterpret_cast<u32x2 *>(cvb + rl * 256 + (p ^ (rl & 15)) * 16 + o) =
                                lo;
                        }
                    }
                    wait_lgkm0();
                    raw_barrier();
                }
                if constexpr (j == 0) { // this unit's scales, before they are refilled
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        usc[mt] = *reinterpret_cast<const u32x4 *>(scs + wave * 1024 +
                                                                   (mt * 16 + li) * 16);
                }
                // A: row li, group ls of the step (with pairs: piece
                // 4 (j % 2) + ls of the pair's 128 bytes of the row)
                const uint8_t *CB = PAIRS ? pairbuf(IntTag<(j / 2) % 2>{}) : S;
                const int kp = 4 * (j % 2) + ls;
                const int aoff = PAIRS ? (li >> 3) * 1024 +
                                             ((li & 7) * 8 + (kp ^ ((li >> 1) & 7))) * 16
                                       : lane * 16;
                constexpr int ASTR = PAIRS ? 2048 : 1024;
                u32x4 cw[MT];
                float scf[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    cw[mt] = *reinterpret_cast<const u32x4 *>(CB + (wave * MT + mt) * ASTR + aoff);
                    scf[mt] = e8m0_operand_of(usc[mt][j], ls);
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    // MFMA column li of tile c: bf16 token 16 c + li, or the
                    // hi / lo row 16 c + li of the split fp32 slab (256-byte
                    // rows, swizzled alike)
                    const uint8_t *B = XBF ? S + ACT_OFF : cvb;
                    bf16x8 bv[NCU];
#pragma unroll
                    for (int c = 0; c < NCU; ++c) {
                        const int r = c * 16 + li;
                        const int p = (4 * ls + m) ^ li;
                        bv[c] = *reinterpret_cast<const bf16x8 *>(B + r * 256 + p * 16);
                    }
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const bf16x8 av = decode8_bf16(cw[mt][m], scf[mt]);
#pragma unroll
                        for (int c = 0; c < NCU; ++c)
                            acc[mt][c] = mfma16x16x32(av, bv[c], acc[mt][c]);
                    }
                }
            };
            step(IntTag<0>{});
            step(IntTag<1>{});
            step(IntTag<2>{});
            step(IntTag<3>{});
            // ---- end of a 512-column unit.  A block's first unit starts its
            // total; the GEMM simply adds it to the zeroed total instead
            // (0 + acc is acc: an MFMA chain from +0 never ends at -0), which
            // changes no bit and only how the loop compiles (measured,
            // 14336x4096: bf16 b = 64 19.5 -> 18.95 us, fp32 b = 32 20.45 ->
            // 20.3 us; the same form costs the expert gate/up 2.5 %)
            const int ub = WALK == 1 ? un : un % nunits;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int c = 0; c < NCU; ++c) {
                    tot[mt][c] = MODE == MODE_GEMM || ub != 0 ? tot[mt][c] + acc[mt][c] : acc[mt][c];
                    acc[mt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        };
        // a block's outputs: a fixed number of stores per wave (RT * NCU * 4),
        // rows past the end and tokens past the item clamped to the last ones,
        // whose values those lanes hold too (their A rows and B columns were
        // loaded clamped the same way)
        auto block_out = [&] __device__(int bk) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int c = 0; c < NCU; ++c) {
                    f32x4 g = tot[rt][c];
                    if (!XBF) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            g[i] += dpp_row_ror8(g[i]);
                    }
                    const int tok = min(XBF ? c * 16 + li : c * 8 + (li & 7), ntok - 1);
                    const int64_t orow = slot0 + tok;
                    const int rbase = row0 + bk * RB + (wave * RT + rt) * 16 + 4 * ls;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        reinterpret_cast<float *>(a.y)[orow * R + min(rbase + i, R - 1)] = g[i];
                }
        };
        // the blocks written out one after the other (no loop around them,
        // so that every path to a wait has the same loads and stores before
        // it and the constant waits above are the only ones)
        if constexpr (WALK == 1) {
            for (int un = 0; un < nunits; ++un)
                unit(un, IntTag<0>{});
        } else {
            for (int un = 0; un < nunits; ++un)
                unit(un, IntTag<0>{});
            block_out(0);
            auto later = [&] __device__(auto bt) {
                constexpr int bk = decltype(bt)::value;
                if constexpr (bk < WALK) {
                    if (nblk > bk) {
                        unit(bk * nunits, IntTag<1>{});
                        for (int un = bk * nunits + 1; un < (bk + 1) * nunits; ++un)
                            unit(un, IntTag<0>{});
                        block_out(bk);
                    }
                }
            };
            later(IntTag<1>{});
            later(IntTag<2>{});
            later(IntTag<3>{});
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
    // the last steps' (clamped, unused) loads land before the workgroup ends
    wait_vmcnt<0>();

    // ---- outputs
    if constexpr (WALK > 1)
        return;
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
            const float pw =
                (MODE == MODE_GATEUP && a.v41) ? a.pair_w[a.pair_of_slot[orow]] : 0.0f;
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
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

namespace {

typedef void (*TiledFn)(SkinnyArgs);

struct TEntry {
    int mode, xbf, nw, rt, nc, pt;
    TiledFn fn;
};

#define MX_T(MODE, XBF, NW, RT, NC, PT) \
    {MODE, XBF, NW, RT, NC, PT, tiled_kernel<NW, RT, NC, (bool)XBF, MODE, (bool)PT>}
#define MX_TX(MODE, NW, RT, NC) MX_T(MODE, 0, NW, RT, NC, 0), MX_T(MODE, 1, NW, RT, NC, 0)
// expert-bank modes also over per-expert pointer tables
#define MX_TXB(MODE, NW, RT, NC) \
    MX_TX(MODE, NW, RT, NC), MX_T(MODE, 0, NW, RT, NC, 1), MX_T(MODE, 1, NW, RT, NC, 1)
// expert bank: gate/up 8 waves x 1 row tile (four 32 KB stages), down 8 x 2
// (one activation slab serves 256 rows: 1.67 -> 1.59 ms on the prefill bank);
// GEMM: 4 waves x 1 row tile (more workgroups on 14336-row weights), or 8
// when the grid keeps enough workgroups
const TEntry kTiled[] = {
    MX_TXB(MODE_GATEUP, 8, 1, 4), MX_TXB(MODE_DOWN, 8, 2, 4),
    MX_TX(MODE_GEMM, 4, 1, 4), MX_TX(MODE_GEMM, 4, 1, 2),
    MX_TX(MODE_GEMM, 8, 1, 4), MX_TX(MODE_GEMM, 8, 1, 2),
};

const TEntry *tfind(int mode, bool xbf, int nw, int rt, int nc, bool pt)
{
    for (const TEntry &e : kTiled)
        if (e.mode == mode && e.xbf == (int)xbf && e.nw == nw && e.rt == rt && e.nc == nc &&
            e.pt == (int)pt)
            return &e;
    return nullptr;
}

} // namespace

bool tiled_supported(int cols) { return cols % 512 == 0; }

int tiled_tokens(bool xbf, int nc) { return xbf ? 16 * nc : 8 * nc; }

int tiled_rows_per_wg(int nw, int rt) { return nw * rt * 16; }

hipError_t tiled_launch(int mode, bool xbf, int nw, int rt, int nc, const SkinnyArgs &a,
                        hipStream_t stream)
{
    const TEntry *e = tfind(mode, xbf, nw, rt, nc, a.ptr_table != 0);
    if (!e)
        return hipErrorInvalidValue;
    const int rpw = tiled_rows_per_wg(nw, rt);
    const int64_t nrb = (a.rows + rpw - 1) / rpw;
    const int64_t nrbw = mode == MODE_DOWN ? (nrb + WALK_DOWN - 1) / WALK_DOWN : nrb;
    hipLaunchKernelGGL(e->fn, dim3((unsigned)(nrbw * a.nch)), dim3(nw * 64), 0, stream, a);
    return hipGetLastError();
}

} // namespace mx
