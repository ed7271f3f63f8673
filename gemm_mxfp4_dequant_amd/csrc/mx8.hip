// Block-scaled FP4 x FP8 product on the CDNA4 matrix cores: the opt-in path
// where MXFP4 weights meet activations quantized to MXFP8 (E4M3 elements,
// one E8M0 power-of-two scale per 32 elements: the OCP MX family that
// "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs" names in its module doc).
//
//  * mxfp8_quantize_kernel: eight lanes per 32-element block of a token row;
//    shared exponent E = floor(log2 max|x|) - 8, stored as the byte E + 127
//    (clamped to [0, 254]); each element is the E4M3 code nearest to
//    x / 2^E, ties to even, saturating at 448, computed with integer
//    operations on the fp32 bits (the same codes as the rule's definition,
//    bit for bit); NaN or inf in a block gives scale 255 and zero codes.
//  * gemm_a8_kernel: v_mfma_scale_f32_16x16x128_f8f6f4 takes the weights as
//    stored (lane (r, g) of the A operand holds the 16 code bytes of row r,
//    32-column group g of the 128-column step, with that group's scale
//    byte) and the quantized activations (lane (c, g) of the B operand holds
//    columns 16g..16g+15 and 64+16g..64+16g+15 of the step for token c; the
//    scale of 32-column block j of token c comes from lane c + 16j).  No
//    decode instructions: the matrix core applies both scales.  A workgroup
//    owns two 16-row tiles and NC tiles of 16 tokens; its 8 waves each walk
//    an eighth of K in 128-column steps (the next step's loads in flight
//    during the current one) into one fp32 accumulator per tile, and the
//    eight partials are summed through LDS in K order.  Used for b <= 16
//    and for widths that are not a multiple of 512.
//  * gemm_a8_tiled_kernel (b > 16, cols % 512 == 0): 64-row workgroups
//    that stream the weights and one LDS copy of the token chunk's
//    quantized activations through a ring of direct global -> LDS loads,
//    the same operand lanes as above read from LDS.
//  * Accuracy (the contract of this entry point, not the 1e-4 rule of the
//    others): the product is the exact product of the weights with the
//    quantized activations up to the matrix core's accumulation, which adds
//    the 32-element blocks exactly but aligns the products inside a block to
//    the block's largest and keeps about 13 bits below it.
#include "../../include/mxfp4.h"
#include "device.h"
#include "launch.h"

namespace mx {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int N> struct IntTag8 {
    static constexpr int value = N;
};

// E4M3 code nearest to v (|v| < 2^9 or saturating), ties to even.
__device__ __forceinline__ uint32_t e4m3_rne_bits(float v)
{
    const uint32_t bits = __float_as_uint(v);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = __builtin_fabsf(v);
    uint32_t code;
    if (a >= 448.0f) {
        code = 0x7Eu; // the largest finite magnitude is the nearest
    } else if (a < 0x1p-6f) {
        // subnormal codes m * 2^-9, m = 0..8 (m = 8 is the smallest normal,
        // whose code is 8 as well); a * 512 is exact, rint rounds to even
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        // normal: round the fp32 mantissa to 3 bits, nearest even, then
        // move the exponent from bias 127 to bias 7 (a carry out of the
        // mantissa bumps the exponent, as it should)
        const uint32_t ab = __float_as_uint(a);
        const uint32_t r = (ab + 0x7FFFFu + ((ab >> 20) & 1u)) >> 20;
        code = r - ((127u - 7u) << 3);
    }
    return sign | code;
}

// Eight consecutive lanes share a 32-element block, four elements each: one
// 16-byte (fp32) or 8-byte (bf16) load per lane, the block's largest
// magnitude and its non-finite flag combined over the eight lanes, one
// 4-byte store of codes per lane and the scale byte from the first.
template <bool XBF>
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const void *x, int64_t blocks,
                                                             uint8_t *q, uint8_t *s)
{
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = gid >> 3;
    const int sub = (int)(gid & 7);
    // a whole block's lanes are in or out together (blocks * 8 threads)
    if (blk >= blocks)
        return;
    const int64_t e0 = blk * 32 + sub * 4;
    float v[4];
    if (XBF) {
        const u32x2 w = *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint16_t *>(x) + e0);
        v[0] = __uint_as_float(w[0] << 16);
        v[1] = __uint_as_float(w[0] & 0xFFFF0000u);
        v[2] = __uint_as_float(w[1] << 16);
        v[3] = __uint_as_float(w[1] & 0xFFFF0000u);
    } else {
        const f32x4 w = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(x) + e0);
        v[0] = w[0];
        v[1] = w[1];
        v[2] = w[2];
        v[3] = w[3];
    }
    float amax = 0.0f;
    int bad = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bad |= !__builtin_isfinite(v[i]);
        amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, m, 8));
        bad |= __shfl_xor(bad, m, 8);
    }
    uint32_t word = 0;
    int k = 0;
    if (bad || amax == 0.0f) {
        k = bad ? 255 : 0;
    } else {
        // floor(log2 amax): the exponent field, or for an fp32 subnormal the
        // position of its leading mantissa bit
        const uint32_t ab = __float_as_uint(amax);
        const int ef = (int)(ab >> 23);
        const int fl = ef ? ef - 127 : (31 - __builtin_clz(ab)) - 149;
        k = fl - 8 + 127;
        k = k < 0 ? 0 : (k > 254 ? 254 : k);
        const int e = k - 127; // x / 2^e, exact (a power-of-two scaling)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            word |= e4m3_rne_bits(__builtin_ldexpf(v[j], -e)) << (8 * j);
    }
    *reinterpret_cast<uint32_t *>(q + e0) = word;
    if (sub == 0)
        s[blk] = (uint8_t)k;
}

constexpr int A8_NWK = 8; // waves per workgroup, each over 1/8 of K
constexpr int A8_RT = 2;  // 16-row tiles per workgroup

// One K step's operands of one wave.
template <int NC> struct A8Step {
    u32x4 a[A8_RT];
    int sa[A8_RT];
    u32x4 blo[NC], bhi[NC];
    int sb[NC];
};

template <int NC>
__global__ __launch_bounds__(A8_NWK * 64) void gemm_a8_kernel(A8Args a)
{
    const int C = a.cols, R = a.rows;
    const int gpr = C / 32;
    const int nsteps = C / 128;
    const int nch = (a.b + 16 * NC - 1) / (16 * NC);
    const int lid = xcd_logical(blockIdx.x, gridDim.x);
    const int ch = lid % nch; // token chunk fastest: a row block's chunks share an XCD
    const int rb = lid / nch;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, ls = lane >> 4;
    const int t0 = ch * 16 * NC;
    const int row0 = rb * (A8_RT * 16);
    const int64_t code_bytes = (int64_t)R * (C / 2);
    // this wave's K steps: a contiguous share, the first waves one more
    const int base = nsteps / A8_NWK, extra = nsteps % A8_NWK;
    const int s0 = wave * base + min(wave, extra);
    const int ns = base + (wave < extra ? 1 : 0);

    // rows past the end read row R - 1 and tokens past b read token b - 1:
    // never stored, and an MFMA output element depends on its own row and
    // column only
    const uint8_t *arow[A8_RT];
    const uint8_t *srow[A8_RT];
#pragma unroll
    for (int rt = 0; rt < A8_RT; ++rt) {
        const int r = min(row0 + rt * 16 + li, R - 1);
        arow[rt] = a.w + (int64_t)r * (C / 2) + ls * 16;
        srow[rt] = a.w + code_bytes + (int64_t)r * gpr + ls;
    }
    const uint8_t *xrow[NC];
    const uint8_t *xsrow[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int t = min(t0 + c * 16 + li, a.b - 1);
        xrow[c] = a.xq + (int64_t)t * C + ls * 16;
        xsrow[c] = a.xs + (int64_t)t * gpr + ls;
    }
    auto load = [&](int L, A8Step<NC> &st) {
#pragma unroll
        for (int rt = 0; rt < A8_RT; ++rt) {
            st.a[rt] = *reinterpret_cast<const u32x4 *>(arow[rt] + (int64_t)L * 64);
            st.sa[rt] = srow[rt][4 * L]; // the scale of this lane's group
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            st.blo[c] = *reinterpret_cast<const u32x4 *>(xrow[c] + (int64_t)L * 128);
            st.bhi[c] = *reinterpret_cast<const u32x4 *>(xrow[c] + (int64_t)L * 128 + 64);
            st.sb[c] = xsrow[c][4 * L]; // block ls of this lane's token
        }
    };

    f32x4 acc[A8_RT][NC];
#pragma unroll
    for (int rt = 0; rt < A8_RT; ++rt)
#pragma unroll
        for (int c = 0; c < NC; ++c)
            acc[rt][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    A8Step<NC> cur, nxt;
    if (ns > 0)
        load(s0, cur);
    for (int i = 0; i < ns; ++i) {
        if (i + 1 < ns)
            load(s0 + i + 1, nxt); // the next step's loads fly during this one
#pragma unroll
        for (int rt = 0; rt < A8_RT; ++rt) {
            const i32x8 A = {(int)cur.a[rt][0], (int)cur.a[rt][1], (int)cur.a[rt][2],
                             (int)cur.a[rt][3], 0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const i32x8 B = {(int)cur.blo[c][0], (int)cur.blo[c][1], (int)cur.blo[c][2],
                                 (int)cur.blo[c][3], (int)cur.bhi[c][0], (int)cur.bhi[c][1],
                                 (int)cur.bhi[c][2], (int)cur.bhi[c][3]};
                acc[rt][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    A, B, acc[rt][c], 4 /* A: FP4 E2M1 */, 0 /* B: FP8 E4M3 */, 0,
                    cur.sa[rt], 0, cur.sb[c]);
            }
        }
        cur = nxt;
    }

    // the waves' K-slice partials, summed in wave (K) order: wave w sums
    // tile w of the A8_RT x NC tiles
    __shared__ f32x4 red[A8_NWK][A8_RT * NC][64];
#pragma unroll
    for (int rt = 0; rt < A8_RT; ++rt)
#pragma unroll
        for (int c = 0; c < NC; ++c)
            red[wave][rt * NC + c][lane] = acc[rt][c];
    __syncthreads();
    for (int tile = wave; tile < A8_RT * NC; tile += A8_NWK) {
        f32x4 v = red[0][tile][lane];
        for (int w = 1; w < A8_NWK; ++w)
            v += red[w][tile][lane];
        const int rt = tile / NC, c = tile % NC;
        // D: lane (li, ls) holds rows 4 ls .. 4 ls + 3 of token column li
        const int t = t0 + c * 16 + li;
        if (t >= a.b)
            continue;
        const int rbase = row0 + rt * 16 + 4 * ls;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rbase + i;
            if (r >= R)
                continue;
            if (a.y_bf16)
                reinterpret_cast<uint16_t *>(a.y)[(int64_t)t * R + r] = f32_to_bf16_bits(v[i]);
            else
                reinterpret_cast<float *>(a.y)[(int64_t)t * R + r] = v[i];
        }
    }
}

// The same product on the tiled schedule (cols % 512 == 0): a workgroup of NW
// waves owns NW 16-row tiles (one per wave) and NC tiles of 16 tokens, and
// runs the whole K loop in 128-column steps (four per 512-column unit).
//  * Activations: a ring of four LDS stages, one per step, filled by direct
//    global -> LDS loads three steps ahead with the step's 16 NC tokens x
//    128 E4M3 bytes (16-byte chunk k of token t at position k ^ (t & 7), so
//    that the sixteen lanes reading one B fragment spread over the banks);
//    with the first step of each unit also the unit's 16 scale bytes of the
//    wave's rows and of one token tile's tokens, which the waves copy to
//    registers at that step.
//  * Weights: a unit's codes of the wave's 16 rows (4 KB) in one of two
//    per-wave buffers (unit parity), loaded as four 1 KB chunks of 4 rows x
//    256 contiguous bytes: lane L of chunk c takes row 4c + L / 16 and the
//    16-byte piece (L & 15) ^ row of its unit slice (so the sixteen lanes
//    reading one A fragment spread over the banks).  Chunks 0-1 of unit v
//    travel with the stage of step 4v - 1, chunks 2-3 with that of step 4v.
//    Whole lines per row and instruction: measured against 16 rows x 64 B
//    per instruction in every step's stage, 14336 x 4096 b = 64 18.8 ->
//    17.9 us, b = 256 51.4 -> 43.1 us, 4096 x 14336 b = 64 45.1 -> 39.8 us.
// Per stage every wave issues the same loads (how many depends only on the
// step's place in its unit), so "stage s has landed" is one constant vmcnt
// wait per step, then one barrier.  Every wave reads the slab from LDS, so
// each activation byte fetched serves 16 NW rows.  One fp32 accumulator per
// token tile, steps in ascending order.
//   Measured at 14336 x 4096, b = 64 (bf16 activations, quantize included),
// before the unit code buffers: scale bytes once per unit instead of 4-byte
// loads of 16 rows' (or tokens') scales every step, 23.8 -> 18.9 us.  Not
// kept: rings of six or eight stages (+4 %, +7 %), and K in two parts over
// eight waves with the parts' sums added through LDS (19.4 us; b = 256: 51.4
// -> 59.5 us).
template <int NW, int NC> struct A8TLayout {
    static_assert((2 * NC) % NW == 0 && NC <= NW, "slab and scale loads spread over the waves");
    static constexpr int STAGE = NC * 16 * 128; // [16 NC tokens][8 chunks][16 B]
    static constexpr int XL = 2 * NC / NW;      // slab loads per wave and step
    // loads issued with the stages of the next two steps, by the place j of
    // the current step in its unit (stage of place 3: two code chunks; place
    // 0: two code chunks and two scale loads)
    static constexpr int ahead(int j)
    {
        return j == 0 ? 2 * XL : j == 1 ? 2 * XL + 2 : j == 2 ? 2 * XL + 6 : 2 * XL + 4;
    }
};

template <int NW, int NC>
__global__ __launch_bounds__(NW * 64) void gemm_a8_tiled_kernel(A8Args a)
{
    using L = A8TLayout<NW, NC>;
    // one variable per buffer: the loads into one and the reads of another
    // are known not to alias
    __shared__ __align__(16) uint8_t st0[L::STAGE], st1[L::STAGE], st2[L::STAGE],
        st3[L::STAGE];
    __shared__ __align__(16) uint8_t cb0[NW * 4096], cb1[NW * 4096];
    // a unit's scale bytes: [NW][64 lanes][16 B], lane li (ls = 0) holding
    // row / token li's 16 (the other lanes load copies)
    __shared__ __align__(16) uint8_t sca[NW * 1024], scb[NW * 1024];
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
    auto codebuf = [&] __device__(auto tag) -> uint8_t * {
        if constexpr (decltype(tag)::value == 0)
            return cb0;
        else
            return cb1;
    };
    const int C = a.cols, R = a.rows;
    const int gpr = C / 32;
    const int nunits = C / 512;
    const int nsteps = nunits * 4;
    const int nch = (a.b + 16 * NC - 1) / (16 * NC);
    const int lid = xcd_logical(blockIdx.x, gridDim.x);
    const int ch = lid % nch; // token chunk fastest: a row block's chunks share an XCD
    const int rb = lid / nch;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, ls = lane >> 4;
    const int t0 = ch * 16 * NC;
    const int ntok = min(16 * NC, a.b - t0);
    const int row0 = rb * (NW * 16);
    const int64_t code_bytes = (int64_t)R * (C / 2);

    // ---- per-lane load sources (rows past the end read row R - 1, tokens
    // past the chunk its last token: never stored, and an MFMA output element
    // depends on its own row and column only)
    const uint8_t *crow[4]; // code chunk c: this lane's row and swizzled piece
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int lr = 4 * c + (lane >> 4);
        const int r = min(row0 + wave * 16 + lr, R - 1);
        crow[c] = a.w + (int64_t)r * (C / 2) + ((lane & 15) ^ lr) * 16;
    }
    const int r = min(row0 + wave * 16 + li, R - 1);
    const uint8_t *asrc = a.w + code_bytes + (int64_t)r * gpr; // 16 scale bytes per unit
    const uint8_t *xsrc[L::XL];
#pragma unroll
    for (int i = 0; i < L::XL; ++i) {
        const int pos = (wave * L::XL + i) * 64 + lane; // slab position (16-byte chunks)
        const int t = pos >> 3, k = (pos & 7) ^ (t & 7);
        xsrc[i] = a.xq + (int64_t)(t0 + min(t, ntok - 1)) * C + k * 16;
    }
    const uint8_t *bsrc = a.xs + (int64_t)(t0 + min((wave % NC) * 16 + li, ntok - 1)) * gpr;
    auto load_codes = [&] __device__(auto bt, int c, int v) {
        lds_dma16(crow[c] + (int64_t)v * 256, codebuf(bt) + wave * 4096 + c * 1024);
    };
    // the loads that travel with step q's stage (q may run past the end:
    // sources clamp to the last step / unit, whose data is then not read);
    // bt: the code buffer of the unit they carry codes for
    auto issue = [&] __device__(auto tag, auto bt, int q) {
        constexpr int st = decltype(tag)::value;
        uint8_t *S = stage(tag);
        const int qs = min(q, nsteps - 1);
        if constexpr (st == 3) {
            const int v = min((q + 1) / 4, nunits - 1);
            load_codes(bt, 0, v);
            load_codes(bt, 1, v);
        }
        if constexpr (st == 0) {
            const int v = min(q / 4, nunits - 1);
            load_codes(bt, 2, v);
            load_codes(bt, 3, v);
        }
#pragma unroll
        for (int i = 0; i < L::XL; ++i)
            lds_dma16(xsrc[i] + (int64_t)qs * 128, S + (wave * L::XL + i) * 1024);
        if constexpr (st == 0) { // a unit's first step: its scales
            lds_dma16(asrc + (qs / 4) * 16, sca + wave * 1024);
            lds_dma16(bsrc + (qs / 4) * 16, scb + wave * 1024);
        }
    };

    f32x4 acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
        acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // prologue: unit 0's code chunks 0-1, then steps 0 .. 2 in flight
    load_codes(IntTag8<0>{}, 0, 0);
    load_codes(IntTag8<0>{}, 1, 0);
    issue(IntTag8<0>{}, IntTag8<0>{}, 0);
    issue(IntTag8<1>{}, IntTag8<0>{}, 1);
    issue(IntTag8<2>{}, IntTag8<0>{}, 2);
    u32x4 usa, usb[NC]; // the unit's scale bytes: word j = step j, byte ls = group ls
    // step j of unit u, whose codes are in buffer bt
    auto step = [&] __device__(auto jt, auto bt, int u) {
        constexpr int j = decltype(jt)::value;
        constexpr int b = decltype(bt)::value;
        const int s = u * 4 + j;
        // stage j (step s) and unit u's codes have landed for every wave;
        // stage j - 1 is free (this wave's reads of it are done before the
        // barrier), and so is the other code buffer from place 0 on
        wait_vmcnt<L::ahead(j)>();
        wait_lgkm0();
        raw_barrier();
        issue(IntTag8<(j + 3) % 4>{}, IntTag8<1 - b>{}, s + 3);
        if constexpr (j == 0) { // this unit's scales, before they are refilled
            usa = *reinterpret_cast<const u32x4 *>(sca + wave * 1024 + li * 16);
#pragma unroll
            for (int c = 0; c < NC; ++c)
                usb[c] = *reinterpret_cast<const u32x4 *>(scb + c * 1024 + li * 16);
        }
        // A: row li, 16-byte piece 4 j + ls of the unit slice
        const int kp = 4 * j + ls;
        const u32x4 av = *reinterpret_cast<const u32x4 *>(
            codebuf(bt) + wave * 4096 + (li >> 2) * 1024 + ((li & 3) * 16 + (kp ^ li)) * 16);
        const i32x8 A = {(int)av[0], (int)av[1], (int)av[2], (int)av[3], 0, 0, 0, 0};
        const int sa = (int)((usa[j] >> (8 * ls)) & 0xFFu); // row li, group ls
        const uint8_t *S = stage(IntTag8<j>{});
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int t = c * 16 + li;
            const uint8_t *row = S + t * 128;
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(row + ((ls ^ (t & 7)) * 16));
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(row + (((4 + ls) ^ (t & 7)) * 16));
            const i32x8 B = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                             (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            const int sb = (int)((usb[c][j] >> (8 * ls)) & 0xFFu); // token t, block ls
            acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                A, B, acc[c], 4 /* A: FP4 E2M1 */, 0 /* B: FP8 E4M3 */, 0, sa, 0, sb);
        }
    };
    auto unit = [&] __device__(auto bt, int u) {
        step(IntTag8<0>{}, bt, u);
        step(IntTag8<1>{}, bt, u);
        step(IntTag8<2>{}, bt, u);
        step(IntTag8<3>{}, bt, u);
    };
    // units in pairs, so that each one's code buffer is known at compile time
    int u = 0;
    for (; u + 1 < nunits; u += 2) {
        unit(IntTag8<0>{}, u);
        unit(IntTag8<1>{}, u + 1);
    }
    if (u < nunits)
        unit(IntTag8<0>{}, u);
    // the last steps' (clamped, unused) loads land before the workgroup ends
    wait_vmcnt<0>();

    // D: lane (li, ls) holds rows 4 ls .. 4 ls + 3 of token column li
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int t = t0 + c * 16 + li;
        if (t >= a.b)
            continue;
        const int rbase = row0 + wave * 16 + 4 * ls;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = rbase + i;
            if (rr >= R)
                continue;
            if (a.y_bf16)
                reinterpret_cast<uint16_t *>(a.y)[(int64_t)t * R + rr] =
                    f32_to_bf16_bits(acc[c][i]);
            else
                reinterpret_cast<float *>(a.y)[(int64_t)t * R + rr] = acc[c][i];
        }
    }
}

} // namespace

hipError_t mxfp8_quantize_launch(const void *x, bool xbf, int64_t b, int64_t cols, uint8_t *q,
                                 uint8_t *s, hipStream_t stream)
{
    const int64_t blocks = b * (cols / 32);
    const unsigned grid = (unsigned)((blocks * 8 + 255) / 256);
    if (xbf)
        hipLaunchKernelGGL(mxfp8_quantize_kernel<true>, dim3(grid), dim3(256), 0, stream, x,
                           blocks, q, s);
    else
        hipLaunchKernelGGL(mxfp8_quantize_kernel<false>, dim3(grid), dim3(256), 0, stream, x,
                           blocks, q, s);
    return hipGetLastError();
}

int a8_rows_per_wg() { return A8_RT * 16; }

hipError_t gemm_a8_launch(const A8Args &a, hipStream_t stream)
{
    // token tiles per workgroup: 4 (64 tokens) when b needs them, else the
    // fewest that hold b (a chunk of tokens re-reads the weights, from L2
    // when the chunks of a row block run together)
    const int nc = a.b > 32 ? 4 : (a.b > 16 ? 2 : 1);
    const int64_t nch = (a.b + 16 * nc - 1) / (16 * nc);
    if (nc >= 2 && a.cols % 512 == 0) {
        // tiled: 64-row workgroups sharing one LDS copy of the activations
        const int64_t nrb = (a.rows + 63) / 64;
        const dim3 grid((unsigned)(nrb * nch)), block(4 * 64);
        if (nc == 4)
            hipLaunchKernelGGL((gemm_a8_tiled_kernel<4, 4>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((gemm_a8_tiled_kernel<4, 2>), grid, block, 0, stream, a);
        return hipGetLastError();
    }
    const int64_t nrb = (a.rows + a8_rows_per_wg() - 1) / a8_rows_per_wg();
    const dim3 grid((unsigned)(nrb * nch)), block(A8_NWK * 64);
    if (nc == 4)
        hipLaunchKernelGGL(gemm_a8_kernel<4>, grid, block, 0, stream, a);
    else if (nc == 2)
        hipLaunchKernelGGL(gemm_a8_kernel<2>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(gemm_a8_kernel<1>, grid, block, 0, stream, a);
    return hipGetLastError();
}

} // namespace mx
