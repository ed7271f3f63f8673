// Block-scaled FP4 x FP8 product on the CDNA4 matrix cores: the opt-in path
// where MXFP4 weights meet activations quantized to MXFP8 (E4M3 elements,
// one E8M0 power-of-two scale per 32 elements: the OCP MX family that
// "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs" names in its module doc).
//
//  * mxfp8_quantize_kernel: one thread per 32-element block of a token row;
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
//    eight partials are summed through LDS in K order.
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

template <bool XBF>
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const void *x, int64_t blocks,
                                                             int gpr, uint8_t *q, uint8_t *s)
{
    const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blk >= blocks)
        return;
    float v[32];
    if (XBF) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(
            reinterpret_cast<const uint16_t *>(x) + blk * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 w = src[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
                v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
            }
        }
    } else {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(x) +
                                                           blk * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 w = src[i];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[4 * i + j] = w[j];
        }
    }
    float amax = 0.0f;
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        bad |= !__builtin_isfinite(v[i]);
        amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    }
    u32x4 out[2];
    if (bad || amax == 0.0f) {
        s[blk] = bad ? 255 : 0;
        out[0] = out[1] = u32x4{0u, 0u, 0u, 0u};
    } else {
        // floor(log2 amax): the exponent field, or for an fp32 subnormal the
        // position of its leading mantissa bit
        const uint32_t ab = __float_as_uint(amax);
        const int ef = (int)(ab >> 23);
        const int fl = ef ? ef - 127 : (31 - __builtin_clz(ab)) - 149;
        int k = fl - 8 + 127;
        k = k < 0 ? 0 : (k > 254 ? 254 : k);
        s[blk] = (uint8_t)k;
        const int e = k - 127; // x / 2^e, exact (a power-of-two scaling)
        uint32_t packed[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                word |= e4m3_rne_bits(__builtin_ldexpf(v[4 * w + j], -e)) << (8 * j);
            packed[w] = word;
        }
        out[0] = u32x4{packed[0], packed[1], packed[2], packed[3]};
        out[1] = u32x4{packed[4], packed[5], packed[6], packed[7]};
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(q + blk * 32);
    dst[0] = out[0];
    dst[1] = out[1];
    (void)gpr;
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

} // namespace

hipError_t mxfp8_quantize_launch(const void *x, bool xbf, int64_t b, int64_t cols, uint8_t *q,
                                 uint8_t *s, hipStream_t stream)
{
    const int64_t blocks = b * (cols / 32);
    const unsigned grid = (unsigned)((blocks + 255) / 256);
    if (xbf)
        hipLaunchKernelGGL(mxfp8_quantize_kernel<true>, dim3(grid), dim3(256), 0, stream, x,
                           blocks, (int)(cols / 32), q, s);
    else
        hipLaunchKernelGGL(mxfp8_quantize_kernel<false>, dim3(grid), dim3(256), 0, stream, x,
                           blocks, (int)(cols / 32), q, s);
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
