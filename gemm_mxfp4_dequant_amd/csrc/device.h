// Device helpers shared by the gfx950 kernels of libmxfp4.
//
// Format decode uses the CDNA4 conversion instructions
// v_cvt_scalef32_pk_{f32,bf16}_fp4: they read two E2M1 nibbles of a byte
// (low nibble first) and scale them by 2^(E-127), E being the exponent field
// of the fp32 scale operand.  Passing the E8M0 byte k as (k << 23) therefore
// applies the format's scale exactly, including k = 0 (2^-127) and k = 255
// (NaN); the products are rounded once (exact for every finite weight).
// This is the decode of the DECODE shader (mx_e2m1, mx_e8m0) of
// "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs", done by the hardware.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// fp32 scale operand carrying E8M0 byte k in its exponent field.
__device__ __forceinline__ float e8m0_operand(uint32_t k) { return __uint_as_float(k << 23); }

// Byte `idx` (0..3) of a word, as the scale operand.
__device__ __forceinline__ float e8m0_operand_of(uint32_t word, uint32_t idx)
{
    return __uint_as_float(((word >> (8u * idx)) & 0xFFu) << 23);
}

// Eight weights (one code word, nibbles 0..7 = elements 0..7) as bf16,
// scaled: the MFMA A/B operand of one lane.
__device__ __forceinline__ bf16x8 decode8_bf16(uint32_t word, float scale)
{
    u32x4 q;
    q[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0));
    q[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1));
    q[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2));
    q[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3));
    return __builtin_bit_cast(bf16x8, q);
}

// Eight weights as fp32 (two per conversion).
__device__ __forceinline__ void decode8_f32(uint32_t word, float scale, float *out)
{
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, 3);
    out[0] = p0[0]; out[1] = p0[1]; out[2] = p1[0]; out[3] = p1[1];
    out[4] = p2[0]; out[5] = p2[1]; out[6] = p3[0]; out[7] = p3[1];
}

// 16x16x32 bf16 MFMA with fp32 accumulate.  Lane l holds A row l%16,
// k = 8*(l/16)..+8; B column l%16, same k; D column l%16, rows
// 4*(l/16)..+4.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Exact-enough split of fp32 into bf16 hi + lo: hi = x truncated to bf16
// (its top 16 bits, one v_perm for two values), lo = RNE(x - hi), where
// x - hi is exact in fp32 and |x - hi| < 2^-7 |x|, so
// |x - hi - lo| <= 2^-8 |x - hi| < 2^-15 |x|.  Truncation keeps hi finite
// for every finite x (nearest-even would round |x| beyond the bf16 maximum
// to infinity), at the cost of the nearest-even split's 2^-16 bound.  NaN
// gives NaN parts; x = +-inf gives hi = x and lo = NaN (inf - inf), so an
// infinite activation makes every output of its token NaN.  Two values,
// packed as one word each (element 0 in the low half).
__device__ __forceinline__ void split_bf16_pair(float x0, float x1, uint32_t &hi, uint32_t &lo)
{
    const uint32_t b0 = __float_as_uint(x0), b1 = __float_as_uint(x1);
    hi = __builtin_amdgcn_perm(b1, b0, 0x07060302u); // bytes 2,3 of b0, then of b1
    const f32x2 r = {x0 - __uint_as_float(b0 & 0xFFFF0000u),
                     x1 - __uint_as_float(b1 & 0xFFFF0000u)};
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
}

// The split of 8 values (MFMA operands).
__device__ __forceinline__ void split_bf16x8(const float *x, bf16x8 &hi, bf16x8 &lo)
{
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t hw, lw;
        split_bf16_pair(x[2 * i], x[2 * i + 1], hw, lw);
        h[i] = hw;
        l[i] = lw;
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// The split of 4 values (half an MFMA operand).
__device__ __forceinline__ void split_bf16x4(f32x4 x, u32x2 &hi, u32x2 &lo)
{
    uint32_t h0, l0, h1, l1;
    split_bf16_pair(x[0], x[1], h0, l0);
    split_bf16_pair(x[2], x[3], h1, l1);
    hi = u32x2{h0, h1};
    lo = u32x2{l0, l1};
}

// Round fp32 to bf16, nearest-even (v_cvt_pk_bf16_f32); inf/NaN kept.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v)
{
    f32x2 p = {v, 0.0f};
    bf16x2 h = __builtin_convertvector(p, bf16x2);
    return (uint16_t)(__builtin_bit_cast(uint32_t, h) & 0xFFFFu);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// DPP rotate by 8 within each 16-lane row: lane l reads lane (l & ~15) | ((l + 8) & 15).
__device__ __forceinline__ float dpp_row_ror8(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// V4.1 expert activation ("cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs",
// dsv4_global_gate_up_mxfp4 with its bf16 flag): gate and up rounded to
// bf16; with lim > 0 up clamped to [-lim, lim] and gate capped at lim; the
// route weight w folded in.  The caller rounds the result to bf16.
__device__ __forceinline__ float swiglu_v41(float g, float u, float w, float lim)
{
    g = bf16_bits_to_f32(f32_to_bf16_bits(g));
    u = bf16_bits_to_f32(f32_to_bf16_bits(u));
    if (lim > 0.0f) {
        u = u < -lim ? -lim : (u > lim ? lim : u);
        g = g > lim ? lim : g;
    }
    return w * (silu(g) * u);
}

// First byte of expert e's tensor in a bank: bank + e * stride for a
// contiguous bank, or entry e of a table of per-expert pointers (PT).  The
// kernels on the measured paths take PT as a template parameter: a runtime
// choice between the two made the 64-expert decode layer 7 % slower
// (111.6 -> 119.8 us), with the same registers.
template <bool PT>
__device__ __forceinline__ const uint8_t *expert_base(const uint8_t *bank, int e, int64_t stride)
{
    if constexpr (PT)
        return reinterpret_cast<const uint8_t *const *>(bank)[e];
    else
        return bank + (int64_t)e * stride;
}

// The same with the choice made at run time (kernels off the measured path).
__device__ __forceinline__ const uint8_t *expert_base_rt(const uint8_t *bank, int ptr_table,
                                                         int e, int64_t stride)
{
    return ptr_table ? expert_base<true>(bank, e, stride) : expert_base<false>(bank, e, stride);
}

// s_waitcnt with vmcnt(n) and the other counters left alone (gfx9 layout).
template <int N> __device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Direct global -> LDS loads: `bytes` (16 or 4) per lane, lane l's bytes to
// lds + l * bytes (lds is wave-uniform).  Kept in plain device functions: the
// kernel templates' host pass must not see the builtin.
__device__ __forceinline__ void lds_dma16(const void *g, void *lds)
{
    __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void *g, void *lds)
{
    __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0);
}

// s_waitcnt lgkmcnt(0) with the other counters left alone: this wave's LDS
// writes are done.
__device__ __forceinline__ void wait_lgkm0()
{
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
}

// Workgroup barrier without a memory fence (a fence would wait for every
// load in flight); the compiler barriers keep LDS accesses on their side.
__device__ __forceinline__ void raw_barrier()
{
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
}

constexpr int NXCD = 8; // MI355X: 8 XCDs, each with its own L2

// Workgroups are dispatched to the XCDs round-robin by id.  This maps the
// dispatch id to a logical id so that each XCD receives a contiguous range
// of logical ids (a bijection on [0, n)).
__device__ __forceinline__ int xcd_logical(int pid, int n)
{
    const int x = pid % NXCD, i = pid / NXCD;
    const int base = n / NXCD, rem = n % NXCD;
    return x < rem ? x * (base + 1) + i : rem * (base + 1) + (x - rem) * base + i;
}

} // namespace mx
