// MXFP4 -> fp32 / bf16 dequantization, bit-exact.
//
// "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs", DECODE shader (mx_e2m1,
// mx_e8m0): weight = E2M1(code) * 2^(k-127).  Every finite product is
// exactly representable in fp32 and in bf16, so the hardware conversion
// (which rounds once) gives the exact value; overflow gives +-inf.  A
// scale-255 group is written as the canonical NaN 0x7FC00000 / 0x7FC0.
//
// One thread per code word (8 consecutive weights of one row: a row's code
// bytes are contiguous, and word i belongs to group i/4, whose scale is byte
// i/4 of the scale plane).  Loads and stores are contiguous across a wave.
#include "device.h"
#include "launch.h"

namespace mx {

template <bool BF16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t *codes, const uint8_t *scales,
                                                      int64_t n_words, void *out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += stride) {
        const uint32_t word = codes[i];
        const uint32_t k = scales[i >> 2];
        const float s = e8m0_operand(k);
        if (BF16) {
            u32x4 v;
            v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 0));
            v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 1));
            v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 2));
            v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 3));
            if (k == 255u)
                v = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
            reinterpret_cast<u32x4 *>(out)[i] = v;
        } else {
            float f[8];
            decode8_f32(word, s, f);
            f32x4 lo = {f[0], f[1], f[2], f[3]};
            f32x4 hi = {f[4], f[5], f[6], f[7]};
            if (k == 255u) {
                const float qnan = __uint_as_float(0x7FC00000u);
                lo = f32x4{qnan, qnan, qnan, qnan};
                hi = lo;
            }
            reinterpret_cast<f32x4 *>(out)[2 * i] = lo;
            reinterpret_cast<f32x4 *>(out)[2 * i + 1] = hi;
        }
    }
}

hipError_t dequant_launch(const uint8_t *w, int64_t rows, int64_t cols, void *out, bool bf16,
                          hipStream_t stream)
{
    const int64_t n_words = rows * cols / 8;
    const uint8_t *scales = w + rows * cols / 2;
    int64_t blocks = (n_words + 255) / 256;
    if (blocks > 256 * 64)
        blocks = 256 * 64;
    if (bf16)
        hipLaunchKernelGGL(dequant_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           reinterpret_cast<const uint32_t *>(w), scales, n_words, out);
    else
        hipLaunchKernelGGL(dequant_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           reinterpret_cast<const uint32_t *>(w), scales, n_words, out);
    return hipGetLastError();
}

} // namespace mx
