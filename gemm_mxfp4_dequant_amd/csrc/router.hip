// Device router for the expert bank: gating logits -> the top-k experts of
// each token and their renormalised weights (a softmax over the logits, the
// k most probable kept, their probabilities divided by the sum of the kept
// ones), i.e. the picks and weights that the MoE frame of "cortiq-engine
// 0.8.40, src/gpu_wgpu/mxfp4.rs" takes as inputs, computed on the device.
// The pages give no router of their own; this is the routing of the
// 64-expert decode workload (softmax over N(0,1) logits, top 6,
// renormalised).
//
// Definition (per token):
//  * order: the larger logit first; equal logits by the lower expert index;
//    -0 equals +0; NaN ranks below every number (-inf included).  Slot k
//    receives the expert of rank k.
//  * weights: w_k = exp(l_k - l_0) / sum_j exp(l_j - l_0) over the k chosen
//    logits, l_0 the largest.  The softmax normaliser over all experts
//    cancels in the renormalisation, so this equals p_k / sum_j p_j.
//
// One wave per token.  Each lane holds up to 16 logits as 64-bit keys
// (order-preserving bits of the value, then the complement of the index, so
// that one unsigned maximum picks the larger value and, on a tie, the lower
// index); top_k rounds of a wave-wide maximum (DPP rotations within each
// 16-lane row, then the four row maxima as scalars) select the slots in rank
// order, the winner's lane retiring its key.  The exponentials are fp32 expf, summed in slot order.
#include "device.h"
#include "launch.h"

namespace mx {

namespace {

constexpr int RT_WAVES = 4; // tokens (waves) per workgroup

__device__ __forceinline__ uint64_t route_key(float v, int e)
{
    uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v); // -0 -> +0
    if (v != v)
        b = 0u; // NaN: below every number
    else        // order-preserving: every number (-inf = 0x007FFFFF) maps above 0
        b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)b << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

// Maximum over the wave: within each 16-lane row by DPP rotations (row_ror
// 1, 2, 4, 8 leave every lane with its row's maximum), then the four row
// maxima read as scalars.  Returns the same value in every lane.
template <int CTRL> __device__ __forceinline__ uint64_t dpp_u64(uint64_t k)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)k, CTRL, 0xF, 0xF, false);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(k >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k)
{
    uint64_t o;
    o = dpp_u64<0x121>(k); // row_ror:1
    k = o > k ? o : k;
    o = dpp_u64<0x122>(k); // row_ror:2
    k = o > k ? o : k;
    o = dpp_u64<0x124>(k); // row_ror:4
    k = o > k ? o : k;
    o = dpp_u64<0x128>(k); // row_ror:8
    k = o > k ? o : k;
    uint64_t m = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)k, 16 * r);
        const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 16 * r);
        const uint64_t v = ((uint64_t)hi << 32) | lo;
        m = v > m ? v : m;
    }
    return m;
}

__device__ __forceinline__ float key_value(uint64_t k)
{
    uint32_t b = (uint32_t)(k >> 32);
    if (b == 0u)
        return __uint_as_float(0x7FC00000u);
    b = (b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b;
    return __uint_as_float(b);
}

// NK: logits per lane (64 * NK >= n_experts; n_experts <= 1024)
template <int NK>
__global__ __launch_bounds__(RT_WAVES * 64) void route_topk_kernel(const float *logits,
                                                                  int n_tokens, int n_experts,
                                                                  int top_k, int32_t *ids,
                                                                  float *w)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * RT_WAVES + (threadIdx.x >> 6);
    if (t >= n_tokens)
        return;
    const float *row = logits + (int64_t)t * n_experts;
    // lane l holds experts l, l + 64, ...; absent experts have key 0, below
    // every real key (a NaN logit keeps its index bits, so it is above 0)
    uint64_t key[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < n_experts ? route_key(row[e], e) : 0ull;
    }
    float mine = 0.0f; // lane k: the logit of slot k
    int my_e = -1;
    for (int k = 0; k < top_k; ++k) {
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < NK; ++i)
            best = key[i] > best ? key[i] : best;
        const uint64_t win = wave_max_u64(best);
        const int e = (int)(0xFFFFFFFFu - (uint32_t)win);
#pragma unroll
        for (int i = 0; i < NK; ++i) // the owner retires the chosen key
            if (lane + 64 * i == e)
                key[i] = 0ull;
        if (lane == k) {
            mine = key_value(win);
            my_e = e;
        }
    }
    const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), 0));
    const float ek = lane < top_k ? expf(mine - l0) : 0.0f;
    float s = 0.0f;
    for (int k = 0; k < top_k; ++k) // slot order
        s += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ek), k));
    if (lane < top_k) {
        ids[(int64_t)t * top_k + lane] = my_e;
        w[(int64_t)t * top_k + lane] = ek / s;
    }
}

} // namespace

hipError_t route_topk_launch(const float *logits, int n_tokens, int n_experts, int top_k,
                             int32_t *ids, float *w, hipStream_t stream)
{
    const int blocks = (n_tokens + RT_WAVES - 1) / RT_WAVES;
    const dim3 grid(blocks), block(RT_WAVES * 64);
    if (n_experts <= 64)
        hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, stream, logits, n_tokens,
                           n_experts, top_k, ids, w);
    else if (n_experts <= 128)
        hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, stream, logits, n_tokens,
                           n_experts, top_k, ids, w);
    else if (n_experts <= 256)
        hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, stream, logits, n_tokens,
                           n_experts, top_k, ids, w);
    else if (n_experts <= 512)
        hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, stream, logits, n_tokens,
                           n_experts, top_k, ids, w);
    else if (n_experts <= 1024)
        hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, stream, logits, n_tokens,
                           n_experts, top_k, ids, w);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

} // namespace mx
