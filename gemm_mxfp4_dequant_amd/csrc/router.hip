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
// index); top_k rounds of a wave-wide maximum (DPP-free butterfly over
// __shfl_xor) select the slots in rank order, the winner's lane retiring
// its key.  The exponentials are fp32 expf, summed in slot order.
#include "device.h"
#include "launch.h"

namespace mx {

namespace {

constexpr int RT_WAVES = 4;        // tokens (waves) per workgroup
constexpr int RT_PER_LANE = 16;    // logits per lane (n_experts <= 1024)

__device__ __forceinline__ uint64_t route_key(float v, int e)
{
    uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v); // -0 -> +0
    if (v != v)
        b = 0u; // NaN: below every number
    else        // order-preserving: every number (-inf = 0x007FFFFF) maps above 0
        b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)b << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)k, off, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(k >> 32), off, 64);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        k = o > k ? o : k;
    }
    return k;
}

__device__ __forceinline__ float key_value(uint64_t k)
{
    uint32_t b = (uint32_t)(k >> 32);
    if (b == 0u)
        return __uint_as_float(0x7FC00000u);
    b = (b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b;
    return __uint_as_float(b);
}

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
    uint64_t key[RT_PER_LANE];
#pragma unroll
    for (int i = 0; i < RT_PER_LANE; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < n_experts ? route_key(row[e], e) : 0ull;
    }
    float mine = 0.0f; // lane k: the logit of slot k
    int my_e = -1;
    for (int k = 0; k < top_k; ++k) {
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < RT_PER_LANE; ++i)
            best = key[i] > best ? key[i] : best;
        const uint64_t win = wave_max_u64(best);
        const int e = (int)(0xFFFFFFFFu - (uint32_t)win);
#pragma unroll
        for (int i = 0; i < RT_PER_LANE; ++i) // the owner retires the chosen key
            if (lane + 64 * i == e)
                key[i] = 0ull;
        if (lane == k) {
            mine = key_value(win);
            my_e = e;
        }
    }
    const float l0 = __shfl(mine, 0, 64);
    const float ek = lane < top_k ? expf(mine - l0) : 0.0f;
    float s = 0.0f;
    for (int k = 0; k < top_k; ++k) // slot order
        s += __shfl(ek, k, 64);
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
    hipLaunchKernelGGL(route_topk_kernel, dim3(blocks), dim3(RT_WAVES * 64), 0, stream, logits,
                       n_tokens, n_experts, top_k, ids, w);
    return hipGetLastError();
}

} // namespace mx
