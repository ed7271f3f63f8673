// Expert-bank plumbing: stable grouping of routed pairs by expert (plus the
// work list of the expert kernels) and the weighted combine.
//
// Grouping follows "rlx-cpu 0.2.17, src/gguf_matmul.rs",
// grouped_moe_sort_plan (counts -> exclusive offsets -> ordered scatter);
// here one workgroup does it deterministically without atomics: the pairs
// are cut into chunks, each chunk counts per expert, a per-expert prefix over
// chunks gives each chunk its starting rank, and each chunk scatters its
// pairs in order.  The result is the pairs sorted by (expert, pair index).
//
// The combine is the weighted sum of "cortiq-engine 0.8.40,
// src/gpu_wgpu/mxfp4.rs" (dsv4_global_down_mxfp4, generic f32 weighting:
// the route weight multiplies the fp32 down output), summed in slot order
// k = 0..top_k-1, and the un-permutation of "rlx-cpu 0.2.17,
// src/gguf_matmul.rs" (grouped_moe_unpermute_out); bf16 output is rounded
// to nearest-even (the mxg_bf16 rule).
#include <atomic>

#include "device.h"
#include "launch.h"

namespace mx {

namespace {
constexpr int GT = 1024;          // grouping threads
constexpr int IDS_IN_LDS = 8192;  // pairs staged in LDS when P is at most this

int group_chunks(int n_pairs, int n_experts)
{
    int nch = 16384 / (n_experts > 0 ? n_experts : 1);
    if (nch > 64)
        nch = 64;
    if (nch > n_pairs)
        nch = n_pairs;
    return nch < 1 ? 1 : nch;
}
} // namespace

int group_max_work(int n_pairs, int n_experts, int tpc)
{
    const int active = n_experts < n_pairs ? n_experts : n_pairs;
    const int bound = (n_pairs + tpc - 1) / tpc + active;
    return bound < n_pairs ? bound : n_pairs;
}

__device__ __forceinline__ int wave_inclusive_scan(int v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d, 64);
        if (lane >= d)
            v += o;
    }
    return v;
}

__global__ __launch_bounds__(GT) void group_kernel(GroupArgs g, int nch)
{
    extern __shared__ __align__(16) int32_t lds[];
    const int E = g.n_experts, P = g.n_pairs, tid = threadIdx.x;
    int32_t *cnt = lds;                 // [nch][E]
    int32_t *tot = cnt + nch * E;       // [E]
    int32_t *scan_a = tot + E;          // [GT] offsets scan
    int32_t *scan_b = scan_a + GT;      // [GT] work-item scan
    int32_t *wsum_a = scan_b + GT;      // [GT / 64] wave totals
    int32_t *wsum_b = wsum_a + GT / 64;
    int32_t *sids = wsum_b + GT / 64;   // [P] when P <= IDS_IN_LDS
    const bool ids_lds = P <= IDS_IN_LDS;
    const int cs = (P + nch - 1) / nch;

    for (int i = tid; i < nch * E; i += GT)
        cnt[i] = 0;
    if (ids_lds)
        for (int p = tid; p < P; p += GT)
            sids[p] = g.ids[p];
    __syncthreads();
    const int32_t *ids = ids_lds ? sids : g.ids;

    // 1. per-chunk counts
    if (tid < nch) {
        const int p1 = min(P, (tid + 1) * cs);
        for (int p = tid * cs; p < p1; ++p) {
            const int e = ids[p];
            if (e >= 0 && e < E)
                cnt[tid * E + e] += 1;
        }
    }
    __syncthreads();
    // 2. per-expert exclusive prefix over chunks
    for (int e = tid; e < E; e += GT) {
        int run = 0;
        for (int c = 0; c < nch; ++c) {
            const int v = cnt[c * E + e];
            cnt[c * E + e] = run;
            run += v;
        }
        tot[e] = run;
    }
    __syncthreads();
    // 3. inclusive scans over experts (E <= GT) of counts and work items:
    //    shuffle scans within waves, then the wave totals
    {
        const int n = tid < E ? tot[tid] : 0;
        int a = wave_inclusive_scan(n);
        int b = wave_inclusive_scan((n + g.tpc - 1) / g.tpc);
        const int wave = tid >> 6;
        if ((tid & 63) == 63) {
            wsum_a[wave] = a;
            wsum_b[wave] = b;
        }
        __syncthreads();
        for (int w = 0; w < wave; ++w) {
            a += wsum_a[w];
            b += wsum_b[w];
        }
        scan_a[tid] = a;
        scan_b[tid] = b;
        __syncthreads();
    }
    // offsets (exclusive) and the total
    if (tid < E) {
        const int excl = scan_a[tid] - tot[tid];
        g.offsets[tid] = excl;
        tot[tid] = excl; // reuse: start slot of expert tid
    }
    if (tid == 0) {
        g.offsets[E] = scan_a[E - 1];
        if (g.n_work)
            *g.n_work = scan_b[E - 1];
    }
    __syncthreads();
    // 4. ordered scatter
    if (tid < nch) {
        const int p1 = min(P, (tid + 1) * cs);
        for (int p = tid * cs; p < p1; ++p) {
            const int e = ids[p];
            if (e >= 0 && e < E) {
                const int s = tot[e] + cnt[tid * E + e]++;
                g.pair_of_slot[s] = p;
                g.slot_of_pair[p] = s;
                if (g.token_of_slot)
                    g.token_of_slot[s] = p / g.top_k;
            } else {
                g.slot_of_pair[p] = -1;
            }
        }
    }
    // 5. work items {expert, first slot, tokens, 0}
    if (g.work && tid < E) {
        const int n = scan_a[tid] - tot[tid];
        const int first_item = scan_b[tid] - (n + g.tpc - 1) / g.tpc;
        for (int c = 0; c * g.tpc < n; ++c) {
            int4 wk;
            wk.x = tid;
            wk.y = tot[tid] + c * g.tpc;
            wk.z = min(g.tpc, n - c * g.tpc);
            wk.w = 0;
            reinterpret_cast<int4 *>(g.work)[first_item + c] = wk;
        }
    }
}

hipError_t group_launch(const GroupArgs &g, hipStream_t stream)
{
    const int nch = group_chunks(g.n_pairs, g.n_experts);
    size_t lds = ((size_t)nch * g.n_experts + g.n_experts + 2 * GT + 2 * (GT / 64)) * 4;
    if (g.n_pairs <= IDS_IN_LDS)
        lds += (size_t)g.n_pairs * 4;
    static std::atomic<uint8_t> opted{0};
    if (lds > 64 * 1024 && !opted.load(std::memory_order_acquire)) {
        hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void *>(group_kernel),
                                            hipFuncAttributeMaxDynamicSharedMemorySize,
                                            160 * 1024);
        if (st != hipSuccess)
            return st;
        opted.store(1, std::memory_order_release);
    }
    hipLaunchKernelGGL(group_kernel, dim3(1), dim3(GT), lds, stream, g, nch);
    return hipGetLastError();
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float *y, const int32_t *slot_of_pair,
                                                      const float *w, int top_k, int hidden,
                                                      int blocks_per_token, void *out)
{
    const int t = blockIdx.x / blocks_per_token;
    const int r = ((blockIdx.x % blocks_per_token) * 256 + threadIdx.x) * 4;
    if (r >= hidden)
        return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // slots in groups of 8: all loads of a group are issued before the sums
    for (int k0 = 0; k0 < top_k; k0 += 8) {
        f32x4 v[8];
        float wk[8];
        bool ok[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = k0 + j;
            const int s = k < top_k ? slot_of_pair[t * top_k + k] : -1;
            ok[j] = s >= 0;
            wk[j] = ok[j] ? w[t * top_k + k] : 0.f;
            v[j] = ok[j] ? *reinterpret_cast<const f32x4 *>(y + (int64_t)s * hidden + r)
                         : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (!ok[j])
                continue;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] += wk[j] * v[j][i];
        }
    }
    if (OUT_BF16) {
        u32x2 o;
        o[0] = (uint32_t)f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
        o[1] = (uint32_t)f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
        *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(out) + (int64_t)t * hidden + r) = o;
    } else {
        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + (int64_t)t * hidden + r) = acc;
    }
}

hipError_t combine_launch(const float *y, const int32_t *slot_of_pair, const float *w,
                          int n_tokens, int top_k, int hidden, void *out, bool out_bf16,
                          hipStream_t stream)
{
    const int bpt = (hidden / 4 + 255) / 256;
    dim3 grid((unsigned)((int64_t)bpt * n_tokens));
    if (out_bf16)
        hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, stream, y, slot_of_pair, w,
                           top_k, hidden, bpt, out);
    else
        hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, stream, y, slot_of_pair, w,
                           top_k, hidden, bpt, out);
    return hipGetLastError();
}

hipError_t copy_launch(void *dst, const void *src, size_t bytes, hipStream_t stream)
{
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, stream);
}

} // namespace mx
