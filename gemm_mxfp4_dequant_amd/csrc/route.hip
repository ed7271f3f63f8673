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
// the route weight multiplies the fp32 down output; in V4.1 mode the weight
// is already folded into the activation and the slots are summed as they
// are), summed in slot order
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

// Inclusive scans over the experts (E <= GT, expert = thread) of the pair
// counts n, the work items ceil(n / tpc) and the cold experts (1 <= n <=
// cold_max): shuffle scans within waves, then the wave totals.  scan
// [3][GT], wsum [3][GT / 64] in LDS.
__device__ void scan_experts(const GroupArgs &g, int n, int32_t *scan, int32_t *wsum)
{
    const int tid = threadIdx.x, wave = tid >> 6;
    int v[3] = {n, (n + g.tpc - 1) / g.tpc, (n > 0 && n <= g.cold_max) ? 1 : 0};
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        v[i] = wave_inclusive_scan(v[i]);
        if ((tid & 63) == 63)
            wsum[i * (GT / 64) + wave] = v[i];
    }
    __syncthreads();
    for (int w = 0; w < wave; ++w)
#pragma unroll
        for (int i = 0; i < 3; ++i)
            v[i] += wsum[i * (GT / 64) + w];
#pragma unroll
    for (int i = 0; i < 3; ++i)
        scan[i * GT + tid] = v[i];
    __syncthreads();
}

// The work items {expert, first slot, pairs, 0} of expert e (first slot s0,
// n pairs), up to tpc pairs each, in work from position item0; with the
// split on, also in work_cold at cold_idx (a cold expert: one item) or in
// work_hot from position hot0.
__device__ void write_items(const GroupArgs &g, int e, int s0, int n, int item0, int hot0,
                            int cold_idx)
{
    const bool cold = n > 0 && n <= g.cold_max;
    for (int c = 0; c * g.tpc < n; ++c) {
        const int4 wk = make_int4(e, s0 + c * g.tpc, min(g.tpc, n - c * g.tpc), 0);
        reinterpret_cast<int4 *>(g.work)[item0 + c] = wk;
        if (cold)
            reinterpret_cast<int4 *>(g.work_cold)[cold_idx] = wk;
        else if (g.cold_max)
            reinterpret_cast<int4 *>(g.work_hot)[hot0 + c] = wk;
    }
}

__global__ __launch_bounds__(GT) void group_kernel(GroupArgs g, int nch)
{
    extern __shared__ __align__(16) int32_t lds[];
    const int E = g.n_experts, P = g.n_pairs, tid = threadIdx.x;
    int32_t *cnt = lds;                 // [nch][E]
    int32_t *tot = cnt + nch * E;       // [E]
    int32_t *scan = tot + E;            // [3][GT] scans over experts
    int32_t *wsum = scan + 3 * GT;      // [3][GT / 64] wave totals
    int32_t *sids = wsum + 3 * (GT / 64); // [P] when P <= IDS_IN_LDS
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
    // 3. inclusive scans over experts of counts and work items
    scan_experts(g, tid < E ? tot[tid] : 0, scan, wsum);
    // offsets (exclusive) and the totals
    if (tid < E) {
        const int excl = scan[tid] - tot[tid];
        g.offsets[tid] = excl;
        tot[tid] = excl; // reuse: start slot of expert tid
    }
    if (tid == 0) {
        g.offsets[E] = scan[E - 1];
        if (g.n_work)
            *g.n_work = scan[GT + E - 1];
        if (g.n_work_hot)
            *g.n_work_hot = scan[GT + E - 1] - scan[2 * GT + E - 1];
        if (g.n_work_cold)
            *g.n_work_cold = scan[2 * GT + E - 1];
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
        const int n = scan[tid] - tot[tid];
        const int item0 = scan[GT + tid] - (n + g.tpc - 1) / g.tpc;
        const int cold_before = scan[2 * GT + tid] - (n > 0 && n <= g.cold_max ? 1 : 0);
        write_items(g, tid, tot[tid], n, item0, item0 - cold_before, scan[2 * GT + tid] - 1);
    }
}

// Fast path for up to GT / 64 * TPW tiles of 64 pairs.  Each wave ranks the
// pairs of its tiles among the lanes with the same expert id with one ballot
// per key bit (the lanes whose key agrees on every bit are the same
// expert), so a pair's rank within its tile is the number of lower lanes
// among its peers, and the lowest peer writes the tile's count for that
// expert.  A per-expert exclusive prefix over tiles, plus the expert
// offsets, gives each pair its slot; the scatter is then one store per
// pair.  Same result as the chunked kernel: pairs sorted by (expert, index).
constexpr int TPW = 8;     // tiles per wave
constexpr int KEYBITS = 11;     // keys: expert ids 0..1023, and NO_EXPERT
constexpr int NO_EXPERT = 2047; // key of a dropped pair (above every expert id)

__global__ __launch_bounds__(GT) void group_tiles_kernel(GroupArgs g, int ntiles)
{
    extern __shared__ __align__(16) int32_t lds[];
    const int E = g.n_experts, P = g.n_pairs, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    int32_t *hist = lds;                 // [ntiles][E]: counts, then prefix over tiles
    int32_t *tot = hist + ntiles * E;    // [E]
    int32_t *scan = tot + E;             // [3][GT] scans over experts
    int32_t *wsum = scan + 3 * GT;       // [3][GT / 64] wave totals

    for (int i = tid; i < ntiles * E; i += GT)
        hist[i] = 0;
    __syncthreads();

    // 1. ranks within tiles and per-tile counts
    int my_e[TPW], my_rank[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        const int tile = wave + (GT / 64) * k;
        const int p = tile * 64 + lane;
        int e = -1;
        if (tile < ntiles && p < P) {
            e = g.ids[p];
            if (e < 0 || e >= E)
                e = -1;
        }
        const int key = e >= 0 ? e : NO_EXPERT;
        uint64_t peers = ~0ull;
#pragma unroll
        for (int b = 0; b < KEYBITS; ++b) {
            const int bit = (key >> b) & 1;
            const uint64_t bal = __ballot(bit);
            peers &= bit ? bal : ~bal;
        }
        const int rank = __popcll(peers & ((1ull << lane) - 1));
        if (e >= 0 && rank == 0)
            hist[tile * E + e] = __popcll(peers);
        my_e[k] = e;
        my_rank[k] = rank;
    }
    __syncthreads();
    // 2. per-expert exclusive prefix over tiles
    for (int e = tid; e < E; e += GT) {
        int run = 0;
        for (int t = 0; t < ntiles; ++t) {
            const int v = hist[t * E + e];
            hist[t * E + e] = run;
            run += v;
        }
        tot[e] = run;
    }
    __syncthreads();
    // 3. inclusive scans over experts of counts and work items
    scan_experts(g, tid < E ? tot[tid] : 0, scan, wsum);
    if (tid < E) {
        const int excl = scan[tid] - tot[tid];
        g.offsets[tid] = excl;
        tot[tid] = excl; // reuse: start slot of expert tid
    }
    if (tid == 0) {
        g.offsets[E] = scan[E - 1];
        if (g.n_work)
            *g.n_work = scan[GT + E - 1];
        if (g.n_work_hot)
            *g.n_work_hot = scan[GT + E - 1] - scan[2 * GT + E - 1];
        if (g.n_work_cold)
            *g.n_work_cold = scan[2 * GT + E - 1];
    }
    __syncthreads();
    // 4. scatter, one pair per lane and tile
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        const int tile = wave + (GT / 64) * k;
        const int p = tile * 64 + lane;
        if (tile >= ntiles || p >= P)
            continue;
        const int e = my_e[k];
        if (e >= 0) {
            const int s = tot[e] + hist[tile * E + e] + my_rank[k];
            g.pair_of_slot[s] = p;
            g.slot_of_pair[p] = s;
            if (g.token_of_slot)
                g.token_of_slot[s] = p / g.top_k;
        } else {
            g.slot_of_pair[p] = -1;
        }
    }
    // 5. work items {expert, first slot, tokens, 0}
    if (g.work && tid < E) {
        const int n = scan[tid] - tot[tid];
        const int item0 = scan[GT + tid] - (n + g.tpc - 1) / g.tpc;
        const int cold_before = scan[2 * GT + tid] - (n > 0 && n <= g.cold_max ? 1 : 0);
        write_items(g, tid, tot[tid], n, item0, item0 - cold_before, scan[2 * GT + tid] - 1);
    }
}

// One wave, up to SMALL_TILES tiles of 64 pairs (decode-sized routing): the
// same tile ranking, then the per-expert prefix and the scans over experts
// in chunks of 64 experts, all within the wave.
constexpr int SMALL_TILES = 8;

__global__ __launch_bounds__(64) void group_small_kernel(GroupArgs g, int ntiles)
{
    extern __shared__ __align__(16) int32_t lds[];
    const int E = g.n_experts, P = g.n_pairs, lane = threadIdx.x;
    int32_t *hist = lds;              // [ntiles][E]
    int32_t *cnt = hist + ntiles * E; // [E] pairs per expert
    int32_t *start = cnt + E;         // [E] first slot
    int32_t *item0 = start + E;       // [E] first work item
    int32_t *split = item0 + E;       // [E] cold item / first item among the hot

    for (int i = lane; i < ntiles * E; i += 64)
        hist[i] = 0;
    __syncthreads();
    int my_e[SMALL_TILES], my_rank[SMALL_TILES];
#pragma unroll
    for (int k = 0; k < SMALL_TILES; ++k) {
        const int p = k * 64 + lane;
        int e = -1;
        if (k < ntiles && p < P) {
            e = g.ids[p];
            if (e < 0 || e >= E)
                e = -1;
        }
        const int key = e >= 0 ? e : NO_EXPERT;
        uint64_t peers = ~0ull;
#pragma unroll
        for (int b = 0; b < KEYBITS; ++b) {
            const int bit = (key >> b) & 1;
            const uint64_t bal = __ballot(bit);
            peers &= bit ? bal : ~bal;
        }
        const int rank = __popcll(peers & ((1ull << lane) - 1));
        if (e >= 0 && rank == 0)
            hist[k * E + e] = __popcll(peers);
        my_e[k] = e;
        my_rank[k] = rank;
    }
    __syncthreads();
    for (int e = lane; e < E; e += 64) {
        int run = 0;
        for (int t = 0; t < ntiles; ++t) {
            const int v = hist[t * E + e];
            hist[t * E + e] = run;
            run += v;
        }
        cnt[e] = run;
    }
    __syncthreads();
    // item0[e]: the expert's first work item; split[e]: its cold item, or
    // its first item among the other experts'
    int carry_a = 0, carry_b = 0, carry_c = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        const int n = e < E ? cnt[e] : 0;
        const bool cold = n > 0 && n <= g.cold_max;
        const int ni = (n + g.tpc - 1) / g.tpc;
        const int a = wave_inclusive_scan(n) + carry_a;
        const int b = wave_inclusive_scan(ni) + carry_b;
        const int c = wave_inclusive_scan(cold ? 1 : 0) + carry_c;
        if (e < E) {
            start[e] = a - n;
            item0[e] = b - ni;
            split[e] = cold ? c - 1 : (b - c) - ni;
            g.offsets[e] = a - n;
        }
        carry_a = __shfl(a, 63, 64);
        carry_b = __shfl(b, 63, 64);
        carry_c = __shfl(c, 63, 64);
    }
    if (lane == 0) {
        g.offsets[E] = carry_a;
        if (g.n_work)
            *g.n_work = carry_b;
        if (g.n_work_hot)
            *g.n_work_hot = carry_b - carry_c;
        if (g.n_work_cold)
            *g.n_work_cold = carry_c;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < SMALL_TILES; ++k) {
        const int p = k * 64 + lane;
        if (k >= ntiles || p >= P)
            continue;
        const int e = my_e[k];
        if (e >= 0) {
            const int s = start[e] + hist[k * E + e] + my_rank[k];
            g.pair_of_slot[s] = p;
            g.slot_of_pair[p] = s;
            if (g.token_of_slot)
                g.token_of_slot[s] = p / g.top_k;
        } else {
            g.slot_of_pair[p] = -1;
        }
    }
    if (g.work) {
        for (int e = lane; e < E; e += 64)
            write_items(g, e, start[e], cnt[e], item0[e], split[e], split[e]);
    }
}

hipError_t group_launch(const GroupArgs &g, hipStream_t stream)
{
    const int ntiles = (g.n_pairs + 63) / 64;
    if (ntiles <= SMALL_TILES) {
        const size_t slds = ((size_t)ntiles * g.n_experts + 4 * (size_t)g.n_experts) * 4;
        // at most (8 + 4) * 1024 * 4 = 48 KB
        hipLaunchKernelGGL(group_small_kernel, dim3(1), dim3(64), slds, stream, g, ntiles);
        return hipGetLastError();
    }
    const size_t tlds =
        ((size_t)ntiles * g.n_experts + g.n_experts + 3 * GT + 3 * (GT / 64)) * 4;
    if (ntiles <= (GT / 64) * TPW && tlds <= 128 * 1024) {
        static std::atomic<uint8_t> topted{0};
        if (tlds > 64 * 1024 && !topted.load(std::memory_order_acquire)) {
            hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void *>(group_tiles_kernel),
                                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                                160 * 1024);
            if (st != hipSuccess)
                return st;
            topted.store(1, std::memory_order_release);
        }
        hipLaunchKernelGGL(group_tiles_kernel, dim3(1), dim3(GT), tlds, stream, g, ntiles);
        return hipGetLastError();
    }

    const int nch = group_chunks(g.n_pairs, g.n_experts);
    size_t lds = ((size_t)nch * g.n_experts + g.n_experts + 3 * GT + 3 * (GT / 64)) * 4;
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
            wk[j] = ok[j] ? (w ? w[t * top_k + k] : 1.f) : 0.f;
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

// V4.1 routing with the shared expert as slot K of every token (expert E,
// weight 1); routed ids outside [0, E) become -1 so that none can alias the
// shared expert.
__global__ __launch_bounds__(256) void augment_kernel(const int32_t *ids, const float *w, int n,
                                                      int top_k, int n_experts, int32_t *ids_aug,
                                                      float *w_aug)
{
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= n)
        return;
    const int t = p / (top_k + 1), k = p % (top_k + 1);
    if (k < top_k) {
        const int e = ids[t * top_k + k];
        ids_aug[p] = (e >= 0 && e < n_experts) ? e : -1;
        w_aug[p] = w[t * top_k + k];
    } else {
        ids_aug[p] = n_experts;
        w_aug[p] = 1.0f;
    }
}

hipError_t augment_launch(const int32_t *ids, const float *w, int n_tokens, int top_k,
                          int n_experts, int32_t *ids_aug, float *w_aug, hipStream_t stream)
{
    const int n = n_tokens * (top_k + 1);
    hipLaunchKernelGGL(augment_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       ids, w, n, top_k, n_experts, ids_aug, w_aug);
    return hipGetLastError();
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
