// C ABI of libmxfp4.so (declared in include/mxfp4.h): argument checks on the
// host, kernel choice by shape, launches on the caller's stream.  No
// allocation, no synchronisation, no CPU fallback.
//
// The checks mirror the refusals of the pages' entry points: matmat in
// "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs" (b == 0, rows == 0,
// cols % 32 != 0, short or mis-shaped buffers) and run_stages in
// "cortiq-engine 0.8.77, src/qtensor/moe_fast.rs" (empty groups, length
// mismatches, out-of-range indices).  Every check runs before any HIP call,
// so refusals work on a machine without a GPU.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/mxfp4.h"
#include "launch.h"

#include <atomic>
#include <cmath>
#include <mutex>

namespace {

thread_local char g_err[512];

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = 0; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int check_tensor(const char *name, const void *w, int64_t rows, int64_t cols)
{
    if (!w)
        return fail(MXFP4_EINVAL, "%s: null pointer", name);
    if (!aligned(w, 16))
        return fail(MXFP4_EALIGN, "%s: pointer not 16-byte aligned", name);
    if (rows < 1 || rows > MXFP4_MAX_ROWS)
        return fail(MXFP4_EINVAL, "%s: rows = %lld outside [1, %d]", name, (long long)rows,
                    MXFP4_MAX_ROWS);
    if (cols < 32 || cols > MXFP4_MAX_COLS || cols % 32 != 0)
        return fail(MXFP4_EINVAL, "%s: cols = %lld must be a multiple of 32 in [32, %d]", name,
                    (long long)cols, MXFP4_MAX_COLS);
    if (mxfp4_nbytes(rows, cols) > MXFP4_MAX_TENSOR_BYTES)
        return fail(MXFP4_EINVAL, "%s: %lld x %lld exceeds %lld bytes", name, (long long)rows,
                    (long long)cols, (long long)MXFP4_MAX_TENSOR_BYTES);
    return MXFP4_OK;
}

int check_dtype(const char *name, int dt)
{
    if (dt != MXFP4_F32 && dt != MXFP4_BF16)
        return fail(MXFP4_EINVAL, "%s: dtype %d is neither MXFP4_F32 nor MXFP4_BF16", name, dt);
    return MXFP4_OK;
}

int check_buffer(const char *name, const void *p, uintptr_t align)
{
    if (!p)
        return fail(MXFP4_EINVAL, "%s: null pointer", name);
    if (!aligned(p, align))
        return fail(MXFP4_EALIGN, "%s: pointer not %d-byte aligned", name, (int)align);
    return MXFP4_OK;
}

int launched(hipError_t st, const char *what)
{
    if (st != hipSuccess)
        return fail(MXFP4_ELAUNCH, "%s: %s", what, hipGetErrorString(st));
    return MXFP4_OK;
}

#define TRY(x)                                                                                     \
    do {                                                                                           \
        int _s = (x);                                                                              \
        if (_s != MXFP4_OK)                                                                        \
            return _s;                                                                             \
    } while (0)

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Tiled path: waves per workgroup (expert bank / GEMM), and the mean pairs
// per touched expert from which the expert bank uses it.
constexpr int TILED_NW_MOE = 8;
constexpr int TILED_RT_GATEUP = 1; // four 32 KB LDS stages
constexpr int TILED_RT_DOWN = 2;   // one activation slab serves 256 rows
constexpr int TILED_NW_GEMM = 4;
constexpr int TILED_NW_GEMM_TALL = 8; // 128-row blocks when the grid stays full
constexpr int TILED_NC = 4;
constexpr int TILED_MIN_TOKENS = 8;
constexpr int TILED_MIN_WGS = 192; // GEMM: tiled only with ~one workgroup per CU
constexpr int TILED_FILL_WGS = 256; // GEMM: one workgroup per CU of MI355X
// Expert bank on the tiled path: the down products of experts with at most
// this many pairs run on the skinny kernel, one item each (measured, 256
// experts of 7168 x 2048, bf16, every expert with c pairs, whole layer on
// the 4-token skinny kernels against tiled: c = 1, 2, 4 in 1050, 1036,
// 1108 us against 1273, 1275, 1302 us; c = 8, two 4-token items, 1830 us
// against 1340 us.  In the 256-expert prefill layer, 99 such experts: down
// 552 -> 378 + 148 us with per-step code loads in the tiled kernels, 510 ->
// 356 + 151 us with paired ones; their gate/up on the skinny kernel too,
// 992 -> 672 + 328 us, so gate/up stays tiled).
constexpr int COLD_MAX = 4;

// Workspace layout of the expert bank.
struct MoeLayout {
    size_t offsets, pair_of_slot, slot_of_pair, token_of_slot, work, n_work, work_cold,
        n_work_cold, work_hot, n_work_hot, h, y, ids_aug, w_aug, total;
};

MoeLayout moe_layout(int64_t n_tokens, int64_t top_k, int64_t n_experts, int64_t hidden,
                     int64_t inter, int x_dtype)
{
    const int64_t P = n_tokens * top_k;
    MoeLayout L;
    size_t o = 0;
    L.offsets = o;
    o += align256((size_t)(n_experts + 1) * 4);
    L.pair_of_slot = o;
    o += align256((size_t)P * 4);
    L.slot_of_pair = o;
    o += align256((size_t)P * 4);
    L.token_of_slot = o;
    o += align256((size_t)P * 4);
    L.work = o;
    o += align256((size_t)P * 16); // at most one item per pair
    L.n_work = o;
    o += 256;
    L.work_cold = o; // one item per expert with few pairs (tiled path)
    o += align256((size_t)(n_experts < P ? n_experts : P) * 16);
    L.n_work_cold = o;
    o += 256;
    L.work_hot = o; // the other experts' items (tiled path)
    o += align256((size_t)P * 16);
    L.n_work_hot = o;
    o += 256;
    L.h = o;
    o += align256((size_t)P * inter * (x_dtype == MXFP4_BF16 ? 2 : 4));
    L.y = o;
    o += align256((size_t)P * hidden * 4);
    L.ids_aug = o; // routing with a shared expert (V4.1)
    o += align256((size_t)P * 4);
    L.w_aug = o;
    o += align256((size_t)P * 4);
    L.total = o;
    return L;
}

// Workspace of the FP4 x FP8 expert bank: the plain bank's (h in fp32) and
// the MXFP8 activations of x and h.
struct MoeA8Layout {
    MoeLayout L;
    size_t xq, xs, hq, hs, total;
};

MoeA8Layout moe_a8_layout(int64_t n_tokens, int64_t top_k, int64_t n_experts, int64_t hidden,
                          int64_t inter)
{
    const int64_t P = n_tokens * top_k;
    MoeA8Layout A;
    A.L = moe_layout(n_tokens, top_k, n_experts, hidden, inter, MXFP4_F32);
    size_t o = A.L.total;
    A.xq = o;
    o += align256((size_t)n_tokens * hidden);
    A.xs = o;
    o += align256((size_t)n_tokens * (hidden / 32));
    A.hq = o;
    o += align256((size_t)P * inter);
    A.hs = o;
    o += align256((size_t)P * (inter / 32));
    A.total = o;
    return A;
}

// Expert-bank variants: the plain bank (route weight on the fp32 down
// output) or the V4.1 bank (bf16 gate/up, SwiGLU limit, route weight folded
// into the bf16 activation, slots summed unweighted, optional shared expert
// applied to every token as slot top_k with weight 1).
struct MoeMode {
    bool v41;
    float lim;
    bool shared;
    bool tables; // gate / up / down are per-expert pointer tables
};

// Stands for the static scratch in the argument checks of the allocation-
// free expert bank (never dereferenced).
void *const NOALLOC_WS = reinterpret_cast<void *>(uintptr_t(1));

// A table of per-expert tensor pointers (device array, 8-byte aligned) for
// rows x cols experts: the table itself and the shape are checked here; its
// entries are device data.
int check_table(const char *name, const void *t, int64_t rows, int64_t cols)
{
    TRY(check_buffer(name, t, 8));
    if (rows < 1 || rows > MXFP4_MAX_ROWS)
        return fail(MXFP4_EINVAL, "%s: rows = %lld outside [1, %d]", name, (long long)rows,
                    MXFP4_MAX_ROWS);
    if (cols < 32 || cols > MXFP4_MAX_COLS || cols % 32 != 0)
        return fail(MXFP4_EINVAL, "%s: cols = %lld must be a multiple of 32 in [32, %d]", name,
                    (long long)cols, MXFP4_MAX_COLS);
    if (mxfp4_nbytes(rows, cols) > MXFP4_MAX_TENSOR_BYTES)
        return fail(MXFP4_EINVAL, "%s: %lld x %lld exceeds %lld bytes", name, (long long)rows,
                    (long long)cols, (long long)MXFP4_MAX_TENSOR_BYTES);
    return MXFP4_OK;
}

int check_moe(const void *gate, const void *up, const void *down, int64_t n_experts,
              int64_t hidden, int64_t inter, const void *x, int x_dtype, int64_t n_tokens,
              const int32_t *topk_ids, const float *topk_w, int64_t top_k, void *out,
              int out_dtype, bool need_out, void *workspace, size_t workspace_bytes,
              bool tables = false)
{
    if (n_experts < 1 || n_experts > MXFP4_MAX_EXPERTS)
        return fail(MXFP4_EINVAL, "n_experts = %lld outside [1, %d]", (long long)n_experts,
                    MXFP4_MAX_EXPERTS);
    if (top_k < 1 || top_k > MXFP4_MAX_TOP_K || top_k > n_experts)
        return fail(MXFP4_EINVAL, "top_k = %lld outside [1, min(%d, n_experts)]",
                    (long long)top_k, MXFP4_MAX_TOP_K);
    if (n_tokens < 1 || n_tokens > MXFP4_MAX_TOKENS)
        return fail(MXFP4_EINVAL, "n_tokens = %lld outside [1, %d]", (long long)n_tokens,
                    MXFP4_MAX_TOKENS);
    if (tables) {
        TRY(check_table("gate", gate, inter, hidden));
        TRY(check_table("up", up, inter, hidden));
        TRY(check_table("down", down, hidden, inter));
    } else {
        TRY(check_tensor("gate", gate, inter, hidden));
        TRY(check_tensor("up", up, inter, hidden));
        TRY(check_tensor("down", down, hidden, inter));
    }
    if (!tables && mxfp4_nbytes(inter, hidden) % 16 != 0)
        return fail(MXFP4_EALIGN, "expert tensor size %lld is not a multiple of 16 bytes",
                    (long long)mxfp4_nbytes(inter, hidden));
    TRY(check_dtype("x_dtype", x_dtype));
    TRY(check_buffer("x", x, 16));
    TRY(check_buffer("topk_ids", topk_ids, 4));
    TRY(check_buffer("topk_w", topk_w, 4));
    if (need_out) {
        TRY(check_dtype("out_dtype", out_dtype));
        TRY(check_buffer("out", out, 16));
    }
    const int64_t P = n_tokens * top_k;
    const int64_t nrb = ((hidden > inter ? hidden : inter) + 15) / 16; // smallest row block
    if (P * nrb > ((int64_t)1 << 31) - 1)
        return fail(MXFP4_EINVAL, "n_tokens * top_k * rows/16 too large for one launch");
    if (workspace == NOALLOC_WS) // the static scratch: size checked by the caller
        return MXFP4_OK;
    TRY(check_buffer("workspace", workspace, 16));
    const size_t need = moe_layout(n_tokens, top_k, n_experts, hidden, inter, x_dtype).total;
    if (workspace_bytes < need)
        return fail(MXFP4_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    return MXFP4_OK;
}

int moe_run(const void *gate, const void *up, const void *down, int64_t n_experts, int64_t hidden,
            int64_t inter, const void *x, int x_dtype, int64_t n_tokens, const int32_t *topk_ids,
            const float *topk_w, int64_t top_k, void *out, int out_dtype, void *workspace,
            const void *h_in, void *h_out, const MoeMode &mode, hipStream_t st)
{
    const bool xbf = x_dtype == MXFP4_BF16;
    const MoeLayout L = moe_layout(n_tokens, top_k + mode.shared, n_experts + mode.shared, hidden,
                                   inter, x_dtype);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    if (mode.shared) {
        // the shared expert becomes slot top_k of every token
        int32_t *ids_aug = reinterpret_cast<int32_t *>(ws + L.ids_aug);
        float *w_aug = reinterpret_cast<float *>(ws + L.w_aug);
        TRY(launched(mx::augment_launch(topk_ids, topk_w, (int)n_tokens, (int)top_k,
                                        (int)n_experts, ids_aug, w_aug, st),
                     "shared-expert routing"));
        topk_ids = ids_aug;
        topk_w = w_aug;
        top_k += 1;
        n_experts += 1;
    }
    const int P = (int)(n_tokens * top_k);
    int32_t *offsets = reinterpret_cast<int32_t *>(ws + L.offsets);
    int32_t *pos = reinterpret_cast<int32_t *>(ws + L.pair_of_slot);
    int32_t *slot = reinterpret_cast<int32_t *>(ws + L.slot_of_pair);
    int32_t *tos = reinterpret_cast<int32_t *>(ws + L.token_of_slot);
    int32_t *work = reinterpret_cast<int32_t *>(ws + L.work);
    int32_t *n_work = reinterpret_cast<int32_t *>(ws + L.n_work);
    void *h = ws + L.h;
    float *y = reinterpret_cast<float *>(ws + L.y);

    // Work items: tokens per item = mean pairs per touched expert, where the
    // touched count is its expectation under uniform routing,
    // E * (1 - (1 - 1/E)^P) (64-expert decode: 48 pairs -> 34 experts -> 2
    // tokens per item, measured best); an expert with more pairs takes
    // several items, each re-reading its rows (from L2 when they run
    // together: items of one row block share an XCD).
    const double touched =
        (double)n_experts * (1.0 - std::pow(1.0 - 1.0 / (double)n_experts, (double)P));
    int want = (int)std::ceil((double)P / (touched > 1.0 ? touched : 1.0));
    // Many pairs per expert (prefill): the tiled kernel, items of up to 64
    // bf16 / 32 fp32 tokens, so a hot expert's rows are streamed once per 64
    // of its tokens.
    const bool tiled = want >= TILED_MIN_TOKENS && mx::tiled_supported((int)hidden) &&
                       mx::tiled_supported((int)inter);
    if (want > 16)
        want = 16;
    int tpc;
    if (tiled) {
        tpc = mx::tiled_tokens(xbf, TILED_NC);
    } else {
        const int tpc_gu = mx::skinny_pick_tpc(mx::MODE_GATEUP, xbf, (int)hidden, want);
        const int tpc_dn = mx::skinny_pick_tpc(mx::MODE_DOWN, xbf, (int)inter, want);
        tpc = tpc_gu < tpc_dn ? tpc_gu : tpc_dn;
    }
    if (tpc < 1)
        return fail(MXFP4_EINVAL, "hidden/inter too large for the on-chip operand buffers");
    const int max_work = mx::group_max_work(P, (int)n_experts, tpc);
    // tiled path: the down products of the experts with at most cold_max
    // pairs, one item each, go to the skinny kernel (their own work list, at
    // most min(E, P) items; the tiled down kernel takes the other experts'
    // list, the tiled gate/up kernel every item, experts ascending: placing
    // the few-pair experts' items last cost 8 us of 992 in the 256-expert
    // prefill gate/up)
    int cold_max = 0;
    if (tiled) {
        cold_max = mx::skinny_pick_tpc(mx::MODE_DOWN, xbf, (int)inter, COLD_MAX);
        if (cold_max > COLD_MAX)
            cold_max = COLD_MAX;
    }
    const int max_cold = (int)(n_experts < P ? n_experts : P);
    int32_t *work_cold = reinterpret_cast<int32_t *>(ws + L.work_cold);
    int32_t *n_work_cold = reinterpret_cast<int32_t *>(ws + L.n_work_cold);
    int32_t *work_hot = reinterpret_cast<int32_t *>(ws + L.work_hot);
    int32_t *n_work_hot = reinterpret_cast<int32_t *>(ws + L.n_work_hot);

    mx::GroupArgs g;
    g.ids = topk_ids;
    g.n_pairs = P;
    g.top_k = (int)top_k;
    g.n_experts = (int)n_experts;
    g.tpc = tpc;
    g.offsets = offsets;
    g.pair_of_slot = pos;
    g.slot_of_pair = slot;
    g.token_of_slot = tos;
    g.work = work;
    g.n_work = n_work;
    g.cold_max = cold_max;
    g.work_hot = cold_max ? work_hot : nullptr;
    g.n_work_hot = cold_max ? n_work_hot : nullptr;
    g.work_cold = cold_max ? work_cold : nullptr;
    g.n_work_cold = cold_max ? n_work_cold : nullptr;
    // Decode-sized routing (at most 64 pairs) into the split-K gate/up
    // kernel: it groups the routing itself (every workgroup ranks the pairs
    // with one wave; workgroup 0 writes the tables the down and combine
    // kernels read), in place of the grouping kernel (measured, 64-expert
    // decode layer: 96.9 -> 94.4 us).
    const mx::SkinnyShape sh_gu =
        tiled ? mx::SkinnyShape{}
              : mx::skinny_shape(mx::MODE_GATEUP, xbf, (int)inter, (int)hidden, tpc, max_work);
    const bool fuse = !tiled && !h_in && !h_out && P <= 64 && sh_gu.kw != 0;
    if (!fuse)
        TRY(launched(mx::group_launch(g, st), "group"));

    const int64_t tbytes = mxfp4_nbytes(inter, hidden);
    if (!h_in) {
        mx::SkinnyArgs a = {};
        a.w0 = static_cast<const uint8_t *>(gate);
        a.w1 = static_cast<const uint8_t *>(up);
        a.expert_stride = tbytes;
        a.rows = (int)inter;
        a.cols = (int)hidden;
        a.x = x;
        a.nch = max_work;
        a.y = h;
        a.y_bf16 = xbf;
        a.work = work;
        a.n_work = n_work;
        a.token_of_slot = tos;
        a.v41 = mode.v41;
        a.lim = mode.lim;
        a.ptr_table = mode.tables;
        a.pair_of_slot = pos;
        a.pair_w = topk_w;
        if (tiled) {
            TRY(launched(mx::tiled_launch(mx::MODE_GATEUP, xbf, TILED_NW_MOE, TILED_RT_GATEUP,
                                          TILED_NC, a, st),
                         "gate/up"));
        } else {
            if (fuse) {
                a.fuse_group = 1 | (P << 1) | ((int)top_k << 8) | ((int)n_experts << 14);
                a.token_of_slot = topk_ids;
                a.pair_of_slot = slot; // slot_of_pair, written by the kernel
            }
            TRY(launched(mx::skinny_launch(mx::MODE_GATEUP, xbf, sh_gu, a, st), "gate/up"));
        }
        if (h_out)
            TRY(launched(mx::copy_launch(h_out, h, (size_t)P * inter * (xbf ? 2 : 4), st),
                         "h copy"));
    }
    if (!out)
        return MXFP4_OK;
    {
        mx::SkinnyArgs a = {};
        a.w0 = static_cast<const uint8_t *>(down);
        a.expert_stride = tbytes;
        a.ptr_table = mode.tables;
        a.rows = (int)hidden;
        a.cols = (int)inter;
        a.x = h_in ? h_in : h;
        a.nch = max_work;
        a.y = y;
        a.y_bf16 = 0;
        a.work = work;
        a.n_work = n_work;
        if (tiled) {
            if (cold_max) {
                mx::SkinnyArgs ac = a;
                ac.nch = max_cold;
                ac.work = work_cold;
                ac.n_work = n_work_cold;
                const mx::SkinnyShape sh = mx::skinny_shape(mx::MODE_DOWN, xbf, (int)hidden,
                                                            (int)inter, cold_max, max_cold);
                TRY(launched(mx::skinny_launch(mx::MODE_DOWN, xbf, sh, ac, st),
                             "down (few-pair experts)"));
                a.work = work_hot;
                a.n_work = n_work_hot;
            }
            TRY(launched(mx::tiled_launch(mx::MODE_DOWN, xbf, TILED_NW_MOE, TILED_RT_DOWN,
                                          TILED_NC, a, st),
                         "down"));
        } else {
            const mx::SkinnyShape sh =
                mx::skinny_shape(mx::MODE_DOWN, xbf, (int)hidden, (int)inter, tpc, max_work);
            TRY(launched(mx::skinny_launch(mx::MODE_DOWN, xbf, sh, a, st), "down"));
        }
    }
    // V4.1: the route weights are already in h; the slots are summed as they are
    TRY(launched(mx::combine_launch(y, slot, mode.v41 ? nullptr : topk_w, (int)n_tokens,
                                    (int)top_k, (int)hidden, out, out_dtype == MXFP4_BF16, st),
                 "combine"));
    return MXFP4_OK;
}


// ---------------------------------------------------------------------------
// Static scratch of the allocation-free expert bank.  The array lives in the
// library's device code (each GPU the library runs on holds its own copy
// until the process ends); its device address is looked up once per device
// with hipGetSymbolAddress, with that device current, and that address, never
// the host-side name, is what the kernels receive.
// ---------------------------------------------------------------------------
constexpr size_t NOALLOC_SCRATCH_BYTES = MXFP4_NOALLOC_SCRATCH_BYTES;
constexpr int NOALLOC_MAX_DEVICES = 64;
std::atomic<void *> g_scratch_ptr[NOALLOC_MAX_DEVICES];
std::mutex g_scratch_mu;

} // namespace

static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

namespace {

int scratch_for_current_device(void **out)
{
    int dev = -1;
    hipError_t st = hipGetDevice(&dev);
    if (st != hipSuccess)
        return fail(MXFP4_ELAUNCH, "hipGetDevice: %s", hipGetErrorString(st));
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
        return fail(MXFP4_EINVAL, "device %d: the static scratch serves devices 0..%d", dev,
                    NOALLOC_MAX_DEVICES - 1);
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_acquire);
        if (!p) {
            st = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (st != hipSuccess || !p)
                return fail(MXFP4_ELAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                            hipGetErrorString(st));
            if (reinterpret_cast<uintptr_t>(p) % 256 != 0)
                return fail(MXFP4_EALIGN, "static scratch at %p is not 256-byte aligned", p);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MXFP4_OK;
}

} // namespace

extern "C" {

int64_t mxfp4_nbytes(int64_t rows, int64_t cols)
{
    if (rows < 0 || cols < 0 || cols % 32 != 0)
        return -1;
    return rows * (cols / 2) + rows * (cols / 32);
}

const char *mxfp4_last_error(void) { return g_err; }

int mxfp4_dequant(const void *w, int64_t rows, int64_t cols, void *out, int out_dtype, void *stream)
{
    clear_error();
    TRY(check_tensor("w", w, rows, cols));
    TRY(check_dtype("out_dtype", out_dtype));
    TRY(check_buffer("out", out, 16));
    return launched(mx::dequant_launch(static_cast<const uint8_t *>(w), rows, cols, out,
                                       out_dtype == MXFP4_BF16, (hipStream_t)stream),
                    "dequant");
}

int mxfp4_gemm(const void *w, int64_t rows, int64_t cols, const void *x, int x_dtype, int64_t b,
               void *y, int y_dtype, void *stream)
{
    clear_error();
    TRY(check_tensor("w", w, rows, cols));
    TRY(check_dtype("x_dtype", x_dtype));
    TRY(check_dtype("y_dtype", y_dtype));
    if (b < 1 || b > MXFP4_MAX_TOKENS)
        return fail(MXFP4_EINVAL, "b = %lld outside [1, %d]", (long long)b, MXFP4_MAX_TOKENS);
    TRY(check_buffer("x", x, 16));
    TRY(check_buffer("y", y, 16));
    const bool xbf = x_dtype == MXFP4_BF16;
    const int maxc = xbf ? 16 : 8;
    // Tiled chunks: two MFMA column tiles (32 bf16 / 16 fp32 tokens) when b
    // fits in them, else four; fp32 tokens also take two when chunks of
    // four would not give each CU a workgroup (measured, 14336 x 4096 fp32
    // b = 32: 224 workgroups of four tiles 26.6 us, 448 of two tiles
    // 24.6 us, the second chunk re-reading the weights from L2; bf16 b = 64
    // is slower with two tiles, 23.1 vs 19.4 us, and fp32 b = 16 with
    // one-tile chunks, 18.5 vs 17.8 us).
    const int rpw = mx::tiled_rows_per_wg(TILED_NW_GEMM, 1);
    const int64_t trb = (rows + rpw - 1) / rpw;
    auto chunks = [&](int nc) {
        return (b + mx::tiled_tokens(xbf, nc) - 1) / mx::tiled_tokens(xbf, nc);
    };
    int tnc = b <= mx::tiled_tokens(xbf, 2) ? 2 : TILED_NC;
    if (!xbf && tnc == TILED_NC && chunks(TILED_NC) * trb < TILED_FILL_WGS)
        tnc = 2;
    const int64_t tnch = chunks(tnc);
    const int64_t twgs = tnch * trb;
    if (b > maxc && mx::tiled_supported((int)cols) && twgs >= TILED_MIN_WGS) {
        // tokens beyond one skinny chunk and enough row blocks to fill the
        // chip: the tiled kernel, one pass over the weights per 64 bf16 / 32
        // fp32 tokens (measured, 14336 x 4096: bf16 b = 64 in 20.9 us
        // against 40.1 us for four skinny chunks; with 64 workgroups,
        // 4096 x 4096, it loses 2x).
        const int nc = tnc;
        const int64_t nch = tnch;
        if (twgs > ((int64_t)1 << 31) - 1)
            return fail(MXFP4_EINVAL, "rows * b too large for one launch");
        // Twice the rows per workgroup (one activation slab serves 128 rows)
        // while the grid keeps TILED_MIN_WGS workgroups (measured, 14336 x
        // 4096 fp32 b = 32, two 16-token chunks: 448 workgroups of 64 rows
        // 24.5 us, 224 of 128 rows 20.4 us; at b = 16 and bf16 b = 64 the 112
        // workgroups of 128 rows lose, 20.5 / 26.8 us against 17.6 / 19.3).
        const int nw = tnch * ((rows + mx::tiled_rows_per_wg(TILED_NW_GEMM_TALL, 1) - 1) /
                               mx::tiled_rows_per_wg(TILED_NW_GEMM_TALL, 1)) >= TILED_MIN_WGS
                           ? TILED_NW_GEMM_TALL
                           : TILED_NW_GEMM;
        mx::SkinnyArgs a = {};
        a.w0 = static_cast<const uint8_t *>(w);
        a.rows = (int)rows;
        a.cols = (int)cols;
        a.x = x;
        a.b = (int)b;
        a.nch = (int)nch;
        a.y = y;
        a.y_bf16 = y_dtype == MXFP4_BF16;
        return launched(
            mx::tiled_launch(mx::MODE_GEMM, xbf, nw, 1, nc, a, (hipStream_t)stream),
            "gemm");
    }
    const int tpc = mx::skinny_pick_tpc(mx::MODE_GEMM, xbf, (int)cols, b < maxc ? (int)b : maxc);
    if (tpc < 1)
        return fail(MXFP4_EINVAL, "cols = %lld too large for the on-chip operand buffers",
                    (long long)cols);
    const int64_t nch = (b + tpc - 1) / tpc;
    const mx::SkinnyShape sh = mx::skinny_shape(mx::MODE_GEMM, xbf, (int)rows, (int)cols, tpc, nch);
    if (mx::skinny_blocks(sh, (int)rows, (int)nch) > ((int64_t)1 << 31) - 1)
        return fail(MXFP4_EINVAL, "rows * b too large for one launch");
    mx::SkinnyArgs a = {};
    a.w0 = static_cast<const uint8_t *>(w);
    a.rows = (int)rows;
    a.cols = (int)cols;
    a.x = x;
    a.b = (int)b;
    a.nch = (int)nch;
    a.y = y;
    a.y_bf16 = y_dtype == MXFP4_BF16;
    return launched(mx::skinny_launch(mx::MODE_GEMM, xbf, sh, a, (hipStream_t)stream), "gemm");
}

size_t mxfp4_gemm_a8_workspace_size(int64_t b, int64_t cols)
{
    if (b < 1 || b > MXFP4_MAX_TOKENS || cols < 128 || cols > MXFP4_MAX_COLS || cols % 128)
        return 0;
    return align256((size_t)b * cols) + align256((size_t)b * (cols / 32));
}

int mxfp8_quantize(const void *x, int x_dtype, int64_t b, int64_t cols, uint8_t *q, uint8_t *s,
                   void *stream)
{
    clear_error();
    TRY(check_dtype("x_dtype", x_dtype));
    if (b < 1 || b > MXFP4_MAX_TOKENS)
        return fail(MXFP4_EINVAL, "b = %lld outside [1, %d]", (long long)b, MXFP4_MAX_TOKENS);
    if (cols < 32 || cols > MXFP4_MAX_COLS || cols % 32)
        return fail(MXFP4_EINVAL, "cols = %lld must be a multiple of 32 in [32, %d]",
                    (long long)cols, MXFP4_MAX_COLS);
    TRY(check_buffer("x", x, 16));
    TRY(check_buffer("q", q, 16));
    TRY(check_buffer("s", s, 1));
    return launched(mx::mxfp8_quantize_launch(x, x_dtype == MXFP4_BF16, b, cols, q, s,
                                              (hipStream_t)stream),
                    "mxfp8 quantize");
}

int mxfp4_gemm_a8(const void *w, int64_t rows, int64_t cols, const void *x, int x_dtype,
                  int64_t b, void *y, int y_dtype, void *workspace, size_t workspace_bytes,
                  void *stream)
{
    clear_error();
    TRY(check_tensor("w", w, rows, cols));
    if (cols % 128)
        return fail(MXFP4_EINVAL, "cols = %lld: the FP4 x FP8 product needs a multiple of 128",
                    (long long)cols);
    TRY(check_dtype("x_dtype", x_dtype));
    TRY(check_dtype("y_dtype", y_dtype));
    if (b < 1 || b > MXFP4_MAX_TOKENS)
        return fail(MXFP4_EINVAL, "b = %lld outside [1, %d]", (long long)b, MXFP4_MAX_TOKENS);
    TRY(check_buffer("x", x, 16));
    TRY(check_buffer("y", y, 16));
    TRY(check_buffer("workspace", workspace, 16));
    const size_t need = mxfp4_gemm_a8_workspace_size(b, cols);
    if (workspace_bytes < need)
        return fail(MXFP4_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    const int64_t nrb = (rows + mx::a8_rows_per_wg() - 1) / mx::a8_rows_per_wg();
    if (nrb * ((b + 15) / 16) > ((int64_t)1 << 31) - 1)
        return fail(MXFP4_EINVAL, "rows * b too large for one launch");
    uint8_t *q = static_cast<uint8_t *>(workspace);
    uint8_t *sc = q + align256((size_t)b * cols);
    const hipStream_t st = (hipStream_t)stream;
    TRY(launched(mx::mxfp8_quantize_launch(x, x_dtype == MXFP4_BF16, b, cols, q, sc, st),
                 "mxfp8 quantize"));
    mx::A8Args a = {};
    a.w = static_cast<const uint8_t *>(w);
    a.rows = (int)rows;
    a.cols = (int)cols;
    a.xq = q;
    a.xs = sc;
    a.b = (int)b;
    a.y = y;
    a.y_bf16 = y_dtype == MXFP4_BF16;
    return launched(mx::gemm_a8_launch(a, st), "gemm a8");
}

int mxfp4_matvec(const void *w, int64_t rows, int64_t cols, const float *x, float *y, void *stream)
{
    return mxfp4_gemm(w, rows, cols, x, MXFP4_F32, 1, y, MXFP4_F32, stream);
}

int moe_route_group(const int32_t *topk_ids, int64_t n_tokens, int64_t top_k, int64_t n_experts,
                    int32_t *offsets, int32_t *pair_of_slot, int32_t *slot_of_pair, void *stream)
{
    clear_error();
    if (n_experts < 1 || n_experts > MXFP4_MAX_EXPERTS)
        return fail(MXFP4_EINVAL, "n_experts = %lld outside [1, %d]", (long long)n_experts,
                    MXFP4_MAX_EXPERTS);
    if (top_k < 1 || top_k > MXFP4_MAX_TOP_K)
        return fail(MXFP4_EINVAL, "top_k = %lld outside [1, %d]", (long long)top_k,
                    MXFP4_MAX_TOP_K);
    if (n_tokens < 1 || n_tokens > MXFP4_MAX_TOKENS)
        return fail(MXFP4_EINVAL, "n_tokens = %lld outside [1, %d]", (long long)n_tokens,
                    MXFP4_MAX_TOKENS);
    TRY(check_buffer("topk_ids", topk_ids, 4));
    TRY(check_buffer("offsets", offsets, 4));
    TRY(check_buffer("pair_of_slot", pair_of_slot, 4));
    TRY(check_buffer("slot_of_pair", slot_of_pair, 4));
    mx::GroupArgs g = {};
    g.ids = topk_ids;
    g.n_pairs = (int)(n_tokens * top_k);
    g.top_k = (int)top_k;
    g.n_experts = (int)n_experts;
    g.tpc = 1;
    g.offsets = offsets;
    g.pair_of_slot = pair_of_slot;
    g.slot_of_pair = slot_of_pair;
    return launched(mx::group_launch(g, (hipStream_t)stream), "group");
}

int moe_route_topk(const float *logits, int64_t n_tokens, int64_t n_experts, int64_t top_k,
                   int32_t *topk_ids, float *topk_w, void *stream)
{
    clear_error();
    if (n_experts < 1 || n_experts > MXFP4_MAX_EXPERTS)
        return fail(MXFP4_EINVAL, "n_experts = %lld outside [1, %d]", (long long)n_experts,
                    MXFP4_MAX_EXPERTS);
    if (top_k < 1 || top_k > MXFP4_MAX_TOP_K || top_k > n_experts)
        return fail(MXFP4_EINVAL, "top_k = %lld outside [1, min(%d, n_experts)]",
                    (long long)top_k, MXFP4_MAX_TOP_K);
    if (n_tokens < 1 || n_tokens > MXFP4_MAX_TOKENS)
        return fail(MXFP4_EINVAL, "n_tokens = %lld outside [1, %d]", (long long)n_tokens,
                    MXFP4_MAX_TOKENS);
    TRY(check_buffer("logits", logits, 4));
    TRY(check_buffer("topk_ids", topk_ids, 4));
    TRY(check_buffer("topk_w", topk_w, 4));
    return launched(mx::route_topk_launch(logits, (int)n_tokens, (int)n_experts, (int)top_k,
                                          topk_ids, topk_w, (hipStream_t)stream),
                    "route");
}

size_t moe_experts_mxfp4_workspace_size(int64_t n_tokens, int64_t top_k, int64_t n_experts,
                                        int64_t hidden, int64_t inter, int x_dtype)
{
    if (n_tokens < 1 || top_k < 1 || n_experts < 1 || hidden < 32 || inter < 32 ||
        hidden % 32 || inter % 32 || (x_dtype != MXFP4_F32 && x_dtype != MXFP4_BF16) ||
        n_tokens > MXFP4_MAX_TOKENS || top_k > MXFP4_MAX_TOP_K || n_experts > MXFP4_MAX_EXPERTS ||
        hidden > MXFP4_MAX_COLS || inter > MXFP4_MAX_COLS)
        return 0;
    return moe_layout(n_tokens, top_k, n_experts, hidden, inter, x_dtype).total;
}

int moe_experts_mxfp4(const void *gate, const void *up, const void *down, int64_t n_experts,
                      int64_t hidden, int64_t inter, const void *x, int x_dtype, int64_t n_tokens,
                      const int32_t *topk_ids, const float *topk_w, int64_t top_k, void *out,
                      int out_dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    clear_error();
    TRY(check_moe(gate, up, down, n_experts, hidden, inter, x, x_dtype, n_tokens, topk_ids,
                  topk_w, top_k, out, out_dtype, true, workspace, workspace_bytes));
    return moe_run(gate, up, down, n_experts, hidden, inter, x, x_dtype, n_tokens, topk_ids,
                   topk_w, top_k, out, out_dtype, workspace, nullptr, nullptr, MoeMode{},
                   (hipStream_t)stream);
}

size_t moe_experts_mxfp4_a8_workspace_size(int64_t n_tokens, int64_t top_k, int64_t n_experts,
                                           int64_t hidden, int64_t inter)
{
    if (n_tokens < 1 || top_k < 1 || n_experts < 1 || hidden < 512 || inter < 512 ||
        hidden % 512 || inter % 512 || n_tokens > MXFP4_MAX_TOKENS ||
        top_k > MXFP4_MAX_TOP_K || n_experts > MXFP4_MAX_EXPERTS || hidden > MXFP4_MAX_COLS ||
        inter > MXFP4_MAX_COLS)
        return 0;
    return moe_a8_layout(n_tokens, top_k, n_experts, hidden, inter).total;
}

int moe_experts_mxfp4_a8(const void *gate, const void *up, const void *down, int64_t n_experts,
                         int64_t hidden, int64_t inter, const void *x, int x_dtype,
                         int64_t n_tokens, const int32_t *topk_ids, const float *topk_w,
                         int64_t top_k, void *out, int out_dtype, void *workspace,
                         size_t workspace_bytes, void *stream)
{
    clear_error();
    // the shared checks (the workspace is checked below, against this
    // entry point's own layout)
    TRY(check_moe(gate, up, down, n_experts, hidden, inter, x, x_dtype, n_tokens, topk_ids,
                  topk_w, top_k, out, out_dtype, true, NOALLOC_WS, 0));
    if (hidden % 512 || inter % 512)
        return fail(MXFP4_EINVAL,
                    "hidden = %lld, inter = %lld: the FP4 x FP8 expert bank needs multiples "
                    "of 512",
                    (long long)hidden, (long long)inter);
    TRY(check_buffer("workspace", workspace, 16));
    const MoeA8Layout A = moe_a8_layout(n_tokens, top_k, n_experts, hidden, inter);
    if (workspace_bytes < A.total)
        return fail(MXFP4_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                    A.total);
    const int P = (int)(n_tokens * top_k);
    const int tpc = mx::moe_a8_tokens();
    const int max_work = mx::group_max_work(P, (int)n_experts, tpc);
    const int64_t rows_max = hidden > inter ? hidden : inter;
    const int64_t nrb = (rows_max + mx::moe_a8_rows_per_wg() - 1) / mx::moe_a8_rows_per_wg();
    if (nrb * max_work > ((int64_t)1 << 31) - 1)
        return fail(MXFP4_EINVAL, "n_tokens * top_k * rows too large for one launch");
    const hipStream_t st = (hipStream_t)stream;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    const MoeLayout &L = A.L;
    int32_t *slot = reinterpret_cast<int32_t *>(ws + L.slot_of_pair);
    int32_t *tos = reinterpret_cast<int32_t *>(ws + L.token_of_slot);
    int32_t *work = reinterpret_cast<int32_t *>(ws + L.work);
    int32_t *n_work = reinterpret_cast<int32_t *>(ws + L.n_work);
    float *h = reinterpret_cast<float *>(ws + L.h);
    float *y = reinterpret_cast<float *>(ws + L.y);
    uint8_t *xq = ws + A.xq, *xs = ws + A.xs, *hq = ws + A.hq, *hs = ws + A.hs;

    TRY(launched(mx::mxfp8_quantize_launch(x, x_dtype == MXFP4_BF16, n_tokens, hidden, xq, xs,
                                           st),
                 "x quantize"));
    mx::GroupArgs g = {};
    g.ids = topk_ids;
    g.n_pairs = P;
    g.top_k = (int)top_k;
    g.n_experts = (int)n_experts;
    g.tpc = tpc;
    g.offsets = reinterpret_cast<int32_t *>(ws + L.offsets);
    g.pair_of_slot = reinterpret_cast<int32_t *>(ws + L.pair_of_slot);
    g.slot_of_pair = slot;
    g.token_of_slot = tos;
    g.work = work;
    g.n_work = n_work;
    TRY(launched(mx::group_launch(g, st), "group"));
    const int64_t tbytes = mxfp4_nbytes(inter, hidden);
    mx::MoeA8Args a = {};
    a.w0 = static_cast<const uint8_t *>(gate);
    a.w1 = static_cast<const uint8_t *>(up);
    a.expert_stride = tbytes;
    a.rows = (int)inter;
    a.cols = (int)hidden;
    a.xq = xq;
    a.xs = xs;
    a.token_of_slot = tos;
    a.work = work;
    a.n_work = n_work;
    a.max_work = max_work;
    a.y = h;
    TRY(launched(mx::moe_a8_launch(mx::MODE_GATEUP, a, st), "gate/up"));
    // h of every slot (those of dropped pairs hold stale values: quantized,
    // never read)
    TRY(launched(mx::mxfp8_quantize_launch(h, false, P, inter, hq, hs, st), "h quantize"));
    a.w0 = static_cast<const uint8_t *>(down);
    a.w1 = nullptr;
    a.rows = (int)hidden;
    a.cols = (int)inter;
    a.xq = hq;
    a.xs = hs;
    a.token_of_slot = nullptr;
    a.y = y;
    TRY(launched(mx::moe_a8_launch(mx::MODE_DOWN, a, st), "down"));
    return launched(mx::combine_launch(y, slot, topk_w, (int)n_tokens, (int)top_k, (int)hidden,
                                       out, out_dtype == MXFP4_BF16, st),
                    "combine");
}

int mxfp4_device_address(const void *p, void **device_ptr)
{
    clear_error();
    if (!p || !device_ptr)
        return fail(MXFP4_EINVAL, "device_address: null pointer");
    *device_ptr = nullptr;
    hipPointerAttribute_t attr;
    const hipError_t st = hipPointerGetAttributes(&attr, p);
    if (st != hipSuccess) {
        (void)hipGetLastError(); // the query's error is not a launch error
        return fail(MXFP4_EINVAL, "%p is neither device memory nor pinned host memory (%s)", p,
                    hipGetErrorString(st));
    }
    if (attr.type == hipMemoryTypeDevice) {
        *device_ptr = const_cast<void *>(p);
        return MXFP4_OK;
    }
    if (attr.type == hipMemoryTypeHost && attr.devicePointer) {
        // the mapped address of the pinned block, at p's offset within it
        const uintptr_t off =
            reinterpret_cast<uintptr_t>(p) - reinterpret_cast<uintptr_t>(attr.hostPointer);
        *device_ptr = static_cast<uint8_t *>(attr.devicePointer) + (attr.hostPointer ? off : 0);
        return MXFP4_OK;
    }
    return fail(MXFP4_EINVAL, "%p is not device-accessible (memory type %d)", p, (int)attr.type);
}

int moe_experts_mxfp4_ptrs(const void *const *gate, const void *const *up,
                           const void *const *down, int64_t n_experts, int64_t hidden,
                           int64_t inter, const void *x, int x_dtype, int64_t n_tokens,
                           const int32_t *topk_ids, const float *topk_w, int64_t top_k,
                           void *out, int out_dtype, void *workspace, size_t workspace_bytes,
                           void *stream)
{
    clear_error();
    TRY(check_moe(gate, up, down, n_experts, hidden, inter, x, x_dtype, n_tokens, topk_ids,
                  topk_w, top_k, out, out_dtype, true, workspace, workspace_bytes, true));
    MoeMode mode = {};
    mode.tables = true;
    return moe_run(gate, up, down, n_experts, hidden, inter, x, x_dtype, n_tokens, topk_ids,
                   topk_w, top_k, out, out_dtype, workspace, nullptr, nullptr, mode,
                   (hipStream_t)stream);
}

int moe_experts_mxfp4_noalloc(const void *gate, const void *up, const void *down,
                              int64_t n_experts, int64_t hidden, int64_t inter, const void *x,
                              int x_dtype, int64_t n_tokens, const int32_t *topk_ids,
                              const float *topk_w, int64_t top_k, void *out, int out_dtype,
                              void *stream)
{
    clear_error();
    TRY(check_moe(gate, up, down, n_experts, hidden, inter, x, x_dtype, n_tokens, topk_ids,
                  topk_w, top_k, out, out_dtype, true, NOALLOC_WS, 0));
    const size_t need = moe_layout(n_tokens, top_k, n_experts, hidden, inter, x_dtype).total;
    if (need > NOALLOC_SCRATCH_BYTES)
        return fail(MXFP4_EWORKSPACE,
                    "these sizes need %zu bytes of scratch; the static scratch holds %zu "
                    "(use moe_experts_mxfp4 with a workspace)",
                    need, NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    TRY(scratch_for_current_device(&ws));
    return moe_run(gate, up, down, n_experts, hidden, inter, x, x_dtype, n_tokens, topk_ids,
                   topk_w, top_k, out, out_dtype, ws, nullptr, nullptr, MoeMode{},
                   (hipStream_t)stream);
}

int moe_experts_mxfp4_stages(const void *gate, const void *up, const void *down,
                             int64_t n_experts, int64_t hidden, int64_t inter, const void *x,
                             int x_dtype, int64_t n_tokens, const int32_t *topk_ids,
                             const float *topk_w, int64_t top_k, void *out, int out_dtype,
                             void *workspace, size_t workspace_bytes, const void *h_in,
                             void *h_out, void *stream)
{
    clear_error();
    TRY(check_moe(gate, up, down, n_experts, hidden, inter, x, x_dtype, n_tokens, topk_ids,
                  topk_w, top_k, out, out_dtype, out != nullptr, workspace, workspace_bytes));
    if (!out && !h_out)
        return fail(MXFP4_EINVAL, "stages: nothing requested (out and h_out are both null)");
    if (h_in)
        TRY(check_buffer("h_in", h_in, 16));
    if (h_out)
        TRY(check_buffer("h_out", h_out, 16));
    if (h_in && h_out)
        return fail(MXFP4_EINVAL, "stages: h_in and h_out are exclusive");
    return moe_run(gate, up, down, n_experts, hidden, inter, x, x_dtype, n_tokens, topk_ids,
                   topk_w, top_k, out, out_dtype, workspace, h_in, h_out, MoeMode{},
                   (hipStream_t)stream);
}

size_t moe_experts_mxfp4_v41_workspace_size(int64_t n_tokens, int64_t top_k, int64_t n_experts,
                                            int64_t hidden, int64_t inter, int has_shared)
{
    if (has_shared != 0 && has_shared != 1)
        return 0;
    return moe_experts_mxfp4_workspace_size(n_tokens, top_k + has_shared, n_experts + has_shared,
                                            hidden, inter, MXFP4_BF16);
}

namespace {

int check_v41(const void *gate, const void *up, const void *down, int64_t n_experts,
              int64_t hidden, int64_t inter, const void *x, int64_t n_tokens,
              const int32_t *topk_ids, const float *topk_w, int64_t top_k, float swiglu_limit,
              int has_shared, void *out, bool need_out, void *workspace, size_t workspace_bytes)
{
    if (has_shared != 0 && has_shared != 1)
        return fail(MXFP4_EINVAL, "has_shared = %d is not 0 or 1", has_shared);
    if (!(swiglu_limit >= 0.0f) || swiglu_limit > 3.0e38f)
        return fail(MXFP4_EINVAL, "swiglu_limit must be finite and >= 0 (0: no limit)");
    if (top_k < 1 || top_k > n_experts)
        return fail(MXFP4_EINVAL, "top_k = %lld outside [1, n_experts]", (long long)top_k);
    // the grouping and kernels see top_k + has_shared slots over
    // n_experts + has_shared experts
    TRY(check_moe(gate, up, down, n_experts + has_shared, hidden, inter, x, MXFP4_BF16, n_tokens,
                  topk_ids, topk_w, top_k + has_shared, out, MXFP4_BF16, need_out, workspace,
                  workspace_bytes));
    return MXFP4_OK;
}

} // namespace

int moe_experts_mxfp4_v41(const void *gate, const void *up, const void *down, int64_t n_experts,
                          int64_t hidden, int64_t inter, const void *x, int64_t n_tokens,
                          const int32_t *topk_ids, const float *topk_w, int64_t top_k,
                          float swiglu_limit, int has_shared, void *out, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    clear_error();
    TRY(check_v41(gate, up, down, n_experts, hidden, inter, x, n_tokens, topk_ids, topk_w, top_k,
                  swiglu_limit, has_shared, out, true, workspace, workspace_bytes));
    return moe_run(gate, up, down, n_experts, hidden, inter, x, MXFP4_BF16, n_tokens, topk_ids,
                   topk_w, top_k, out, MXFP4_BF16, workspace, nullptr, nullptr,
                   MoeMode{true, swiglu_limit, has_shared != 0}, (hipStream_t)stream);
}

int moe_experts_mxfp4_v41_stages(const void *gate, const void *up, const void *down,
                                 int64_t n_experts, int64_t hidden, int64_t inter, const void *x,
                                 int64_t n_tokens, const int32_t *topk_ids, const float *topk_w,
                                 int64_t top_k, float swiglu_limit, int has_shared, void *out,
                                 void *workspace, size_t workspace_bytes, const void *h_in,
                                 void *h_out, void *stream)
{
    clear_error();
    TRY(check_v41(gate, up, down, n_experts, hidden, inter, x, n_tokens, topk_ids, topk_w, top_k,
                  swiglu_limit, has_shared, out, out != nullptr, workspace, workspace_bytes));
    if (!out && !h_out)
        return fail(MXFP4_EINVAL, "stages: nothing requested (out and h_out are both null)");
    if (h_in)
        TRY(check_buffer("h_in", h_in, 16));
    if (h_out)
        TRY(check_buffer("h_out", h_out, 16));
    if (h_in && h_out)
        return fail(MXFP4_EINVAL, "stages: h_in and h_out are exclusive");
    return moe_run(gate, up, down, n_experts, hidden, inter, x, MXFP4_BF16, n_tokens, topk_ids,
                   topk_w, top_k, out, MXFP4_BF16, workspace, h_in, h_out,
                   MoeMode{true, swiglu_limit, has_shared != 0}, (hipStream_t)stream);
}

} // extern "C"
