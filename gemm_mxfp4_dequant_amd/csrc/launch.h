// Internal interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mx {

enum { MODE_GEMM = 0, MODE_GATEUP = 1, MODE_DOWN = 2 };

// Arguments of the skinny MFMA kernels (one struct for all modes).
struct SkinnyArgs {
    const uint8_t *w0;        // GEMM: the tensor; GATEUP: gate bank; DOWN: down bank
    const uint8_t *w1;        // GATEUP: up bank
    int64_t expert_stride;    // bytes between experts in a bank
    int rows, cols;           // of one tensor
    const void *x;            // GEMM: x [b][cols]; GATEUP: x [T][cols]; DOWN: h [slots][cols]
    int b;                    // GEMM: tokens
    int nch;                  // GEMM: token chunks; MoE: work item bound
    int nrb;                  // row blocks of rows_per_wg rows (set by skinny_launch)
    int rbw;                  // row blocks walked by one workgroup (set by skinny_launch;
                              // -1: one, with reduction buffers of its own)
    void *y;                  // GEMM: y [b][rows]; GATEUP: h [slots][rows]; DOWN: y [slots][rows]
    int y_bf16;               // output element type (GEMM, GATEUP)
    const int *work;          // MoE: int4 {expert, first slot, tokens, 0} per item
    const int *n_work;        // MoE: number of items (device)
    const int *token_of_slot; // GATEUP: token row of each slot
    // GATEUP, V4.1 activation (v41 != 0): h = bf16(w * silu(min(bf16 g, lim)) *
    // clamp(bf16 u, -lim, lim)), clamping only when lim > 0; w = pair_w of the
    // slot's pair
    int v41;
    float lim;
    const int *pair_of_slot;
    const float *pair_w;
    // MoE: w0 / w1 are tables of per-expert tensor pointers (device arrays
    // of n_experts pointers; an entry may point to device memory or to
    // device-mapped pinned host memory) instead of contiguous banks.
    int ptr_table;
    // GATEUP (split-K kernel): 0, or routing that the kernel groups itself
    // (at most 64 pairs), packed as 1 | P << 1 | top_k << 8 | n_experts << 14.
    // Then token_of_slot holds the routing ids [P] and pair_of_slot the
    // slot_of_pair table [P], which workgroup 0 writes together with work and
    // n_work for the down and combine kernels.
    // This last field also pads the struct to 128 bytes, so the hidden
    // launch arguments the compiler appends (grid and workgroup sizes) start
    // at offset 128.  Measured against the unpadded 120 bytes, same code
    // otherwise: 4096 x 4096 matvec 5.04 -> 4.85 us, b = 8 6.97 -> 6.77 us,
    // 64-expert decode -0.4 %, 14336 x 4096 b = 8 +0.9 %.
    int fuse_group;
};
static_assert(sizeof(SkinnyArgs) == 128, "SkinnyArgs layout: see fuse_group");

// Launch shape of one skinny call: K slab width (0 = generic kernel),
// tokens per workgroup, row tiles per matrix, threads, row blocks walked by
// one workgroup, LDS bytes.
struct SkinnyShape {
    int kw, tpc, nr, threads, rows_per_wg, rbw;
    size_t lds;
    int64_t persist_wgs; // expert bank: the grid the items share (0: GEMM)
};

// Tokens per workgroup for a call that wants `want` columns (fits LDS).
int skinny_pick_tpc(int mode, bool xbf, int cols, int want);
// Shape for `items` token chunks / work items per row block.
SkinnyShape skinny_shape(int mode, bool xbf, int rows, int cols, int tpc, int64_t items);
// Workgroups of a launch: ceil(ceil(rows / rows_per_wg) / |rbw|) * nch.
int64_t skinny_blocks(const SkinnyShape &s, int rows, int nch);
hipError_t skinny_launch(int mode, bool xbf, const SkinnyShape &s, SkinnyArgs a,
                         hipStream_t stream);

// Tiled path (items of tens of tokens): NW waves x RT x 16 rows per workgroup,
// NC column tiles of 16 MFMA columns, K streamed in 128-column steps.
bool tiled_supported(int cols);     // cols % 512 == 0
int tiled_tokens(bool xbf, int nc); // tokens per work item
int tiled_rows_per_wg(int nw, int rt);
// grid = ceil(rows / tiled_rows_per_wg(nw, rt)) * a.nch
hipError_t tiled_launch(int mode, bool xbf, int nw, int rt, int nc, const SkinnyArgs &a,
                        hipStream_t stream);

// Block-scaled FP4 x FP8 product (mx8.hip): activations quantized to MXFP8
// (E4M3 codes xq [b][cols], E8M0 scale bytes xs [b][cols / 32]), then
// v_mfma_scale_f32_16x16x128_f8f6f4 with the weights as stored.
struct A8Args {
    const uint8_t *w;
    int rows, cols; // cols % 128 == 0
    const uint8_t *xq, *xs;
    int b;
    void *y; // [b][rows]
    int y_bf16;
};
hipError_t mxfp8_quantize_launch(const void *x, bool xbf, int64_t b, int64_t cols, uint8_t *q,
                                 uint8_t *s, hipStream_t stream);
hipError_t gemm_a8_launch(const A8Args &a, hipStream_t stream);
int a8_rows_per_wg();

// Expert bank on the block-scaled FP4 x FP8 product (moe_a8.hip), for work
// items of up to moe_a8_tokens() tokens of one expert.  Activations MXFP8:
// codes xq [rows of x][cols], scales xs [rows of x][cols / 32].  GATEUP:
// x rows gathered by token_of_slot, y = h [slot][rows] = silu(g) u (fp32);
// DOWN: x rows are slots, y [slot][rows] (fp32).  cols % 512 == 0.
struct MoeA8Args {
    const uint8_t *w0, *w1; // GATEUP: gate / up banks; DOWN: down bank
    int64_t expert_stride;  // bytes between experts in a bank
    int rows, cols;         // of one tensor
    const uint8_t *xq, *xs;
    const int *token_of_slot; // GATEUP
    const int *work;          // int4 {expert, first slot, tokens, 0} per item
    const int *n_work;        // number of items (device)
    int max_work;             // bound on the items (grid)
    float *y;
};
// grid = ceil(rows / moe_a8_rows_per_wg()) * max_work
hipError_t moe_a8_launch(int mode, const MoeA8Args &a, hipStream_t stream);
int moe_a8_rows_per_wg();
int moe_a8_tokens();

hipError_t dequant_launch(const uint8_t *w, int64_t rows, int64_t cols, void *out, bool bf16,
                          hipStream_t stream);

// Grouping of pairs by expert (one workgroup) and the work list for the
// expert kernels.  ws_* are device arrays inside the caller's workspace.
struct GroupArgs {
    const int32_t *ids;
    int n_pairs, top_k, n_experts, tpc;
    int32_t *offsets;       // [E+1]
    int32_t *pair_of_slot;  // [P]
    int32_t *slot_of_pair;  // [P]
    int32_t *token_of_slot; // [P] (may be null)
    int32_t *work;          // [max_work][4] (may be null)
    int32_t *n_work;        // [1] (may be null)
    // 0, or: besides work (every item, experts ascending), the items of the
    // experts with 1..cold_max pairs (one each) also go to work_cold
    // [min(E, P)][4] and those of the other experts to work_hot [max_work][4]
    // (counts in n_work_cold / n_work_hot [1])
    int cold_max;
    int32_t *work_hot;
    int32_t *n_work_hot;
    int32_t *work_cold;
    int32_t *n_work_cold;
};
hipError_t group_launch(const GroupArgs &g, hipStream_t stream);
int group_max_work(int n_pairs, int n_experts, int tpc);

// V4.1 routing with a shared expert: ids_aug[t][k] = ids[t][k] for k < K
// (ids outside [0, E) become -1) and E for k = K; w_aug likewise with 1.
hipError_t augment_launch(const int32_t *ids, const float *w, int n_tokens, int top_k,
                          int n_experts, int32_t *ids_aug, float *w_aug, hipStream_t stream);

// out[t][r] = sum_k w[t][k] * y[slot_of_pair[t*K+k]][r] (w == nullptr: unit weights)
hipError_t combine_launch(const float *y, const int32_t *slot_of_pair, const float *w,
                          int n_tokens, int top_k, int hidden, void *out, bool out_bf16,
                          hipStream_t stream);

// Top-k routing of gating logits [n_tokens][n_experts] (n_experts <= 1024,
// top_k <= 32): ids / w [n_tokens][top_k] in rank order, weights renormalised.
hipError_t route_topk_launch(const float *logits, int n_tokens, int n_experts, int top_k,
                             int32_t *ids, float *w, hipStream_t stream);

// Copy h rows (slot order) between a caller buffer and the workspace.
hipError_t copy_launch(void *dst, const void *src, size_t bytes, hipStream_t stream);

} // namespace mx
