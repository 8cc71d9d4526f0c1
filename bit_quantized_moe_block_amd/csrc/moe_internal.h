// Internal structures shared by the host side of the C ABI and the gfx950
// kernels of the routed-experts decode step. Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kThreads = 256;       // every kernel: 4 wave64s
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 16;
constexpr int kMaxTokens = 512;
// Bucket rows: k routed rows per token, plus one per token for a shared expert.
constexpr int kMaxPairs = kMaxTokens * (kMaxTopK + 1);
constexpr int kGroupRows = 16;      // rows of one MFMA token block
// Row groups: each hit expert's bucket split into groups of <= 16 rows.
constexpr int kMaxGroups = kMaxExperts + kMaxPairs / kGroupRows;
constexpr int kLdsPadHalves = 8;    // 16 B row padding of the staged activations

constexpr int kFmtCodebook = 1;
constexpr int kFmtNvfp4 = 2;

// Cross-block counters (rb_done, h_ready) sit one per 128-byte line:
// blocks polling one counter must not queue behind traffic to its
// neighbours, as they would when packed.
constexpr int kCtrStride = 32;  // uint32 per counter slot

// Error bits of Counters::error_word.
constexpr uint32_t kErrSpinLimit = 1u;

// One stored expert projection on the device (copied from moe_tensor_desc).
struct DevTensor {
    const void *codes;
    const void *scales;
    const uint16_t *lut;
    float tensor_scale;
    int32_t bits;
};

// Routing result of one run, written by the route kernel's bucketing block.
struct Plan {
    int32_t m;
    int32_t n_groups;      // row groups (<= group_rows rows each)
    int32_t n_items1;      // gate/up work items
    int32_t n_items;       // all work items
    int32_t n_sgroups;     // row groups of the shared expert (groups 0 .. n_sgroups-1)
    int32_t n_wide;        // routed groups whose gate/up items span span1 row blocks;
                           // the routed groups after them take one row block per item
    int32_t pad[2];
    int32_t g_expert[kMaxGroups];  // expert of group u (groups in expert order)
    int32_t g_off[kMaxGroups];     // first row of u in the bucket row list
    int32_t g_rows[kMaxGroups];    // rows of u (1..group_rows)
};

// Completed work items are counted on kDoneSlots counters (block b adds to
// slot b % kDoneSlots) so that no single address takes every block's atomic.
constexpr int kDoneSlots = 8;

struct Counters {
    uint32_t items_done[kDoneSlots];  // work items completed (statistics)
    uint32_t error_word;              // kErr* bits
    uint32_t route_done;              // top-k blocks finished (route kernel)
    uint32_t pad[6];
};

// Everything a kernel needs, passed by value.
struct Params {
    int32_t format, E, k, H, I, max_tokens;
    int32_t ks1, kc1;      // gate/up: column splits and columns per split
    int32_t ks2, kc2;      // down: column splits and columns per split (kc1 = kc2)
    int32_t span1;         // gate/up: 128-row blocks per work item (set per run)
    int32_t n_rb1;         // I / 128 gate/up row blocks of 128 (one rotation block each)
    int32_t n_rb2;         // H / 256 down row blocks of 256
    int32_t pair_cap;      // bucket row capacity: max_tokens * (k + has_shared)
    int32_t has6;          // 1: some tensor has 6-bit codes (selects the kernel with that path)
    int32_t has_shared;    // 1: an always-on shared expert (tensors 3E..3E+2, bucket
                           // rows m*k + t, group expert id E)
    int32_t sh_half;       // 1: the shared expert's items cover half row blocks (its
                           // 6-bit codes make a full row block three 2-bit ones)
    int32_t group_rows;    // rows per row group: 16 (persistent decode kernel) or 64 (prefill)
    int32_t gcap;          // row-group table entries in LDS (bound on the groups of a run)
    int32_t egrid;         // expert-kernel blocks of the run (set per run)
    int32_t lds_tab;       // byte offset of that table in the expert kernel's dynamic LDS
    uint32_t spin_limit;   // polls before a dependency wait gives up
    float *out;            // [m][H] result of the current launch
    const DevTensor *tensors;   // [E*3 + 3] (the last three: the shared expert)
    const int8_t *signs_h;      // [H]
    const int8_t *signs_i;      // [I]
    int32_t *ids;          // [pair_cap] expert of (t, j)
    float *wts;            // [pair_cap] router weight of (t, j)
    int32_t *counts;       // [E]
    int32_t *offsets;      // [E+1]
    int32_t *rows;         // [pair_cap] bucket row list, entry t*k+j (routed rows)
    int32_t *pos;          // [pair_cap] bucket position of (t, j)
    Plan *plan;
    _Float16 *xr;          // [max_tokens][H] rotated activations (fp16)
    float *gu_part;        // [ks1][pair_cap][2][I] gate/up partial sums
    _Float16 *hr;          // [pair_cap][I] rotated SiLU(g)*u (fp16)
    float *y_part;         // [ks2][pair_cap][H] down partial sums
    Counters *ctr;
    uint32_t *rb_done;     // [kMaxGroups][n_rb1] finished column splits per row block
    uint32_t *h_ready;     // [kMaxGroups] finished row blocks of h per row group
                           // (both: one counter per kCtrStride uint32)
};

// Kernel launchers (kernels.hip).
size_t route_lds_bytes(int E, int m);
hipError_t launch_route(const Params &p, const uint16_t *x, const float *logits, int m,
                        hipStream_t s);
hipError_t launch_expert(const Params &p, int grid, size_t lds_bytes, hipStream_t s);
hipError_t launch_combine(const Params &p, int m, hipStream_t s);
// Prefill kernels (gate/up, then down) over up to grid_groups row groups of
// up to 64 rows.
hipError_t launch_prefill(const Params &p, int grid_groups, hipStream_t s);
constexpr int kPrefillRows = 64;  // rows per prefill row group
// Occupancy of the expert kernel for a given dynamic LDS size.
hipError_t expert_occupancy(int format, int ng, bool six, int *blocks_per_cu, size_t lds_bytes);
// Small-m kernel (runs of up to kSmallMaxTokens tokens when no tensor has
// 6-bit codes): gate/up items of 32 rows and down items of 64 rows over all
// columns, persistent grid; it stages R x max(H, I) fp16 activation rows with
// at most kSmallStageElems elements.
hipError_t launch_small(const Params &p, int grid, size_t lds_bytes, hipStream_t s);
hipError_t small_occupancy(int format, int *blocks_per_cu, size_t lds_bytes);
constexpr int kSmallMaxTokens = 4;
constexpr int kSmallStageElems = 8 * 256 * 8;  // staging loads per thread x threads x 8 halves

}  // namespace moe
