// Internal launch interface between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpt {

struct TopkLaunch {
    const float* logits;
    const float* bias;
    int64_t M;
    int E, k, scoring, renorm;
    int vector_rows;  // rows are 16-byte aligned and E % 4 == 0
    int32_t* inds;
    float* weights;
};

// Gate weight formats: bf16, or block-scaled (OCP MX: E8M0 scale per 32
// elements) with FP4 E2M1 or FP8 E4M3 elements.
enum GateFormat : int { kGateBf16 = 0, kGateMxfp4 = 1, kGateMxfp8 = 2 };

// Decode: M <= 64 tokens.  Grid = R row blocks x B expert blocks x S H-splits.
struct DecodeLaunch {
    const uint16_t* x;
    const uint16_t* w;      // bf16 gate [E, H], or NULL with a block-scaled gate below
    int w_format;           // GateFormat
    const uint8_t* w_codes; // block-scaled gate codes: MXFP4 [E, H/2] (even element in the
                            // low nibble) or MXFP8 [E, H] (one E4M3 code per byte)
    const uint8_t* w_scale; // block-scaled gate: E8M0 scales [E, H/32]
    const float* bias;
    int M, H, E, k, scoring, renorm;
    int32_t* inds;
    float* weights;
    float* logits_out;      // optional
    int32_t* table_ids;     // unique-route table, M*k <= 64 (all four set or all NULL)
    int32_t* table_mask;
    int32_t* table_s2u;
    int32_t* table_count;
    float* partials;        // workspace [S][M][256] (value, tag) pairs, zero-filled at init
    uint32_t* counters;     // workspace, kDecodeCounters words (8-byte words for the
                            // split kernel: epoch << 8 | count), zero-filled at init
    int S;                  // H splits
    int ks_per_split;       // k units per split: 32-wide k-steps (bf16 gate), 128-wide blocks (MX)
    int load_waves;         // geometry: kDecodeWide.load_waves
    // one-expert-per-workgroup kernel (M <= kExpertMaxRows)
    uint32_t* xslots;       // workspace [kExpertMaxRows][256] (logit bits, tag) pairs, tag 0 between calls
    uint64_t* xcounters;    // workspace, kExpertCounterWords words: group words (epoch << 8 | count)
    uint32_t* status;       // workspace: sticky status bits (kStatus*)
    uint32_t wait_ticks;    // bound on the finisher's wait (100 MHz realtime ticks)
};

struct PrefillLaunch {
    const uint16_t* x;
    const uint16_t* w;      // bf16 gate [E, H], or NULL with a block-scaled gate below
    int w_format;           // GateFormat
    const uint8_t* w_codes; // MXFP4 [E, H/2] or MXFP8 [E, H] codes (H % 128 == 0)
    const uint8_t* w_scale; // E8M0 scales [E, H/32], 4-byte aligned
    const float* bias;
    int64_t M;
    int H, E, k, scoring, renorm;
    int32_t* inds;
    float* weights;
    float* logits_out;      // optional
    float* partials;        // workspace [tile][S][128][256] (S > 1 only)
    uint32_t* counters;     // workspace [tile][kPrefillCountersPerTile], zero between calls
    int S;                  // K splits per 128-row tile
    int k_per_split;        // H elements per split (multiple of 64)
    uint32_t spin_ticks;    // bounded wait for sibling splits (100 MHz realtime ticks)
};

// Routed gather + shared-expert add: out[t] = bf16(bf16(sum_j w[t,j] y[row(t,j)]) + shared[t]).
struct GatherLaunch {
    const uint16_t* y;               // expert output rows, bf16 [y_rows, D]
    int64_t y_rows;                  // rows outside [0, y_rows) add nothing
    const int32_t* slot_rows;        // [M, k] rows of y, -1 = none; NULL: rows from the table
    const int32_t* token_mask;       // unique-route table (rows in its compact layout)
    const int32_t* slot_to_unique;
    const int32_t* unique_count;
    const float* weights;            // [M, k]
    const uint16_t* shared;          // bf16 [M, D]
    uint16_t* out;                   // bf16 [M, D] (may be `shared`)
    int64_t M;
    int k, D;
};

// Expert GEMM1 on the unique-route table's compact rows.
struct Gemm1Launch {
    const uint16_t* x;               // bf16 [M, D] token activations
    const uint16_t* w1;              // bf16 [E, F, D] every expert's GEMM1 weights
    const int32_t* unique_ids;       // the table (device)
    const int32_t* token_mask;
    const int32_t* unique_count;
    uint16_t* out;                   // bf16 [M*k, F] compact rows
    int64_t E, F, D;
    int M, k;
};

hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream);
hipError_t launch_gemm1(const Gemm1Launch& a, hipStream_t stream);
hipError_t launch_gather(const GatherLaunch& a, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream);
hipError_t launch_decode_expert(const DecodeLaunch& a, hipStream_t stream);
// The allocation-free variant: the kernel's workspace in static device memory
// (the launch's xslots, xcounters and status are ignored and replaced).
hipError_t launch_decode_expert_noalloc(DecodeLaunch a, hipStream_t stream);
hipError_t noalloc_scratch(int device, void** out);  // this device's copy of that memory
size_t noalloc_scratch_bytes();
hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream);
int prefill_splits(int64_t M);

// Decode geometry shared by the host (workspace sizing) and the launcher.
constexpr int kDecodeTile = 16;        // rows per row block, experts per expert block
constexpr int kDecodeMaxSplits = 8;    // H splits
constexpr int kDecodeMaxM = 256;
constexpr int kDecodeMaxRowBlocks = kDecodeMaxM / kDecodeTile;
constexpr int kDecodeMaxBlocks = 256 / kDecodeTile;  // expert blocks at E = 256
// Arrival counters, one 64-byte line (16 4-byte words) apart: per (row
// block, expert block), then per row block.
constexpr int kDecodeCounterStride = 16;
// ... then the unique-route table's (index, tag) slots, one per routed slot
// t*k + j of the row block that builds it (M*k <= 64).
constexpr int kDecodeTableSlotWord =
    kDecodeCounterStride * (kDecodeMaxRowBlocks * kDecodeMaxBlocks + kDecodeMaxRowBlocks);
constexpr int kDecodeCounters = kDecodeTableSlotWord + 2 * 64;

// One-expert-per-workgroup decode kernel: token counts up to kExpertMaxRows;
// arrival counters for groups of kExpertGroup workgroups, one 64-byte line
// (kExpertCounterStride 8-byte words) apart, then the group counter.
constexpr int kExpertMaxRows = 8;
// From this many tokens on, router_fwd (and router_fwd_route_table, which
// must give the same bytes) takes the H-split kernel: measured at H = 7168,
// 5 to 8 tokens there take 6.5-6.6 us against 7.6-8.7 us here (one finisher
// per row beats one workgroup routing every row); up to 4 tokens this kernel
// is as fast or faster, and the allocation-free entry point (up to 4 tokens)
// shares it.
constexpr int kExpertSplitMinRows = 5;
// Allocation-free decode entry point: up to this many tokens.
constexpr int kNoAllocMaxRows = 4;
constexpr int kExpertGroup = 16;
constexpr int kExpertGroups = 256 / kExpertGroup;
constexpr int kExpertCounterStride = 8;
constexpr int kExpertCounterWords = kExpertCounterStride * (kExpertGroups + 1);
// Sticky status bits (workspace word, read and cleared by router_status).
constexpr uint32_t kStatusWaitLimit = 1u;  // a finisher stopped waiting at the time limit
// Default bound on a decode finisher's wait: 100 ms (100 MHz realtime clock).
constexpr uint32_t kDecodeWaitTicksDefault = 10000000u;

// Split decode geometry (kExpertSplitMinRows tokens and more): workgroups of
// 8 load waves, so a finisher has enough waves to route its rows, plus one
// control wave; as many H-splits (up to max_splits) as keep the grid within
// target_workgroups, one per CU.
struct DecodeGeometry {
    int load_waves;
    int target_workgroups;
    int max_splits;
};
constexpr DecodeGeometry kDecodeWide{8, 256, kDecodeMaxSplits};

// Prefill geometry: 128-row tiles; K split S ways (16, 8, 4 or 2) while
// tiles (padded to the 8 XCDs) * S <= 256.
constexpr int kPrefillTileRows = 128;
constexpr int kPrefillMaxPairs = 256;          // (tile, split) pairs with published partials
constexpr int kPrefillCountersPerTile = 32;    // arrive, done, abandoned[16], pad
constexpr int kPrefillMaxSplitTiles = kPrefillMaxPairs / 2;

}  // namespace gpt
