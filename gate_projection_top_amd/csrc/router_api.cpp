// C-ABI layer of librouter: argument validation, the per-device workspace,
// and the choice between the decode and prefill kernels.  No arithmetic of
// the router happens here; every step runs in the HIP kernels.
#include "router.h"

#include <atomic>
#include <mutex>

#include "launch.hpp"

namespace {

struct DeviceWorkspace {
    float* partials = nullptr;          // decode H-split partial logits [S][M][256] (value, tag), zero-filled
    uint32_t* counters = nullptr;       // decode arrival counters (two levels)
    uint32_t* xslots = nullptr;         // one-expert decode: tagged logit slots, zero-filled
    uint64_t* xcounters = nullptr;      // one-expert decode: epoch/arrival words, zero-filled
    uint32_t* status = nullptr;         // sticky status bits
    float* pf_partials = nullptr;       // prefill split partials [tile][S][128][256]
    uint32_t* pf_counters = nullptr;    // prefill per-tile counters
};

constexpr int kMaxDevices = 64;
constexpr size_t kPartialFloats =
    (size_t)gpt::kDecodeMaxSplits * gpt::kDecodeMaxM * ROUTER_MAX_E * 2;  // (value, tag) pairs: 4 MiB
constexpr int kCounters = gpt::kDecodeCounters;
constexpr size_t kPfPartialFloats =
    (size_t)gpt::kPrefillMaxPairs * gpt::kPrefillTileRows * ROUTER_MAX_E;  // 32 MiB
constexpr size_t kPfCounters = (size_t)gpt::kPrefillMaxSplitTiles * gpt::kPrefillCountersPerTile;
constexpr size_t kXSlotWords = (size_t)gpt::kExpertMaxRows * ROUTER_MAX_E * 2;  // (logit, tag) pairs

// A device's workspaces: one per stream that has called a fused entry
// point, up to ROUTER_MAX_STREAMS, all allocated by router_init.  A stream
// keeps its slot until router_release_stream; calls on one stream are
// ordered by the stream, so no two launches that can overlap share a slot.
struct DevicePool {
    bool ready = false;
    DeviceWorkspace ws[ROUTER_MAX_STREAMS];
    hipStream_t owner[ROUTER_MAX_STREAMS] = {};
    bool taken[ROUTER_MAX_STREAMS] = {};
};

DevicePool g_pool[kMaxDevices];
std::atomic<uint32_t> g_spin_ticks{20000};  // 200 us at the 100 MHz realtime clock
std::atomic<uint32_t> g_decode_wait_ticks{gpt::kDecodeWaitTicksDefault};
std::mutex g_ws_mutex;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

void free_workspace(DeviceWorkspace& ws)
{
    void* bufs[] = {ws.partials, ws.counters, ws.xslots, ws.xcounters, ws.status, ws.pf_partials, ws.pf_counters};
    for (void* b : bufs)
        if (b) (void)hipFree(b);
    ws = DeviceWorkspace{};
}

// Allocates one workspace and zeroes what must start at zero (on the null
// stream; the caller synchronises the device before first use).
hipError_t alloc_workspace(DeviceWorkspace& ws)
{
    hipError_t e = hipMalloc((void**)&ws.partials, kPartialFloats * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void**)&ws.counters, kCounters * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMalloc((void**)&ws.pf_partials, kPfPartialFloats * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void**)&ws.pf_counters, kPfCounters * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMalloc((void**)&ws.xslots, kXSlotWords * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMalloc((void**)&ws.xcounters, gpt::kExpertCounterWords * sizeof(uint64_t));
    if (e == hipSuccess) e = hipMalloc((void**)&ws.status, sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(ws.xslots, 0, kXSlotWords * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(ws.xcounters, 0, gpt::kExpertCounterWords * sizeof(uint64_t));
    if (e == hipSuccess) e = hipMemset(ws.status, 0, sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(ws.partials, 0, kPartialFloats * sizeof(float));
    if (e == hipSuccess) e = hipMemset(ws.counters, 0, kCounters * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(ws.pf_counters, 0, kPfCounters * sizeof(uint32_t));
    return e;
}

int init_device(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return ROUTER_ERR_INVALID_ARGUMENT;
    std::lock_guard<std::mutex> guard(g_ws_mutex);
    DevicePool& pool = g_pool[dev];
    if (pool.ready) return ROUTER_OK;

    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return ROUTER_ERR_HIP;
    if (prev != dev && hipSetDevice(dev) != hipSuccess) return ROUTER_ERR_HIP;
    hipError_t e = hipSuccess;
    for (int i = 0; i < ROUTER_MAX_STREAMS && e == hipSuccess; ++i) e = alloc_workspace(pool.ws[i]);
    // The counters must read zero before any stream (blocking or not) runs a
    // kernel; init is rare, so a device-wide wait is acceptable here.
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (prev != dev) (void)hipSetDevice(prev);
    if (e != hipSuccess) {
        for (DeviceWorkspace& ws : pool.ws) free_workspace(ws);
        return ROUTER_ERR_NO_WORKSPACE;
    }
    pool.ready = true;
    return ROUTER_OK;
}

// The workspace of `stream` on the current device: its slot, or a free slot
// it now takes.  A device not yet initialised is initialised here, except
// under stream capture (allocation and a device-wide wait cannot be
// captured): then ROUTER_ERR_NOT_INITIALIZED.
int current_workspace(hipStream_t stream, DeviceWorkspace* out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return ROUTER_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return ROUTER_ERR_INVALID_ARGUMENT;
    for (int attempt = 0; attempt < 2; ++attempt) {
        {
            std::lock_guard<std::mutex> guard(g_ws_mutex);
            DevicePool& pool = g_pool[dev];
            if (pool.ready) {
                int free_slot = -1;
                for (int i = 0; i < ROUTER_MAX_STREAMS; ++i) {
                    if (pool.taken[i] && pool.owner[i] == stream) {
                        *out = pool.ws[i];
                        return ROUTER_OK;
                    }
                    if (!pool.taken[i] && free_slot < 0) free_slot = i;
                }
                if (free_slot < 0) return ROUTER_ERR_BUSY;
                pool.taken[free_slot] = true;
                pool.owner[free_slot] = stream;
                *out = pool.ws[free_slot];
                return ROUTER_OK;
            }
        }
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return ROUTER_ERR_HIP;
        if (cs != hipStreamCaptureStatusNone) return ROUTER_ERR_NOT_INITIALIZED;
        const int rc = init_device(dev);
        if (rc != ROUTER_OK) return rc;
    }
    return ROUTER_ERR_NO_WORKSPACE;
}

int check_common(int64_t M, int E, int k, int scoring, int renorm)
{
    if (scoring != ROUTER_SCORING_SOFTMAX && scoring != ROUTER_SCORING_SQRT_SOFTPLUS)
        return ROUTER_ERR_INVALID_ARGUMENT;
    if (renorm != 0 && renorm != 1) return ROUTER_ERR_INVALID_ARGUMENT;
    if (M < 0 || E < 1 || k < 1 || k > E) return ROUTER_ERR_INVALID_ARGUMENT;
    if (E > ROUTER_MAX_E || k > ROUTER_MAX_K) return ROUTER_ERR_UNSUPPORTED;
    return ROUTER_OK;
}

int check_hidden(int H)
{
    if (H < 1) return ROUTER_ERR_INVALID_ARGUMENT;
    if (H % 8 != 0) return ROUTER_ERR_UNSUPPORTED;
    return ROUTER_OK;
}

int check_projection(const void* x, const void* w)
{
    if (!x || !w) return ROUTER_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(w)) return ROUTER_ERR_MISALIGNED;
    return ROUTER_OK;
}

// Decode split choice: about the geometry's target workgroup count, with at
// least one k unit (a 32-wide k-step, or a 128-wide block-scaled block) per load
// wave in every split.
void decode_splits(int M, int KS, int E, int* S_out, int* ks_per_split_out, int* load_waves_out)
{
    const gpt::DecodeGeometry g = gpt::kDecodeWide;
    const int R = (M + gpt::kDecodeTile - 1) / gpt::kDecodeTile;
    const int B = (E + gpt::kDecodeTile - 1) / gpt::kDecodeTile;
    // As many splits as keep one workgroup per CU (256): a second workgroup
    // on a CU shares its load path (measured at 320 tokens: 36 us against 20
    // us at 256), while more workgroups up to that point shorten each one's
    // k range (32-64 tokens: 9.8-13.1 us at 128 workgroups, 8.6-10.0 us at
    // 256).
    int S = g.target_workgroups / (R * B);
    const int by_work = KS / g.load_waves > 1 ? KS / g.load_waves : 1;
    if (S > by_work) S = by_work;
    if (S > g.max_splits) S = g.max_splits;
    if (S < 1) S = 1;
    const int per = (KS + S - 1) / S;
    *ks_per_split_out = per;
    *S_out = (KS + per - 1) / per;
    *load_waves_out = g.load_waves;
}

// format kGateBf16 reads w; the block-scaled formats read w_codes and w_scale.
int run_fused(const void* x, const void* w, int format, const uint8_t* w_codes, const uint8_t* w_scale,
              const float* bias, int64_t M, int H, int E, int k, int scoring, int renorm,
              int32_t* inds, float* weights, float* logits, int32_t* t_ids, int32_t* t_mask,
              int32_t* t_s2u, int32_t* t_count, hipStream_t stream)
{
    hipError_t e;
    DeviceWorkspace ws;
    const int rc = current_workspace(stream, &ws);
    if (rc != ROUTER_OK) return rc;
    if (M <= ROUTER_DECODE_MAX_M) {
        gpt::DecodeLaunch a{};
        a.x = static_cast<const uint16_t*>(x);
        a.w = static_cast<const uint16_t*>(w);
        a.w_format = format;
        a.w_codes = w_codes;
        a.w_scale = w_scale;
        a.bias = bias;
        a.M = (int)M;
        a.H = H;
        a.E = E;
        a.k = k;
        a.scoring = scoring;
        a.renorm = renorm;
        a.inds = inds;
        a.weights = weights;
        a.logits_out = logits;
        a.table_ids = t_ids;
        a.table_mask = t_mask;
        a.table_s2u = t_s2u;
        a.table_count = t_count;
        a.partials = ws.partials;
        a.counters = ws.counters;
        a.xslots = ws.xslots;
        a.xcounters = ws.xcounters;
        a.status = ws.status;
        a.wait_ticks = g_decode_wait_ticks.load(std::memory_order_relaxed);
        // One gate row per workgroup up to kExpertMaxRows tokens (with or
        // without the route table, so both give the same bytes); the H-split
        // kernel above, one finisher per row.
        if (M < gpt::kExpertSplitMinRows) {
            e = gpt::launch_decode_expert(a, stream);
        } else {
            const int units = format != gpt::kGateBf16 ? (H + 127) / 128 : (H + 31) / 32;
            decode_splits((int)M, units, E, &a.S, &a.ks_per_split, &a.load_waves);
            e = gpt::launch_decode(a, stream);
        }
    } else {
        gpt::PrefillLaunch a{};
        a.x = static_cast<const uint16_t*>(x);
        a.w = static_cast<const uint16_t*>(w);
        a.w_format = format;
        a.w_codes = w_codes;
        a.w_scale = w_scale;
        a.bias = bias;
        a.M = M;
        a.H = H;
        a.E = E;
        a.k = k;
        a.scoring = scoring;
        a.renorm = renorm;
        a.inds = inds;
        a.weights = weights;
        a.logits_out = logits;
        a.partials = ws.pf_partials;
        a.counters = ws.pf_counters;
        a.S = gpt::prefill_splits(M);
        const int k_steps = (H + 63) / 64;
        a.k_per_split = ((k_steps + a.S - 1) / a.S) * 64;
        a.spin_ticks = g_spin_ticks.load(std::memory_order_relaxed);
        e = gpt::launch_prefill(a, stream);
    }
    return e == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
}

}  // namespace

extern "C" {

int router_init(int device)
{
    if (device < 0) {
        if (hipGetDevice(&device) != hipSuccess) return ROUTER_ERR_HIP;
    }
    const int rc = init_device(device);
    if (rc != ROUTER_OK) return rc;
    // resolve this device's copy of the allocation-free entry's static scratch
    void* scratch = nullptr;
    return gpt::noalloc_scratch(device, &scratch) == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
}

int router_fwd(const void* x, const void* w, const float* bias, int64_t M, int H, int E, int k,
               int scoring, int renorm, int32_t* out_inds, float* out_weights,
               float* opt_out_logits, hipStream_t stream)
{
    int rc = check_common(M, E, k, scoring, renorm);
    if (rc == ROUTER_OK) rc = check_hidden(H);
    if (rc != ROUTER_OK) return rc;
    if (M == 0) return ROUTER_OK;
    rc = check_projection(x, w);
    if (rc != ROUTER_OK) return rc;
    if (!out_inds || !out_weights) return ROUTER_ERR_INVALID_ARGUMENT;
    if (M > 0x7fffffffLL / 256) return ROUTER_ERR_UNSUPPORTED;
    // 32-bit byte offsets inside one 128-row tile of X and inside W
    if ((int64_t)H * 2 * 256 > 0x7fff0000LL) return ROUTER_ERR_UNSUPPORTED;
    return run_fused(x, w, gpt::kGateBf16, nullptr, nullptr, bias, M, H, E, k, scoring, renorm, out_inds,
                     out_weights, opt_out_logits, nullptr, nullptr, nullptr, nullptr, stream);
}

int router_fwd_noalloc(const void* x, const void* w, const float* bias, int64_t M, int H, int E, int k,
                       int scoring, int renorm, int32_t* out_inds, float* out_weights, float* opt_out_logits,
                       hipStream_t stream)
{
    int rc = check_common(M, E, k, scoring, renorm);
    if (rc == ROUTER_OK) rc = check_hidden(H);
    if (rc != ROUTER_OK) return rc;
    if (M == 0) return ROUTER_OK;
    if (M > ROUTER_NOALLOC_MAX_M) return ROUTER_ERR_UNSUPPORTED;
    rc = check_projection(x, w);
    if (rc != ROUTER_OK) return rc;
    if (!out_inds || !out_weights) return ROUTER_ERR_INVALID_ARGUMENT;
    if ((int64_t)H * 2 * 256 > 0x7fff0000LL) return ROUTER_ERR_UNSUPPORTED;
    gpt::DecodeLaunch a{};
    a.x = static_cast<const uint16_t*>(x);
    a.w = static_cast<const uint16_t*>(w);
    a.w_format = gpt::kGateBf16;
    a.bias = bias;
    a.M = (int)M;
    a.H = H;
    a.E = E;
    a.k = k;
    a.scoring = scoring;
    a.renorm = renorm;
    a.inds = out_inds;
    a.weights = out_weights;
    a.logits_out = opt_out_logits;
    a.wait_ticks = g_decode_wait_ticks.load(std::memory_order_relaxed);
    return gpt::launch_decode_expert_noalloc(a, stream) == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
}

// The table is built by the finisher of the single row block, in one wavefront.
static_assert(ROUTER_TABLE_MAX_M <= gpt::kDecodeTile, "table rows share one row block");
static_assert(ROUTER_TABLE_MAX_SLOTS <= 64, "table slots fit one wavefront");
static_assert(ROUTER_TABLE_MAX_M <= ROUTER_DECODE_MAX_M, "table calls take the decode path");

int router_fwd_route_table(const void* x, const void* w, const float* bias, int M, int H, int E,
                           int k, int scoring, int renorm, int32_t* out_inds, float* out_weights,
                           float* opt_out_logits, int32_t* out_unique_ids,
                           int32_t* out_token_mask, int32_t* out_slot_to_unique,
                           int32_t* out_unique_count, hipStream_t stream)
{
    int rc = check_common(M, E, k, scoring, renorm);
    if (rc == ROUTER_OK) rc = check_hidden(H);
    if (rc == ROUTER_OK) rc = check_projection(x, w);
    if (rc != ROUTER_OK) return rc;
    if (M < 1) return ROUTER_ERR_INVALID_ARGUMENT;
    if (M > ROUTER_TABLE_MAX_M || M * k > ROUTER_TABLE_MAX_SLOTS) return ROUTER_ERR_UNSUPPORTED;
    if (!out_inds || !out_weights || !out_unique_ids || !out_token_mask || !out_slot_to_unique ||
        !out_unique_count)
        return ROUTER_ERR_INVALID_ARGUMENT;
    return run_fused(x, w, gpt::kGateBf16, nullptr, nullptr, bias, M, H, E, k, scoring, renorm, out_inds,
                     out_weights, opt_out_logits, out_unique_ids, out_token_mask,
                     out_slot_to_unique, out_unique_count, stream);
}

int router_fwd_m2_table(const void* x, const void* w, const float* bias, int H, int E, int k,
                        int scoring, int renorm, int32_t* out_inds, float* out_weights,
                        float* opt_out_logits, int32_t* out_unique_ids,
                        int32_t* out_token_mask, int32_t* out_slot_to_unique,
                        int32_t* out_unique_count, hipStream_t stream)
{
    return router_fwd_route_table(x, w, bias, 2, H, E, k, scoring, renorm, out_inds, out_weights,
                                  opt_out_logits, out_unique_ids, out_token_mask,
                                  out_slot_to_unique, out_unique_count, stream);
}

// Shared checks and launch of the block-scaled gate formats.
static int run_block_scaled(int format, const void* x, const uint8_t* w_codes, const uint8_t* w_scale,
                            const float* bias, int64_t M, int H, int E, int k, int scoring, int renorm,
                            int32_t* out_inds, float* out_weights, float* opt_out_logits,
                            hipStream_t stream)
{
    int rc = check_common(M, E, k, scoring, renorm);
    if (rc == ROUTER_OK) rc = check_hidden(H);
    if (rc != ROUTER_OK) return rc;
    if (H % 32 != 0) return ROUTER_ERR_UNSUPPORTED;
    // the prefill kernel moves a 64-wide stage's two scales as one aligned dword
    if (M > ROUTER_DECODE_MAX_M && H % 128 != 0) return ROUTER_ERR_UNSUPPORTED;
    if (M == 0) return ROUTER_OK;
    rc = check_projection(x, w_codes);
    if (rc != ROUTER_OK) return rc;
    if (!w_scale || !out_inds || !out_weights) return ROUTER_ERR_INVALID_ARGUMENT;
    if (M > ROUTER_DECODE_MAX_M && ((uintptr_t)w_scale & 3u) != 0) return ROUTER_ERR_MISALIGNED;
    if (M > 0x7fffffffLL / 256) return ROUTER_ERR_UNSUPPORTED;
    // 32-bit byte offsets inside one 128-row tile of X and inside the codes
    if ((int64_t)H * 2 * 256 > 0x7fff0000LL) return ROUTER_ERR_UNSUPPORTED;
    return run_fused(x, nullptr, format, w_codes, w_scale, bias, M, H, E, k, scoring, renorm, out_inds,
                     out_weights, opt_out_logits, nullptr, nullptr, nullptr, nullptr, stream);
}

int router_fwd_mxfp4(const void* x, const uint8_t* w_fp4, const uint8_t* w_scale,
                     const float* bias, int64_t M, int H, int E, int k, int scoring, int renorm,
                     int32_t* out_inds, float* out_weights, float* opt_out_logits,
                     hipStream_t stream)
{
    return run_block_scaled(gpt::kGateMxfp4, x, w_fp4, w_scale, bias, M, H, E, k, scoring, renorm,
                            out_inds, out_weights, opt_out_logits, stream);
}

int router_fwd_mxfp8(const void* x, const uint8_t* w_fp8, const uint8_t* w_scale,
                     const float* bias, int64_t M, int H, int E, int k, int scoring, int renorm,
                     int32_t* out_inds, float* out_weights, float* opt_out_logits,
                     hipStream_t stream)
{
    return run_block_scaled(gpt::kGateMxfp8, x, w_fp8, w_scale, bias, M, H, E, k, scoring, renorm,
                            out_inds, out_weights, opt_out_logits, stream);
}

int router_gather_shared_add(const void* y, int64_t y_rows, const int32_t* slot_rows,
                             const float* weights, const void* shared, int64_t M, int k, int D,
                             void* out, hipStream_t stream)
{
    if (M < 0 || k < 1 || D < 1 || y_rows < 0) return ROUTER_ERR_INVALID_ARGUMENT;
    if (k > ROUTER_MAX_K || D % 8 != 0) return ROUTER_ERR_UNSUPPORTED;
    if (M == 0) return ROUTER_OK;
    if (!slot_rows || !weights || !shared || !out || (!y && y_rows > 0)) return ROUTER_ERR_INVALID_ARGUMENT;
    if (!aligned16(y) || !aligned16(shared) || !aligned16(out)) return ROUTER_ERR_MISALIGNED;
    if (M * (((int64_t)D + 1023) / 1024) > 0x7fffffffLL) return ROUTER_ERR_UNSUPPORTED;
    gpt::GatherLaunch a{};
    a.y = static_cast<const uint16_t*>(y);
    a.y_rows = y_rows;
    a.slot_rows = slot_rows;
    a.weights = weights;
    a.shared = static_cast<const uint16_t*>(shared);
    a.out = static_cast<uint16_t*>(out);
    a.M = M;
    a.k = k;
    a.D = D;
    return gpt::launch_gather(a, stream) == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
}

int router_gather_shared_add_table(const void* y, const int32_t* token_mask,
                                   const int32_t* slot_to_unique, const int32_t* unique_count,
                                   const float* weights, const void* shared, int M, int k, int D,
                                   void* out, hipStream_t stream)
{
    if (M < 1 || k < 1 || D < 1) return ROUTER_ERR_INVALID_ARGUMENT;
    if (k > ROUTER_MAX_K || D % 8 != 0 || M > ROUTER_TABLE_MAX_M || M * k > ROUTER_TABLE_MAX_SLOTS)
        return ROUTER_ERR_UNSUPPORTED;
    if (!y || !token_mask || !slot_to_unique || !unique_count || !weights || !shared || !out)
        return ROUTER_ERR_INVALID_ARGUMENT;
    if (!aligned16(y) || !aligned16(shared) || !aligned16(out)) return ROUTER_ERR_MISALIGNED;
    gpt::GatherLaunch a{};
    a.y = static_cast<const uint16_t*>(y);
    a.y_rows = (int64_t)M * k;  // the compact layout never has more rows than slots
    a.token_mask = token_mask;
    a.slot_to_unique = slot_to_unique;
    a.unique_count = unique_count;
    a.weights = weights;
    a.shared = static_cast<const uint16_t*>(shared);
    a.out = static_cast<uint16_t*>(out);
    a.M = M;
    a.k = k;
    a.D = D;
    return gpt::launch_gather(a, stream) == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
}

int router_expert_gemm1_table(const void* x, const void* w1, int E, int64_t F, int D,
                              const int32_t* unique_ids, const int32_t* token_mask,
                              const int32_t* unique_count, int M, int k, void* out,
                              hipStream_t stream)
{
    if (M < 1 || k < 1 || E < 1 || F < 1 || D < 1) return ROUTER_ERR_INVALID_ARGUMENT;
    if (k > ROUTER_MAX_K || M > ROUTER_TABLE_MAX_M || M * k > ROUTER_TABLE_MAX_SLOTS || D % 8 != 0)
        return ROUTER_ERR_UNSUPPORTED;
    if ((int64_t)M * k * ((F + 63) / 64) > 0x7fffffffLL) return ROUTER_ERR_UNSUPPORTED;
    if (!x || !w1 || !unique_ids || !token_mask || !unique_count || !out)
        return ROUTER_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(w1)) return ROUTER_ERR_MISALIGNED;
    gpt::Gemm1Launch a{};
    a.x = static_cast<const uint16_t*>(x);
    a.w1 = static_cast<const uint16_t*>(w1);
    a.unique_ids = unique_ids;
    a.token_mask = token_mask;
    a.unique_count = unique_count;
    a.out = static_cast<uint16_t*>(out);
    a.E = E;
    a.F = F;
    a.D = D;
    a.M = M;
    a.k = k;
    return gpt::launch_gemm1(a, stream) == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
}

int router_topk_from_logits(const float* logits, const float* bias, int64_t M, int E, int k,
                            int scoring, int renorm, int32_t* out_inds, float* out_weights,
                            hipStream_t stream)
{
    const int rc = check_common(M, E, k, scoring, renorm);
    if (rc != ROUTER_OK) return rc;
    if (M == 0) return ROUTER_OK;
    if (!logits || !out_inds || !out_weights) return ROUTER_ERR_INVALID_ARGUMENT;
    gpt::TopkLaunch a{};
    a.logits = logits;
    a.bias = bias;
    a.M = M;
    a.E = E;
    a.k = k;
    a.scoring = scoring;
    a.renorm = renorm;
    a.vector_rows = (E % 4 == 0) && aligned16(logits);
    a.inds = out_inds;
    a.weights = out_weights;
    return gpt::launch_topk(a, stream) == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
}

int router_set_exchange_timeout_us(int microseconds)
{
    if (microseconds < 0) return ROUTER_ERR_INVALID_ARGUMENT;
    const uint64_t ticks = (uint64_t)microseconds * 100u;
    g_spin_ticks.store(ticks > 0xffffffffu ? 0xffffffffu : (uint32_t)ticks, std::memory_order_relaxed);
    return ROUTER_OK;
}

int router_set_decode_wait_limit_us(int microseconds)
{
    if (microseconds < 0) return ROUTER_ERR_INVALID_ARGUMENT;
    const uint64_t ticks = (uint64_t)microseconds * 100u;
    g_decode_wait_ticks.store(ticks > 0xffffffffu ? 0xffffffffu : (uint32_t)ticks, std::memory_order_relaxed);
    return ROUTER_OK;
}

int router_status(int device, int clear, uint32_t* out_flags)
{
    if (!out_flags) return ROUTER_ERR_INVALID_ARGUMENT;
    if (device < 0) {
        if (hipGetDevice(&device) != hipSuccess) return ROUTER_ERR_HIP;
    }
    if (device >= kMaxDevices) return ROUTER_ERR_INVALID_ARGUMENT;
    uint32_t* words[ROUTER_MAX_STREAMS + 1] = {};  // every workspace's status word, then the scratch's
    {
        std::lock_guard<std::mutex> guard(g_ws_mutex);
        if (g_pool[device].ready)
            for (int i = 0; i < ROUTER_MAX_STREAMS; ++i) words[i] = g_pool[device].ws[i].status;
    }
    *out_flags = 0;
    if (!words[0]) return ROUTER_OK;  // nothing has run on this device through this library
    void* scratch = nullptr;
    if (gpt::noalloc_scratch(device, &scratch) == hipSuccess)
        words[ROUTER_MAX_STREAMS] =
            reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(scratch) + gpt::noalloc_scratch_bytes() - 256);
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return ROUTER_ERR_HIP;
    if (prev != device && hipSetDevice(device) != hipSuccess) return ROUTER_ERR_HIP;
    hipError_t e = hipDeviceSynchronize();
    for (uint32_t* st : words) {
        if (!st || e != hipSuccess) continue;
        uint32_t f = 0;
        e = hipMemcpy(&f, st, sizeof(uint32_t), hipMemcpyDeviceToHost);
        *out_flags |= f;
        if (e == hipSuccess && clear) e = hipMemset(st, 0, sizeof(uint32_t));
    }
    if (e == hipSuccess && clear) e = hipDeviceSynchronize();
    if (prev != device) (void)hipSetDevice(prev);
    return e == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
}

int router_release_stream(hipStream_t stream)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return ROUTER_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return ROUTER_ERR_INVALID_ARGUMENT;
    std::lock_guard<std::mutex> guard(g_ws_mutex);
    DevicePool& pool = g_pool[dev];
    for (int i = 0; i < ROUTER_MAX_STREAMS; ++i)
        if (pool.taken[i] && pool.owner[i] == stream) pool.taken[i] = false;
    return ROUTER_OK;
}

const char* router_strerror(int code)
{
    switch (code) {
    case ROUTER_OK: return "ok";
    case ROUTER_ERR_INVALID_ARGUMENT: return "invalid argument";
    case ROUTER_ERR_UNSUPPORTED: return "shape outside the supported limits";
    case ROUTER_ERR_MISALIGNED: return "x or the gate weights are not 16-byte aligned";
    case ROUTER_ERR_HIP: return "HIP runtime error";
    case ROUTER_ERR_NO_WORKSPACE: return "workspace allocation failed";
    case ROUTER_ERR_BUSY: return "every workspace of the device is held by another stream (router_release_stream)";
    case ROUTER_ERR_NOT_INITIALIZED: return "first call on the device under stream capture: call router_init first";
    default: return "unknown router error";
    }
}

}  // extern "C"
