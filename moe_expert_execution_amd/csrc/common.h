// Internal declarations shared by the ftmoe library sources (gfx950, HIP).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <string>

#include "ftmoe.h"

namespace ftmoe {

// ---- limits ---------------------------------------------------------------
constexpr int kMaxExperts = 4096;      // E
constexpr int kMaxSlots = 32768;       // N
constexpr int kMaxTopK = 16;           // k
constexpr int kCtrlThreads = 1024;     // one control workgroup
constexpr int kKeysPerThread = kMaxSlots / kCtrlThreads;   // victim keys held per thread
constexpr uint64_t kStampLimit = 1ull << 40;               // stamps fit 40 bits; slot 24 bits
constexpr int kChunkTokens = 64;       // tokens per stable-sort chunk (one 64-bit mask)
constexpr int kSmallPlanRoutes = 1024; // routes handled by the one-workgroup planner
constexpr int kLargeKeySpace = 8192;   // slots (or experts) addressable by the chunked planner
constexpr int kGemvMaxTokens = 4;      // tokens per call served by the GEMV path
constexpr size_t kStaticScratchBytes = 16u << 20;   // the per-GPU static scratch of ft_moe_forward_noalloc

// device counters (ft_stats order)
enum { C_CALLS, C_ROUTES, C_UNIQUE, C_HITS, C_MISSES, C_FILLS, C_CPU, C_EVICT, C_BYTES, C_STREAMED,
       C_GEMV_EXPERTS, C_GEMV_ROWS, C_GEMM_EXPERTS, C_GEMM_ROWS, C_N };

// ---- error plumbing -----------------------------------------------------------
void set_error(const char* fmt, ...);
void clear_error();

#define FT_HIP(call)                                                                    \
    do {                                                                                \
        hipError_t e_ = (call);                                                         \
        if (e_ != hipSuccess) {                                                         \
            ::ftmoe::set_error("%s failed: %s (%s:%d)", #call, hipGetErrorString(e_),   \
                               __FILE__, __LINE__);                                     \
            return FT_ERR_HIP;                                                          \
        }                                                                               \
    } while (0)

#define FT_REQUIRE(cond, ...)                          \
    do {                                               \
        if (!(cond)) {                                 \
            ::ftmoe::set_error(__VA_ARGS__);           \
            return FT_ERR_ARG;                         \
        }                                              \
    } while (0)

// ---- record geometry ------------------------------------------------------------
struct RecordLayout {
    int64_t S;             // bytes per record (the host bank's record stride)
    int64_t P;             // slot stride of the device pool: S rounded up to 256 bytes, so every slot's
                           // record starts aligned for 16-byte loads (block-FP8 records of small d, f
                           // are not multiples of 16 bytes)
    int64_t off_gate, off_up, off_down;         // code / value offsets
    int64_t off_sg, off_su, off_sd;             // scale offsets (fp8, mxfp4)
};
bool record_layout(const ft_shape& s, RecordLayout* out);

// ---- the host branch ------------------------------------------------------------
struct HostBranch;
HostBranch* host_branch_create(const ft_shape& sh, const RecordLayout& rl, const uint8_t* const* bank_layers,
                               int32_t max_tokens);
void host_branch_destroy(HostBranch* hb);
// Pinned staging owned by the host branch (device-visible for async copies).
struct HostStaging {
    uint16_t* x;       // [max_tokens x d]
    int32_t* routes;   // [max_tokens x k]
    float* w;          // [max_tokens x k]
    float* P;          // [max_tokens x d]
};
HostStaging host_branch_staging(HostBranch* hb);
// How a forward call hands work to the host branch.  Mailbox: the planner
// stores `seq` to *seq_word (pinned) after staging; a polling host thread runs
// the call and stores `seq` to *done_word, which the combine kernel polls
// (bounded) before it reads the host partials.  Otherwise a stream host
// function runs the call.
// Graph mailbox (calls captured into a graph): the planner draws the call's
// number from a device counter, stores layer and T, then the number, to the
// mailbox's graph words; the poller answers in gdone, which the combine
// kernel polls against the device counter (numbers fixed at capture could not
// be replayed).
struct HostSignal {
    bool mailbox;
    uint64_t seq;
    uint64_t* seq_word;
    uint64_t* done_word;
    uint64_t* gmbox;            // graph words: [0] number, [8] done, [16] layer, [17] T (null = none)
    uint64_t* gseq_dev;         // device counter of graph calls
    int32_t layer, T;
};
HostSignal host_branch_prepare(HostBranch* hb, int32_t layer, int32_t T);
// The graph mailbox for a captured call (gmbox null when no poller runs).
HostSignal host_branch_graph_signal(HostBranch* hb, uint64_t* gseq_dev, int32_t layer, int32_t T);
// Enqueue the host computation of layer `layer` for T tokens on `stream`
// (staging must already hold routes, w and x for those tokens).
hipError_t host_branch_enqueue(HostBranch* hb, int32_t layer, int32_t T, hipStream_t stream);
// The same for a call being captured into a graph: a host function whose
// context lives as long as the branch, so the graph can replay it.
hipError_t host_branch_enqueue_captured(HostBranch* hb, int32_t layer, int32_t T, hipStream_t stream);
int host_branch_threads(HostBranch* hb);
// Run one host-branch call on the calling thread (staging must hold its routes,
// weights and activations); no GPU work may be pending on the host branch.
void host_branch_run_sync(HostBranch* hb, int32_t layer, int32_t T);
// bytes of expert records the workers read, and seconds spent in host calls with work
void host_branch_counters(HostBranch* hb, uint64_t* bytes, double* seconds, uint64_t* experts);

// ---- optional expert-kernel timing ------------------------------------------------
struct Timing;
Timing* timing_create();
void timing_destroy(Timing* t);
// Events that hipExtLaunchKernelGGL stamps at the start and end of one launch
// of class `cls` (both null when `t` is null, i.e. timing is off).
struct TimedLaunch {
    hipEvent_t start = nullptr, stop = nullptr;
};
TimedLaunch timing_launch(Timing* t, int cls);
void timing_read(Timing* t, uint64_t* launches, double* ms);   // synchronises on pending events

// ---- the cache handle ---------------------------------------------------------
struct PlanBuffers {
    int32_t* meta;          // [4]: n_active, n_tiles, n_gpu_routes, unused
    int32_t* active_slot;   // [cap]
    int32_t* seg;           // [cap + 1]: sorted-row offset of each active slot
    int32_t* perm;          // [cap]: route index of each sorted row
    int32_t* route_pos;     // [cap]: sorted row of each route, -1 if not on the GPU
    int32_t* tile_active;   // [max tiles]
    int32_t* tile_row0;     // [max tiles]
    int32_t* tile_first;    // [cap + 1]: first tile of each active slot (then the tile count)
    int32_t* chunk_counts;  // [chunks x kLargeKeySpace] (large planner)
    // (sized for any slot count at creation, so resize never reallocates them)
    int64_t max_tiles;
};

}  // namespace ftmoe

namespace ftmoe {
// Cache state the kernels read at run time rather than from their arguments,
// so that a call captured into a graph sees it as it is at replay: the profile
// (ft_cache_set_profile) and the generation of the slot pool, which
// ft_cache_resize advances (classify compares it with the generation the
// call was enqueued under).  Lives in device memory until the cache is
// destroyed.
struct DevState {
    uint32_t gen;
    uint32_t bp_mbps, bh_mbps;
    int32_t max_fetch;
};
}  // namespace ftmoe

struct ft_cache {
    ft_shape sh;
    ft_profile prof;
    ftmoe::RecordLayout rl;
    int64_t N;
    int32_t max_tokens;
    int32_t cap;               // max_tokens * k
    int device;
    const uint8_t** bank_host; // [L] host address of layer l's E records (pinned; entries may repeat)
    const uint8_t** bank_dev;  // [L] in device memory: the device-visible addresses of the same banks
    uint8_t* pool;             // N * S bytes of HBM
    // control state (device)
    int32_t* slot_for_id;      // [L*E]
    int32_t* id_of_slot;       // [kMaxSlots]: entries past N unused (never reallocated)
    uint64_t* stamp;           // [kMaxSlots]
    uint64_t* clock;           // [1]
    unsigned long long* counters;  // [C_N]
    int32_t* errflag;          // [1]
    ftmoe::DevState* dstate;   // [1] profile and pool generation (device)
    uint32_t gen;              // the pool generation calls are enqueued under
    uint32_t host_wait_polls;  // bound of the combine's wait for the host branch (FTMOE_HOST_WAIT_POLLS)
    uint64_t* gseq_dev;        // [1] number of the last host-branch call made by a graph replay
    // internal copy of the last classify's fill worklist and counts
    int32_t* wl_counts;        // [4]
    int32_t* wl_slot;          // [cap]
    int32_t* wl_src;           // [cap]
    // forward scratch
    ftmoe::PlanBuffers plan;
    uint16_t* H;               // [cap x f] bf16 (GEMM path)
    uint16_t* Y;               // [cap x d] bf16 expert outputs, one row per GPU route
    int32_t cap_gemv;          // rows served by the GEMV path
    int32_t gv_kq;             // K-parts of the gate/up GEMV
    float* gv_part;            // [2 x gv_kq x cap_gemv x f] fp32 K-part sums of g and u (GEMV path)
    float* dpart;              // [groups x k x d] fp32 partial outputs of the one-token decode kernel
                               // (null: one-token calls take the two-kernel GEMV path)
    // streams and events
    hipStream_t xfer;          // transfer stream (fills, full-layer loads)
    hipStream_t hstream;       // host-branch copies and host function
    hipEvent_t ev_ctrl, ev_fwd, ev_host, ev_xlast, ev_fence;
    bool xfer_pending;         // ev_xlast recorded
    bool fill_pending;         // the last classify's fills are not enqueued yet
    hipStream_t fill_stream;   // the stream of that classify
    bool streaming;            // inside a run of STREAMED calls (beginning fence taken)
    // full-layer buffers
    int buf_layer[2];
    hipEvent_t ready[2], release[2];
    bool release_recorded[2];
    ftmoe::HostBranch* host;
    ftmoe::Timing* timing;     // null unless timing is enabled
};

namespace ftmoe {
// ---- kernel launchers (each returns hipGetLastError() of its launches) ----
hipError_t launch_route(const uint16_t* x, const uint16_t* wr, int T, int d, int E, int k, int32_t* ids,
                        float* w, hipStream_t st);
hipError_t launch_classify(ft_cache* c, int32_t layer, int32_t* ids, int32_t R, const ft_classify_out* out,
                           hipStream_t st);
hipError_t launch_fill(ft_cache* c, hipStream_t st, TimedLaunch tl = TimedLaunch());
hipError_t launch_invalidate(ft_cache* c, int buf, hipStream_t st);
hipError_t launch_register(ft_cache* c, int layer, int buf, hipStream_t st);
hipError_t launch_resize_gather(const uint8_t* old_pool, uint8_t* new_pool, int64_t P, const int32_t* src_slots,
                                int n, hipStream_t st);
// plan: routes -> active slots, sorted rows, tiles.  slot_base >= 0 means routes
// are raw expert ids mapped to slot slot_base + e (full-layer buffer).
// `work_counter` (C_GEMV_EXPERTS or C_GEMM_EXPERTS) receives the active-slot
// count and the next counter the row count.
// With `stage`, routes, w and x of the call are also copied into the host
// branch's pinned staging.  With `fill` (R <= kSmallPlanRoutes only), the
// pending fill runs in the same launch, timed by those events.
// With `decode_hits` (and `fill`), the launch also runs the one-token decode
// kernel's workgroups for the call's GPU routes whose slots are not being
// filled (the filled ones follow in a launch of their own).
hipError_t launch_plan(ft_cache* c, const int32_t* routes, int T, int slot_base, int bm, int work_counter,
                       const float* w, const uint16_t* x, const HostStaging* stage, const HostSignal* sig,
                       hipStream_t st, const TimedLaunch* fill = nullptr, bool decode_hits = false);
hipError_t launch_gemv(ft_cache* c, const uint16_t* x, int T, hipStream_t st);
int gemv_kparts(const ft_shape& s);
hipError_t launch_gemm(ft_cache* c, const uint16_t* x, int T, hipStream_t st);
// P: the host branch's partial sums [T x d] in pinned host memory (null when
// the call has no host branch).  With a mailbox or graph-mailbox `wait`, the
// kernel itself first waits (bounded, error flag 8) for the host branch's
// answer to the call.
hipError_t launch_combine(ft_cache* c, const int32_t* routes, const float* w, int T, const float* P,
                          uint16_t* y, hipStream_t st, const HostSignal* wait = nullptr);
int gemm_tile_m();
enum { DEC_ALL = 0, DEC_HITS = 1, DEC_FILLS = 2 };   // the GPU routes a decode launch serves
// The one-token decode kernel (one launch: gate/up, SwiGLU, down partials)
// and its combine.  subset: DEC_ALL / DEC_HITS / DEC_FILLS (decode_wg.h);
// slot_base < 0: routes are classify's slot ids, else expert ids of the
// full-layer buffer starting at that slot (STREAMED, subset DEC_ALL).
int decode_groups(const ft_shape& s);          // neuron groups (workgroups per route)
bool decode_fits(const ft_shape& s);           // shapes the kernel serves
hipError_t launch_decode(ft_cache* c, const uint16_t* x, const int32_t* routes, int subset, hipStream_t st,
                         int slot_base = -1);
hipError_t launch_combine_part(ft_cache* c, const int32_t* routes, const float* w, const float* P, uint16_t* y,
                               hipStream_t st, const HostSignal* wait);
// The per-GPU static scratch: its device address is looked up once per device
// (setup: `device` current), then read back by static_scratch (null if not set up).
hipError_t static_scratch_setup(int device);
void* static_scratch(int device);
}  // namespace ftmoe
