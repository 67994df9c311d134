/*
 * ftmoe.h — C ABI of the routed-expert MoE layer with a GPU slot cache
 * (MI355X / gfx950, HIP).
 *
 * The layer follows the FreeToken pages: the full routed-expert pool lives in
 * host memory and is the source of truth; a slot cache in HBM holds complete
 * layer-expert records shared by all layers; one control kernel per layer
 * dedupes the routed experts, classifies each as a hit or a miss, derives the
 * fill count q, picks LRU victims and rewrites the routes into slot ids; the
 * expert FFN runs on the GPU for hits and fills and on host cores for the
 * remaining misses, and the two partial sums merge into the layer output.
 * Prefill instead streams whole layers through two full-layer buffers.
 *
 * Conventions shared by every call
 *  - All functions return ft_status.  On error nothing has been enqueued and
 *    ft_last_error() (thread-local) describes the problem.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    GPU step of a call is enqueued on it, except the full-layer loads of
 *    STREAMED mode (the library's transfer stream, ordered by events); only
 *    create, resize, profile, set_profile, stats, timing, snapshot, read_slot
 *    and destroy synchronise with the device.
 *  - Device pointers must be allocated on the device that created the cache.
 *  - A handle is used from one host thread at a time.
 *  - bf16 values are passed as uint16_t bit patterns.
 *  - No C++ exception crosses this boundary.
 */
#ifndef FTMOE_H
#define FTMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FT_OK = 0,
    FT_ERR_ARG = 1,          /* invalid argument or shape                       */
    FT_ERR_NOMEM = 2,        /* device or pinned allocation failed              */
    FT_ERR_HIP = 3,          /* a HIP runtime call failed                       */
    FT_ERR_STATE = 4,        /* call not valid in the cache's current state     */
    FT_ERR_UNSUPPORTED = 5   /* combination not implemented                     */
} ft_status;

/* Weight formats of a layer-expert record. */
enum {
    FT_FMT_BF16 = 0,         /* bf16 weights                                     */
    FT_FMT_FP8_B128 = 1,     /* e4m3fn codes, one fp32 scale per 128x128 block   */
    FT_FMT_MXFP4_B32 = 2     /* e2m1 codes, one e8m0 scale per 32 along K        */
};

/* Layer geometry.  d_model and d_ff must be multiples of 128, with
 * d_model <= 32768 and d_ff <= 8192. */
typedef struct {
    int32_t layers;          /* L: MoE layers held by the host bank              */
    int32_t experts;         /* E: routed experts per layer (<= 4096)            */
    int32_t top_k;           /* k: experts per token (1..E, <= 16)               */
    int32_t d_model;         /* d: hidden size                                   */
    int32_t d_ff;            /* f: expert FFN width                              */
    int32_t fmt;             /* FT_FMT_*                                         */
} ft_shape;

/* Profiled bandwidths that set the fill/host split.  q = 0 if m = 0, else
 * min(max(round_half_up(m * bp / bh), 1), m, slots - hits, cap) with
 * cap = max_fetch when max_fetch >= 0 (no cap when -1).  Derivation:
 * "Making Large MoE Models Practical on a Single Machine", section 5
 * "Deriving q*" (T_fill = qS/B_P balanced against T_cpu = (m-q)S/(B_H-B_P));
 * at-least-one-fill rule: txtmix article, q* policy paragraph. */
typedef struct {
    uint32_t bp_mbps;        /* B_P, MB/s, > 0                                   */
    uint32_t bh_mbps;        /* B_H, MB/s, > 0                                   */
    int32_t max_fetch;       /* -1 = no cap; >= 0 caps fills per call            */
} ft_profile;

typedef struct ft_cache ft_cache;

/* Unique-id classes written by ft_cache_classify. */
enum { FT_HIT = 0, FT_FILL = 1, FT_CPU = 2 };

/* Forward modes and flags. */
enum {
    FT_MODE_CACHED = 0,      /* consume routes rewritten by ft_cache_classify    */
    FT_MODE_STREAMED = 1,    /* compute from the full-layer buffer of `layer`    */
    FT_PREFETCH_NEXT = 0x100,/* STREAMED: also enqueue layer+1's load            */
    FT_SINGLE_BUFFER = 0x200,/* STREAMED: one full-layer buffer (the ablation)  */
    FT_WARM_DECODE = 0x400   /* STREAMED: the streamed layer stays resident     */
};

/* Output of one classify call: caller-owned DEVICE arrays of `capacity`
 * entries (capacity >= T * top_k).  Entries past the valid counts are left
 * unspecified ("The Expert Cache That Follows the Router", section "How
 * residency follows demand without leaving the device": fixed-size device
 * buffers with a valid count keep the dynamic miss count out of graph shapes).
 *   counts[0] n_uniq   unique flat ids (flat id = layer * E + expert)
 *   counts[1] hits
 *   counts[2] m        misses
 *   counts[3] q        fills (the first q misses in ascending flat-id order)
 *   uniq[i]            ascending unique flat ids, i < n_uniq
 *   cls[i]             FT_HIT / FT_FILL / FT_CPU of uniq[i]
 *   slot[i]            slot holding uniq[i] after the call, -1 for FT_CPU
 *   ev_slot[i], ev_old[i], ev_new[i]   i < q: the i-th fill's victim slot, the
 *                      flat id it evicted (-1 if the slot was empty) and the
 *                      flat id admitted
 *   cpu_ids[i]         i < m - q: flat ids executed on the host            */
typedef struct {
    int32_t* counts;         /* int32[4] */
    int32_t* uniq;
    uint8_t* cls;
    int32_t* slot;
    int32_t* ev_slot;
    int32_t* ev_old;
    int32_t* ev_new;
    int32_t* cpu_ids;
    int32_t capacity;
} ft_classify_out;

/* Cumulative counters (read by ft_cache_stats, which synchronises). */
typedef struct {
    uint64_t calls;          /* classify calls                                   */
    uint64_t routes;         /* routed (token, expert) pairs seen by classify    */
    uint64_t unique;         /* unique layer-experts                             */
    uint64_t hits, misses, fills, cpu_experts, evictions;
    uint64_t bytes_filled;   /* record bytes copied host -> slot by fills        */
    uint64_t layers_streamed;/* full-layer loads into the two buffers            */
    uint64_t clock;          /* LRU clock (starts at 1)                          */
    int32_t error_flags;     /* sticky device flags: 1 = expert id or route out of
                                range (ignored), 2 = LRU clock past 2^40, 4 =
                                repeated expert in a token's routes (the repeat
                                is dropped), 8 = a call gave up waiting for the
                                host experts (seconds; its output is invalid),
                                16 = a graph captured before ft_cache_resize
                                was replayed (it did nothing; output zero) */
    int32_t num_slots;
    uint64_t host_experts;   /* expert FFNs run by the host workers               */
    uint64_t host_bytes;     /* expert-record bytes the host workers read         */
    double host_seconds;     /* wall time of host-branch calls that had work      */
} ft_stats;

/* ---------------------------------------------------------------------------
 * ft_cache_create — build a cold slot cache over a host bank.
 *
 * host_bank: caller-owned PINNED host memory (ft_host_alloc, or any
 *   hipHostMalloc allocation) holding layers * experts records of
 *   ft_record_bytes() bytes, record r = layer * E + expert at offset r * S
 *   (flat-id-major banks: txtmix article, section on the FTW format; the host
 *   pool is authoritative: "The Expert Cache That Follows the Router", section
 *   "One logical expert, two physical levels of memory").  It must stay valid
 *   and unchanged until ft_cache_destroy.
 * num_slots: N complete records allocated in HBM (1..32768), one slot every
 *   ft_record_bytes() rounded up to 256 bytes (so each slot's record starts
 *   aligned; a bank record is copied into a slot whole).
 * max_tokens: largest T any later call will pass (sizes internal buffers),
 *   1..65535, with max_tokens * top_k * d_ff * 2 below 4 GiB (the expert
 *   GEMMs reach activation rows through 32-bit byte offsets).
 * Errors: FT_ERR_ARG (shape, null, N, max_tokens; a host_bank that is not
 *   pinned, or whose allocation is known to end before layers * experts
 *   records), FT_ERR_NOMEM, FT_ERR_HIP.
 * Synchronises the current device.  The host workers it starts use AVX-512
 *   (F, BW, VL, DQ and the BF16 extension) on the host CPU.
 *
 * Record layout (S bytes), matrices [rows x K] in this order:
 *   BF16       WgT [f x d] | WuT [f x d] | WdT [d x f]                  (bf16)
 *   FP8_B128   codes WgT | WuT | WdT (u8 e4m3fn), then fp32 scales
 *              sg [f/128 x d/128] | su [f/128 x d/128] | sd [d/128 x f/128]
 *   MXFP4_B32  codes WgT [f x d/2] | WuT [f x d/2] | WdT [d x f/2]
 *              (two e2m1 per byte, low nibble = even k), then e8m0 scales
 *              sg [f x d/32] | su [f x d/32] | sd [d x f/32]
 * where FFN(x) = (silu(x WgT^T) * (x WuT^T)) WdT^T.
 * Panel order: every code matrix and every e8m0 scale matrix is stored in
 * 32-row panels, panel p (rows 32p .. 32p+31) one contiguous block of
 * 32 * (row bytes); inside it, unit c of row r — 16 bytes of codes (8 bf16,
 * 16 e4m3 or 32 e2m1 values along K), or one e8m0 byte — is at unit index
 * (c / 2) * 64 + (c % 2) * 32 + (r % 32).  So 64 lanes reading 16 bytes each at
 * consecutive addresses receive one 32-row x 2-unit tile, the operand layout
 * of a 32x32 matrix-core step, and a streaming reader sees 1 KiB runs.  The
 * fp8 block scales are row-major.  d and f must be multiples of 128.
 * ------------------------------------------------------------------------- */
ft_status ft_cache_create(const ft_shape* shape, const ft_profile* profile, const void* host_bank,
                          int64_t num_slots, int32_t max_tokens, ft_cache** out);

/* ---------------------------------------------------------------------------
 * ft_cache_create_layers — ft_cache_create over one bank per layer.
 * layer_banks[l] (l < layers): PINNED host memory holding layer l's `experts`
 *   records back to back (record e at offset e * ft_record_bytes()); the
 *   table itself is copied, the banks are caller-owned and must stay valid
 *   and unchanged until ft_cache_destroy.  Entries may point to the same
 *   memory (layers that share weights); flat ids, and so residency and LRU
 *   decisions, stay per layer.  ft_cache_create(host_bank) is this call with
 *   layer_banks[l] = host_bank + l * experts * ft_record_bytes().
 * Everything else, errors included, is as ft_cache_create (FT_ERR_ARG names
 * a layer whose bank is null, not pinned, or whose allocation is known to
 * end before its E records).
 * ------------------------------------------------------------------------- */
ft_status ft_cache_create_layers(const ft_shape* shape, const ft_profile* profile, const void* const* layer_banks,
                                 int64_t num_slots, int32_t max_tokens, ft_cache** out);

/* Release every resource of the cache (synchronises).  NULL is accepted. */
ft_status ft_cache_destroy(ft_cache* cache);

/* Bytes of one layer-expert record for a shape (0 for an invalid shape). */
int64_t ft_record_bytes(const ft_shape* shape);

/* ---------------------------------------------------------------------------
 * ft_moe_route — top-k softmax routing ("Making Large MoE Models Practical on
 * a Single Machine", section 1: each token selects a few of the layer's
 * experts).
 * x  [T x d]   bf16, device, row-major
 * wr [d x E]   bf16, device, row-major (z = x wr)
 * ids [T x k]  int32, device, out: experts by logit descending, ties to the
 *              lower expert index
 * w  [T x k]   fp32, device, out: softmax over the k chosen logits
 * Logits are accumulated in fp64 from exact bf16 products.  T >= 0 (T = 0
 * enqueues nothing).  Keeps no state between calls, with one restriction: a
 * call of T <= 16 tokens passes its partial logits from its first kernel to
 * its second through one device-wide scratch area of the library, so two such
 * calls must not run at the same time (e.g. on two streams); calls on one
 * stream, and calls of more tokens, are unrestricted.  Errors: FT_ERR_ARG,
 * FT_ERR_HIP.
 * ------------------------------------------------------------------------- */
ft_status ft_moe_route(const ft_shape* shape, const uint16_t* x, const uint16_t* wr, int32_t T,
                       int32_t* ids, float* w, void* stream);

/* ---------------------------------------------------------------------------
 * ft_cache_classify — the per-layer control step ("The Expert Cache That
 * Follows the Router", section "How residency follows demand without leaving
 * the device"; hyper.ai summary, section 方法: one single-pass kernel dedupes,
 * classifies against the residency table, derives q and selects victims;
 * txtmix article, section "CUDA-graph 兼容的 LRU 缓存": one scan yields the
 * LRU candidates and the miss path takes the first q).
 * ids [T x k]  int32, device, IN: expert ids 0..E-1 of `layer`;
 *              OUT (in place): the route of each (token, j): the slot id for a
 *              hit or fill, -(1 + expert) for an expert run on the host.
 *              An id outside 0..E-1 sets error flag 1 (ft_stats) and its route
 *              becomes INT32_MIN, which ft_moe_forward ignores.
 * out          caller-owned device arrays (see ft_classify_out); may be NULL
 *              when the caller does not need them.
 * Enqueues the control kernel on `stream`; never synchronises with the host.
 * The fills it chooses (device-initiated copies of whole records from the
 * pinned host bank into the victim slots) are enqueued by the next call on the
 * cache, on that call's stream: normally the CACHED ft_moe_forward of the same
 * layer, which first stages the host branch's inputs so that the PCIe pull
 * and the host experts run at the same time; any other call (or a sync point)
 * enqueues them first on the classify's stream.
 * Policy: unique ids ascend by flat id; hits are stamped clock+r, fills
 * clock+hits+i, clock += hits+q; victims are the q smallest (stamp, slot)
 * among slots not hit by this call (empty slots have stamp 0); the i-th fill
 * takes the i-th victim; host-run misses leave residency and recency unchanged.
 * Errors: FT_ERR_ARG (layer, T outside 1..max_tokens, null ids), FT_ERR_HIP.
 * ------------------------------------------------------------------------- */
ft_status ft_cache_classify(ft_cache* cache, int32_t layer, int32_t* ids, int32_t T,
                            const ft_classify_out* out, void* stream);

/* ---------------------------------------------------------------------------
 * ft_moe_forward — the routed SwiGLU expert FFN and the weighted top-k
 * combine: y[t] = sum_j w[t,j] * FFN_{layer, e(t,j)}(x[t]), accumulated in
 * fp32, written as bf16 (expert FFN with a gate/up and a down projection read
 * from one slot record: "The Expert Cache That Follows the Router", section
 * "One logical expert, two physical levels of memory"; exact merge of the GPU
 * and host partial sums: METAL MEDIA summary, Figure 2 caption).
 * mode FT_MODE_CACHED: routes are the in-place output of the preceding
 *   ft_cache_classify for this layer.  Slot routes run on the GPU from the
 *   slot pool, after that call's fills, which this call enqueues on `stream`
 *   once the host branch's inputs are staged; -(1+e) routes (0 <= e < E) run
 *   on the library's host workers from the host bank (never from a slot,
 *   residency unchanged: same page, paragraph on the host source as
 *   fallback); the partial sums merge before the bf16 rounding.  INT32_MIN
 *   routes are skipped; any other value raises error flag 1 and is skipped.
 *   A call of more than 1,024 routes (T * top_k) needs num_slots <= 8,192
 *   (the key space of the many-route planner): FT_ERR_UNSUPPORTED otherwise.
 * mode FT_MODE_STREAMED (needs num_slots >= 2E, else FT_ERR_STATE): routes are
 *   raw expert ids 0..E-1; the layer is computed from full-layer buffer
 *   layer % 2 (slots [b*E, (b+1)*E)), loading it first on the transfer stream
 *   if it does not already hold `layer`; loading invalidates the previous
 *   owners of those slots ("The Expert Cache That Follows the Router",
 *   paragraphs on prefill buffers and on the release event and beginning
 *   fence).  With FT_PREFETCH_NEXT the load of layer+1 into the other buffer
 *   is enqueued after this layer's compute is issued, so that it overlaps it
 *   ("Making Large MoE Models Practical on a Single Machine", section 2).
 *   With FT_SINGLE_BUFFER (needs num_slots >= E) every layer uses buffer 0,
 *   so a layer's load waits for the previous layer's compute and no transfer
 *   overlaps compute: the one-buffer ablation of the txtmix article's
 *   "prefill 不是稀疏的" section (its −19/−25/−26% at 4k/8k/16k tokens).
 *   With FT_WARM_DECODE the layer's experts in the buffer become decode
 *   residents after its compute (a variant: the pages leave buffer contents
 *   volatile but note that a full-layer prefill may warm experts for the
 *   next phase, "The Expert Cache That Follows the Router", paragraph on the
 *   costs of flexibility): expert e in ascending order is registered when it
 *   is resident nowhere, at slot b*E + e with stamp clock + e; the clock
 *   then advances by E.  Reloading the buffer evicts them again.
 * x [T x d] bf16, routes [T x k] int32, w [T x k] fp32, y [T x d] bf16: device.
 * Graph capture: a decode layer step — ft_moe_route, ft_cache_classify and a
 *   CACHED ft_moe_forward on one stream — may be captured into a HIP graph
 *   and replayed, so that the step needs no host involvement beyond the
 *   graph launch ("Making Large MoE Models Practical on a Single Machine",
 *   section 10; the txtmix article's "CUDA-graph 兼容的 LRU 缓存" section:
 *   fixed-size device buffers, routing-dependent control as data).  A captured
 *   call hands its host experts to the polling host thread through the
 *   mailbox with a number drawn from a device counter (so every replay posts
 *   a new one), and a one-wave kernel polls for the answer, bounded: after a
 *   few seconds it sets error flag 8 and lets the stream go on.  With stream
 *   host functions (FTMOE_HOST_SIGNAL=callback) the host experts become a
 *   captured host function instead (its context lives until
 *   ft_cache_destroy).  A replay reads the cache's current profile (set by
 *   ft_cache_set_profile or ft_cache_profile after the capture).  A graph
 *   captured before ft_cache_resize must be captured again: replayed, each of
 *   its calls does nothing except set its routes to INT32_MIN and its output
 *   y to zero, and raises error flag 16.  A graph must not be replayed after
 *   ft_cache_destroy.  Kernel timing must be off (FT_ERR_STATE); STREAMED
 *   calls cannot be captured (FT_ERR_UNSUPPORTED).
 * Errors: FT_ERR_ARG (layer, T outside 1..max_tokens, null pointers, flags
 *   with CACHED mode), FT_ERR_STATE, FT_ERR_UNSUPPORTED, FT_ERR_HIP.  A
 *   refused call enqueues nothing and changes no state.
 * ------------------------------------------------------------------------- */
ft_status ft_moe_forward(ft_cache* cache, int32_t layer, int32_t mode, const uint16_t* x,
                         const int32_t* routes, const float* w, int32_t T, uint16_t* y, void* stream);

/* ---------------------------------------------------------------------------
 * ft_moe_forward_noalloc — ft_moe_forward in FT_MODE_CACHED for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid it): the same computation and results, with
 * the call's scratch (planner lists; at one token the decode kernel's
 * partial outputs, (f/32) k d fp32 ((f/64) for MXFP4); at 2 to 4 tokens the
 * GEMV K-part sums, h and expert outputs) taken from one static device array
 * of 16 MiB per GPU instead of the cache's buffers; the call allocates and
 * frees nothing.
 * Arguments, ordering and errors are those of ft_moe_forward with mode
 * FT_MODE_CACHED, plus: calls of more than 4 tokens, or whose scratch would
 * exceed the 16 MiB (about 2 kq T k f 4 + T k (f + d) 2 bytes, kq <= 8),
 * are refused with FT_ERR_UNSUPPORTED before anything is enqueued.  The
 * array lives from the first cache created on a GPU until the process ends
 * and keeps the last call's contents; every call on a GPU uses the same
 * array, so calls that overlap in time on one GPU (on different streams, or
 * from several caches) race: order them on one stream.
 * ------------------------------------------------------------------------- */
ft_status ft_moe_forward_noalloc(ft_cache* cache, int32_t layer, const uint16_t* x, const int32_t* routes,
                                 const float* w, int32_t T, uint16_t* y, void* stream);

/* ---------------------------------------------------------------------------
 * ft_cache_resize — rebuild the slot cache for a new slot count at a safe
 * point (METAL MEDIA summary, item 4; hyper.ai summary, section 方法: the GPU
 * expert cache is rebuilt against a revised VRAM budget without restarting).
 * The caller guarantees no work is pending on this cache.  Keeps the
 * min(new_num_slots, residents) entries with the largest stamps, packed into
 * slots 0.. in ascending old-slot order, stamps and clock unchanged; every
 * other new slot is empty.  Graphs captured before the resize are void (see
 * ft_moe_forward).  Synchronises.  Errors: FT_ERR_ARG; FT_ERR_NOMEM and
 * FT_ERR_HIP while the new pool is built (the cache is then unchanged);
 * FT_ERR_HIP from the final map writes (the device failed part-way: destroy
 * the cache).
 * ------------------------------------------------------------------------- */
ft_status ft_cache_resize(ft_cache* cache, int64_t new_num_slots);

/* ---------------------------------------------------------------------------
 * ft_cache_profile — measure this machine's B_P and B_H on the real paths
 * ("Making Large MoE Models Practical on a Single Machine", section 7: the
 * split uses measured, not nominal, bandwidths; the txtmix.com FreeToken
 * article's quick start: one bandwidth benchmark per GPU and expert format).
 * B_P: the fill kernel pulls `records` layer-0 records from the pinned host
 * bank into slots 0 .. records-1, max_tokens * k records per launch (best of
 * three passes, HIP events).  B_H: the host workers run `records` records as
 * host experts of up to max_tokens tokens per call (best of three passes
 * after a warm-up, the workers' own clock).  Each pass reads records of its own
 * (pass p: p * records + i, modulo E), so no pass is timed on data a previous
 * one left in a host cache.  Both are record bytes / time in MB/s, written to `out`
 * (max_fetch copied from the cache's profile).  Safe point: the caller
 * guarantees no work is pending on this cache.  The slots are overwritten, so
 * the cache restarts empty (every map entry absent, stamps 0, clock 1); the
 * cache's own profile is not changed (see ft_cache_set_profile).
 * records: 1 .. min(E, num_slots).  Synchronises.
 * Errors: FT_ERR_ARG, FT_ERR_HIP.
 * ------------------------------------------------------------------------- */
ft_status ft_cache_profile(ft_cache* cache, int32_t records, ft_profile* out);

/* Replace the cache's B_P / B_H / max_fetch (for example with a measured
 * profile).  Later classify calls, and replays of graphs captured earlier,
 * compute q* from it; calls already enqueued keep the profile they were
 * enqueued under (this call synchronises first).  Errors: FT_ERR_ARG,
 * FT_ERR_HIP. */
ft_status ft_cache_set_profile(ft_cache* cache, const ft_profile* profile);

/* Counters and sticky error flags (synchronises). */
ft_status ft_cache_stats(const ft_cache* cache, ft_stats* out);

/* Expert-kernel timing (measurement support).  When enabled, every
 * ft_moe_forward brackets its expert kernels, and every fill launch its
 * kernel, with HIP events on the stream the kernel runs on;
 * ft_cache_timing synchronises and returns, per kernel class (0 GEMV gate/up,
 * or at one token the decode kernel doing gate/up, SwiGLU and down in one
 * launch; 1 GEMV down, none at one token; 2 GEMM gate/up, 3 GEMM down,
 * 4 fill), the number of launches
 * and their summed event durations, plus device-side counts of the work those
 * launches did: expert records read (one per active slot per call) and GPU
 * rows (routes) computed. */
enum { FT_K_GEMV_GU = 0, FT_K_GEMV_DOWN = 1, FT_K_GEMM_GU = 2, FT_K_GEMM_DOWN = 3, FT_K_FILL = 4, FT_K_COUNT = 5 };
typedef struct {
    uint64_t launches[FT_K_COUNT];
    double ms[FT_K_COUNT];
    uint64_t gemv_experts, gemv_rows;   /* summed over GEMV-path calls */
    uint64_t gemm_experts, gemm_rows;   /* summed over GEMM-path calls */
} ft_timing;
ft_status ft_cache_set_timing(ft_cache* cache, int32_t enable);   /* also resets the totals */
ft_status ft_cache_timing(const ft_cache* cache, ft_timing* out);

/* Copy the maps to host memory (synchronises): slot_for_id [L*E],
 * id_of_slot [N], stamp [N]; any pointer may be NULL. */
ft_status ft_cache_snapshot(const ft_cache* cache, int32_t* slot_for_id, int32_t* id_of_slot,
                            uint64_t* stamp, uint64_t* clock);

/* Copy slot `slot`'s S record bytes to host memory `dst` (synchronises). */
ft_status ft_cache_read_slot(const ft_cache* cache, int64_t slot, void* dst);

/* Pinned, device-mapped host memory for host banks (hipHostMalloc).  Banks
 * larger than torch's power-of-two pinned allocator can serve come from here. */
ft_status ft_host_alloc(size_t bytes, void** ptr);
ft_status ft_host_free(void* ptr);

/* Description of the last error on the calling thread ("" if none). */
const char* ft_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FTMOE_H */
