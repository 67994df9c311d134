// The C ABI of the routed-expert MoE layer (include/ftmoe.h): argument
// validation, resource ownership, stream/event ordering, and the calls that
// enqueue the kernels.  No C++ exception crosses the boundary.
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "common.h"

namespace ftmoe {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

void clear_error() { g_err[0] = 0; }

static bool record_layout_packed(const ft_shape& s, RecordLayout* o) {
    const int64_t d = s.d_model, f = s.d_ff, fd = d * f;
    if (d <= 0 || f <= 0 || d % 128 || f % 128 || d > 32768 || f > 8192) return false;
    switch (s.fmt) {
        case FT_FMT_BF16:
            o->off_gate = 0;
            o->off_up = 2 * fd;
            o->off_down = 4 * fd;
            o->off_sg = o->off_su = o->off_sd = 0;
            o->S = 6 * fd;
            return true;
        case FT_FMT_FP8_B128: {
            const int64_t nb = (d / 128) * (f / 128);
            o->off_gate = 0;
            o->off_up = fd;
            o->off_down = 2 * fd;
            o->off_sg = 3 * fd;
            o->off_su = 3 * fd + 4 * nb;
            o->off_sd = 3 * fd + 8 * nb;
            o->S = 3 * fd + 12 * nb;
            return true;
        }
        case FT_FMT_MXFP4_B32: {
            const int64_t cb = fd / 2, sb = fd / 32;
            o->off_gate = 0;
            o->off_up = cb;
            o->off_down = 2 * cb;
            o->off_sg = 3 * cb;
            o->off_su = 3 * cb + sb;
            o->off_sd = 3 * cb + 2 * sb;
            o->S = 3 * cb + 3 * sb;
            return true;
        }
    }
    return false;
}

bool record_layout(const ft_shape& s, RecordLayout* o) {
    if (!record_layout_packed(s, o)) return false;
    o->P = (o->S + 255) & ~(int64_t)255;
    return true;
}

// ---- expert-kernel timing: a ring of event pairs, folded into totals when a
// pair is reused or read
struct Timing {
    static constexpr int kRing = 4096;
    hipEvent_t ev[kRing][2];
    int cls[kRing];
    bool live[kRing];
    int next = 0;
    uint64_t launches[FT_K_COUNT] = {};
    double ms[FT_K_COUNT] = {};
    bool ok = true;
};

static void fold(Timing* t, int i) {
    if (!t->live[i]) return;
    float msec = 0.f;
    if (hipEventSynchronize(t->ev[i][1]) == hipSuccess && hipEventElapsedTime(&msec, t->ev[i][0], t->ev[i][1]) == hipSuccess) {
        t->ms[t->cls[i]] += msec;
        t->launches[t->cls[i]] += 1;
    }
    t->live[i] = false;
}

Timing* timing_create() {
    auto* t = new Timing();
    for (int i = 0; i < Timing::kRing; ++i) {
        t->live[i] = false;
        if (hipEventCreate(&t->ev[i][0]) != hipSuccess || hipEventCreate(&t->ev[i][1]) != hipSuccess) t->ok = false;
    }
    return t;
}

void timing_destroy(Timing* t) {
    if (!t) return;
    for (int i = 0; i < Timing::kRing; ++i) {
        (void)hipEventDestroy(t->ev[i][0]);
        (void)hipEventDestroy(t->ev[i][1]);
    }
    delete t;
}

TimedLaunch timing_launch(Timing* t, int cls) {
    TimedLaunch tl;
    if (!t) return tl;
    const int i = t->next;
    t->next = (t->next + 1) % Timing::kRing;
    fold(t, i);     // the pair used kRing launches ago has long completed
    t->cls[i] = cls;
    t->live[i] = true;
    tl.start = t->ev[i][0];
    tl.stop = t->ev[i][1];
    return tl;
}

void timing_read(Timing* t, uint64_t* launches, double* ms) {
    for (int i = 0; i < Timing::kRing; ++i) fold(t, i);
    for (int k = 0; k < FT_K_COUNT; ++k) {
        launches[k] = t->launches[k];
        ms[k] = t->ms[k];
    }
}

namespace {

ft_status flush_fill(ft_cache* c, hipStream_t st);

template <typename T>
hipError_t dalloc(T** p, size_t n) {
    return hipMalloc(reinterpret_cast<void**>(p), n * sizeof(T) + 256);
}

constexpr int64_t kDecodePartMaxBytes = 256ll << 20;   // partial outputs of the one-token decode kernel

ft_status check_shape(const ft_shape* s) {
    FT_REQUIRE(s, "shape is null");
    FT_REQUIRE(s->layers >= 1, "layers must be >= 1");
    FT_REQUIRE(s->experts >= 1 && s->experts <= kMaxExperts, "experts must be in 1..%d", kMaxExperts);
    FT_REQUIRE(s->top_k >= 1 && s->top_k <= kMaxTopK && s->top_k <= s->experts, "top_k must be in 1..min(E, %d)",
               kMaxTopK);
    FT_REQUIRE((int64_t)s->layers * s->experts < (1ll << 31), "layers * experts too large");
    RecordLayout rl;
    FT_REQUIRE(record_layout(*s, &rl), "d_model and d_ff must be positive multiples of 128 and fmt valid");
    return FT_OK;
}

void free_cache(ft_cache* c) {
    if (!c) return;
    if (c->fill_pending) (void)flush_fill(c, c->fill_stream);
    (void)hipDeviceSynchronize();
    if (c->host) host_branch_destroy(c->host);
    if (c->timing) timing_destroy(c->timing);
    void* bufs[] = {c->pool, c->slot_for_id, c->id_of_slot, c->stamp, c->clock, c->counters, c->errflag, c->gseq_dev,
                    c->dstate,
                    c->wl_counts, c->wl_slot, c->wl_src, c->plan.meta, c->plan.active_slot, c->plan.seg,
                    c->plan.perm, c->plan.route_pos, c->plan.tile_active, c->plan.tile_row0, c->plan.tile_first,
                    c->plan.chunk_counts, c->H, c->Y, c->gv_part, c->bank_dev, c->dpart};
    for (void* b : bufs)
        if (b) (void)hipFree(b);
    hipEvent_t evs[] = {c->ev_ctrl, c->ev_fwd, c->ev_host, c->ev_xlast, c->ev_fence,
                        c->ready[0], c->ready[1], c->release[0], c->release[1]};
    for (hipEvent_t e : evs)
        if (e) (void)hipEventDestroy(e);
    if (c->xfer) (void)hipStreamDestroy(c->xfer);
    if (c->hstream) (void)hipStreamDestroy(c->hstream);
    delete[] c->bank_host;
    delete c;
}

// The planner's tile lists and chunk counts, sized for any slot count (a call
// has at most one active slot per route), so that resize never reallocates
// buffers a captured call may hold.
hipError_t alloc_plan(ft_cache* c) {
    const int64_t cap = c->cap;
    c->plan.max_tiles = (cap + gemm_tile_m() - 1) / gemm_tile_m() + cap + 1;
    const int64_t chunks = (c->max_tokens + kChunkTokens - 1) / kChunkTokens;
    hipError_t e;
    if ((e = dalloc(&c->plan.tile_active, c->plan.max_tiles))) return e;
    if ((e = dalloc(&c->plan.tile_row0, c->plan.max_tiles))) return e;
    if ((e = dalloc(&c->plan.tile_first, cap + 1))) return e;
    if ((e = dalloc(&c->plan.chunk_counts, chunks * kLargeKeySpace))) return e;
    return hipSuccess;
}

// Write the profile and pool generation the kernels read at run time.
hipError_t write_dstate(ft_cache* c) {
    DevState ds{c->gen, c->prof.bp_mbps, c->prof.bh_mbps, c->prof.max_fetch};
    return hipMemcpy(c->dstate, &ds, sizeof(ds), hipMemcpyHostToDevice);
}

// Enqueue the fills chosen by the last classify (if not yet enqueued) on `st`.
// Classify leaves them pending so that forward can first stage the host
// branch's inputs: the copy over PCIe and the host experts then run together.
// Every later call on the cache flushes a pending fill before it can read a slot.
ft_status flush_fill(ft_cache* c, hipStream_t st) {
    if (!c->fill_pending) return FT_OK;
    FT_HIP(launch_fill(c, st, timing_launch(c->timing, FT_K_FILL)));
    c->fill_pending = false;
    return FT_OK;
}

// Flush on the stream of the classify that chose the fills (sync points).
ft_status flush_fill_sync(ft_cache* c) {
    ft_status s = flush_fill(c, c->fill_stream);
    if (s != FT_OK) return s;
    FT_HIP(hipDeviceSynchronize());
    return FT_OK;
}

ft_status enqueue_load(ft_cache* c, int layer, int buf, hipStream_t st) {
    // the buffer's previous layer must be done; the first load after decode
    // work waits for everything already on the caller's stream (beginning fence)
    if (!c->streaming) {
        FT_HIP(hipEventRecord(c->ev_fence, st));
        FT_HIP(hipStreamWaitEvent(c->xfer, c->ev_fence, 0));
        c->streaming = true;
    }
    if (c->release_recorded[buf]) FT_HIP(hipStreamWaitEvent(c->xfer, c->release[buf], 0));
    FT_HIP(launch_invalidate(c, buf, c->xfer));
    const int64_t E = c->sh.experts, S = c->rl.S, P = c->rl.P;
    if (P == S) {
        FT_HIP(hipMemcpyAsync(c->pool + (int64_t)buf * E * P, c->bank_host[layer], E * S,
                              hipMemcpyHostToDevice, c->xfer));
    } else {   // records of S bytes into slots P bytes apart
        FT_HIP(hipMemcpy2DAsync(c->pool + (int64_t)buf * E * P, (size_t)P, c->bank_host[layer],
                                (size_t)S, (size_t)S, (size_t)E, hipMemcpyHostToDevice, c->xfer));
    }
    FT_HIP(hipEventRecord(c->ready[buf], c->xfer));
    FT_HIP(hipEventRecord(c->ev_xlast, c->xfer));
    c->xfer_pending = true;
    c->buf_layer[buf] = layer;
    return FT_OK;
}

// A CACHED call: host-branch staging, the pending fills, the planner, the GPU
// experts and the combine.  `c` holds the cache's state; `bufs` supplies the
// per-call scratch the kernels use (planner lists, GEMV K-part sums, h, expert
// outputs): the cache itself, or a view of it over the static scratch.
ft_status forward_cached(ft_cache* c, ft_cache* bufs, int32_t layer, const uint16_t* x, const int32_t* routes,
                         const float* w, int32_t T, uint16_t* y, hipStream_t st, bool capturing) {
    const int k = c->sh.top_k;
    const bool gemv = T <= kGemvMaxTokens;
    // one token: the one-launch decode kernel (gate/up, SwiGLU, down partials)
    const bool fused = T == 1 && bufs->dpart != nullptr;
    if ((int64_t)T * k > kSmallPlanRoutes && c->N > kLargeKeySpace) {
        set_error("a CACHED call of more than %d routes needs num_slots <= %d (the chunked planner's key space)",
                  kSmallPlanRoutes, kLargeKeySpace);
        return FT_ERR_UNSUPPORTED;
    }
    // host branch: the planner copies the call's routes, weights and
    // activations into pinned staging and, with the mailbox, posts the
    // call's sequence number; the host workers run the host experts and
    // leave their partial sums in pinned memory.  A call being captured
    // into a graph posts to the mailbox's graph words instead, numbered by
    // a device counter so that every replay posts a new number; the
    // combine kernel waits for the answer (bounded).  Without a poller,
    // it uses a captured host function.
    HostStaging hs = host_branch_staging(c->host);
    HostSignal sig = capturing ? host_branch_graph_signal(c->host, c->gseq_dev, layer, T)
                               : host_branch_prepare(c->host, layer, T);
    // with a mailbox, this call's pending fill rides in the planner's
    // launch (a host function, in contrast, must follow the staging at once)
    const bool plan_fill =
        c->fill_pending && (sig.mailbox || sig.gmbox) && (int64_t)T * k <= kSmallPlanRoutes;
    const TimedLaunch ftl = plan_fill ? timing_launch(c->timing, FT_K_FILL) : TimedLaunch();
    // the hit experts' decode workgroups ride in that launch too, beside the
    // pull (with kernel timing on they run in the decode launch, so that its
    // events time every GPU expert)
    const bool hits_in_fill = fused && plan_fill && !c->timing;
    FT_HIP(launch_plan(bufs, routes, T, -1, gemm_tile_m(), gemv ? C_GEMV_EXPERTS : C_GEMM_EXPERTS, w, x, &hs, &sig,
                       st, plan_fill ? &ftl : nullptr, hits_in_fill));
    if (plan_fill) c->fill_pending = false;
    if (!sig.mailbox && !sig.gmbox) {
        FT_HIP(hipEventRecord(c->ev_fwd, st));
        FT_HIP(hipStreamWaitEvent(c->hstream, c->ev_fwd, 0));
        FT_HIP(capturing ? host_branch_enqueue_captured(c->host, layer, T, c->hstream)
                         : host_branch_enqueue(c->host, layer, T, c->hstream));
        FT_HIP(hipEventRecord(c->ev_host, c->hstream));
    }
    // this layer's fills, then the GPU experts (hits and fills) from the slot pool
    ft_status fs = flush_fill(c, st);
    if (fs != FT_OK) return fs;
    if (c->xfer_pending) FT_HIP(hipStreamWaitEvent(st, c->ev_xlast, 0));
    if (fused)
        FT_HIP(launch_decode(bufs, x, routes, hits_in_fill ? DEC_FILLS : DEC_ALL, st));
    else
        FT_HIP(gemv ? launch_gemv(bufs, x, T, st) : launch_gemm(bufs, x, T, st));
    // the combine waits for the host branch's answer itself (a stream wait
    // packet costs ~4.5 us even when the answer is already there); with
    // a host function, the stream waits for its event
    if (!sig.mailbox && !sig.gmbox) FT_HIP(hipStreamWaitEvent(st, c->ev_host, 0));
    FT_HIP(fused ? launch_combine_part(bufs, routes, w, hs.P, y, st, &sig)
                 : launch_combine(bufs, routes, w, T, hs.P, y, st, &sig));
    return FT_OK;
}

}  // namespace
}  // namespace ftmoe

using namespace ftmoe;

extern "C" {

const char* ft_last_error(void) { return g_err; }

int64_t ft_record_bytes(const ft_shape* shape) {
    RecordLayout rl;
    if (!shape || !record_layout(*shape, &rl)) return 0;
    return rl.S;
}

ft_status ft_host_alloc(size_t bytes, void** ptr) {
    clear_error();
    FT_REQUIRE(ptr && bytes > 0, "ptr must be non-null and bytes > 0");
    hipError_t e = hipHostMalloc(ptr, bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
        set_error("hipHostMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
        *ptr = nullptr;
        return FT_ERR_NOMEM;
    }
    return FT_OK;
}

ft_status ft_host_free(void* ptr) {
    clear_error();
    if (ptr) FT_HIP(hipHostFree(ptr));
    return FT_OK;
}

ft_status ft_cache_create_layers(const ft_shape* shape, const ft_profile* profile, const void* const* layer_banks,
                                 int64_t num_slots, int32_t max_tokens, ft_cache** out) {
    clear_error();
    FT_REQUIRE(out, "out is null");
    *out = nullptr;
    ft_status st = check_shape(shape);
    if (st != FT_OK) return st;
    FT_REQUIRE(profile && profile->bp_mbps > 0 && profile->bh_mbps > 0, "profile bandwidths must be > 0");
    FT_REQUIRE(profile->max_fetch >= -1, "max_fetch must be >= -1");
    FT_REQUIRE(layer_banks, "layer bank table is null");
    for (int32_t l = 0; l < shape->layers; ++l) FT_REQUIRE(layer_banks[l], "bank of layer %d is null", l);
    FT_REQUIRE(num_slots >= 1 && num_slots <= kMaxSlots, "num_slots must be in 1..%d", kMaxSlots);
    FT_REQUIRE(max_tokens >= 1 && max_tokens <= 65535, "max_tokens must be in 1..65535");
    FT_REQUIRE((int64_t)max_tokens * shape->top_k <= (1 << 24), "max_tokens * top_k too large");
    FT_REQUIRE((int64_t)max_tokens * shape->top_k * shape->d_ff * 2 <= 0xFFFFFFFFll,
               "max_tokens * top_k * d_ff * 2 must be below 4 GiB");

    ft_cache* c = new (std::nothrow) ft_cache();
    if (!c) return FT_ERR_NOMEM;
    memset(c, 0, sizeof(*c));
    c->sh = *shape;
    c->prof = *profile;
    record_layout(*shape, &c->rl);
    c->N = num_slots;
    c->max_tokens = max_tokens;
    c->cap = max_tokens * shape->top_k;
    c->buf_layer[0] = c->buf_layer[1] = -1;
#define CK(call)                                                                             \
    do {                                                                                     \
        hipError_t e_ = (call);                                                              \
        if (e_ != hipSuccess) {                                                              \
            set_error("%s failed: %s", #call, hipGetErrorString(e_));                        \
            free_cache(c);                                                                   \
            return e_ == hipErrorOutOfMemory ? FT_ERR_NOMEM : FT_ERR_HIP;                    \
        }                                                                                    \
    } while (0)
    CK(hipGetDevice(&c->device));
    CK(static_scratch_setup(c->device));      // ft_moe_forward_noalloc's array on this device
    const int64_t L = shape->layers, E = shape->experts, S = c->rl.S, d = shape->d_model, f = shape->d_ff;
    c->bank_host = new (std::nothrow) const uint8_t*[L];
    if (!c->bank_host) {
        free_cache(c);
        return FT_ERR_NOMEM;
    }
    std::vector<const uint8_t*> dev_banks(L);
    for (int64_t l = 0; l < L; ++l) {
        void* hp = const_cast<void*>(layer_banks[l]);
        void* dptr = nullptr;
        if (hipHostGetDevicePointer(&dptr, hp, 0) != hipSuccess || !dptr) {
            (void)hipGetLastError();
            free_cache(c);
            set_error("bank of layer %lld must be pinned host memory (ft_host_alloc / hipHostMalloc)", (long long)l);
            return FT_ERR_ARG;
        }
        // Where the runtime knows the bank's allocation (hipHostMalloc memory),
        // it must hold the layer's E records: fills and layer loads read the
        // bank from the device, where a short bank faults.
        hipDeviceptr_t base = nullptr;
        size_t size = 0;
        if (hipMemGetAddressRange(&base, &size, hp) == hipSuccess && base && size) {
            const int64_t avail =
                (int64_t)(static_cast<const uint8_t*>(base) + size - static_cast<const uint8_t*>(hp));
            if (avail < E * S) {
                free_cache(c);
                set_error("bank of layer %lld: its allocation holds %lld bytes from the pointer; %lld records need "
                          "%lld", (long long)l, (long long)avail, (long long)E, (long long)(E * S));
                return FT_ERR_ARG;
            }
        } else {
            (void)hipGetLastError();   // an untracked pointer: no check, and no stale error left behind
        }
        c->bank_host[l] = static_cast<const uint8_t*>(hp);
        dev_banks[l] = static_cast<const uint8_t*>(dptr);
    }
    CK(dalloc(&c->bank_dev, L));
    CK(hipMemcpy(c->bank_dev, dev_banks.data(), sizeof(const uint8_t*) * L, hipMemcpyHostToDevice));
    const int64_t cap = c->cap;
    CK(hipMalloc(reinterpret_cast<void**>(&c->pool), (size_t)(c->N * c->rl.P)));
    CK(dalloc(&c->slot_for_id, L * E));
    CK(dalloc(&c->id_of_slot, kMaxSlots));
    CK(dalloc(&c->stamp, kMaxSlots));
    CK(dalloc(&c->dstate, 1));
    CK(dalloc(&c->clock, 1));
    CK(dalloc(&c->counters, C_N));
    CK(dalloc(&c->errflag, 1));
    CK(dalloc(&c->gseq_dev, 1));
    CK(dalloc(&c->wl_counts, 4));
    CK(dalloc(&c->wl_slot, cap));
    CK(dalloc(&c->wl_src, cap));
    CK(dalloc(&c->plan.meta, 4));
    CK(dalloc(&c->plan.active_slot, cap));
    CK(dalloc(&c->plan.seg, cap + 1));
    CK(dalloc(&c->plan.perm, cap));
    CK(dalloc(&c->plan.route_pos, cap));
    CK(alloc_plan(c));
    CK(dalloc(&c->H, cap * f));
    CK(dalloc(&c->Y, cap * d));
    c->cap_gemv = std::min<int32_t>(max_tokens, kGemvMaxTokens) * shape->top_k;
    c->gv_kq = gemv_kparts(*shape);
    CK(dalloc(&c->gv_part, 2ll * c->gv_kq * c->cap_gemv * f));
    // the one-token decode kernel's partial outputs (shapes it serves)
    if (decode_fits(*shape) && decode_groups(*shape) <= 64 &&
        (int64_t)decode_groups(*shape) * shape->top_k * d * 4 <= kDecodePartMaxBytes)
        CK(dalloc(&c->dpart, (int64_t)decode_groups(*shape) * shape->top_k * d));
    // seconds of polls, each a PCIe read: far beyond any host call (a test
    // lowers it to force the time-out path)
    c->host_wait_polls = 1u << 22;
    if (const char* e = getenv("FTMOE_HOST_WAIT_POLLS")) c->host_wait_polls = (uint32_t)strtoul(e, nullptr, 10);
    CK(hipMemset(c->slot_for_id, 0xFF, sizeof(int32_t) * L * E));
    CK(hipMemset(c->id_of_slot, 0xFF, sizeof(int32_t) * kMaxSlots));
    CK(hipMemset(c->stamp, 0, sizeof(uint64_t) * kMaxSlots));
    CK(write_dstate(c));
    const uint64_t one = 1;
    CK(hipMemcpy(c->clock, &one, sizeof(one), hipMemcpyHostToDevice));
    CK(hipMemset(c->counters, 0, sizeof(unsigned long long) * C_N));
    CK(hipMemset(c->errflag, 0, sizeof(int32_t)));
    CK(hipMemset(c->gseq_dev, 0, sizeof(uint64_t)));
    CK(hipMemset(c->plan.meta, 0, sizeof(int32_t) * 4));
    CK(hipStreamCreateWithFlags(&c->xfer, hipStreamNonBlocking));
    CK(hipStreamCreateWithFlags(&c->hstream, hipStreamNonBlocking));
    hipEvent_t* evs[] = {&c->ev_ctrl, &c->ev_fwd, &c->ev_host, &c->ev_xlast, &c->ev_fence,
                         &c->ready[0], &c->ready[1], &c->release[0], &c->release[1]};
    for (hipEvent_t* e : evs) CK(hipEventCreateWithFlags(e, hipEventDisableTiming));
    CK(hipDeviceSynchronize());
#undef CK
    c->host = host_branch_create(*shape, c->rl, c->bank_host, max_tokens);
    if (!c->host) {
        free_cache(c);
        set_error("host branch: pinned staging allocation failed");
        return FT_ERR_NOMEM;
    }
    *out = c;
    return FT_OK;
}

ft_status ft_cache_create(const ft_shape* shape, const ft_profile* profile, const void* host_bank,
                          int64_t num_slots, int32_t max_tokens, ft_cache** out) {
    clear_error();
    FT_REQUIRE(out, "out is null");
    *out = nullptr;
    ft_status st = check_shape(shape);
    if (st != FT_OK) return st;
    FT_REQUIRE(host_bank, "host bank is null");
    const int64_t stride = (int64_t)shape->experts * ft_record_bytes(shape);
    std::vector<const void*> layers(shape->layers);
    for (int32_t l = 0; l < shape->layers; ++l) layers[l] = static_cast<const uint8_t*>(host_bank) + l * stride;
    return ft_cache_create_layers(shape, profile, layers.data(), num_slots, max_tokens, out);
}

ft_status ft_cache_destroy(ft_cache* cache) {
    clear_error();
    free_cache(cache);
    return FT_OK;
}

ft_status ft_moe_route(const ft_shape* shape, const uint16_t* x, const uint16_t* wr, int32_t T, int32_t* ids,
                       float* w, void* stream) {
    clear_error();
    FT_REQUIRE(shape, "shape is null");
    FT_REQUIRE(shape->experts >= 1 && shape->experts <= 256, "routing supports 1..256 experts");
    FT_REQUIRE(shape->top_k >= 1 && shape->top_k <= shape->experts && shape->top_k <= kMaxTopK, "bad top_k");
    FT_REQUIRE(shape->d_model >= 1, "bad d_model");
    FT_REQUIRE(T >= 0, "T must be >= 0");
    if (T == 0) return FT_OK;
    FT_REQUIRE(x && wr && ids && w, "null pointer");
    FT_HIP(launch_route(x, wr, T, shape->d_model, shape->experts, shape->top_k, ids, w, (hipStream_t)stream));
    return FT_OK;
}

ft_status ft_cache_classify(ft_cache* c, int32_t layer, int32_t* ids, int32_t T, const ft_classify_out* out,
                            void* stream) {
    clear_error();
    FT_REQUIRE(c, "cache is null");
    FT_REQUIRE(layer >= 0 && layer < c->sh.layers, "layer %d out of range", layer);
    FT_REQUIRE(T >= 1 && T <= c->max_tokens, "T must be in 1..max_tokens (%d)", c->max_tokens);
    FT_REQUIRE(ids, "ids is null");
    if (out) {
        FT_REQUIRE(out->counts, "out->counts is null");
        FT_REQUIRE(out->capacity >= T * c->sh.top_k, "out capacity %d < T*k", out->capacity);
    }
    hipStream_t st = (hipStream_t)stream;
    // fills of a previous classify that no forward consumed, and full-layer
    // loads, land before this call reads the maps
    ft_status fs = flush_fill(c, st);
    if (fs != FT_OK) return fs;
    if (c->xfer_pending) FT_HIP(hipStreamWaitEvent(st, c->ev_xlast, 0));
    c->streaming = false;
    c->buf_layer[0] = c->buf_layer[1] = -1;     // decode fills may reuse buffer slots
    FT_HIP(launch_classify(c, layer, ids, T * c->sh.top_k, out, st));
    c->fill_pending = true;
    c->fill_stream = st;
    return FT_OK;
}

ft_status ft_moe_forward(ft_cache* c, int32_t layer, int32_t mode, const uint16_t* x, const int32_t* routes,
                         const float* w, int32_t T, uint16_t* y, void* stream) {
    clear_error();
    FT_REQUIRE(c, "cache is null");
    FT_REQUIRE(layer >= 0 && layer < c->sh.layers, "layer %d out of range", layer);
    FT_REQUIRE(T >= 1 && T <= c->max_tokens, "T must be in 1..max_tokens (%d)", c->max_tokens);
    FT_REQUIRE(x && routes && w && y, "null pointer");
    const int m = mode & 0xFF;
    FT_REQUIRE(m == FT_MODE_CACHED || m == FT_MODE_STREAMED, "unknown mode %d", m);
    FT_REQUIRE((mode & ~(0xFF | FT_PREFETCH_NEXT | FT_SINGLE_BUFFER | FT_WARM_DECODE)) == 0, "unknown flags");
    FT_REQUIRE(m == FT_MODE_STREAMED || (mode & ~0xFF) == 0, "flags apply to STREAMED mode only");
    hipStream_t st = (hipStream_t)stream;
    const int k = c->sh.top_k;
    const int64_t d = c->sh.d_model;
    const bool gemv = T <= kGemvMaxTokens;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    FT_HIP(hipStreamIsCapturing(st, &cap));
    const bool capturing = cap != hipStreamCaptureStatusNone;
    if (capturing && c->timing) {
        set_error("kernel timing must be off while a call is captured into a graph");
        return FT_ERR_STATE;
    }
    if (m == FT_MODE_CACHED) return forward_cached(c, c, layer, x, routes, w, T, y, st, capturing);
    if (capturing) {
        set_error("STREAMED calls cannot be captured into a graph (their loads follow host-side buffer state)");
        return FT_ERR_UNSUPPORTED;
    }
    // STREAMED: full-layer buffer layer % 2 (buffer 0 for every layer with
    // FT_SINGLE_BUFFER, whose loads then wait for the previous layer's compute)
    ft_status fs = flush_fill(c, st);
    if (fs != FT_OK) return fs;
    const int E = c->sh.experts;
    const bool single = (mode & FT_SINGLE_BUFFER) != 0;
    const int64_t need = single ? (int64_t)E : 2 * (int64_t)E;
    if (c->N < need) {
        set_error("STREAMED mode needs num_slots >= %lld (%lld slots)", (long long)need, (long long)c->N);
        return FT_ERR_STATE;
    }
    const int b = single ? 0 : layer % 2;
    if (c->buf_layer[b] != layer) {
        ft_status s = enqueue_load(c, layer, b, st);
        if (s != FT_OK) return s;
    }
    FT_HIP(hipStreamWaitEvent(st, c->ready[b], 0));
    FT_HIP(launch_plan(c, routes, T, b * E, gemm_tile_m(), gemv ? C_GEMV_EXPERTS : C_GEMM_EXPERTS, w, x, nullptr,
                       nullptr, st));
    if (T == 1 && c->dpart) {
        // one token: the decode kernel over the buffer's records, then the
        // combine of its partial outputs (the planner's route positions
        // tell which routes it ran)
        FT_HIP(launch_decode(c, x, routes, DEC_ALL, st, (int)(b * E)));
        FT_HIP(launch_combine_part(c, routes, w, nullptr, y, st, nullptr));
    } else {
        FT_HIP(gemv ? launch_gemv(c, x, T, st) : launch_gemm(c, x, T, st));
        FT_HIP(launch_combine(c, routes, w, T, nullptr, y, st));
    }
    if (mode & FT_WARM_DECODE) FT_HIP(launch_register(c, layer, b, st));
    FT_HIP(hipEventRecord(c->release[b], st));
    c->release_recorded[b] = true;
    if ((mode & FT_PREFETCH_NEXT) && layer + 1 < c->sh.layers) {
        const int nb = single ? 0 : (layer + 1) % 2;
        if (c->buf_layer[nb] != layer + 1) {
            ft_status s = enqueue_load(c, layer + 1, nb, st);
            if (s != FT_OK) return s;
        }
    }
    return FT_OK;
}

ft_status ft_moe_forward_noalloc(ft_cache* c, int32_t layer, const uint16_t* x, const int32_t* routes, const float* w,
                                 int32_t T, uint16_t* y, void* stream) {
    clear_error();
    FT_REQUIRE(c, "cache is null");
    FT_REQUIRE(layer >= 0 && layer < c->sh.layers, "layer %d out of range", layer);
    FT_REQUIRE(T >= 1 && T <= c->max_tokens, "T must be in 1..max_tokens (%d)", c->max_tokens);
    FT_REQUIRE(x && routes && w && y, "null pointer");
    if (T > kGemvMaxTokens) {
        set_error("ft_moe_forward_noalloc serves calls of at most %d tokens", kGemvMaxTokens);
        return FT_ERR_UNSUPPORTED;
    }
    uint8_t* base = static_cast<uint8_t*>(static_scratch(c->device));
    if (!base) {
        set_error("the static scratch of device %d is not set up", c->device);
        return FT_ERR_STATE;
    }
    // the call's scratch, carved from the static array (256-byte aligned pieces)
    const int64_t R = (int64_t)T * c->sh.top_k, d = c->sh.d_model, f = c->sh.d_ff;
    size_t off = 0;
    auto take = [&](int64_t bytes) {
        uint8_t* p = base + off;
        off = (off + (size_t)bytes + 255) & ~(size_t)255;
        return p;
    };
    ft_cache v = *c;
    v.plan.meta = reinterpret_cast<int32_t*>(take(4 * sizeof(int32_t)));
    v.plan.active_slot = reinterpret_cast<int32_t*>(take(R * sizeof(int32_t)));
    v.plan.seg = reinterpret_cast<int32_t*>(take((R + 1) * sizeof(int32_t)));
    v.plan.perm = reinterpret_cast<int32_t*>(take(R * sizeof(int32_t)));
    v.plan.route_pos = reinterpret_cast<int32_t*>(take(R * sizeof(int32_t)));
    v.plan.max_tiles = R + 2;                 // one tile per active slot on the GEMV path
    v.plan.tile_active = reinterpret_cast<int32_t*>(take(v.plan.max_tiles * sizeof(int32_t)));
    v.plan.tile_row0 = reinterpret_cast<int32_t*>(take(v.plan.max_tiles * sizeof(int32_t)));
    v.plan.tile_first = reinterpret_cast<int32_t*>(take((R + 1) * sizeof(int32_t)));
    v.plan.chunk_counts = nullptr;            // the one-workgroup planner only (R <= 64)
    v.cap_gemv = (int32_t)R;
    if (T == 1 && c->dpart) {        // the one-token decode kernel: its partial outputs only
        v.dpart = reinterpret_cast<float*>(take((int64_t)decode_groups(c->sh) * R * d * sizeof(float)));
        v.gv_part = nullptr;
        v.H = v.Y = nullptr;
    } else {                         // the two-kernel GEMV
        v.dpart = nullptr;
        v.gv_part = reinterpret_cast<float*>(take(2ll * c->gv_kq * R * f * sizeof(float)));
        v.H = reinterpret_cast<uint16_t*>(take(R * f * sizeof(uint16_t)));
        v.Y = reinterpret_cast<uint16_t*>(take(R * d * sizeof(uint16_t)));
    }
    if (off > kStaticScratchBytes) {
        set_error("this call needs %zu bytes of scratch; the static scratch holds %zu", off, kStaticScratchBytes);
        return FT_ERR_UNSUPPORTED;
    }
    hipStream_t st = (hipStream_t)stream;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    FT_HIP(hipStreamIsCapturing(st, &cap));
    const bool capturing = cap != hipStreamCaptureStatusNone;
    if (capturing && c->timing) {
        set_error("kernel timing must be off while a call is captured into a graph");
        return FT_ERR_STATE;
    }
    return forward_cached(c, &v, layer, x, routes, w, T, y, st, capturing);
}

ft_status ft_cache_resize(ft_cache* c, int64_t new_num_slots) {
    clear_error();
    FT_REQUIRE(c, "cache is null");
    FT_REQUIRE(new_num_slots >= 1 && new_num_slots <= kMaxSlots, "num_slots must be in 1..%d", kMaxSlots);
    ft_status fs = flush_fill_sync(c);
    if (fs != FT_OK) return fs;
    const int64_t L = c->sh.layers, E = c->sh.experts, N = c->N, Nn = new_num_slots;
    std::vector<int32_t> ios(N);
    std::vector<uint64_t> stamp(N);
    FT_HIP(hipMemcpy(ios.data(), c->id_of_slot, sizeof(int32_t) * N, hipMemcpyDeviceToHost));
    FT_HIP(hipMemcpy(stamp.data(), c->stamp, sizeof(uint64_t) * N, hipMemcpyDeviceToHost));
    // the min(Nn, residents) most recent residents, in ascending old-slot order
    std::vector<int32_t> res;
    for (int64_t s = 0; s < N; ++s)
        if (ios[s] >= 0) res.push_back((int32_t)s);
    std::stable_sort(res.begin(), res.end(), [&](int32_t a, int32_t b) { return stamp[a] > stamp[b]; });
    if ((int64_t)res.size() > Nn) res.resize(Nn);
    std::sort(res.begin(), res.end());
    std::vector<int32_t> h_ios(Nn, -1), h_sfi(L * E, -1);
    std::vector<uint64_t> h_st(Nn, 0);
    for (size_t i = 0; i < res.size(); ++i) {
        h_ios[i] = ios[res[i]];
        h_st[i] = stamp[res[i]];
        h_sfi[ios[res[i]]] = (int32_t)i;
    }
    // The new pool is built first; a failure up to the commit leaves the cache
    // as it was.
    uint8_t* npool = nullptr;
    int32_t* src = nullptr;
    auto fail = [&](hipError_t e, const char* what) {
        (void)hipFree(npool);
        (void)hipFree(src);
        set_error("resize: %s failed: %s", what, hipGetErrorString(e));
        return e == hipErrorOutOfMemory ? FT_ERR_NOMEM : FT_ERR_HIP;
    };
    hipError_t e;
    if ((e = hipMalloc(reinterpret_cast<void**>(&npool), (size_t)(Nn * c->rl.P)))) return fail(e, "pool allocation");
    if ((e = dalloc(&src, std::max<size_t>(res.size(), 1)))) return fail(e, "gather list allocation");
    if (!res.empty()) {
        if ((e = hipMemcpy(src, res.data(), sizeof(int32_t) * res.size(), hipMemcpyHostToDevice)))
            return fail(e, "gather list copy");
        if ((e = launch_resize_gather(c->pool, npool, c->rl.P, src, (int)res.size(), 0))) return fail(e, "gather");
        if ((e = hipDeviceSynchronize())) return fail(e, "gather");
    }
    (void)hipFree(src);
    src = nullptr;
    // Commit.  The maps are rewritten in place (they are sized for any slot
    // count) and the pool generation advances, so that a call replayed from a
    // graph captured before this resize does nothing (error flag 16).  A HIP
    // failure from here on means the device failed part-way: the cache must
    // then be destroyed.
    if ((e = hipMemcpy(c->id_of_slot, h_ios.data(), sizeof(int32_t) * Nn, hipMemcpyHostToDevice)) ||
        (e = hipMemcpy(c->stamp, h_st.data(), sizeof(uint64_t) * Nn, hipMemcpyHostToDevice)) ||
        (e = hipMemcpy(c->slot_for_id, h_sfi.data(), sizeof(int32_t) * L * E, hipMemcpyHostToDevice))) {
        (void)hipFree(npool);
        set_error("resize: writing the maps failed: %s (destroy the cache)", hipGetErrorString(e));
        return FT_ERR_HIP;
    }
    (void)hipFree(c->pool);
    c->pool = npool;
    c->N = Nn;
    c->gen += 1;
    c->buf_layer[0] = c->buf_layer[1] = -1;
    c->release_recorded[0] = c->release_recorded[1] = false;
    c->xfer_pending = false;
    c->streaming = false;
    FT_HIP(write_dstate(c));
    FT_HIP(hipDeviceSynchronize());
    return FT_OK;
}

ft_status ft_cache_set_profile(ft_cache* c, const ft_profile* p) {
    clear_error();
    FT_REQUIRE(c && p, "null pointer");
    FT_REQUIRE(p->bp_mbps > 0 && p->bh_mbps > 0, "bandwidths must be positive");
    FT_REQUIRE(p->max_fetch >= -1, "max_fetch must be -1 or >= 0");
    // calls already enqueued run with the profile they were enqueued under
    ft_status fs = flush_fill_sync(c);
    if (fs != FT_OK) return fs;
    c->prof = *p;
    FT_HIP(write_dstate(c));
    return FT_OK;
}

ft_status ft_cache_profile(ft_cache* c, int32_t records, ft_profile* out) {
    clear_error();
    FT_REQUIRE(c && out, "null pointer");
    const int64_t lim = std::min<int64_t>(c->sh.experts, c->N);
    FT_REQUIRE(records >= 1 && records <= lim, "records must be in 1..min(E, num_slots) = %lld", (long long)lim);
    ft_status fs = flush_fill_sync(c);
    if (fs != FT_OK) return fs;
    FT_HIP(hipDeviceSynchronize());
    const int64_t S = c->rl.S;
    const int k = c->sh.top_k;
    const int batch = c->cap;                 // worklist and host-staging capacity
    const int E = c->sh.experts;
    // Every fill repetition and host pass reads its own records (pass p reads
    // layer-0 records p*records .. p*records + records - 1, modulo E), so that
    // neither path is timed on data a previous pass left in a host cache.
    auto rec_of = [&](int pass, int i) { return (int32_t)(((int64_t)pass * records + i) % E); };
    // B_P: the fill kernel pulls `records` records into slots 0 .. records-1,
    // in launches of at most `batch` records
    hipEvent_t e0, e1;
    FT_HIP(hipEventCreate(&e0));
    FT_HIP(hipEventCreate(&e1));
    double best_ms = 1e30;
    for (int rep = 0; rep < 3; ++rep) {
        double ms_rep = 0.0;
        for (int b0 = 0; b0 < records; b0 += batch) {
            const int n = std::min(batch, records - b0);
            std::vector<int32_t> idx(n);
            std::vector<int32_t> src(n);
            for (int i = 0; i < n; ++i) {
                idx[i] = b0 + i;
                src[i] = rec_of(rep, b0 + i);
            }
            const int32_t counts[4] = {n, 0, n, n};
            FT_HIP(hipMemcpy(c->wl_slot, idx.data(), sizeof(int32_t) * n, hipMemcpyHostToDevice));
            FT_HIP(hipMemcpy(c->wl_src, src.data(), sizeof(int32_t) * n, hipMemcpyHostToDevice));
            FT_HIP(hipMemcpy(c->wl_counts, counts, sizeof(counts), hipMemcpyHostToDevice));
            TimedLaunch tl;
            tl.start = e0;
            tl.stop = e1;
            FT_HIP(launch_fill(c, 0, tl));
            FT_HIP(hipEventSynchronize(e1));
            float ms = 0.0f;
            FT_HIP(hipEventElapsedTime(&ms, e0, e1));
            ms_rep += ms;
        }
        best_ms = std::min(best_ms, ms_rep);
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    const double bp = (double)records * S / (best_ms / 1e3) / 1e6;
    // B_H: the host workers run the same records as host routes of up to
    // max_tokens tokens per call (zero activations; the time does not depend on values)
    HostStaging hs = host_branch_staging(c->host);
    auto host_pass = [&](int pass) {
        for (int b0 = 0; b0 < records; b0 += batch) {
            const int n = std::min(batch, records - b0);
            const int T = (n + k - 1) / k;
            memset(hs.x, 0, sizeof(uint16_t) * (size_t)T * c->sh.d_model);
            for (int r = 0; r < T * k; ++r) {
                hs.routes[r] = r < n ? -(1 + rec_of(pass, b0 + r)) : INT32_MIN;
                hs.w[r] = 1.0f / k;
            }
            host_branch_run_sync(c->host, 0, T);
        }
    };
    // best of three passes, as for B_P: one pass is a millisecond or so, and a
    // worker the OS delays for part of it stretches the whole pass
    host_pass(3);                      // warm-up (worker wake-up), records not timed
    double bh = 0.0;
    for (int pass = 4; pass < 7; ++pass) {
        uint64_t b0c, b1c, x0, x1;
        double s0, s1;
        host_branch_counters(c->host, &b0c, &s0, &x0);
        host_pass(pass);
        host_branch_counters(c->host, &b1c, &s1, &x1);
        bh = std::max(bh, (double)(b1c - b0c) / std::max(s1 - s0, 1e-9) / 1e6);
    }
    // the pool's slots were overwritten: the cache restarts empty
    const int64_t nids = (int64_t)c->sh.layers * c->sh.experts;
    const uint64_t one = 1;
    FT_HIP(hipMemset(c->slot_for_id, 0xFF, sizeof(int32_t) * nids));
    FT_HIP(hipMemset(c->id_of_slot, 0xFF, sizeof(int32_t) * c->N));
    FT_HIP(hipMemset(c->stamp, 0, sizeof(uint64_t) * c->N));
    FT_HIP(hipMemcpy(c->clock, &one, sizeof(one), hipMemcpyHostToDevice));
    FT_HIP(hipMemset(c->wl_counts, 0, sizeof(int32_t) * 4));
    c->buf_layer[0] = c->buf_layer[1] = -1;
    c->release_recorded[0] = c->release_recorded[1] = false;
    c->xfer_pending = false;
    c->streaming = false;
    FT_HIP(hipDeviceSynchronize());
    out->bp_mbps = (uint32_t)std::min(bp, 4.0e9);
    out->bh_mbps = (uint32_t)std::min(bh, 4.0e9);
    out->max_fetch = c->prof.max_fetch;
    return FT_OK;
}

ft_status ft_cache_stats(const ft_cache* c, ft_stats* o) {
    clear_error();
    FT_REQUIRE(c && o, "null pointer");
    ft_status fs = flush_fill_sync(const_cast<ft_cache*>(c));
    if (fs != FT_OK) return fs;
    unsigned long long cnt[C_N];
    uint64_t clk;
    int32_t err;
    FT_HIP(hipMemcpy(cnt, c->counters, sizeof(cnt), hipMemcpyDeviceToHost));
    FT_HIP(hipMemcpy(&clk, c->clock, sizeof(clk), hipMemcpyDeviceToHost));
    FT_HIP(hipMemcpy(&err, c->errflag, sizeof(err), hipMemcpyDeviceToHost));
    o->calls = cnt[C_CALLS];
    o->routes = cnt[C_ROUTES];
    o->unique = cnt[C_UNIQUE];
    o->hits = cnt[C_HITS];
    o->misses = cnt[C_MISSES];
    o->fills = cnt[C_FILLS];
    o->cpu_experts = cnt[C_CPU];
    o->evictions = cnt[C_EVICT];
    o->bytes_filled = cnt[C_BYTES];
    o->layers_streamed = cnt[C_STREAMED];
    o->clock = clk;
    o->error_flags = err;
    o->num_slots = (int32_t)c->N;
    host_branch_counters(c->host, &o->host_bytes, &o->host_seconds, &o->host_experts);
    return FT_OK;
}

ft_status ft_cache_set_timing(ft_cache* c, int32_t enable) {
    clear_error();
    FT_REQUIRE(c, "cache is null");
    ft_status fs = flush_fill_sync(c);
    if (fs != FT_OK) return fs;
    if (c->timing) {
        timing_destroy(c->timing);
        c->timing = nullptr;
    }
    const unsigned long long z[4] = {0, 0, 0, 0};
    FT_HIP(hipMemcpy(c->counters + C_GEMV_EXPERTS, z, sizeof(z), hipMemcpyHostToDevice));
    if (enable) {
        c->timing = timing_create();
        if (!c->timing->ok) {
            timing_destroy(c->timing);
            c->timing = nullptr;
            set_error("timing events could not be created");
            return FT_ERR_HIP;
        }
    }
    return FT_OK;
}

ft_status ft_cache_timing(const ft_cache* c, ft_timing* o) {
    clear_error();
    FT_REQUIRE(c && o, "null pointer");
    ft_status fs = flush_fill_sync(const_cast<ft_cache*>(c));
    if (fs != FT_OK) return fs;
    memset(o, 0, sizeof(*o));
    if (c->timing) timing_read(c->timing, o->launches, o->ms);
    unsigned long long w[4];
    FT_HIP(hipMemcpy(w, c->counters + C_GEMV_EXPERTS, sizeof(w), hipMemcpyDeviceToHost));
    o->gemv_experts = w[0];
    o->gemv_rows = w[1];
    o->gemm_experts = w[2];
    o->gemm_rows = w[3];
    return FT_OK;
}

ft_status ft_cache_snapshot(const ft_cache* c, int32_t* slot_for_id, int32_t* id_of_slot, uint64_t* stamp,
                            uint64_t* clock) {
    clear_error();
    FT_REQUIRE(c, "cache is null");
    ft_status fs = flush_fill_sync(const_cast<ft_cache*>(c));
    if (fs != FT_OK) return fs;
    const int64_t LE = (int64_t)c->sh.layers * c->sh.experts;
    if (slot_for_id) FT_HIP(hipMemcpy(slot_for_id, c->slot_for_id, sizeof(int32_t) * LE, hipMemcpyDeviceToHost));
    if (id_of_slot) FT_HIP(hipMemcpy(id_of_slot, c->id_of_slot, sizeof(int32_t) * c->N, hipMemcpyDeviceToHost));
    if (stamp) FT_HIP(hipMemcpy(stamp, c->stamp, sizeof(uint64_t) * c->N, hipMemcpyDeviceToHost));
    if (clock) FT_HIP(hipMemcpy(clock, c->clock, sizeof(uint64_t), hipMemcpyDeviceToHost));
    return FT_OK;
}

ft_status ft_cache_read_slot(const ft_cache* c, int64_t slot, void* dst) {
    clear_error();
    FT_REQUIRE(c && dst, "null pointer");
    FT_REQUIRE(slot >= 0 && slot < c->N, "slot out of range");
    ft_status fs = flush_fill_sync(const_cast<ft_cache*>(c));
    if (fs != FT_OK) return fs;
    FT_HIP(hipMemcpy(dst, c->pool + slot * c->rl.P, (size_t)c->rl.S, hipMemcpyDeviceToHost));
    return FT_OK;
}

}  // extern "C"
