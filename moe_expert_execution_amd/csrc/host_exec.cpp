// Host branch of the bandwidth-adaptive split: misses that are not filled run
// on host cores straight from the pinned host bank, never touching a slot or
// the residency maps.  Persistent worker threads pinned to cores compute each
// host expert's SwiGLU FFN for its routed tokens and accumulate the
// gate-weighted outputs into the partial sum P [T x d] (fp32), which the GPU
// adds in the combine ("Making Large MoE Models Practical on a Single
// Machine", sections 4 and 10; hyper.ai summary, section 方法: persistent C++
// workers pinned to physical cores; "The Expert Cache That Follows the
// Router": a host-run miss reads the source without changing residency).
//
// Signalling: the planner kernel copies the call's routes, weights and
// activations into pinned staging and posts the call's sequence number to a
// pinned mailbox; a poller thread runs the call with the workers and posts
// it done.  The partial sum P stays in pinned memory, where the combine
// kernel reads it after waiting (bounded) for the done word; the GPU experts
// and fills run meanwhile.  Without the poller (FTMOE_HOST_SIGNAL=callback)
// the call is a host function on a stream of the library's, and the caller's
// stream waits for its event before the combine.
#include <hip/hip_runtime.h>
#include <immintrin.h>
#include <pthread.h>
#include <sched.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include "common.h"
#include "host_dots.h"

namespace ftmoe {
namespace {

constexpr int kRing = 256;
constexpr size_t kMailboxBytes = 512;

struct Job {
    int layer = 0, T = 0;
    // host experts of this call: expert id, and its (token, weight) list
    std::vector<int> experts;
    std::vector<int> tok_off;          // [n_experts + 1]
    std::vector<int> tok;              // token index per entry
    std::vector<float> wt;             // gate weight per entry
};

}  // namespace

struct HostBranch {
    ft_shape sh;
    RecordLayout rl;
    std::vector<const uint8_t*> bank;   // [L]: layer l's E records (host addresses)
    int32_t max_tokens;
    HostStaging stg;
    int nthreads;
    std::vector<std::thread> workers;
    // job dispatch
    std::mutex mu;
    std::condition_variable cv;
    std::atomic<uint64_t> gen{0};
    std::atomic<bool> stop{false};          // workers
    std::atomic<bool> stop_poller{false};   // the mailbox poller (stopped first)
    Job job;
    int cur_expert = 0;
    std::atomic<int> next_block{0};
    std::atomic<int> arrived{0};
    std::atomic<int> phase{0};
    std::atomic<int> finished{0};
    // per-call scratch shared by the workers
    std::vector<float> xf;             // [max_tokens x d] fp32 activations of the tokens with host routes
    std::vector<uint16_t> xb;          // the same in bf16
    std::vector<float> hbuf;           // SwiGLU outputs [rows x f]: every (expert, token) entry of a call
    std::vector<uint16_t> hbuf16;      // the same in bf16, for experts with many tokens
                                       // with up to max(max_tokens, 2k, min(max_tokens k, 2^21 / f)) entries
    // host-function contexts of calls captured into graphs: each captured
    // call owns one for the life of the branch (a graph may replay it any
    // number of times)
    struct GraphCall {
        HostBranch* hb;
        int layer, T;
    };
    std::vector<std::unique_ptr<GraphCall>> graph_calls;
    // ring of host-function contexts
    struct Call {
        HostBranch* hb;
        int layer, T;
        std::atomic<int> busy{0};
    } ring[kRing];
    uint64_t ring_next = 0;
    // mailbox (pinned, u64 words): [0] seq posted by the GPU, [8] done posted
    // by the poller; graph calls: [16] number, [24] done, [32] layer, [33] T
    bool use_mailbox = false;
    uint64_t* mbox = nullptr;
    uint64_t next_seq = 0;                   // last seq handed out (enqueuing thread)
    std::atomic<uint64_t> processed{0};      // last seq the poller finished
    struct Params {
        int layer, T;
    } params[kRing];
    std::thread poller;
    // counters (read after a device synchronisation)
    std::atomic<uint64_t> c_bytes{0}, c_experts{0};
    std::atomic<uint64_t> c_ns{0};
};

namespace {

inline float silu(float z) { return z / (1.0f + std::exp(-z)); }

// spin barrier over all participants (workers + the calling thread)
void barrier(HostBranch* hb, int participants) {
    const int ph = hb->phase.load(std::memory_order_acquire);
    if (hb->arrived.fetch_add(1, std::memory_order_acq_rel) == participants - 1) {
        hb->arrived.store(0, std::memory_order_relaxed);
        hb->next_block.store(0, std::memory_order_relaxed);
        hb->phase.store(ph + 1, std::memory_order_release);
    } else {
        while (hb->phase.load(std::memory_order_acquire) == ph) _mm_pause();
    }
}

// Per-thread scratch of the host workers.
struct WorkerScratch {
    std::vector<float> g, u, y;         // 16 * tokens dot results (32 for one token: a whole panel)
    std::vector<const float*> vec;      // token vectors
    std::vector<float> wdec;            // one decoded half panel, 16 x K (fp32)
    std::vector<uint16_t> wdec16;       // one decoded half panel, 16 x K (bf16, many-token dots)
    std::vector<const uint16_t*> vec16; // token vectors in bf16
    void fit(int nt, int kmax) {
        if ((int64_t)wdec.size() < 16ll * kmax) wdec.resize(16 * (size_t)kmax);
        if ((int64_t)wdec16.size() < 16 * hostk::decoded_ld(kmax)) wdec16.resize(16 * (size_t)hostk::decoded_ld(kmax));
        if ((int)vec16.size() < nt) vec16.resize(nt);
        if ((int)vec.size() < nt) {
            const size_t n = std::max<size_t>(32, 16 * (size_t)nt);
            g.resize(n);
            u.resize(n);
            y.resize(n);
            vec.resize(nt);
        }
    }
};

// All participants run this for the current job.  A work item is a whole
// 32-row panel, computed as its two 16-row halves one after the other: the
// halves interleave within every 1 KiB lane block (256-byte runs), so one
// core reads every line of the item once, where half-panel items on two
// cores each fetched (and prefetched) lines of the other's half (decode:
// 145 -> 162-174 GB/s of host experts).  When the SwiGLU outputs of every
// (expert, token) entry fit the scratch (decode: a few host experts of one
// token), the call runs in two phases over all its experts at once: (1) 32
// rows of one expert's gate and up matrices per item, h of that expert's
// tokens; (2) 32 output columns per item, every expert's down matrix in
// expert order, so each output element still receives its experts' terms in
// the same order.  Otherwise the experts run one after the other, two phases
// each.  An expert's token count picks its dot form (host_dots.h), the same
// in both phases: one token, the whole-panel pass; up to
// stream_max_vectors(fmt), the streaming pass with h kept in fp32; more, the
// half panel decoded once to bf16 and h kept in bf16.
void run_job(HostBranch* hb, int participants, WorkerScratch& ws) {
    const Job& jb = hb->job;
    const int d = hb->sh.d_model, f = hb->sh.d_ff, E = hb->sh.experts, fmt = hb->sh.fmt;
    const int64_t S = hb->rl.S;
    float* P = hb->stg.P;
    const int nx = (int)jb.experts.size();
    const bool together = (int64_t)jb.tok.size() * f <= (int64_t)hb->hbuf.size();
    // phase 1 of experts [x0, x1): items (expert, panel); h rows are indexed by entry
    auto phase1 = [&](int x0, int x1) {
        const int per = f / 32;
        const int nblk = (x1 - x0) * per;
        for (;;) {
            const int it = hb->next_block.fetch_add(1, std::memory_order_relaxed);
            if (it >= nblk) break;
            const int xi = x0 + it / per, p = it % per;
            const int e = jb.experts[xi];
            const int t0 = jb.tok_off[xi], nt = jb.tok_off[xi + 1] - t0;
            const uint8_t* rec = hb->bank[jb.layer] + (int64_t)e * S;
            ws.fit(nt, std::max(d, f));
            for (int i = 0; i < nt; ++i) ws.vec[i] = hb->xf.data() + (int64_t)jb.tok[t0 + i] * d;
            const int64_t hrow0 = together ? t0 : 0;
            if (nt == 1) {      // one token: each lane block read in one or two passes
                hostk::panel_dots_1(fmt, rec, hb->rl.off_gate, hb->rl.off_sg, p, d, ws.vec[0], ws.g.data());
                hostk::panel_dots_1(fmt, rec, hb->rl.off_up, hb->rl.off_su, p, d, ws.vec[0], ws.u.data());
                for (int r = 0; r < 32; ++r) hb->hbuf[hrow0 * f + 32 * p + r] = silu(ws.g[r]) * ws.u[r];
                continue;
            }
            if (nt > hostk::stream_max_vectors(fmt)) {      // many tokens: bf16 rows and vectors, h kept in bf16
                for (int i = 0; i < nt; ++i) ws.vec16[i] = hb->xb.data() + (int64_t)jb.tok[t0 + i] * d;
                const int64_t ld = hostk::decoded_ld(d);
                for (int h = 0; h < 2; ++h) {
                    hostk::half_panel_decode_bf16(fmt, rec, hb->rl.off_gate, hb->rl.off_sg, p, h, d, ws.wdec16.data(), ld);
                    hostk::dots_16xT_bf16(ws.wdec16.data(), ld, d, ws.vec16.data(), nt, ws.g.data());
                    hostk::half_panel_decode_bf16(fmt, rec, hb->rl.off_up, hb->rl.off_su, p, h, d, ws.wdec16.data(), ld);
                    hostk::dots_16xT_bf16(ws.wdec16.data(), ld, d, ws.vec16.data(), nt, ws.u.data());
                    const int b = 2 * p + h;  // rows 16 b .. 16 b + 15
                    for (int i = 0; i < nt; ++i) {
                        alignas(64) float hv[16];
                        for (int r = 0; r < 16; ++r) hv[r] = silu(ws.g[i * 16 + r]) * ws.u[i * 16 + r];
                        const __m256bh hb16 = _mm512_cvtneps_pbh(_mm512_load_ps(hv));
                        _mm256_storeu_si256(reinterpret_cast<__m256i*>(&hb->hbuf16[(hrow0 + i) * f + 16 * b]),
                                            (__m256i)hb16);
                    }
                }
                continue;
            }
            for (int h = 0; h < 2; ++h) {
                hostk::half_panel_dots(fmt, rec, hb->rl.off_gate, hb->rl.off_sg, p, h, d, ws.vec.data(), nt,
                                       ws.wdec.data(), ws.g.data());
                hostk::half_panel_dots(fmt, rec, hb->rl.off_up, hb->rl.off_su, p, h, d, ws.vec.data(), nt,
                                       ws.wdec.data(), ws.u.data());
                const int b = 2 * p + h;      // rows 16 b .. 16 b + 15
                for (int i = 0; i < nt; ++i)
                    for (int r = 0; r < 16; ++r)
                        hb->hbuf[(hrow0 + i) * f + 16 * b + r] = silu(ws.g[i * 16 + r]) * ws.u[i * 16 + r];
            }
        }
    };
    // phase 2 of experts [x0, x1): items are output panels, over the experts in order
    auto phase2 = [&](int x0, int x1) {
        const int nblk = d / 32;
        for (;;) {
            const int p = hb->next_block.fetch_add(1, std::memory_order_relaxed);
            if (p >= nblk) break;
            for (int xi = x0; xi < x1; ++xi) {            // each output element: its experts in order
                const int e = jb.experts[xi];
                const int t0 = jb.tok_off[xi], nt = jb.tok_off[xi + 1] - t0;
                const uint8_t* rec = hb->bank[jb.layer] + (int64_t)e * S;
                ws.fit(nt, std::max(d, f));
                const int64_t hrow0 = together ? t0 : 0;
                for (int i = 0; i < nt; ++i) ws.vec[i] = hb->hbuf.data() + (hrow0 + i) * f;
                if (nt > hostk::stream_max_vectors(fmt)) {      // many tokens: bf16 (h as phase 1 left it)
                    for (int i = 0; i < nt; ++i) ws.vec16[i] = hb->hbuf16.data() + (hrow0 + i) * f;
                    const int64_t ld = hostk::decoded_ld(f);
                    for (int b = 2 * p; b < 2 * p + 2; ++b) {
                        hostk::half_panel_decode_bf16(fmt, rec, hb->rl.off_down, hb->rl.off_sd, b >> 1, b & 1, f,
                                                      ws.wdec16.data(), ld);
                        hostk::dots_16xT_bf16(ws.wdec16.data(), ld, f, ws.vec16.data(), nt, ws.y.data());
                        for (int i = 0; i < nt; ++i) {
                            float* pr = P + (int64_t)jb.tok[t0 + i] * d + 16 * b;
                            const float wt = jb.wt[t0 + i];
                            for (int r = 0; r < 16; ++r) pr[r] += wt * ws.y[i * 16 + r];
                        }
                    }
                    continue;
                }
                if (nt == 1) {      // one token: the whole output panel in one call
                    hostk::panel_dots_1(fmt, rec, hb->rl.off_down, hb->rl.off_sd, p, f, ws.vec[0], ws.y.data());
                    float* pr = P + (int64_t)jb.tok[t0] * d + 32 * p;
                    const float wt = jb.wt[t0];
                    for (int r = 0; r < 32; ++r) pr[r] += wt * ws.y[r];
                    continue;
                }
                for (int b = 2 * p; b < 2 * p + 2; ++b) {    // output columns 16 b .. 16 b + 15
                    hostk::half_panel_dots(fmt, rec, hb->rl.off_down, hb->rl.off_sd, b >> 1, b & 1, f,
                                           ws.vec.data(), nt, ws.wdec.data(), ws.y.data());
                    for (int i = 0; i < nt; ++i) {
                        float* pr = P + (int64_t)jb.tok[t0 + i] * d + 16 * b;
                        const float wt = jb.wt[t0 + i];
                        for (int r = 0; r < 16; ++r) pr[r] += wt * ws.y[i * 16 + r];
                    }
                }
            }
        }
    };
    if (together) {
        phase1(0, nx);
        barrier(hb, participants);
        phase2(0, nx);
        barrier(hb, participants);
    } else {
        for (int xi = 0; xi < nx; ++xi) {
            phase1(xi, xi + 1);
            barrier(hb, participants);
            phase2(xi, xi + 1);
            barrier(hb, participants);
        }
    }
}

void worker_main(HostBranch* hb, int idx, int cpu) {
    if (cpu >= 0) {
        cpu_set_t set;
        CPU_ZERO(&set);
        CPU_SET(cpu, &set);
        pthread_setaffinity_np(pthread_self(), sizeof(set), &set);
    }
    WorkerScratch ws;
    uint64_t seen = 0;
    for (;;) {
        // spin briefly, then block
        int spins = 0;
        while (hb->gen.load(std::memory_order_acquire) == seen && !hb->stop.load()) {
            if (++spins < 20000) {
                _mm_pause();
            } else {
                std::unique_lock<std::mutex> lk(hb->mu);
                hb->cv.wait(lk, [&] { return hb->gen.load() != seen || hb->stop.load(); });
            }
        }
        if (hb->stop.load()) return;
        seen = hb->gen.load(std::memory_order_acquire);
        run_job(hb, hb->nthreads + 1, ws);
        hb->finished.fetch_add(1, std::memory_order_acq_rel);
    }
    (void)idx;
}

// One host-branch call: read the staged routes, run the host experts with the
// worker pool, leave the partial sums in staging P.
void run_call(HostBranch* hb, int layer, int T) {
    const int k = hb->sh.top_k, d = hb->sh.d_model, E = hb->sh.experts;
    Job& jb = hb->job;
    jb.layer = layer;
    jb.T = T;
    jb.experts.clear();
    jb.tok_off.clear();
    jb.tok.clear();
    jb.wt.clear();
    // host routes -(1+e); a repeated expert of a token is dropped (the planner does the same)
    std::vector<std::pair<int, int>> pairs;   // (expert, route)
    const int32_t* routes = hb->stg.routes;
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            const int32_t rv = routes[t * k + j];
            if (rv >= 0 || rv == INT32_MIN) continue;
            const int e = -rv - 1;
            if (e < 0 || e >= E) continue;
            bool dup = false;
            for (int jj = 0; jj < j; ++jj) dup |= routes[t * k + jj] == rv;
            if (!dup) pairs.emplace_back(e, t * k + j);
        }
    }
    std::sort(pairs.begin(), pairs.end());
    std::vector<char> has(T, 0);
    for (size_t i = 0; i < pairs.size(); ++i) {
        if (i == 0 || pairs[i].first != pairs[i - 1].first) {
            jb.experts.push_back(pairs[i].first);
            jb.tok_off.push_back((int)jb.tok.size());
        }
        const int r = pairs[i].second;
        jb.tok.push_back(r / k);
        jb.wt.push_back(hb->stg.w[r]);
        has[r / k] = 1;
    }
    jb.tok_off.push_back((int)jb.tok.size());
    if (!jb.experts.empty()) {
        const auto t_start = std::chrono::steady_clock::now();
        for (int t = 0; t < T; ++t)
            if (has[t]) memset(hb->stg.P + (int64_t)t * d, 0, sizeof(float) * d);
        // the activations of every token with host routes, out of the pinned
        // staging (read once here; the dot loops read them many times): fp32,
        // and bf16 as they are
        for (int t = 0; t < T; ++t) {
            if (!has[t]) continue;
            const uint16_t* xr = hb->stg.x + (int64_t)t * d;
            float* o = hb->xf.data() + (int64_t)t * d;
            uint16_t* ob = hb->xb.data() + (int64_t)t * d;
            for (int c = 0; c < d; ++c) {
                ob[c] = xr[c];
                o[c] = __builtin_bit_cast(float, (uint32_t)xr[c] << 16);
            }
        }
        hb->finished.store(0);
        {
            std::lock_guard<std::mutex> lk(hb->mu);
            hb->gen.fetch_add(1, std::memory_order_acq_rel);
        }
        hb->cv.notify_all();
        static thread_local WorkerScratch ws;
        run_job(hb, hb->nthreads + 1, ws);
        while (hb->finished.load(std::memory_order_acquire) < hb->nthreads) _mm_pause();
        const auto ns = std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() -
                                                                             t_start).count();
        hb->c_ns.fetch_add((uint64_t)ns);
        hb->c_experts.fetch_add(jb.experts.size());
        hb->c_bytes.fetch_add(jb.experts.size() * (uint64_t)hb->rl.S);
    }
}

// Runs on the HIP runtime's callback thread, in stream order.
void host_fn(void* p) {
    auto* call = static_cast<HostBranch::Call*>(p);
    run_call(call->hb, call->layer, call->T);
    call->busy.store(0, std::memory_order_release);
}

void graph_host_fn(void* p) {
    auto* call = static_cast<HostBranch::GraphCall*>(p);
    run_call(call->hb, call->layer, call->T);
}

// Mailbox poller: waits for the GPU to post a sequence number, runs that call,
// posts it as done.  Every posted number is answered, in order.
void poller_main(HostBranch* hb, int cpu) {
    if (cpu >= 0) {
        cpu_set_t set;
        CPU_ZERO(&set);
        CPU_SET(cpu, &set);
        pthread_setaffinity_np(pthread_self(), sizeof(set), &set);
    }
    volatile uint64_t* seq_word = hb->mbox;
    uint64_t* done_word = hb->mbox + 8;
    uint64_t* g = hb->mbox + 16;              // graph calls
    uint64_t last = 0, glast = 0;
    int idle = 0;
    while (!hb->stop_poller.load(std::memory_order_relaxed)) {
        const uint64_t gs = __atomic_load_n(g, __ATOMIC_ACQUIRE);
        if (gs != glast) {
            idle = 0;
            const int layer = (int)__atomic_load_n(g + 16, __ATOMIC_RELAXED);
            const int T = (int)__atomic_load_n(g + 17, __ATOMIC_RELAXED);
            run_call(hb, layer, T);
            __atomic_store_n(g + 8, gs, __ATOMIC_RELEASE);
            glast = gs;
            continue;
        }
        const uint64_t s = __atomic_load_n(seq_word, __ATOMIC_ACQUIRE);
        if (s == last) {
            if (++idle < 200000) {
                _mm_pause();
            } else {
                std::this_thread::sleep_for(std::chrono::microseconds(20));
            }
            continue;
        }
        idle = 0;
        for (uint64_t n = last + 1; n <= s && !hb->stop_poller.load(std::memory_order_relaxed); ++n) {
            const HostBranch::Params p = hb->params[n % kRing];
            run_call(hb, p.layer, p.T);
            __atomic_store_n(done_word, n, __ATOMIC_RELEASE);
            hb->processed.store(n, std::memory_order_release);
        }
        last = s;
    }
}

}  // namespace

HostBranch* host_branch_create(const ft_shape& sh, const RecordLayout& rl, const uint8_t* const* bank_layers,
                               int32_t max_tokens) {
    auto* hb = new HostBranch();
    hb->sh = sh;
    hb->rl = rl;
    hb->bank.assign(bank_layers, bank_layers + sh.layers);
    hb->max_tokens = max_tokens;
    const int64_t d = sh.d_model, k = sh.top_k, f = sh.d_ff;
    void* p = nullptr;
    bool ok = true;
    ok &= hipHostMalloc(&p, sizeof(uint16_t) * max_tokens * d, hipHostMallocDefault) == hipSuccess;
    hb->stg.x = (uint16_t*)p;
    ok &= hipHostMalloc(&p, sizeof(int32_t) * max_tokens * k, hipHostMallocDefault) == hipSuccess;
    hb->stg.routes = (int32_t*)p;
    ok &= hipHostMalloc(&p, sizeof(float) * max_tokens * k, hipHostMallocDefault) == hipSuccess;
    hb->stg.w = (float*)p;
    ok &= hipHostMalloc(&p, sizeof(float) * max_tokens * d, hipHostMallocDefault) == hipSuccess;
    hb->stg.P = (float*)p;
    ok &= hipHostMalloc(&p, kMailboxBytes, hipHostMallocDefault) == hipSuccess;
    hb->mbox = (uint64_t*)p;
    if (hb->mbox) memset(hb->mbox, 0, kMailboxBytes);
    // the kernels write and read the staging through these same addresses
    for (void* hp : {(void*)hb->stg.x, (void*)hb->stg.routes, (void*)hb->stg.w, (void*)hb->stg.P, (void*)hb->mbox}) {
        void* dp = nullptr;
        ok &= hp && hipHostGetDevicePointer(&dp, hp, 0) == hipSuccess && dp == hp;
    }
    if (!ok) {
        host_branch_destroy(hb);
        return nullptr;
    }
    hb->xf.resize((size_t)max_tokens * d);
    hb->xb.resize((size_t)max_tokens * d);
    // SwiGLU outputs: one row per token for experts run one at a time, or one
    // row per (expert, token) entry when a call's entries fit (at least 2k rows)
    const int64_t hrows = std::max<int64_t>(std::max<int64_t>(max_tokens, 2 * (int64_t)sh.top_k),
                                            std::min<int64_t>((int64_t)max_tokens * sh.top_k, (1 << 21) / f));
    hb->hbuf.resize((size_t)hrows * f);
    hb->hbuf16.resize((size_t)hrows * f);
    for (int i = 0; i < kRing; ++i) hb->ring[i].hb = hb;
    // worker count: cores in the affinity mask minus four (the caller's thread,
    // the mailbox poller, the HIP runtime's threads), at least one: spinning
    // workers that share cores with those threads stall the pooled phases
    // (decode, 16 cores: 155 GB/s of host experts with 12 workers, 111 with 14)
    cpu_set_t set;
    CPU_ZERO(&set);
    std::vector<int> cpus;
    if (sched_getaffinity(0, sizeof(set), &set) == 0)
        for (int c = 0; c < CPU_SETSIZE; ++c)
            if (CPU_ISSET(c, &set)) cpus.push_back(c);
    int n = (int)cpus.size() - 4;
    if (const char* env = getenv("FTMOE_HOST_THREADS")) n = atoi(env) - 1;
    n = std::max(0, std::min(n, 63));
    hb->nthreads = n;
    for (int i = 0; i < n; ++i) {
        int cpu = cpus.empty() ? -1 : cpus[(i + 2) % cpus.size()];
        hb->workers.emplace_back(worker_main, hb, i, cpu);
    }
    // signalling: a polled mailbox in pinned memory, whose done word the
    // combine kernel polls (FTMOE_HOST_SIGNAL=callback forces stream host
    // functions)
    const char* sig = getenv("FTMOE_HOST_SIGNAL");
    hb->use_mailbox = !(sig && strcmp(sig, "callback") == 0);
    if (hb->use_mailbox) hb->poller = std::thread(poller_main, hb, cpus.empty() ? -1 : cpus[1 % cpus.size()]);
    return hb;
}

void host_branch_run_sync(HostBranch* hb, int32_t layer, int32_t T) { run_call(hb, layer, T); }

HostSignal host_branch_prepare(HostBranch* hb, int32_t layer, int32_t T) {
    HostSignal s{};
    s.mailbox = hb->use_mailbox;
    if (!s.mailbox) return s;
    const uint64_t n = ++hb->next_seq;
    // the poller reads params[n % kRing] only after the GPU posted n; keep it
    // from lapping an entry that is still unread
    while (n - hb->processed.load(std::memory_order_acquire) >= (uint64_t)kRing) std::this_thread::yield();
    hb->params[n % kRing].layer = layer;
    hb->params[n % kRing].T = T;
    std::atomic_thread_fence(std::memory_order_release);
    s.seq = n;
    s.seq_word = hb->mbox;
    s.done_word = hb->mbox + 8;
    return s;
}

HostSignal host_branch_graph_signal(HostBranch* hb, uint64_t* gseq_dev, int32_t layer, int32_t T) {
    HostSignal s{};
    if (!hb->use_mailbox) return s;
    s.gmbox = hb->mbox + 16;
    s.gseq_dev = gseq_dev;
    s.layer = layer;
    s.T = T;
    return s;
}

void host_branch_destroy(HostBranch* hb) {
    if (!hb) return;
    // the poller first: a call it is running needs every worker, so the
    // workers stop only once it has returned (the host can still be behind
    // the device here, when a combine gave up waiting for it)
    hb->stop_poller.store(true);
    if (hb->poller.joinable()) hb->poller.join();
    {
        std::lock_guard<std::mutex> lk(hb->mu);
        hb->stop.store(true);
    }
    hb->cv.notify_all();
    for (auto& t : hb->workers) t.join();
    if (hb->stg.x) (void)hipHostFree(hb->stg.x);
    if (hb->stg.routes) (void)hipHostFree(hb->stg.routes);
    if (hb->stg.w) (void)hipHostFree(hb->stg.w);
    if (hb->stg.P) (void)hipHostFree(hb->stg.P);
    if (hb->mbox) (void)hipHostFree(hb->mbox);
    delete hb;
}

HostStaging host_branch_staging(HostBranch* hb) { return hb->stg; }

void host_branch_counters(HostBranch* hb, uint64_t* bytes, double* seconds, uint64_t* experts) {
    *bytes = hb->c_bytes.load();
    *seconds = hb->c_ns.load() * 1e-9;
    *experts = hb->c_experts.load();
}


int host_branch_threads(HostBranch* hb) { return hb->nthreads + 1; }

hipError_t host_branch_enqueue(HostBranch* hb, int32_t layer, int32_t T, hipStream_t stream) {
    auto& call = hb->ring[hb->ring_next % kRing];
    // a context is reused only after its previous host function finished
    while (call.busy.load(std::memory_order_acquire)) std::this_thread::yield();
    hb->ring_next++;
    call.layer = layer;
    call.T = T;
    call.busy.store(1, std::memory_order_release);
    hipError_t e = hipLaunchHostFunc(stream, host_fn, &call);
    if (e != hipSuccess) call.busy.store(0);
    return e;
}

hipError_t host_branch_enqueue_captured(HostBranch* hb, int32_t layer, int32_t T, hipStream_t stream) {
    hb->graph_calls.emplace_back(new HostBranch::GraphCall{hb, layer, T});
    return hipLaunchHostFunc(stream, graph_host_fn, hb->graph_calls.back().get());
}

}  // namespace ftmoe
