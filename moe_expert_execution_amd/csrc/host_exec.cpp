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
// The GPU side never waits on the host: the work is enqueued as a stream host
// function after the routes, weights and activations are copied to pinned
// staging, and the partial sum is copied back on the same stream.
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
#include <mutex>
#include <thread>
#include <vector>

#include "common.h"

namespace ftmoe {
namespace {

constexpr int kRing = 256;
constexpr int kRowBlock = 16;

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
    const uint8_t* bank;
    int32_t max_tokens;
    HostStaging stg;
    int nthreads;
    std::vector<std::thread> workers;
    // job dispatch
    std::mutex mu;
    std::condition_variable cv;
    std::atomic<uint64_t> gen{0};
    std::atomic<bool> stop{false};
    Job job;
    int cur_expert = 0;
    std::atomic<int> next_block{0};
    std::atomic<int> arrived{0};
    std::atomic<int> phase{0};
    std::atomic<int> finished{0};
    // per-call scratch shared by the workers
    std::vector<float> xf;             // [max_tokens x d] fp32 activations of the tokens with host routes
    std::vector<float> hbuf;           // [max_tokens x f] SwiGLU output of the current expert
    // ring of host-function contexts
    struct Call {
        HostBranch* hb;
        int layer, T;
        std::atomic<int> busy{0};
    } ring[kRing];
    uint64_t ring_next = 0;
    // mailbox (pinned): [0] seq posted by the GPU, [8] done posted by the poller
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

// ---- row decoders: one weight row -> fp32 ------------------------------------
inline float e4m3_to_f32(uint8_t c) {
    const uint32_t s = (c & 0x80u) << 24;
    const uint32_t e = (c >> 3) & 0xF, m = c & 7;
    float v;
    if (e == 0) {
        v = (float)m * (1.0f / 512.0f);
    } else {
        v = __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
    }
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) | s);
}

const float kE2M1[16] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f,
                         -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};

// Decode row n of a [rows x K] matrix stored at `off` (scales at `soff`).
void decode_row(const HostBranch* hb, const uint8_t* rec, int64_t off, int64_t soff, int n, int K, float* out) {
    switch (hb->sh.fmt) {
        case FT_FMT_BF16: {
            const uint16_t* r = reinterpret_cast<const uint16_t*>(rec + off) + (int64_t)n * K;
            int i = 0;
            for (; i + 16 <= K; i += 16) {
                __m256i w16 = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(r + i));
                __m512i w32 = _mm512_slli_epi32(_mm512_cvtepu16_epi32(w16), 16);
                _mm512_storeu_ps(out + i, _mm512_castsi512_ps(w32));
            }
            for (; i < K; ++i) out[i] = __builtin_bit_cast(float, (uint32_t)r[i] << 16);
            break;
        }
        case FT_FMT_FP8_B128: {
            const uint8_t* r = rec + off + (int64_t)n * K;
            const float* sc = reinterpret_cast<const float*>(rec + soff) + (int64_t)(n >> 7) * (K >> 7);
            for (int b = 0; b < K; b += 128) {
                const float s = sc[b >> 7];
                for (int i = 0; i < 128; ++i) out[b + i] = e4m3_to_f32(r[b + i]) * s;
            }
            break;
        }
        case FT_FMT_MXFP4_B32: {
            const uint8_t* r = rec + off + (int64_t)n * (K / 2);
            const uint8_t* sc = rec + soff + (int64_t)n * (K >> 5);
            for (int b = 0; b < K; b += 32) {
                const float s = ldexpf(1.0f, (int)sc[b >> 5] - 127);
                for (int i = 0; i < 16; ++i) {
                    const uint8_t v = r[(b >> 1) + i];
                    out[b + 2 * i] = kE2M1[v & 0xF] * s;
                    out[b + 2 * i + 1] = kE2M1[v >> 4] * s;
                }
            }
            break;
        }
    }
}

inline float dot_f32(const float* a, const float* b, int n) {
    __m512 acc0 = _mm512_setzero_ps(), acc1 = _mm512_setzero_ps();
    int i = 0;
    for (; i + 32 <= n; i += 32) {
        acc0 = _mm512_fmadd_ps(_mm512_loadu_ps(a + i), _mm512_loadu_ps(b + i), acc0);
        acc1 = _mm512_fmadd_ps(_mm512_loadu_ps(a + i + 16), _mm512_loadu_ps(b + i + 16), acc1);
    }
    float s = _mm512_reduce_add_ps(_mm512_add_ps(acc0, acc1));
    for (; i < n; ++i) s += a[i] * b[i];
    return s;
}

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

// All participants run this for the current job.
void run_job(HostBranch* hb, int participants, std::vector<float>& rowbuf) {
    const Job& jb = hb->job;
    const int d = hb->sh.d_model, f = hb->sh.d_ff, E = hb->sh.experts;
    const int64_t S = hb->rl.S;
    float* P = hb->stg.P;
    for (size_t xi = 0; xi < jb.experts.size(); ++xi) {
        const int e = jb.experts[xi];
        const int t0 = jb.tok_off[xi], t1 = jb.tok_off[xi + 1], nt = t1 - t0;
        const uint8_t* rec = hb->bank + ((int64_t)jb.layer * E + e) * S;
        // phase 1: h[i][n] = silu(x_i . WgT[n]) * (x_i . WuT[n])
        const int nblk1 = (f + kRowBlock - 1) / kRowBlock;
        for (;;) {
            const int b = hb->next_block.fetch_add(1, std::memory_order_relaxed);
            if (b >= nblk1) break;
            for (int n = b * kRowBlock; n < std::min(f, (b + 1) * kRowBlock); ++n) {
                decode_row(hb, rec, hb->rl.off_gate, hb->rl.off_sg, n, d, rowbuf.data());
                decode_row(hb, rec, hb->rl.off_up, hb->rl.off_su, n, d, rowbuf.data() + d);
                for (int i = 0; i < nt; ++i) {
                    const float* xr = hb->xf.data() + (int64_t)jb.tok[t0 + i] * d;
                    const float g = dot_f32(xr, rowbuf.data(), d);
                    const float u = dot_f32(xr, rowbuf.data() + d, d);
                    hb->hbuf[(int64_t)i * f + n] = silu(g) * u;
                }
            }
        }
        barrier(hb, participants);
        // phase 2: P[t][c] += w * (h_i . WdT[c])
        const int nblk2 = (d + kRowBlock - 1) / kRowBlock;
        for (;;) {
            const int b = hb->next_block.fetch_add(1, std::memory_order_relaxed);
            if (b >= nblk2) break;
            for (int c = b * kRowBlock; c < std::min(d, (b + 1) * kRowBlock); ++c) {
                decode_row(hb, rec, hb->rl.off_down, hb->rl.off_sd, c, f, rowbuf.data());
                for (int i = 0; i < nt; ++i) {
                    const float y = dot_f32(hb->hbuf.data() + (int64_t)i * f, rowbuf.data(), f);
                    P[(int64_t)jb.tok[t0 + i] * d + c] += jb.wt[t0 + i] * y;
                }
            }
        }
        barrier(hb, participants);
    }
}

void worker_main(HostBranch* hb, int idx, int cpu) {
    if (cpu >= 0) {
        cpu_set_t set;
        CPU_ZERO(&set);
        CPU_SET(cpu, &set);
        pthread_setaffinity_np(pthread_self(), sizeof(set), &set);
    }
    std::vector<float> rowbuf(2 * (size_t)std::max(hb->sh.d_model, hb->sh.d_ff) + 64);
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
        run_job(hb, hb->nthreads + 1, rowbuf);
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
        // fp32 activations of every token with host routes
        for (int t = 0; t < T; ++t) {
            if (!has[t]) continue;
            const uint16_t* xr = hb->stg.x + (int64_t)t * d;
            float* o = hb->xf.data() + (int64_t)t * d;
            for (int c = 0; c < d; ++c) o[c] = __builtin_bit_cast(float, (uint32_t)xr[c] << 16);
        }
        hb->finished.store(0);
        {
            std::lock_guard<std::mutex> lk(hb->mu);
            hb->gen.fetch_add(1, std::memory_order_acq_rel);
        }
        hb->cv.notify_all();
        std::vector<float> rowbuf(2 * (size_t)std::max(hb->sh.d_model, hb->sh.d_ff) + 64);
        run_job(hb, hb->nthreads + 1, rowbuf);
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
    uint64_t last = 0;
    int idle = 0;
    while (!hb->stop.load(std::memory_order_relaxed)) {
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
        for (uint64_t n = last + 1; n <= s; ++n) {
            const HostBranch::Params p = hb->params[n % kRing];
            run_call(hb, p.layer, p.T);
            __atomic_store_n(done_word, n, __ATOMIC_RELEASE);
            hb->processed.store(n, std::memory_order_release);
        }
        last = s;
    }
}

}  // namespace

HostBranch* host_branch_create(const ft_shape& sh, const RecordLayout& rl, const uint8_t* bank_host,
                               int32_t max_tokens) {
    auto* hb = new HostBranch();
    hb->sh = sh;
    hb->rl = rl;
    hb->bank = bank_host;
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
    ok &= hipHostMalloc(&p, 128, hipHostMallocDefault) == hipSuccess;
    hb->mbox = (uint64_t*)p;
    if (hb->mbox) memset(hb->mbox, 0, 128);
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
    hb->hbuf.resize((size_t)max_tokens * f);
    for (int i = 0; i < kRing; ++i) hb->ring[i].hb = hb;
    // worker count: cores in the affinity mask minus two (runtime threads, caller), at least one
    cpu_set_t set;
    CPU_ZERO(&set);
    std::vector<int> cpus;
    if (sched_getaffinity(0, sizeof(set), &set) == 0)
        for (int c = 0; c < CPU_SETSIZE; ++c)
            if (CPU_ISSET(c, &set)) cpus.push_back(c);
    int n = (int)cpus.size() - 2;
    if (const char* env = getenv("FTMOE_HOST_THREADS")) n = atoi(env) - 1;
    n = std::max(0, std::min(n, 63));
    hb->nthreads = n;
    for (int i = 0; i < n; ++i) {
        int cpu = cpus.empty() ? -1 : cpus[(i + 2) % cpus.size()];
        hb->workers.emplace_back(worker_main, hb, i, cpu);
    }
    // signalling: a polled mailbox when the device can wait on a memory value
    // (FTMOE_HOST_SIGNAL=callback forces stream host functions)
    int dev = 0, can_wait = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&can_wait, hipDeviceAttributeCanUseStreamWaitValue, dev) != hipSuccess)
        can_wait = 0;
    const char* sig = getenv("FTMOE_HOST_SIGNAL");
    hb->use_mailbox = can_wait && !(sig && strcmp(sig, "callback") == 0);
    if (hb->use_mailbox) hb->poller = std::thread(poller_main, hb, cpus.empty() ? -1 : cpus[1 % cpus.size()]);
    return hb;
}

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

void host_branch_destroy(HostBranch* hb) {
    if (!hb) return;
    {
        std::lock_guard<std::mutex> lk(hb->mu);
        hb->stop.store(true);
    }
    hb->cv.notify_all();
    if (hb->poller.joinable()) hb->poller.join();
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

}  // namespace ftmoe
