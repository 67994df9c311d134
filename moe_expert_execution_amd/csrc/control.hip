// Per-layer control of the slot cache: one workgroup dedupes the routed
// experts, classifies them against the residency table, derives the fill count
// q, stamps LRU recency, selects the q least-recently-used victims in one scan
// of the slots, admits the fills into the maps and rewrites the routes into
// slot ids — all on the device, with no host synchronisation ("The Expert
// Cache That Follows the Router", section "How residency follows demand without
// leaving the device"; hyper.ai summary, section 方法; txtmix article, section
// "CUDA-graph 兼容的 LRU 缓存").  Also: the fill copy (device-initiated pull of
// whole records from the pinned host bank into the victim slots), the
// invalidation of a full-layer buffer before it is overwritten, and the record
// gather used by resize.
#include "common.h"
#include "fill.h"

namespace ftmoe {
namespace {

struct CtrlArgs {
    int32_t* ids;
    int32_t R, layer, E, N;
    int32_t* slot_for_id;
    int32_t* id_of_slot;
    uint64_t* stamp;
    uint64_t* clock;
    unsigned long long* counters;
    int32_t* errflag;
    const DevState* ds;     // profile and pool generation, read at run time
    uint32_t gen;           // the pool generation this call was enqueued under
    int64_t S;
    // caller outputs (any may be null)
    int32_t* o_counts;
    int32_t* o_uniq;
    uint8_t* o_cls;
    int32_t* o_slot;
    int32_t* o_ev_slot;
    int32_t* o_ev_old;
    int32_t* o_ev_new;
    int32_t* o_cpu;
    // internal fill worklist
    int32_t* wl_counts;
    int32_t* wl_slot;
    int32_t* wl_src;
};

constexpr int kWaves = kCtrlThreads / 64;

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

// Exclusive scan over the workgroup; every thread gets its prefix and the total.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int* total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int incl = wave_incl_scan(v, lane);
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        int s = wsum[i];
        base += (i < wid) ? s : 0;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    uint32_t lo = __shfl_xor((unsigned)(v & 0xffffffffu), m, 64);
    uint32_t hi = __shfl_xor((unsigned)(v >> 32), m, 64);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ int fill_count(int m, int h, int N, uint32_t bp, uint32_t bh, int max_fetch) {
    if (m <= 0) return 0;
    int64_t q = (2ll * m * bp + bh) / (2ll * bh);   // round half up of m * B_P / B_H
    if (q < 1) q = 1;
    if (q > m) q = m;
    if (q > N - h) q = N - h;
    if (max_fetch >= 0 && q > max_fetch) q = max_fetch;
    return q < 0 ? 0 : (int)q;
}

// KPT: victim keys per thread, ceil(N / kCtrlThreads) rounded up to a power of two
template <int KPT>
__global__ void __launch_bounds__(kCtrlThreads) classify_kernel(CtrlArgs a) {
    static_assert(KPT * kCtrlThreads <= kMaxSlots, "keys per thread beyond the slot limit");
    __shared__ uint32_t ebits[kMaxExperts / 32];
    __shared__ int wordbase[kMaxExperts / 32];
    __shared__ int16_t pos_of_e[kMaxExperts];     // expert -> unique index
    __shared__ int16_t e_of_u[kMaxExperts];       // unique index -> expert
    __shared__ int32_t uslot[kMaxExperts];        // unique index -> slot or -1
    __shared__ uint8_t ucls[kMaxExperts];
    __shared__ int16_t miss_list[kMaxExperts];    // miss rank -> unique index
    __shared__ uint32_t hitbits[kMaxSlots / 32];
    __shared__ int16_t victims[kMaxExperts];     // slots fit 15 bits (N <= 32768)
    __shared__ int32_t victim_old[kMaxExperts];  // each victim's owner (flat id) or -1
    __shared__ int wsum[kWaves];
    __shared__ uint64_t wmin[2][kWaves];
    __shared__ int sh_nuniq, sh_evict;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int E = a.E, N = a.N, R = a.R;
    const int ewords = (E + 31) >> 5, nwords = (N + 31) >> 5;
    const uint64_t clk = *a.clock;
    const uint32_t gen_now = a.ds->gen;
    const uint32_t bp = a.ds->bp_mbps, bh = a.ds->bh_mbps;
    const int32_t max_fetch = a.ds->max_fetch;

    // Every map read of the call is issued here, together: the layer's
    // slot_for_id entries (expert tid + j * kCtrlThreads), and the stamp and
    // owner of each slot this thread keys in the victim scan (slot
    // tid + j * kCtrlThreads).  The rest of the kernel then works on chip
    // and only stores.  (Stamps of slots hit in this call change below, but
    // those slots never compete as victims.)
    constexpr int kEPerThread = kMaxExperts / kCtrlThreads;
    int sfi[kEPerThread];
#pragma unroll
    for (int j = 0; j < kEPerThread; ++j) {
        const int e = tid + j * kCtrlThreads;
        sfi[j] = e < E ? a.slot_for_id[(int64_t)a.layer * E + e] : -1;
    }
    uint64_t pst[KPT];
    int pown[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int s = tid + j * kCtrlThreads;
        pst[j] = s < N ? a.stamp[s] : 0;
        pown[j] = s < N ? a.id_of_slot[s] : -1;
    }

    // A call replayed from a graph captured before ft_cache_resize: its slot
    // count and pool are gone.  It changes nothing but its routes, which all
    // become INT32_MIN (so the rest of the call has no expert to run), and
    // raises error flag 16.  The loads above stay within the maps, which
    // resize never reallocates.
    if (gen_now != a.gen) {
        for (int r = tid; r < R; r += kCtrlThreads) a.ids[r] = INT32_MIN;
        if (tid < 4) {
            a.wl_counts[tid] = 0;
            if (a.o_counts) a.o_counts[tid] = 0;
        }
        if (tid == 0) atomicOr(a.errflag, 16);
        return;
    }

    for (int i = tid; i < ewords; i += kCtrlThreads) ebits[i] = 0;
    for (int i = tid; i < nwords; i += kCtrlThreads) hitbits[i] = 0;
    if (tid == 0) sh_evict = 0;
    __syncthreads();

    // 1. mark the routed experts (dedupe)
    for (int r = tid; r < R; r += kCtrlThreads) {
        int e = a.ids[r];
        if (e < 0 || e >= E) {
            atomicOr(a.errflag, 1);
        } else {
            atomicOr(&ebits[e >> 5], 1u << (e & 31));
        }
    }
    __syncthreads();

    // 2. ascending compaction: prefix popcount over the bitmap words
    if (wid == 0) {
        int c0 = (2 * lane < ewords) ? __popc(ebits[2 * lane]) : 0;
        int c1 = (2 * lane + 1 < ewords) ? __popc(ebits[2 * lane + 1]) : 0;
        int incl = wave_incl_scan(c0 + c1, lane);
        int excl = incl - c0 - c1;
        if (2 * lane < ewords) wordbase[2 * lane] = excl;
        if (2 * lane + 1 < ewords) wordbase[2 * lane + 1] = excl + c0;
        if (lane == 63) sh_nuniq = incl;
    }
    __syncthreads();
    const int nu = sh_nuniq;

    // 3. unique index of every routed expert, and its residency
#pragma unroll
    for (int j = 0; j < kEPerThread; ++j) {
        const int e = tid + j * kCtrlThreads;
        if (e >= E) break;
        uint32_t wv = ebits[e >> 5];
        if (wv & (1u << (e & 31))) {
            int idx = wordbase[e >> 5] + __popc(wv & ((1u << (e & 31)) - 1u));
            pos_of_e[e] = (int16_t)idx;
            e_of_u[idx] = (int16_t)e;
            const int s = sfi[j];
            uslot[idx] = (s >= 0 && s < N) ? s : -1;
        }
    }
    __syncthreads();

    // 4. ranks among hits (ascending) and the ordered miss list
    const int per = (nu + kCtrlThreads - 1) / kCtrlThreads;   // <= 4
    const int i0 = tid * per;
    int myhits = 0;
    for (int j = 0; j < per; ++j) {
        int i = i0 + j;
        if (i < nu && uslot[i] >= 0) ++myhits;
    }
    int htot;
    int hb = block_excl_scan(myhits, wsum, &htot);
    const int h = htot, m = nu - htot;
    const int q = fill_count(m, h, N, bp, bh, max_fetch);
    for (int j = 0; j < per; ++j) {
        int i = i0 + j;
        if (i >= nu) break;
        int s = uslot[i];
        if (s >= 0) {                       // hit: refresh recency, protect the slot
            a.stamp[s] = clk + (uint64_t)hb;
            atomicOr(&hitbits[s >> 5], 1u << (s & 31));
            ucls[i] = FT_HIT;
            ++hb;
        } else {
            int mr = i - hb;                 // rank among misses
            miss_list[mr] = (int16_t)i;
        }
    }
    __syncthreads();

    // 5. one scan of the slots: each thread keeps its (stamp, slot) keys; the
    //    q smallest keys among slots not hit in this call are the victims
    if (q > 0) {
        uint64_t keys[KPT];
        uint64_t lmin = ~0ull;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            int s = tid + j * kCtrlThreads;
            uint64_t k = ~0ull;
            if (s < N && !(hitbits[s >> 5] & (1u << (s & 31)))) {
                uint64_t st = pst[j];
                if (st >= kStampLimit) st = kStampLimit - 1;
                k = (st << 24) | (uint64_t)s;
            }
            keys[j] = k;
            lmin = k < lmin ? k : lmin;
        }
        for (int i = 0; i < q; ++i) {
            uint64_t v = lmin;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                uint64_t o = shfl_xor_u64(v, off);
                v = o < v ? o : v;
            }
            if (lane == 0) wmin[i & 1][wid] = v;
            __syncthreads();
            uint64_t g = ~0ull;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                uint64_t o = wmin[i & 1][w];
                g = o < g ? o : g;
            }
            if (tid == 0) victims[i] = (int16_t)(g & 0xFFFFFFu);
            if (lmin == g) {
                uint64_t nm = ~0ull;
#pragma unroll
                for (int j = 0; j < KPT; ++j) {
                    uint64_t k = keys[j];
                    if (k == g && g != ~0ull) victim_old[i] = pown[j];   // keys are unique (slot in the low bits)
                    if (k > g && k < nm) nm = k;
                }
                lmin = nm;
            }
        }
    }
    __syncthreads();

    // 6. admit the first q misses into the victims; the rest run on the host
    for (int r = tid; r < m; r += kCtrlThreads) {
        int i = miss_list[r];
        int e = e_of_u[i];
        int32_t u = a.layer * E + e;
        if (r < q) {
            int v = victims[r];
            int old = victim_old[r];
            if (old >= 0) {
                a.slot_for_id[old] = -1;
                atomicAdd(&sh_evict, 1);
            }
            a.id_of_slot[v] = u;
            a.slot_for_id[u] = v;
            a.stamp[v] = clk + (uint64_t)(h + r);
            uslot[i] = v;
            ucls[i] = FT_FILL;
            a.wl_slot[r] = v;
            a.wl_src[r] = u;
            if (a.o_ev_slot) a.o_ev_slot[r] = v;
            if (a.o_ev_old) a.o_ev_old[r] = old;
            if (a.o_ev_new) a.o_ev_new[r] = u;
        } else {
            uslot[i] = -1;
            ucls[i] = FT_CPU;
            if (a.o_cpu) a.o_cpu[r - q] = u;
        }
    }
    __syncthreads();

    // 7. outputs and the in-place route rewrite
    for (int i = tid; i < nu; i += kCtrlThreads) {
        if (a.o_uniq) a.o_uniq[i] = a.layer * E + e_of_u[i];
        if (a.o_cls) a.o_cls[i] = ucls[i];
        if (a.o_slot) a.o_slot[i] = uslot[i];
    }
    for (int r = tid; r < R; r += kCtrlThreads) {
        int e = a.ids[r];
        int out;
        if (e < 0 || e >= E) {
            out = INT32_MIN;
        } else {
            int s = uslot[pos_of_e[e]];
            out = s >= 0 ? s : -(1 + e);
        }
        a.ids[r] = out;
    }
    if (tid == 0) {
        if (a.o_counts) {
            a.o_counts[0] = nu;
            a.o_counts[1] = h;
            a.o_counts[2] = m;
            a.o_counts[3] = q;
        }
        a.wl_counts[0] = nu;
        a.wl_counts[1] = h;
        a.wl_counts[2] = m;
        a.wl_counts[3] = q;
        uint64_t nc = clk + (uint64_t)(h + q);
        if (nc >= kStampLimit) atomicOr(a.errflag, 2);
        *a.clock = nc;
        atomicAdd(&a.counters[C_CALLS], 1ull);
        atomicAdd(&a.counters[C_ROUTES], (unsigned long long)R);
        atomicAdd(&a.counters[C_UNIQUE], (unsigned long long)nu);
        atomicAdd(&a.counters[C_HITS], (unsigned long long)h);
        atomicAdd(&a.counters[C_MISSES], (unsigned long long)m);
        atomicAdd(&a.counters[C_FILLS], (unsigned long long)q);
        atomicAdd(&a.counters[C_CPU], (unsigned long long)(m - q));
        atomicAdd(&a.counters[C_EVICT], (unsigned long long)sh_evict);
        atomicAdd(&a.counters[C_BYTES], (unsigned long long)q * (unsigned long long)a.S);
    }
}

// The decode fill as a kernel of its own (the planner's launch carries it
// when the call posts to the host branch through a mailbox).
constexpr int kFillThreads = 256;
constexpr int kFillBlocks = 512;

__global__ void __launch_bounds__(kFillThreads)
    fill_kernel(const int32_t* wl_counts, const int32_t* wl_slot, const int32_t* wl_src,
                const uint8_t* const* __restrict__ banks, int E, uint8_t* __restrict__ pool, int64_t S, int64_t P) {
    fill_records<kFillThreads>(wl_counts, wl_slot, wl_src, banks, E, pool, S, P, blockIdx.x, gridDim.x);
}

// Clear the owners of full-layer buffer slots [s0, s0 + E) before a layer is
// copied in: the old flat ids become absent and the slots empty.
__global__ void invalidate_kernel(int32_t s0, int32_t E, int32_t* slot_for_id, int32_t* id_of_slot,
                                  uint64_t* stamp, unsigned long long* counters) {
    for (int i = threadIdx.x; i < E; i += blockDim.x) {
        int s = s0 + i;
        int old = id_of_slot[s];
        if (old >= 0) slot_for_id[old] = -1;
        id_of_slot[s] = -1;
        stamp[s] = 0;
    }
    if (threadIdx.x == 0) atomicAdd(&counters[C_STREAMED], 1ull);
}

// Prefill-warms-decode variant: the layer just computed from a full-layer
// buffer (slots s0 .. s0 + E - 1, expert e in slot s0 + e) becomes a set of
// decode residents.  Expert e is registered when it is resident nowhere and
// its buffer slot is free (the load cleared it), with stamp clock + e; the
// clock then advances by E.  One workgroup; the flat ids are distinct, so the
// threads touch distinct entries.
__global__ void register_kernel(int32_t layer, int32_t s0, int32_t E, int32_t* slot_for_id, int32_t* id_of_slot,
                                uint64_t* stamp, uint64_t* clock, int32_t* errflag) {
    __shared__ uint64_t clk;
    if (threadIdx.x == 0) clk = *clock;
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int32_t u = layer * E + e, s = s0 + e;
        if (slot_for_id[u] < 0 && id_of_slot[s] < 0) {
            slot_for_id[u] = s;
            id_of_slot[s] = u;
            stamp[s] = clk + (uint64_t)e;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint64_t nc = clk + (uint64_t)E;
        if (nc >= kStampLimit) atomicOr(errflag, 2);
        *clock = nc;
    }
}

// new_pool[i] = old_pool[src_slots[i]] for i < n (whole slots of P bytes, P a
// multiple of 256).
__global__ void __launch_bounds__(kFillThreads)
    gather_kernel(const uint8_t* __restrict__ old_pool, uint8_t* __restrict__ new_pool, int64_t P,
                  const int32_t* src_slots, int n) {
    const int64_t cpr = (P + kFillChunk - 1) / kFillChunk;
    const int64_t total = (int64_t)n * cpr;
    for (int64_t c = blockIdx.x; c < total; c += gridDim.x) {
        const int64_t i = c / cpr;
        const int64_t off = (c - i * cpr) * kFillChunk;
        const int64_t len = (P - off) < kFillChunk ? (P - off) : kFillChunk;
        const uint4* src = reinterpret_cast<const uint4*>(old_pool + (int64_t)src_slots[i] * P + off);
        uint4* dst = reinterpret_cast<uint4*>(new_pool + i * P + off);
        for (int64_t b = threadIdx.x; b < len / 16; b += kFillThreads) dst[b] = src[b];
    }
}

}  // namespace

hipError_t launch_classify(ft_cache* c, int32_t layer, int32_t* ids, int32_t R, const ft_classify_out* out,
                           hipStream_t st) {
    CtrlArgs a;
    a.ids = ids;
    a.R = R;
    a.layer = layer;
    a.E = c->sh.experts;
    a.N = (int32_t)c->N;
    a.slot_for_id = c->slot_for_id;
    a.id_of_slot = c->id_of_slot;
    a.stamp = c->stamp;
    a.clock = c->clock;
    a.counters = c->counters;
    a.errflag = c->errflag;
    a.ds = c->dstate;
    a.gen = c->gen;
    a.S = c->rl.S;
    a.o_counts = out ? out->counts : nullptr;
    a.o_uniq = out ? out->uniq : nullptr;
    a.o_cls = out ? out->cls : nullptr;
    a.o_slot = out ? out->slot : nullptr;
    a.o_ev_slot = out ? out->ev_slot : nullptr;
    a.o_ev_old = out ? out->ev_old : nullptr;
    a.o_ev_new = out ? out->ev_new : nullptr;
    a.o_cpu = out ? out->cpu_ids : nullptr;
    a.wl_counts = c->wl_counts;
    a.wl_slot = c->wl_slot;
    a.wl_src = c->wl_src;
    const int kpt = (a.N + kCtrlThreads - 1) / kCtrlThreads;
    if (kpt <= 1) hipLaunchKernelGGL(classify_kernel<1>, dim3(1), dim3(kCtrlThreads), 0, st, a);
    else if (kpt <= 2) hipLaunchKernelGGL(classify_kernel<2>, dim3(1), dim3(kCtrlThreads), 0, st, a);
    else if (kpt <= 4) hipLaunchKernelGGL(classify_kernel<4>, dim3(1), dim3(kCtrlThreads), 0, st, a);
    else if (kpt <= 8) hipLaunchKernelGGL(classify_kernel<8>, dim3(1), dim3(kCtrlThreads), 0, st, a);
    else if (kpt <= 16) hipLaunchKernelGGL(classify_kernel<16>, dim3(1), dim3(kCtrlThreads), 0, st, a);
    else hipLaunchKernelGGL(classify_kernel<kKeysPerThread>, dim3(1), dim3(kCtrlThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_fill(ft_cache* c, hipStream_t st, TimedLaunch tl) {
    hipExtLaunchKernelGGL(fill_kernel, dim3(kFillBlocks), dim3(kFillThreads), 0, st, tl.start, tl.stop, 0,
                          (const int32_t*)c->wl_counts, (const int32_t*)c->wl_slot, (const int32_t*)c->wl_src,
                          (const uint8_t* const*)c->bank_dev, (int)c->sh.experts, c->pool, c->rl.S, c->rl.P);
    return hipGetLastError();
}

hipError_t launch_invalidate(ft_cache* c, int buf, hipStream_t st) {
    hipLaunchKernelGGL(invalidate_kernel, dim3(1), dim3(256), 0, st, (int32_t)(buf * c->sh.experts),
                       (int32_t)c->sh.experts, c->slot_for_id, c->id_of_slot, c->stamp, c->counters);
    return hipGetLastError();
}

hipError_t launch_register(ft_cache* c, int layer, int buf, hipStream_t st) {
    hipLaunchKernelGGL(register_kernel, dim3(1), dim3(256), 0, st, (int32_t)layer, (int32_t)(buf * c->sh.experts),
                       (int32_t)c->sh.experts, c->slot_for_id, c->id_of_slot, c->stamp, c->clock, c->errflag);
    return hipGetLastError();
}

hipError_t launch_resize_gather(const uint8_t* old_pool, uint8_t* new_pool, int64_t P, const int32_t* src_slots,
                                int n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(gather_kernel, dim3(kFillBlocks), dim3(kFillThreads), 0, st, old_pool, new_pool, P,
                       src_slots, n);
    return hipGetLastError();
}

}  // namespace ftmoe
