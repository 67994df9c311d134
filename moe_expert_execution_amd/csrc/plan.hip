// Token-to-slot sort/scan that builds the expert kernels' work lists.
//
// Input: routes [T x k] (slot ids for GPU routes; negative = host or invalid;
// or, for a full-layer buffer, raw expert ids mapped to slot base + e).
// Output (PlanBuffers): the GPU rows sorted by (slot, route index) — a stable
// counting sort — with
//   perm[p]        route index of sorted row p
//   route_pos[r]   sorted row of route r, -1 when r is not a GPU route
//   active_slot[a] the a-th slot with rows, ascending
//   seg[a]         first sorted row of active slot a (seg[n_active] = rows)
//   tile_active / tile_row0: BM-row tiles of each active slot
//   meta           {n_active, n_tiles, n_rows}
// A token that lists the same expert twice keeps only its first route; the
// duplicate is dropped and error flag 4 is raised.
//
// Up to 1024 routes: one workgroup, bitonic sort of (slot, route) keys.
// More: three kernels over 64-token chunks — per-chunk slot masks and counts,
// one scan, then rank = chunk offset + popcount(mask below the token).
#include "common.h"
#include "decode_wg.h"
#include "fill.h"

namespace ftmoe {
namespace {

constexpr int kPlanThreads = 1024;

struct PlanArgs {
    const int32_t* routes;
    int32_t R, k, T;
    int32_t slot_base;      // >= 0: routes are expert ids, slot = base + e
    int32_t E;              // expert count (validates raw ids)
    int32_t N;              // slots
    int32_t bm;             // tile rows
    int32_t key_space;      // large planner: keys 0..key_space-1
    int32_t* errflag;
    int32_t* meta;
    int32_t* active_slot;
    int32_t* seg;
    int32_t* perm;
    int32_t* route_pos;
    int32_t* tile_active;
    int32_t* tile_row0;
    int32_t* tile_first;
    int32_t* chunk_counts;
    unsigned long long* work;   // [2]: active slots, rows (accumulated)
    // host-branch staging (pinned, device-visible; null = none): the call's
    // routes, weights and activations for the host workers
    const float* w;
    const uint16_t* x;
    int32_t d;
    int32_t* h_routes;
    float* h_w;
    uint16_t* h_x;
    uint64_t* seq_word;      // mailbox: store seq here once staging is visible (null = none)
    uint64_t seq;
    uint64_t* gmbox;         // graph mailbox words (null = none)
    uint64_t* gseq_dev;      // device counter of graph calls
    int32_t glayer;
};

// Post the call to the host branch's mailbox after the staging writes of the
// whole workgroup (system-scope release).
__device__ __forceinline__ void post_mailbox(const PlanArgs& a) {
    if (a.seq_word && threadIdx.x == 0) {
        __threadfence_system();
        __hip_atomic_store(a.seq_word, a.seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    if (a.gmbox && threadIdx.x == 0) {
        const uint64_t n = *a.gseq_dev + 1;          // calls on one stream run in order
        *a.gseq_dev = n;
        __hip_atomic_store(a.gmbox + 16, (uint64_t)a.glayer, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(a.gmbox + 17, (uint64_t)a.T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __threadfence_system();
        __hip_atomic_store(a.gmbox, n, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// Copy routes, weights and activations of the call into pinned host staging
// (zero-copy writes over PCIe) with the whole workgroup / grid.
__device__ __forceinline__ void stage_to_host(const PlanArgs& a, int tid, int nthr) {
    for (int r = tid; r < a.R; r += nthr) {
        a.h_routes[r] = a.routes[r];
        a.h_w[r] = a.w[r];
    }
    const int nx = a.T * a.d / 8;   // 16-byte chunks (d % 128 == 0)
    const uint4* xs = reinterpret_cast<const uint4*>(a.x);
    uint4* xd = reinterpret_cast<uint4*>(a.h_x);
    for (int i = tid; i < nx; i += nthr) xd[i] = xs[i];
}

// Slot of route r, or -1 when it is not a GPU route (host, invalid, duplicate).
// A value that is neither a route of the call's mode nor INT32_MIN (the mark
// classify leaves on an id it already flagged) raises error flag 1 and is
// ignored, as the host branch and the combine ignore it.
__device__ __forceinline__ int route_slot(const PlanArgs& a, int r) {
    int v = a.routes[r];
    int s;
    bool ok;
    if (a.slot_base >= 0) {            // raw expert ids of a full-layer buffer
        ok = v >= 0 && v < a.E;
        s = ok ? a.slot_base + v : -1;
    } else {                           // slot ids, or host routes -(1 + e)
        ok = (v >= 0 && v < a.N) || (v < 0 && v >= -a.E);
        s = (v >= 0 && v < a.N) ? v : -1;
    }
    if (!ok && v != INT32_MIN) atomicOr(a.errflag, 1);
    if (s < 0) return -1;
    const int t = r / a.k, j = r - t * a.k;
    for (int jj = 0; jj < j; ++jj) {          // drop a repeated expert of the same token
        if (a.routes[t * a.k + jj] == v) {
            atomicOr(a.errflag, 4);
            return -1;
        }
    }
    return s;
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int* total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int incl = wave_incl_scan(v, lane);
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    int base = 0, tot = 0;
    for (int i = 0; i < kPlanThreads / 64; ++i) {
        int s = wsum[i];
        base += (i < wid) ? s : 0;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

// Tiles of every active slot, in order.  Thread i handles active i.
__device__ void emit_tiles(const PlanArgs& a, int n_active, int* wsum) {
    int total_tiles = 0;
    for (int base = 0; base < n_active; base += kPlanThreads) {
        const int i = base + threadIdx.x;
        int nt = 0, rows = 0, r0 = 0;
        if (i < n_active) {
            r0 = a.seg[i];
            rows = a.seg[i + 1] - r0;
            nt = (rows + a.bm - 1) / a.bm;
        }
        int tot;
        int off = block_excl_scan(nt, wsum, &tot) + total_tiles;
        if (i < n_active) a.tile_first[i] = off;
        for (int j = 0; j < nt; ++j) {
            a.tile_active[off + j] = i;
            a.tile_row0[off + j] = r0 + j * a.bm;
        }
        total_tiles += tot;
    }
    if (threadIdx.x == 0) {
        a.meta[1] = total_tiles;
        a.tile_first[n_active] = total_tiles;
    }
}

// ---- one-workgroup planner (R <= 1024) ------------------------------------------
__device__ __forceinline__ void plan_small(const PlanArgs& a) {
    __shared__ uint32_t keys[kSmallPlanRoutes];
    __shared__ int wsum[kPlanThreads / 64];
    const int tid = threadIdx.x;
    if (a.h_routes) {
        stage_to_host(a, tid, kPlanThreads);
        __syncthreads();
        post_mailbox(a);
    }
    int P = 1;
    while (P < a.R) P <<= 1;

    // key = slot << 10 | route (slot < 32768, route < 1024); non-GPU routes last
    if (tid < P) {
        uint32_t key = 0xFFFFFFFFu;
        if (tid < a.R) {
            int s = route_slot(a, tid);
            if (s >= 0) key = ((uint32_t)s << 10) | (uint32_t)tid;
            a.route_pos[tid] = -1;
        }
        keys[tid] = key;
    }
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (tid < P) {
                int partner = tid ^ stride;
                if (partner > tid) {
                    uint32_t x = keys[tid], y = keys[partner];
                    bool up = (tid & size) == 0;
                    if ((x > y) == up) {
                        keys[tid] = y;
                        keys[partner] = x;
                    }
                }
            }
            __syncthreads();
        }
    }
    // rows, heads, active list
    int valid = (tid < a.R && keys[tid] != 0xFFFFFFFFu) ? 1 : 0;
    int rows;
    block_excl_scan(valid, wsum, &rows);
    int head = 0;
    if (valid) {
        uint32_t kk = keys[tid];
        int r = (int)(kk & 1023u);
        a.perm[tid] = r;
        a.route_pos[r] = tid;
        head = (tid == 0 || (keys[tid - 1] >> 10) != (kk >> 10)) ? 1 : 0;
    }
    int n_active;
    int ai = block_excl_scan(head, wsum, &n_active);
    if (head) {
        a.active_slot[ai] = (int)(keys[tid] >> 10);
        a.seg[ai] = tid;
    }
    if (tid == 0) {
        a.seg[n_active] = rows;
        a.meta[0] = n_active;
        a.meta[2] = rows;
        atomicAdd(&a.work[0], (unsigned long long)n_active);
        atomicAdd(&a.work[1], (unsigned long long)rows);
    }
    __syncthreads();
    emit_tiles(a, n_active, wsum);
}

__global__ void __launch_bounds__(kPlanThreads) plan_small_kernel(PlanArgs a) { plan_small(a); }

struct FillArgs {
    const int32_t* wl_counts;
    const int32_t* wl_slot;
    const int32_t* wl_src;
    const uint8_t* const* banks;   // device addresses of each layer's host bank
    int E;
    uint8_t* pool;
    int64_t S, P;   // bank record stride, pool slot stride
};
constexpr int kPlanFillBlocks = 512;   // fill workgroups of kPlanThreads beside the planner: one 64 KiB chunk each for q <= 3 at decode sizes

// The planner and the call's fill in one launch: workgroup 0 plans, the next
// kPlanFillBlocks pull the filled records.  Neither reads what the other
// writes (the plan reads the routes, the fill the worklist; classify wrote
// both), and the planner's few microseconds disappear under the PCIe pull.
// DECODE: the workgroups after them run the one-token decode kernel for the
// GPU routes whose slots this call does not fill (hits), beside the pull; the
// filled routes' workgroups follow in the next launch.
constexpr int kDecFillWaves = kPlanThreads / 64;   // the decode workgroups use all 16 waves (fewer loads per lane)
template <int FMT, bool DECODE>
__global__ void __launch_bounds__(kPlanThreads) plan_fill_kernel(PlanArgs a, FillArgs f, DecodeArgs da) {
    if (blockIdx.x == 0) {
        plan_small(a);
        return;
    }
    if (blockIdx.x <= kPlanFillBlocks) {
        // 256 threads per workgroup pull, as in the fill kernel: a workgroup's
        // host reads in flight set the PCIe rate
        if (threadIdx.x < 256)
            fill_records<256>(f.wl_counts, f.wl_slot, f.wl_src, f.banks, f.E, f.pool, f.S, f.P, blockIdx.x - 1,
                              kPlanFillBlocks);
        return;
    }
    if constexpr (DECODE) {
        extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
        decode_route_group<FMT, kDecFillWaves, DecodeShape<FMT>::BU16, DEC_HITS>(da, blockIdx.x - 1 - kPlanFillBlocks, xs);
    }
}

template <int FMT, bool DECODE>
void launch_plan_fill(const PlanArgs& a, const FillArgs& f, const DecodeArgs& da, const TimedLaunch* fill,
                      hipStream_t st) {
    const unsigned grid = 1 + kPlanFillBlocks + (DECODE ? (unsigned)(da.k * (da.f / DecodeShape<FMT>::NPW)) : 0u);
    const size_t lds = DECODE ? decode_lds_bytes(da.d) : 0;
    hipExtLaunchKernelGGL((plan_fill_kernel<FMT, DECODE>), dim3(grid), dim3(kPlanThreads), lds, st, fill->start,
                          fill->stop, 0, a, f, da);
}

// ---- chunked planner (any R; key space <= 8192) --------------------------------
// Kernel A: per 64-token chunk, the mask of tokens routed to each key, and its popcount.
__global__ void __launch_bounds__(kPlanThreads) plan_count_kernel(PlanArgs a) {
    __shared__ unsigned long long mask[kLargeKeySpace];
    const int c = blockIdx.x, K = a.key_space;
    for (int i = threadIdx.x; i < K; i += kPlanThreads) mask[i] = 0ull;
    __syncthreads();
    const int r = c * kChunkTokens * a.k + threadIdx.x;
    if (threadIdx.x < kChunkTokens * a.k && r < a.R) {
        int s = route_slot(a, r);
        if (s >= 0) {
            int key = a.slot_base >= 0 ? s - a.slot_base : s;
            atomicOr(&mask[key], 1ull << (threadIdx.x / a.k));
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < K; i += kPlanThreads)
        a.chunk_counts[(int64_t)c * K + i] = __popcll(mask[i]);
}

// Kernel B: per-key totals, segment starts, per-chunk offsets, active list, tiles.
// G threads share a key (each sums a contiguous range of chunks); keys are
// processed in ascending passes of 1024 / G.
__global__ void __launch_bounds__(kPlanThreads) plan_scan_kernel(PlanArgs a, int nchunks) {
    post_mailbox(a);   // the staging kernel ran earlier on this stream
    __shared__ int part[kPlanThreads];
    __shared__ int kstart[kPlanThreads];
    __shared__ int kact[kPlanThreads];
    __shared__ int wsum[kPlanThreads / 64];
    const int tid = threadIdx.x, K = a.key_space;
    int G = 1;
    while (G * 2 * K <= kPlanThreads) G *= 2;
    const int kpp = kPlanThreads / G;
    const int cpg = (nchunks + G - 1) / G;
    const int g = tid % G;
    const int c0 = g * cpg, c1 = (c0 + cpg) < nchunks ? (c0 + cpg) : nchunks;
    int run_rows = 0, run_active = 0;
    for (int kb = 0; kb < K; kb += kpp) {
        const int key = kb + tid / G;
        int s = 0;
        if (key < K)
            for (int c = c0; c < c1; ++c) s += a.chunk_counts[(int64_t)c * K + key];
        part[tid] = s;
        __syncthreads();
        const int gb = tid - g;
        int pre = 0, tot = 0;
        for (int i = 0; i < G; ++i) {
            int v = part[gb + i];
            pre += (i < g) ? v : 0;
            tot += v;
        }
        const bool lead = (g == 0) && key < K;
        int pass_rows, pass_active;
        int ex = block_excl_scan(lead ? tot : 0, wsum, &pass_rows);
        int ax = block_excl_scan((lead && tot > 0) ? 1 : 0, wsum, &pass_active);
        if (g == 0) {
            kstart[tid / G] = run_rows + ex;
            kact[tid / G] = run_active + ax;
        }
        __syncthreads();
        if (key < K) {
            const int start = kstart[tid / G];
            int off = start + pre;
            for (int c = c0; c < c1; ++c) {
                int64_t o = (int64_t)c * K + key;
                int cnt = a.chunk_counts[o];
                a.chunk_counts[o] = off;     // counts become offsets
                off += cnt;
            }
            if (lead && tot > 0) {
                const int ai = kact[tid / G];
                a.active_slot[ai] = a.slot_base >= 0 ? a.slot_base + key : key;
                a.seg[ai] = start;
            }
        }
        run_rows += pass_rows;
        run_active += pass_active;
        __syncthreads();
    }
    if (tid == 0) {
        a.seg[run_active] = run_rows;
        a.meta[0] = run_active;
        a.meta[2] = run_rows;
        atomicAdd(&a.work[0], (unsigned long long)run_active);
        atomicAdd(&a.work[1], (unsigned long long)run_rows);
    }
    __syncthreads();
    emit_tiles(a, run_active, wsum);
}

// Host staging for the chunked planner's calls.
__global__ void __launch_bounds__(256) stage_kernel(PlanArgs a) {
    stage_to_host(a, blockIdx.x * 256 + threadIdx.x, gridDim.x * 256);
}

// Kernel C: stable scatter.
__global__ void __launch_bounds__(kPlanThreads) plan_scatter_kernel(PlanArgs a) {
    __shared__ unsigned long long mask[kLargeKeySpace];
    const int c = blockIdx.x, K = a.key_space;
    for (int i = threadIdx.x; i < K; i += kPlanThreads) mask[i] = 0ull;
    __syncthreads();
    const int r = c * kChunkTokens * a.k + threadIdx.x;
    const bool mine = threadIdx.x < kChunkTokens * a.k && r < a.R;
    int key = -1, tl = 0;
    if (mine) {
        int s = route_slot(a, r);
        if (s >= 0) {
            key = a.slot_base >= 0 ? s - a.slot_base : s;
            tl = threadIdx.x / a.k;
            atomicOr(&mask[key], 1ull << tl);
        }
    }
    __syncthreads();
    if (mine) {
        if (key >= 0) {
            unsigned long long below = tl ? (mask[key] & ((1ull << tl) - 1ull)) : 0ull;
            int p = a.chunk_counts[(int64_t)c * K + key] + __popcll(below);
            a.perm[p] = r;
            a.route_pos[r] = p;
        } else {
            a.route_pos[r] = -1;
        }
    }
}

}  // namespace

hipError_t launch_plan(ft_cache* c, const int32_t* routes, int T, int slot_base, int bm, int work_counter,
                       const float* w, const uint16_t* x, const HostStaging* stage, const HostSignal* sig,
                       hipStream_t st, const TimedLaunch* fill, bool decode_hits) {
    PlanArgs a;
    a.seq_word = (sig && sig->mailbox) ? sig->seq_word : nullptr;
    a.seq = sig ? sig->seq : 0;
    a.gmbox = sig ? sig->gmbox : nullptr;
    a.gseq_dev = sig ? sig->gseq_dev : nullptr;
    a.glayer = sig ? sig->layer : 0;
    a.w = w;
    a.x = x;
    a.d = c->sh.d_model;
    a.h_routes = stage ? stage->routes : nullptr;
    a.h_w = stage ? stage->w : nullptr;
    a.h_x = stage ? stage->x : nullptr;
    a.routes = routes;
    a.k = c->sh.top_k;
    a.T = T;
    a.R = T * a.k;
    a.slot_base = slot_base;
    a.E = c->sh.experts;
    a.N = (int32_t)c->N;
    a.bm = bm;
    a.key_space = slot_base >= 0 ? c->sh.experts : (int32_t)c->N;
    a.errflag = c->errflag;
    a.meta = c->plan.meta;
    a.active_slot = c->plan.active_slot;
    a.seg = c->plan.seg;
    a.perm = c->plan.perm;
    a.route_pos = c->plan.route_pos;
    a.tile_active = c->plan.tile_active;
    a.tile_row0 = c->plan.tile_row0;
    a.tile_first = c->plan.tile_first;
    a.chunk_counts = c->plan.chunk_counts;
    a.work = c->counters + work_counter;
    if (fill) {
        if (a.R > kSmallPlanRoutes) return hipErrorInvalidValue;
        FillArgs f{c->wl_counts, c->wl_slot, c->wl_src, (const uint8_t* const*)c->bank_dev, (int)c->sh.experts,
                   c->pool, c->rl.S, c->rl.P};
        if (decode_hits && (T != 1 || !c->dpart)) return hipErrorInvalidValue;
        const DecodeArgs da = decode_args(c, x, routes);
        switch (decode_hits ? c->sh.fmt : -1) {
            case FT_FMT_BF16: launch_plan_fill<FT_FMT_BF16, true>(a, f, da, fill, st); break;
            case FT_FMT_FP8_B128: launch_plan_fill<FT_FMT_FP8_B128, true>(a, f, da, fill, st); break;
            case FT_FMT_MXFP4_B32: launch_plan_fill<FT_FMT_MXFP4_B32, true>(a, f, da, fill, st); break;
            default: launch_plan_fill<FT_FMT_BF16, false>(a, f, da, fill, st); break;
        }
    } else if (a.R <= kSmallPlanRoutes) {
        hipLaunchKernelGGL(plan_small_kernel, dim3(1), dim3(kPlanThreads), 0, st, a);
    } else {
        if (a.key_space > kLargeKeySpace) return hipErrorInvalidValue;
        int nchunks = (T + kChunkTokens - 1) / kChunkTokens;
        if (stage) hipLaunchKernelGGL(stage_kernel, dim3(256), dim3(256), 0, st, a);
        hipLaunchKernelGGL(plan_count_kernel, dim3(nchunks), dim3(kPlanThreads), 0, st, a);
        hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a, nchunks);
        hipLaunchKernelGGL(plan_scatter_kernel, dim3(nchunks), dim3(kPlanThreads), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace ftmoe
