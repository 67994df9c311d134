// Weighted top-k combine: y[t] = sum over the token's GPU routes, j ascending,
// of w[t,j] * Y[row(t,j)] (bf16 expert outputs), plus the host branch's partial
// sum P[t] when the token has a host route -(1+e), 0 <= e < E (the routes the
// host branch runs and whose P rows it writes); accumulated in fp32 and
// rounded once to bf16.  The GPU and host partial outputs merge into the layer output
// (METAL MEDIA summary, Figure 2 caption; hyper.ai summary, section 方法).
#include "wfmt.h"

namespace ftmoe {
namespace {

constexpr int kCombThreads = 256;

// With `done`, each workgroup first waits until the host branch has answered
// the call: *done (pinned memory) reaches the call's number — `seq`, or
// *seq_dev when the number is drawn on the device (graph calls).  The wait is
// bounded: past `limit` polls it raises error flag 8 and goes on, so every
// wave ends.
__global__ void __launch_bounds__(kCombThreads)
    combine_kernel(const int32_t* __restrict__ routes, const int32_t* __restrict__ route_pos,
                   const float* __restrict__ w, const uint16_t* __restrict__ Y, const float* P, int T, int k, int d, int E,
                   uint16_t* __restrict__ y, const uint64_t* done, const uint64_t* seq_dev, uint64_t seq,
                   uint32_t limit, int32_t* errflag) {
    if (done) {
        if (threadIdx.x == 0) {
            const uint64_t n = seq_dev ? *seq_dev : seq;
            for (uint32_t it = 0; __hip_atomic_load(done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) < n; ++it) {
                if (it >= limit) {
                    atomicOr(errflag, 8);
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
        }
        __syncthreads();
    }
    const int t = blockIdx.y;
    const int c = (blockIdx.x * kCombThreads + threadIdx.x) * 4;
    if (t >= T || c >= d) return;
    // the token's route metadata first, then all its expert rows at once
    // (a route not run on the GPU loads row 0 and adds nothing)
    int rp[kMaxTopK], rv[kMaxTopK];
    float wj[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
        if (j < k) {
            const int r = t * k + j;
            rp[j] = route_pos[r];
            rv[j] = routes[r];
            wj[j] = w[r];
        }
    uint2 v[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
        if (j < k) v[j] = *reinterpret_cast<const uint2*>(Y + (int64_t)(rp[j] > 0 ? rp[j] : 0) * d + c);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    bool host = false;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
        if (j < k) {
            if (rp[j] >= 0) {
                acc.x = fmaf(wj[j], bf16lo(v[j].x), acc.x);
                acc.y = fmaf(wj[j], bf16hi(v[j].x), acc.y);
                acc.z = fmaf(wj[j], bf16lo(v[j].y), acc.z);
                acc.w = fmaf(wj[j], bf16hi(v[j].y), acc.w);
            } else {
                host |= (rv[j] < 0 && rv[j] >= -E);
            }
        }
    if (P && host) {
        // pinned host memory written by the host workers: system-scope loads
        const float* p = P + (int64_t)t * d + c;
        acc.x += __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        acc.y += __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        acc.z += __hip_atomic_load(p + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        acc.w += __hip_atomic_load(p + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    uint2 o;
    o.x = (uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
    o.y = (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
    *reinterpret_cast<uint2*>(y + (int64_t)t * d + c) = o;
}

// The one-token decode's combine (decode_wg.h): route j's expert output is
// the sum of its G neuron groups' partial rows part[g][j][0..d).  A
// workgroup covers 64 output columns: 16 column quads x 16 slices of the
// groups; slice s sums groups s, s + 16, ... (at most kCPMaxPerSlice) of
// every GPU route, weighted, and the slices are added in order, so the result
// is deterministic.  Every load is issued at once, and the wait for the host
// branch's answer overlaps them; only the host partial is read after it.
constexpr int kCPSlices = 16;
constexpr int kCPMaxPerSlice = 4;       // groups per slice: G <= 64
__global__ void __launch_bounds__(kCombThreads)
    combine_part_kernel(const int32_t* __restrict__ routes, const int32_t* __restrict__ route_pos,
                        const float* __restrict__ w, const float* __restrict__ part, const float* P, int k, int d,
                        int G, int E, uint16_t* __restrict__ y, const uint64_t* done, const uint64_t* seq_dev,
                        uint64_t seq, uint32_t limit, int32_t* errflag) {
    __shared__ float4 red[kCPSlices][16];
    const int quad = threadIdx.x & 15, sl = threadIdx.x >> 4;
    const int c = blockIdx.x * 64 + quad * 4;
    // partial rows of every route (a route not run on the GPU reads rows it
    // does not add)
    float4 v[kCPMaxPerSlice][kMaxTopK];
#pragma unroll
    for (int i = 0; i < kCPMaxPerSlice; ++i)
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            const int g = sl + i * kCPSlices;
            v[i][j] = (j < k && g < G) ? *reinterpret_cast<const float4*>(part + ((int64_t)g * k + j) * d + c)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    // the route metadata, issued behind the partial rows so that one round
    // trip covers both: lane j of each wave loads route j's, then every route's values are broadcast from their lane
    const int lane = threadIdx.x & 63;
    const int rpl = lane < k ? route_pos[lane] : -1;
    const int rvl = lane < k ? routes[lane] : INT32_MIN;
    const int wl = lane < k ? __float_as_int(w[lane]) : 0;
    int rp[kMaxTopK], rv[kMaxTopK];
    float wj[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        rp[j] = __builtin_amdgcn_readlane(rpl, j);
        rv[j] = __builtin_amdgcn_readlane(rvl, j);
        wj[j] = __int_as_float(__builtin_amdgcn_readlane(wl, j));
    }
    // the first poll of the host's answer goes out behind the loads; polls are
    // relaxed, and one acquire follows once the number is seen (a system-scope
    // acquire invalidates L2 on this part, so it must not sit before the loads)
    uint64_t want = 0, seen = ~0ull;
    if (done && threadIdx.x == 0) {
        want = seq_dev ? *seq_dev : seq;
        seen = __hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    bool host = false;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
        if (j < k) {
            if (rp[j] >= 0) {
                float4 s = v[0][j];
#pragma unroll
                for (int i = 1; i < kCPMaxPerSlice; ++i) {
                    s.x += v[i][j].x;
                    s.y += v[i][j].y;
                    s.z += v[i][j].z;
                    s.w += v[i][j].w;
                }
                acc.x = fmaf(wj[j], s.x, acc.x);
                acc.y = fmaf(wj[j], s.y, acc.y);
                acc.z = fmaf(wj[j], s.z, acc.z);
                acc.w = fmaf(wj[j], s.w, acc.w);
            } else {
                host |= (rv[j] < 0 && rv[j] >= -E);
            }
        }
    red[sl][quad] = acc;
    if (done && threadIdx.x == 0) {
        for (uint32_t it = 0; seen < want; ++it) {
            if (it >= limit) {
                atomicOr(errflag, 8);
                break;
            }
            __builtin_amdgcn_s_sleep(8);
            seen = __hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        // synchronise with the host's release of its number: the host partial
        // sums it wrote before are visible after this (read below only when the
        // call has host experts)
        if (P && host) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
    }
    __syncthreads();
    if (sl == 0) {
        float4 t = red[0][quad];
        for (int s2 = 1; s2 < kCPSlices; ++s2) {
            const float4 u = red[s2][quad];
            t.x += u.x;
            t.y += u.y;
            t.z += u.z;
            t.w += u.w;
        }
        if (P && host) {
            // pinned host memory written by the host workers: system-scope loads
            const float* p = P + c;
            t.x += __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            t.y += __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            t.z += __hip_atomic_load(p + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            t.w += __hip_atomic_load(p + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        uint2 o;
        o.x = (uint32_t)f32_to_bf16_rne(t.x) | ((uint32_t)f32_to_bf16_rne(t.y) << 16);
        o.y = (uint32_t)f32_to_bf16_rne(t.z) | ((uint32_t)f32_to_bf16_rne(t.w) << 16);
        *reinterpret_cast<uint2*>(y + c) = o;
    }
}

}  // namespace

hipError_t launch_combine(ft_cache* c, const int32_t* routes, const float* w, int T, const float* P, uint16_t* y,
                          hipStream_t st, const HostSignal* wait) {
    if (T <= 0) return hipSuccess;
    const int d = c->sh.d_model;
    dim3 grid((d / 4 + kCombThreads - 1) / kCombThreads, T);
    const uint64_t* done = nullptr;
    const uint64_t* seq_dev = nullptr;
    uint64_t seq = 0;
    if (wait && wait->gmbox) {
        done = wait->gmbox + 8;
        seq_dev = wait->gseq_dev;
    } else if (wait && wait->mailbox) {
        done = wait->done_word;
        seq = wait->seq;
    }
    hipLaunchKernelGGL(combine_kernel, grid, dim3(kCombThreads), 0, st, routes, c->plan.route_pos, w, c->Y, P, T,
                       c->sh.top_k, d, c->sh.experts, y, done, seq_dev, seq, c->host_wait_polls, c->errflag);
    return hipGetLastError();
}

hipError_t launch_combine_part(ft_cache* c, const int32_t* routes, const float* w, const float* P, uint16_t* y,
                               hipStream_t st, const HostSignal* wait) {
    const int d = c->sh.d_model;
    const uint64_t* done = nullptr;
    const uint64_t* seq_dev = nullptr;
    uint64_t seq = 0;
    if (wait && wait->gmbox) {
        done = wait->gmbox + 8;
        seq_dev = wait->gseq_dev;
    } else if (wait && wait->mailbox) {
        done = wait->done_word;
        seq = wait->seq;
    }
    hipLaunchKernelGGL(combine_part_kernel, dim3(d / 64), dim3(kCombThreads), 0, st, routes, c->plan.route_pos, w,
                       c->dpart, P, c->sh.top_k, d, decode_groups(c->sh), c->sh.experts, y, done, seq_dev, seq,
                       c->host_wait_polls, c->errflag);
    return hipGetLastError();
}

}  // namespace ftmoe
