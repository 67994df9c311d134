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
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    bool host = false;
    for (int j = 0; j < k; ++j) {
        const int r = t * k + j;
        const int p = route_pos[r];
        if (p >= 0) {
            const float wj = w[r];
            const uint2 v = *reinterpret_cast<const uint2*>(Y + (int64_t)p * d + c);
            acc.x = fmaf(wj, bf16lo(v.x), acc.x);
            acc.y = fmaf(wj, bf16hi(v.x), acc.y);
            acc.z = fmaf(wj, bf16lo(v.y), acc.z);
            acc.w = fmaf(wj, bf16hi(v.y), acc.w);
        } else {
            const int rv = routes[r];
            host |= (rv < 0 && rv >= -E);
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

}  // namespace ftmoe
