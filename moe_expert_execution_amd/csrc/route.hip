// Top-k softmax routing: z = x Wr with every bf16 product exact and the sum
// accumulated in fp64; the k largest logits per token (ties to the lower
// expert); weights = softmax over the chosen k.  The router picks k of the
// layer's E experts per token ("Making Large MoE Models Practical on a Single
// Machine", section 1).
//
// Calls with T <= 16 use a file-scope device array for partial logits, shared
// by every such call on the device: concurrent small-T calls on different
// streams must be ordered by the caller.
#include "common.h"

namespace ftmoe {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteTokens = 16;     // tokens per workgroup
constexpr int kRouteMaxE = 256;      // experts supported by this kernel
constexpr int kDChunk = 256;         // hidden-size chunk staged in LDS

__device__ __forceinline__ double bf16_to_f64(uint16_t u) {
    return (double)__uint_as_float((uint32_t)u << 16);
}

// One wave selects the k largest of the logits zl (lane l holds experts
// l + 64 j; taken marks slots to skip), ties to the lower expert, and writes
// the ids and the softmax of the chosen logits (fp64, stored fp32).
__device__ __forceinline__ void topk_softmax_wave(double (&zl)[kRouteMaxE / 64], bool (&taken)[kRouteMaxE / 64], int lane, int k,
                                  int32_t* __restrict__ ids, float* __restrict__ w) {
    double zsel[kMaxTopK];
    int esel[kMaxTopK];
    for (int r = 0; r < k; ++r) {
        // best of this lane: largest z, ties to lower expert index; then across the wave
        double bz = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < kRouteMaxE / 64; ++j) {
            const int ee = lane + 64 * j;
            if (!taken[j] && (zl[j] > bz || (zl[j] == bz && ee < be))) {
                bz = zl[j];
                be = ee;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const double oz = __shfl_xor(bz, off, 64);
            const int oe = __shfl_xor(be, off, 64);
            if (oz > bz || (oz == bz && oe < be)) {
                bz = oz;
                be = oe;
            }
        }
        zsel[r] = bz;
        esel[r] = be;
#pragma unroll
        for (int j = 0; j < kRouteMaxE / 64; ++j)
            if (lane + 64 * j == be) taken[j] = true;
    }
    if (lane == 0) {
        double s = 0.0, ex[kMaxTopK];
        for (int r = 0; r < k; ++r) {
            ex[r] = exp(zsel[r] - zsel[0]);
            s += ex[r];
        }
        for (int r = 0; r < k; ++r) {
            ids[r] = esel[r];
            w[r] = (float)(ex[r] / s);
        }
    }
}

// Logits of kRouteTokens tokens: thread (g, e) sums the k-slice i = g, g + G,
// ... of column e; the G partial sums are added in a fixed order.
__global__ void __launch_bounds__(kRouteThreads)
    route_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int d, int E, int k,
                 int32_t* __restrict__ ids, float* __restrict__ w) {
    __shared__ uint16_t xs[kRouteTokens][kDChunk];
    __shared__ double zs[kRouteTokens][kRouteMaxE];

    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * kRouteTokens;
    const int G = kRouteThreads / E > 0 ? kRouteThreads / E : 1;   // k-splits per column
    const int e = tid % E;
    const int g = tid / E;
    const bool active = g < G && tid < G * E;

    for (int i = tid; i < kRouteTokens * E; i += kRouteThreads) zs[i / E][i % E] = 0.0;

    double acc[kRouteTokens];
#pragma unroll
    for (int t = 0; t < kRouteTokens; ++t) acc[t] = 0.0;

    for (int c0 = 0; c0 < d; c0 += kDChunk) {
        const int cl = (d - c0) < kDChunk ? (d - c0) : kDChunk;
        __syncthreads();
        for (int i = tid; i < kRouteTokens * kDChunk; i += kRouteThreads) {
            int t = i / kDChunk, c = i % kDChunk;
            uint16_t v = 0;
            if (t0 + t < T && c < cl) v = x[(int64_t)(t0 + t) * d + c0 + c];
            xs[t][c] = v;
        }
        __syncthreads();
        if (active) {
            for (int c = g; c < cl; c += G) {
                double wv = bf16_to_f64(wr[(int64_t)(c0 + c) * E + e]);
#pragma unroll
                for (int t = 0; t < kRouteTokens; ++t) acc[t] = fma(bf16_to_f64(xs[t][c]), wv, acc[t]);
            }
        }
    }
    __syncthreads();
    // fixed-order reduction of the G partial sums
    for (int gg = 0; gg < G; ++gg) {
        if (active && g == gg) {
#pragma unroll
            for (int t = 0; t < kRouteTokens; ++t) zs[t][e] += acc[t];
        }
        __syncthreads();
    }

    // top-k and softmax: one wave per token
    const int lane = tid & 63, wid = tid >> 6;
    for (int t = wid; t < kRouteTokens; t += kRouteThreads / 64) {
        if (t0 + t >= T) break;
        double zl[kRouteMaxE / 64];
        bool taken[kRouteMaxE / 64];
#pragma unroll
        for (int j = 0; j < kRouteMaxE / 64; ++j) {
            int ee = lane + 64 * j;
            zl[j] = ee < E ? zs[t][ee] : -INFINITY;
            taken[j] = ee >= E;
        }
        topk_softmax_wave(zl, taken, lane, k, ids + (int64_t)(t0 + t) * k, w + (int64_t)(t0 + t) * k);
    }
}

// ---- small T (decode): the d-range is split over kRouteDS workgroups so the
// router matrix streams through many CUs; partial logits go to a file-scope
// device array and a second kernel adds them in a fixed order, then selects.
// The array is shared by every call on the device, so two small-T calls must
// not run concurrently (on one stream they are ordered).
constexpr int kRouteSmallT = 16;
constexpr int kRouteDS = 32;
__device__ double g_route_part[kRouteDS * kRouteSmallT * kRouteMaxE];

template <int TT>
__global__ void __launch_bounds__(kRouteThreads)
    route_partial_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int d, int E) {
    __shared__ double red[kRouteThreads][TT];
    const int tid = threadIdx.x;
    const int ds = blockIdx.x;
    const int span = (d + kRouteDS - 1) / kRouteDS;
    const int r0 = ds * span, r1 = (r0 + span) < d ? (r0 + span) : d;
    const int G = kRouteThreads / E > 0 ? kRouteThreads / E : 1;
    const int e = tid % E, g = tid / E;
    const bool active = g < G && tid < G * E;
    double acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.0;
    if (active) {
#pragma unroll 4
        for (int r = r0 + g; r < r1; r += G) {
            const double wv = bf16_to_f64(wr[(int64_t)r * E + e]);
#pragma unroll
            for (int t = 0; t < TT; ++t)
                if (t < T) acc[t] = fma(bf16_to_f64(x[(int64_t)t * d + r]), wv, acc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) red[tid][t] = acc[t];
    __syncthreads();
    if (tid < E) {
        for (int t = 0; t < T && t < TT; ++t) {
            double s = 0.0;
            for (int gg = 0; gg < G; ++gg) s += red[gg * E + tid][t];
            g_route_part[((int64_t)ds * kRouteSmallT + t) * kRouteMaxE + tid] = s;
        }
    }
}

// One token, E % 8 == 0: each thread streams 16-byte pieces (8 experts) of
// router rows; a workgroup covers d / kRouteDS rows.
__global__ void __launch_bounds__(kRouteThreads)
    route_partial_vec_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int d, int E) {
    __shared__ double red[kRouteThreads][8];   // [row sub-group * ncg + column group][8 experts]
    const int tid = threadIdx.x;
    const int ds = blockIdx.x;
    const int ncg = E / 8;                      // 16-byte column groups per row
    const int rpi = kRouteThreads / ncg;        // rows per iteration
    const int cg = tid % ncg, rs = tid / ncg;
    const int span = (d + kRouteDS - 1) / kRouteDS;
    const int r0 = ds * span, r1 = (r0 + span) < d ? (r0 + span) : d;
    double acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0;
    if (rs < rpi) {
#pragma unroll 2
        for (int r = r0 + rs; r < r1; r += rpi) {
            const uint4 wv = *reinterpret_cast<const uint4*>(wr + (int64_t)r * E + cg * 8);
            const double xv = bf16_to_f64(x[r]);
            const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[2 * j] = fma(xv, (double)__uint_as_float(ww[j] << 16), acc[2 * j]);
                acc[2 * j + 1] = fma(xv, (double)__uint_as_float(ww[j] & 0xFFFF0000u), acc[2 * j + 1]);
            }
        }
        const int slot = rs * ncg + cg;
#pragma unroll
        for (int j = 0; j < 8; ++j) red[slot][j] = acc[j];
    }
    __syncthreads();
    if (tid < E) {
        const int g = tid / 8, j = tid % 8;
        double s = 0.0;
        for (int q = 0; q < rpi; ++q) s += red[q * ncg + g][j];
        g_route_part[((int64_t)ds * kRouteSmallT) * kRouteMaxE + tid] = s;
    }
}

// one wave per token: z = sum of the kRouteDS partials (fixed order), top-k, softmax
__global__ void __launch_bounds__(64) route_select_kernel(int T, int E, int k, int32_t* __restrict__ ids,
                                                          float* __restrict__ w) {
    const int t = blockIdx.x, lane = threadIdx.x;
    if (t >= T) return;
    double zl[kRouteMaxE / 64];
    bool taken[kRouteMaxE / 64];
#pragma unroll
    for (int j = 0; j < kRouteMaxE / 64; ++j) {
        const int ee = lane + 64 * j;
        double z = -INFINITY;
        if (ee < E) {
            // all partials in flight at once, then added in their fixed order
            double p[kRouteDS];
#pragma unroll
            for (int ds = 0; ds < kRouteDS; ++ds) p[ds] = g_route_part[((int64_t)ds * kRouteSmallT + t) * kRouteMaxE + ee];
            z = 0.0;
#pragma unroll
            for (int ds = 0; ds < kRouteDS; ++ds) z += p[ds];
        }
        zl[j] = z;
        taken[j] = ee >= E;
    }
    topk_softmax_wave(zl, taken, lane, k, ids + (int64_t)t * k, w + (int64_t)t * k);
}

// Many tokens, E in {64, 128, 256}: the logits are a [T x d] x [d x E] product
// on the fp64 matrix cores (v_mfma_f64_16x16x4_f64; bf16 inputs are exact in
// fp64, the sums are fp64).  A workgroup covers 16 tokens x all E experts with
// 2 E / 64 waves: wave (h, e64) computes 16 tokens x 64 experts over the K half
// h of each 128-wide K-chunk, and the two halves' logits are added in a fixed
// order at the end (two waves per SIMD keep the fp64 matrix pipe busy).  Per
// chunk the activations [16 x 128] and the router rows [128 x E] are staged in
// LDS as they are (the next chunk is prefetched into registers meanwhile).
// Lane group g = l / 16 takes k in [16 g, 16 g + 16) of its 64-wide half, so
// MFMA step s contracts k = 16 g + s over the four groups; column c = l % 16
// of matrix tile nt is expert 4 c + nt of the wave's 64, so one 8-byte LDS
// read gives a lane its four tiles' router values for a step.  The logits then
// go through LDS to the one-wave-per-token selection.
template <int EE>
__global__ void __launch_bounds__(2 * EE, 1)
    route_mfma_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int d, int k,
                      int32_t* __restrict__ ids, float* __restrict__ w) {
    constexpr int NW = EE / 64;            // waves per K half, one per 64 experts
    constexpr int NT = 2 * NW * 64;        // threads
    constexpr int KC = 128;
    constexpr int LDX = KC + 8;            // padded activation row (bf16)
    constexpr int LDW = EE + 8;            // padded router row (bf16)
    constexpr int XC = 16 * KC / 8;        // 16-byte pieces of a chunk: activations
    constexpr int WC = KC * EE / 8;        //                                router rows
    constexpr int XPT = (XC + NT - 1) / NT, WPT = WC / NT;
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // kept in registers (no stack copy)
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    typedef double f64x4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) uint16_t xs[16 * LDX];
    __shared__ __attribute__((aligned(16))) uint16_t ws[KC * LDW];
    __shared__ double zs[16][EE];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int kh = wid / NW, wv = wid % NW;
    const int g = lane >> 4, c16 = lane & 15;
    const int t0 = blockIdx.x * 16;
    f64x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = f64x4{0.0, 0.0, 0.0, 0.0};

    u32x4_t rx[XPT], rw[WPT];
    auto gload = [&](int c0) {
#pragma unroll
        for (int e = 0; e < XPT; ++e) {
            const int i = tid + NT * e;
            const int t = i / (KC / 8), c8 = i - t * (KC / 8);
            rx[e] = u32x4_t{0u, 0u, 0u, 0u};
            if (i < XC && t0 + t < T) rx[e] = *reinterpret_cast<const u32x4_t*>(x + (int64_t)(t0 + t) * d + c0 + 8 * c8);
        }
#pragma unroll
        for (int e = 0; e < WPT; ++e) {
            const int i = tid + NT * e;
            const int kk = i / (EE / 8), e8 = i - kk * (EE / 8);
            rw[e] = *reinterpret_cast<const u32x4_t*>(wr + (int64_t)(c0 + kk) * EE + 8 * e8);
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int e = 0; e < XPT; ++e) {
            const int i = tid + NT * e;
            const int t = i / (KC / 8), c8 = i - t * (KC / 8);
            if (i < XC) *reinterpret_cast<u32x4_t*>(&xs[t * LDX + 8 * c8]) = rx[e];
        }
#pragma unroll
        for (int e = 0; e < WPT; ++e) {
            const int i = tid + NT * e;
            const int kk = i / (EE / 8), e8 = i - kk * (EE / 8);
            *reinterpret_cast<u32x4_t*>(&ws[kk * LDW + 8 * e8]) = rw[e];
        }
    };
    gload(0);
    lstore();
    __syncthreads();
    for (int c0 = 0; c0 < d; c0 += KC) {
        const bool more = c0 + KC < d;
        if (more) gload(c0 + KC);
        const uint16_t* xr = &xs[c16 * LDX + 64 * kh + 16 * g];
        const u32x4_t xa0 = *reinterpret_cast<const u32x4_t*>(xr);
        const u32x4_t xa1 = *reinterpret_cast<const u32x4_t*>(xr + 8);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const uint32_t xw = s < 8 ? xa0[s >> 1] : xa1[(s - 8) >> 1];
            const double a = (double)__uint_as_float((s & 1) ? (xw & 0xFFFF0000u) : (xw << 16));
            const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(&ws[(64 * kh + 16 * g + s) * LDW + wv * 64 + 4 * c16]);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const uint32_t u = bb[nt >> 1];
                const double b = (double)__uint_as_float((nt & 1) ? (u & 0xFFFF0000u) : (u << 16));
                acc[nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[nt], 0, 0, 0);
            }
        }
        __syncthreads();
        if (more) {
            lstore();
            __syncthreads();
        }
    }
    // accumulator element v of lane l: token 4 v + l / 16; tile nt column l % 16 = expert 4 (l % 16) + nt.
    // The K halves are added in a fixed order: half 0, then half 1.
    if (kh == 0) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v) zs[4 * v + g][wv * 64 + 4 * c16 + nt] = acc[nt][v];
    }
    __syncthreads();
    if (kh == 1) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v) zs[4 * v + g][wv * 64 + 4 * c16 + nt] += acc[nt][v];
    }
    __syncthreads();
    for (int t = wid; t < 16; t += 2 * NW) {
        if (t0 + t >= T) break;
        double zl[kRouteMaxE / 64];
        bool taken[kRouteMaxE / 64];
#pragma unroll
        for (int j = 0; j < kRouteMaxE / 64; ++j) {
            const int ee = lane + 64 * j;
            zl[j] = ee < EE ? zs[t][ee] : -INFINITY;
            taken[j] = ee >= EE;
        }
        topk_softmax_wave(zl, taken, lane, k, ids + (int64_t)(t0 + t) * k, w + (int64_t)(t0 + t) * k);
    }
}

}  // namespace

hipError_t launch_route(const uint16_t* x, const uint16_t* wr, int T, int d, int E, int k, int32_t* ids, float* w,
                        hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (T <= kRouteSmallT) {
        if (T == 1 && E % 8 == 0)
            hipLaunchKernelGGL(route_partial_vec_kernel, dim3(kRouteDS), dim3(kRouteThreads), 0, st, x, wr, d, E);
        else if (T == 1)
            hipLaunchKernelGGL(route_partial_kernel<1>, dim3(kRouteDS), dim3(kRouteThreads), 0, st, x, wr, T, d, E);
        else
            hipLaunchKernelGGL(route_partial_kernel<kRouteSmallT>, dim3(kRouteDS), dim3(kRouteThreads), 0, st, x, wr,
                               T, d, E);
        hipLaunchKernelGGL(route_select_kernel, dim3(T), dim3(64), 0, st, T, E, k, ids, w);
        return hipGetLastError();
    }
    if (d % 128 == 0 && (E == 64 || E == 128 || E == 256)) {
        const dim3 grid((T + 15) / 16);
        if (E == 64)
            hipLaunchKernelGGL(route_mfma_kernel<64>, grid, dim3(128), 0, st, x, wr, T, d, k, ids, w);
        else if (E == 128)
            hipLaunchKernelGGL(route_mfma_kernel<128>, grid, dim3(256), 0, st, x, wr, T, d, k, ids, w);
        else
            hipLaunchKernelGGL(route_mfma_kernel<256>, grid, dim3(512), 0, st, x, wr, T, d, k, ids, w);
        return hipGetLastError();
    }
    int blocks = (T + kRouteTokens - 1) / kRouteTokens;
    hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(kRouteThreads), 0, st, x, wr, T, d, E, k, ids, w);
    return hipGetLastError();
}

}  // namespace ftmoe
