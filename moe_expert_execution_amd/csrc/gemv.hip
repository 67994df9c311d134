// Decode expert FFN: bandwidth-bound split-K GEMVs over the active slots.
//
// Each active slot serves a few token rows (decode: usually one).  Gate/up:
// every workgroup item is (slot, 8 neurons): the 16 gate and up rows are read
// with coalesced 16-byte loads, K split over the four waves (each lane one
// 16-byte chunk of every row per step, so 16 loads are in flight per lane);
// wave sums and then the four K-quarters are added in a fixed order inside the
// workgroup — no cross-workgroup reduction, no device-scope fence — and SwiGLU,
// h = silu(g) * u, is written to fp32 H.  Work items are counted from the
// device-side number of active slots, so one fixed grid serves any hit/fill
// mix.  Down: (slot, 16 output columns) items read the down rows and H and
// write fp32 Y per sorted row.  The expert FFN (gate/up
// then down, from one slot record) is the one "The Expert Cache That Follows
// the Router" describes in section "One logical expert, two physical levels of
// memory"; SwiGLU is this build's activation.
#include "wfmt.h"

namespace ftmoe {

constexpr int kGemvThreads = 256;
constexpr int kGemvBlocks = 1024;
constexpr int kGemvNeurons = 8;     // per gate/up item: 8 gate + 8 up rows, K split over the 4 waves
constexpr int kGemvCols = 16;       // per down item (4 waves x 4)

struct GemvArgs {
    const uint16_t* x;
    int T, k, d, f;
    const int32_t* meta;
    const int32_t* active_slot;
    const int32_t* seg;
    const int32_t* perm;
    const uint8_t* pool;
    int64_t S;
    int64_t off_gate, off_up, off_down, off_sg, off_su, off_sd;
    float* Hf;          // [cap_g][f]
    float* Y;           // [cap][d]
    int cap_g;
};

namespace {

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// dot of one weight chunk with EPC activations given as packed bf16 pairs
template <int FMT>
__device__ __forceinline__ float chunk_dot_bf16x(const uint4 w, float scale, const uint32_t* xw);

template <>
__device__ __forceinline__ float chunk_dot_bf16x<FT_FMT_BF16>(const uint4 w, float, const uint32_t* xw) {
    float s = dot2_bf16(w.x, xw[0], 0.0f);
    s = dot2_bf16(w.y, xw[1], s);
    s = dot2_bf16(w.z, xw[2], s);
    return dot2_bf16(w.w, xw[3], s);
}

template <>
__device__ __forceinline__ float chunk_dot_bf16x<FT_FMT_FP8_B128>(const uint4 w, float scale, const uint32_t* xw) {
    float v[16];
    WF<FT_FMT_FP8_B128>::to_f32(w, v);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        s = fmaf(v[2 * i], bf16lo(xw[i]), s);
        s = fmaf(v[2 * i + 1], bf16hi(xw[i]), s);
    }
    return s * scale;
}

template <>
__device__ __forceinline__ float chunk_dot_bf16x<FT_FMT_MXFP4_B32>(const uint4 w, float scale, const uint32_t* xw) {
    float v[32];
    WF<FT_FMT_MXFP4_B32>::to_f32(w, scale, v);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        s = fmaf(v[2 * i], bf16lo(xw[i]), s);
        s = fmaf(v[2 * i + 1], bf16hi(xw[i]), s);
    }
    return s;
}

// dot of one weight chunk with EPC fp32 activations
template <int FMT>
__device__ __forceinline__ float chunk_dot_f32x(const uint4 w, float scale, const float* h);

template <>
__device__ __forceinline__ float chunk_dot_f32x<FT_FMT_BF16>(const uint4 w, float, const float* h) {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s = fmaf(bf16lo(ww[i]), h[2 * i], s);
        s = fmaf(bf16hi(ww[i]), h[2 * i + 1], s);
    }
    return s;
}

template <>
__device__ __forceinline__ float chunk_dot_f32x<FT_FMT_FP8_B128>(const uint4 w, float scale, const float* h) {
    float v[16];
    WF<FT_FMT_FP8_B128>::to_f32(w, v);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s = fmaf(v[i], h[i], s);
    return s * scale;
}

template <>
__device__ __forceinline__ float chunk_dot_f32x<FT_FMT_MXFP4_B32>(const uint4 w, float scale, const float* h) {
    float v[32];
    WF<FT_FMT_MXFP4_B32>::to_f32(w, scale, v);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) s = fmaf(v[i], h[i], s);
    return s;
}

// scale of the chunk starting at (row n, column k0) of a [rows x K] matrix
template <int FMT>
__device__ __forceinline__ float chunk_scale(const uint8_t* rec, int64_t off_s, int n, int k0, int K) {
    if constexpr (FMT == FT_FMT_FP8_B128) {
        return reinterpret_cast<const float*>(rec + off_s)[(n >> 7) * (K >> 7) + (k0 >> 7)];
    } else if constexpr (FMT == FT_FMT_MXFP4_B32) {
        return e8m0_to_f32(rec[off_s + (int64_t)n * (K >> 5) + (k0 >> 5)]);
    } else {
        return 1.0f;
    }
}

template <int FMT, int TG>
__global__ void __launch_bounds__(kGemvThreads) gemv_gateup_kernel(GemvArgs a) {
    constexpr int EPC = WF<FMT>::EPC;
    constexpr int XW = EPC / 2;     // packed bf16 words of x per chunk
    constexpr int NN = kGemvNeurons;
    __shared__ float red[4][NN][2][TG];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int n_active = a.meta[0];
    const int d = a.d, f = a.f;
    const int NB = f / NN;
    const int items = n_active * NB;
    const int cpr = d / EPC;                 // 16-byte chunks per row
    const int cpw = (cpr + 3) / 4;           // the K quarter of each wave
    const int c_begin = wid * cpw;
    const int c_end = (c_begin + cpw) < cpr ? (c_begin + cpw) : cpr;
    const int64_t rowb = WF<FMT>::row_bytes(d);

    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int ai = item / NB;
        const int nb = item - ai * NB;
        const int slot = a.active_slot[ai];
        const int r0 = a.seg[ai];
        int nrows = a.seg[ai + 1] - r0;
        nrows = nrows > TG ? TG : nrows;
        const uint8_t* rec = a.pool + (int64_t)slot * a.S;
        const int n0 = nb * NN;

        const uint16_t* xr[TG];
#pragma unroll
        for (int t = 0; t < TG; ++t) {
            const int rr = r0 + (t < nrows ? t : nrows - 1);
            xr[t] = a.x + (int64_t)(a.perm[rr] / a.k) * d;
        }
        float acc[NN][2][TG];
#pragma unroll
        for (int i = 0; i < NN; ++i)
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int t = 0; t < TG; ++t) acc[i][g][t] = 0.0f;

        for (int c = c_begin + lane; c < c_end; c += 64) {
            const int k0 = c * EPC;
            uint4 wv[NN][2];
#pragma unroll
            for (int i = 0; i < NN; ++i) {
                wv[i][0] = *reinterpret_cast<const uint4*>(rec + a.off_gate + (int64_t)(n0 + i) * rowb + c * 16);
                wv[i][1] = *reinterpret_cast<const uint4*>(rec + a.off_up + (int64_t)(n0 + i) * rowb + c * 16);
            }
            float sc[NN][2];
#pragma unroll
            for (int i = 0; i < NN; ++i) {
                // FP8: the NN neurons share one 128-row scale block; MXFP4: one scale per row
                const int nr = (FMT == FT_FMT_MXFP4_B32) ? n0 + i : n0;
                sc[i][0] = chunk_scale<FMT>(rec, a.off_sg, nr, k0, d);
                sc[i][1] = chunk_scale<FMT>(rec, a.off_su, nr, k0, d);
            }
            uint32_t xw[TG][XW];
#pragma unroll
            for (int t = 0; t < TG; ++t)
#pragma unroll
                for (int q = 0; q < XW / 4; ++q) {
                    const uint4 v = *reinterpret_cast<const uint4*>(xr[t] + k0 + 8 * q);
                    xw[t][4 * q] = v.x;
                    xw[t][4 * q + 1] = v.y;
                    xw[t][4 * q + 2] = v.z;
                    xw[t][4 * q + 3] = v.w;
                }
#pragma unroll
            for (int i = 0; i < NN; ++i)
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    if constexpr (FMT == FT_FMT_BF16) {
#pragma unroll
                        for (int t = 0; t < TG; ++t) acc[i][g][t] += chunk_dot_bf16x<FMT>(wv[i][g], 1.0f, xw[t]);
                    } else {
                        // decode the chunk once, use it for every token
                        float v[EPC];
                        if constexpr (FMT == FT_FMT_FP8_B128) {
                            WF<FMT>::to_f32(wv[i][g], v);
                        } else {
                            WF<FMT>::to_f32(wv[i][g], sc[i][g], v);
                        }
#pragma unroll
                        for (int t = 0; t < TG; ++t) {
                            float sacc = 0.0f;
#pragma unroll
                            for (int j = 0; j < XW; ++j) {
                                sacc = fmaf(v[2 * j], bf16lo(xw[t][j]), sacc);
                                sacc = fmaf(v[2 * j + 1], bf16hi(xw[t][j]), sacc);
                            }
                            acc[i][g][t] += (FMT == FT_FMT_FP8_B128) ? sacc * sc[i][g] : sacc;
                        }
                    }
                }
        }
        // K-split partials: wave sums, then the four waves in a fixed order
#pragma unroll
        for (int i = 0; i < NN; ++i)
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int t = 0; t < TG; ++t) {
                    const float v = wave_sum(acc[i][g][t]);
                    if (lane == 0) red[wid][i][g][t] = v;
                }
        __syncthreads();
        const int tid = threadIdx.x;
        if (tid < NN * nrows) {
            const int i = tid % NN, t = tid / NN;
            const float gs = (red[0][i][0][t] + red[1][i][0][t]) + (red[2][i][0][t] + red[3][i][0][t]);
            const float us = (red[0][i][1][t] + red[1][i][1][t]) + (red[2][i][1][t] + red[3][i][1][t]);
            a.Hf[(int64_t)(r0 + t) * f + n0 + i] = silu(gs) * us;
        }
        __syncthreads();
    }
}

template <int FMT, int TG>
__global__ void __launch_bounds__(kGemvThreads) gemv_down_kernel(GemvArgs a) {
    constexpr int EPC = WF<FMT>::EPC;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int n_active = a.meta[0];
    const int d = a.d, f = a.f;
    const int CB = d / kGemvCols;
    const int cpr = f / EPC;
    const int items = n_active * CB;
    const int64_t rowb = WF<FMT>::row_bytes(f);
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int ai = item / CB;
        const int cb = item - ai * CB;
        const int slot = a.active_slot[ai];
        const int r0 = a.seg[ai];
        int nrows = a.seg[ai + 1] - r0;
        nrows = nrows > TG ? TG : nrows;
        const uint8_t* rec = a.pool + (int64_t)slot * a.S;
        const int c0 = cb * kGemvCols + wid * 4;
        float acc[4][TG];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < TG; ++t) acc[i][t] = 0.0f;
        for (int c = lane; c < cpr; c += 64) {
            const int k0 = c * EPC;
            uint4 wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wv[i] = *reinterpret_cast<const uint4*>(rec + a.off_down + (int64_t)(c0 + i) * rowb + c * 16);
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sc[i] = chunk_scale<FMT>(rec, a.off_sd, FMT == FT_FMT_MXFP4_B32 ? c0 + i : c0, k0, f);
#pragma unroll
            for (int t = 0; t < TG; ++t) {
                const int rr = r0 + (t < nrows ? t : nrows - 1);
                float h[EPC];
#pragma unroll
                for (int q = 0; q < EPC / 4; ++q) {
                    float4 v = *reinterpret_cast<const float4*>(a.Hf + (int64_t)rr * f + k0 + 4 * q);
                    h[4 * q] = v.x;
                    h[4 * q + 1] = v.y;
                    h[4 * q + 2] = v.z;
                    h[4 * q + 3] = v.w;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i][t] += chunk_dot_f32x<FMT>(wv[i], sc[i], h);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < TG; ++t) {
                float v = wave_sum(acc[i][t]);
                if (lane == 0 && t < nrows) a.Y[(int64_t)(r0 + t) * d + c0 + i] = v;
            }
    }
}

template <int FMT, int TG>
hipError_t launch_fmt(const GemvArgs& a, Timing* tm, hipStream_t st) {
    TimedLaunch t1 = timing_launch(tm, FT_K_GEMV_GU);
    hipExtLaunchKernelGGL((gemv_gateup_kernel<FMT, TG>), dim3(kGemvBlocks), dim3(kGemvThreads), 0, st, t1.start,
                          t1.stop, 0, a);
    TimedLaunch t2 = timing_launch(tm, FT_K_GEMV_DOWN);
    hipExtLaunchKernelGGL((gemv_down_kernel<FMT, TG>), dim3(kGemvBlocks), dim3(kGemvThreads), 0, st, t2.start,
                          t2.stop, 0, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(ft_cache* c, const uint16_t* x, int T, hipStream_t st) {
    GemvArgs a;
    a.x = x;
    a.T = T;
    a.k = c->sh.top_k;
    a.d = c->sh.d_model;
    a.f = c->sh.d_ff;
    a.meta = c->plan.meta;
    a.active_slot = c->plan.active_slot;
    a.seg = c->plan.seg;
    a.perm = c->plan.perm;
    a.pool = c->pool;
    a.S = c->rl.S;
    a.off_gate = c->rl.off_gate;
    a.off_up = c->rl.off_up;
    a.off_down = c->rl.off_down;
    a.off_sg = c->rl.off_sg;
    a.off_su = c->rl.off_su;
    a.off_sd = c->rl.off_sd;
    a.Hf = c->gv_H;
    a.Y = c->Y;
    a.cap_g = c->cap_gemv;
    const bool one = T == 1;
    switch (c->sh.fmt) {
        case FT_FMT_BF16:
            return one ? launch_fmt<FT_FMT_BF16, 1>(a, c->timing, st) : launch_fmt<FT_FMT_BF16, kGemvMaxTokens>(a, c->timing, st);
        case FT_FMT_FP8_B128:
            return one ? launch_fmt<FT_FMT_FP8_B128, 1>(a, c->timing, st) : launch_fmt<FT_FMT_FP8_B128, kGemvMaxTokens>(a, c->timing, st);
        case FT_FMT_MXFP4_B32:
            return one ? launch_fmt<FT_FMT_MXFP4_B32, 1>(a, c->timing, st)
                       : launch_fmt<FT_FMT_MXFP4_B32, kGemvMaxTokens>(a, c->timing, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ftmoe
