// Decode expert FFN: bandwidth-bound GEMVs over the active slots.
//
// Each active slot serves a few token rows (decode: usually one).  Weights are
// panel-ordered (32 rows per panel; one 16-byte load per lane at consecutive
// addresses fetches rows 32p..32p+31 at two adjacent chunk columns — a "lane
// block" of 1 KiB), so every weight load of these kernels is a 1 KiB
// contiguous run.
//
// Gate/up: a workgroup owns (active slot, 32-neuron panel, K-part): its four
// waves split the K-part's lane blocks of the gate and the up panel, dot them
// with the token rows (staged once in LDS), and add the wave partials in a
// fixed order; the K-part sums of g and u go to a small fp32 buffer.
// Down: a workgroup owns (active slot, 32 output columns); its prologue forms
// h = silu(sum g) * (sum u) for the slot's rows in LDS (the K-parts added in a
// fixed order, rounded to bf16), then four waves split K = f and reduce
// through LDS into Y (bf16).
// No atomics and no cross-workgroup ordering: results are deterministic.
// Work items are counted from the device-side number of active slots, so one
// grid serves any hit/fill mix.  The expert FFN (gate/up then down, from one
// slot record) is the one "The Expert Cache That Follows the Router"
// describes in section "One logical expert, two physical levels of memory";
// SwiGLU is this library's activation.
#include "wfmt.h"

namespace ftmoe {

constexpr int kGuWaves = 4;          // waves per gate/up workgroup
constexpr int kDnWaves = 4;          // waves per down workgroup
constexpr int kBatch = 8;            // gate/up: lane blocks per matrix held in flight per lane
constexpr int kDnBatch = 16;         // down: lane blocks held in flight per lane
constexpr int kMaxSpan = 4096;       // K elements of x staged per gate/up workgroup
constexpr int kMaxKq = 8;            // most K-parts of gate/up

struct GemvArgs {
    const uint16_t* x;
    int T, k, d, f;
    const int32_t* meta;
    const int32_t* active_slot;
    const int32_t* seg;
    const int32_t* perm;
    const uint8_t* pool;
    int64_t S;          // slot stride of the pool (bytes)
    int64_t off_gate, off_up, off_down, off_sg, off_su, off_sd;
    float* part;        // [2][kq][cap_g][f]: K-part sums of g (0) and u (1)
    uint16_t* hb;       // [cap_g][f] bf16 h, when formed once by the finalize kernel
    uint16_t* Y;        // [cap][d] bf16
    int cap_g;
    int kq;             // K-parts of gate/up
    int lbq;            // lane blocks per K-part
};

// K-parts of the gate/up GEMV for a shape: at most kBatch lane blocks per wave
// and matrix (all in flight at once), and at most kMaxSpan activations staged
// per workgroup.
// Whether h is formed once by a separate kernel rather than in every down
// workgroup's prologue: when the down workgroups' repeated reads of the K-part
// sums (d/32 workgroups x 2 kq f fp32 per expert) would exceed the down
// weights themselves (d f bytes-per-element).
bool gemv_finalize(const ft_shape& s, int kq) {
    const double bpe = s.fmt == FT_FMT_BF16 ? 2.0 : s.fmt == FT_FMT_FP8_B128 ? 1.0 : 0.5;
    return kq >= 4.0 * bpe;
}

int gemv_kparts(const ft_shape& s) {
    const int64_t rb = s.fmt == FT_FMT_BF16 ? 2ll * s.d_model : s.fmt == FT_FMT_FP8_B128 ? s.d_model : s.d_model / 2;
    const int64_t lb = rb / 32;
    int kq = (int)((lb + kGuWaves * kBatch - 1) / (kGuWaves * kBatch));
    const int need = (int)((s.d_model + kMaxSpan - 1) / kMaxSpan);
    if (kq < need) kq = need;
    if (kq < 1) kq = 1;
    if (kq > kMaxKq) kq = kMaxKq;
    return kq;
}

namespace {

// silu with a hardware reciprocal (1 ulp): z / (1 + e^-z)
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

__device__ __forceinline__ float swap_halves_sum(float v) { return v + __shfl_xor(v, 32, 64); }

// dot of one 16-byte weight chunk with EPC bf16 activations (xw: EPC/2 packed pairs)
template <int FMT>
__device__ __forceinline__ float chunk_dot(const u32x4_t w, float scale, const uint32_t* xw) {
    if constexpr (FMT == FT_FMT_BF16) {
        float s = dot2_bf16(w[0], xw[0], 0.0f);
        s = dot2_bf16(w[1], xw[1], s);
        s = dot2_bf16(w[2], xw[2], s);
        return dot2_bf16(w[3], xw[3], s);
    } else if constexpr (FMT == FT_FMT_FP8_B128) {
        // e4m3 values are exact in bf16; the block scale multiplies the chunk sum
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false);
            const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true);
            s = __builtin_amdgcn_fdot2_f32_bf16(lo, __builtin_bit_cast(bf16x2_t, xw[2 * i]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(hi, __builtin_bit_cast(bf16x2_t, xw[2 * i + 1]), s, false);
        }
        return s * scale;
    } else {
        // e2m1 times a power-of-two scale is exact in bf16
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 0);
            const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 1);
            const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 2);
            const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 3);
            s = __builtin_amdgcn_fdot2_f32_bf16(p0, __builtin_bit_cast(bf16x2_t, xw[4 * i]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(p1, __builtin_bit_cast(bf16x2_t, xw[4 * i + 1]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(p2, __builtin_bit_cast(bf16x2_t, xw[4 * i + 2]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(p3, __builtin_bit_cast(bf16x2_t, xw[4 * i + 3]), s, false);
        }
        return s;
    }
}

// Scale of lane block j of a panel for this lane: FP8 — the fp32 scale of the
// 128 x 128 block (uniform over the panel's 32 rows and the block's two chunk
// columns); MXFP4 — the lane's own e8m0 byte, stored in the same panel order.
template <int FMT>
__device__ __forceinline__ float lane_scale(const uint8_t* rec, int64_t off_s, int p, int j, int lane, int K) {
    if constexpr (FMT == FT_FMT_FP8_B128) {
        return reinterpret_cast<const float*>(rec + off_s)[(p >> 2) * (K >> 7) + (j >> 2)];
    } else if constexpr (FMT == FT_FMT_MXFP4_B32) {
        return e8m0_to_f32(rec[off_s + (int64_t)p * K + j * 64 + lane]);
    } else {
        return 1.0f;
    }
}

template <int FMT, int TG>
__global__ void __launch_bounds__(kGuWaves * 64) gemv_gateup_kernel(GemvArgs a) {
    constexpr int EPC = WF<FMT>::EPC;
    constexpr int XW = EPC / 2;                                  // packed bf16 pairs of x per chunk
    constexpr int XPT = TG * (kMaxSpan / 8) / (kGuWaves * 64);    // 16-byte x chunks per thread
    constexpr int NB = TG == 1 ? kBatch : kBatch / 2;            // lane blocks per matrix in flight
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [TG][span]
    __shared__ float red[kGuWaves][2][TG][32];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, tid = threadIdx.x;
    const int d = a.d, f = a.f;
    const int P = f >> 5;
    const int item = blockIdx.x;
    const int kq = item % a.kq;
    const int rest = item / a.kq;
    const int p = rest % P;
    const int ai = rest / P;
    // independent metadata loads (ai is below the buffers' capacity)
    const int n_active = a.meta[0];
    const int slot = a.active_slot[ai];
    const int r0 = a.seg[ai];
    const int r1 = a.seg[ai + 1];
    if (ai >= n_active) return;
    int nrows = r1 - r0;
    nrows = nrows > TG ? TG : nrows;
    const uint8_t* rec = a.pool + (int64_t)slot * a.S;
    const int64_t rowb = WF<FMT>::row_bytes(d);
    const int LB = (int)(rowb >> 5);                       // lane blocks per panel
    const int jq0 = kq * a.lbq;
    const int jq1 = min(LB, jq0 + a.lbq);
    const int nq = jq1 - jq0;
    const int jw0 = jq0 + (wid * nq) / kGuWaves;
    const int jw1 = jq0 + ((wid + 1) * nq) / kGuWaves;
    const uint8_t* gp = rec + a.off_gate + (int64_t)p * 32 * rowb + lane * 16;
    const uint8_t* up = rec + a.off_up + (int64_t)p * 32 * rowb + lane * 16;

    // the token rows' activations of this K-part (one call of T = 1 has the
    // single row x[0]; otherwise the sorted rows' tokens come from perm)
    const int k0 = 2 * jq0 * EPC;
    const int span = 2 * nq * EPC;
    const int c8n = span >> 3;
    const uint16_t* xr[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) {
        if (TG == 1) {
            xr[t] = a.x + k0;
        } else {
            const int rr = r0 + (t < nrows ? t : nrows - 1);
            xr[t] = a.x + (int64_t)(a.perm[rr] / a.k) * d + k0;
        }
    }
    u32x4_t xv[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int q = tid + kGuWaves * 64 * i;
        if (q < TG * c8n) {
            const int t = q / c8n, c8 = q - t * c8n;
            xv[i] = *reinterpret_cast<const u32x4_t*>(xr[t] + 8 * c8);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // then the weights: the whole K range of this wave in flight at once
    u32x4_t wg[NB], wu[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
        if (jw0 + i < jw1) {
            wg[i] = *reinterpret_cast<const u32x4_t*>(gp + (int64_t)(jw0 + i) * 1024);
            wu[i] = *reinterpret_cast<const u32x4_t*>(up + (int64_t)(jw0 + i) * 1024);
        }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int q = tid + kGuWaves * 64 * i;
        if (q < TG * c8n) {
            const int t = q / c8n, c8 = q - t * c8n;
            *reinterpret_cast<u32x4_t*>(&xs[t * span + 8 * c8]) = xv[i];
        }
    }
    __syncthreads();

    float ag[TG], au[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) ag[t] = au[t] = 0.0f;
    for (int j0 = jw0; j0 < jw1; j0 += NB) {
        if (j0 != jw0) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
                if (j0 + i < jw1) {
                    wg[i] = *reinterpret_cast<const u32x4_t*>(gp + (int64_t)(j0 + i) * 1024);
                    wu[i] = *reinterpret_cast<const u32x4_t*>(up + (int64_t)(j0 + i) * 1024);
                }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int j = j0 + i;
            if (j < jw1) {
                const float sg = lane_scale<FMT>(rec, a.off_sg, p, j, lane, d);
                const float su = lane_scale<FMT>(rec, a.off_su, p, j, lane, d);
                const int xo = (2 * (j - jq0) + (lane >> 5)) * EPC;    // this lane's chunk inside the span
#pragma unroll
                for (int t = 0; t < TG; ++t) {
                    uint32_t xw[XW];
#pragma unroll
                    for (int q = 0; q < XW / 4; ++q) {
                        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&xs[t * span + xo + 8 * q]);
                        xw[4 * q] = v[0];
                        xw[4 * q + 1] = v[1];
                        xw[4 * q + 2] = v[2];
                        xw[4 * q + 3] = v[3];
                    }
                    ag[t] += chunk_dot<FMT>(wg[i], sg, xw);
                    au[t] += chunk_dot<FMT>(wu[i], su, xw);
                }
            }
        }
    }
    // lanes l and l + 32 hold the same row's two chunk columns
#pragma unroll
    for (int t = 0; t < TG; ++t) {
        const float g = swap_halves_sum(ag[t]);
        const float u = swap_halves_sum(au[t]);
        if (lane < 32) {
            red[wid][0][t][lane] = g;
            red[wid][1][t][lane] = u;
        }
    }
    __syncthreads();
    if (tid < 2 * TG * 32) {
        const int n = tid & 31, t = (tid >> 5) % TG, m = tid / (32 * TG);
        if (t < nrows) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < kGuWaves; ++w) s += red[w][m][t][n];
            a.part[(((int64_t)m * a.kq + kq) * a.cap_g + r0 + t) * f + 32 * p + n] = s;
        }
    }
}

// h = silu(sum g) * (sum u) in bf16 for every GPU row, the K-parts added in
// order; 1,024 elements of one active slot's rows per workgroup.
template <int TG>
__global__ void __launch_bounds__(256) gemv_swiglu_kernel(GemvArgs a) {
    const int f = a.f;
    const int nch = (TG * f + 1023) / 1024;
    const int ai = blockIdx.x / nch, ch = blockIdx.x - ai * nch;
    const int n_active = a.meta[0];
    const int r0 = a.seg[ai];
    const int r1 = a.seg[ai + 1];
    if (ai >= n_active) return;
    int nrows = r1 - r0;
    nrows = nrows > TG ? TG : nrows;
    float vg[4][kMaxKq], vu[4][kMaxKq];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = ch * 1024 + e * 256 + threadIdx.x;
        const int t = i / f, n = i - t * f;
#pragma unroll
        for (int kk = 0; kk < kMaxKq; ++kk)
            if (kk < a.kq && t < nrows) {
                vg[e][kk] = a.part[((int64_t)kk * a.cap_g + r0 + t) * f + n];
                vu[e][kk] = a.part[(((int64_t)a.kq + kk) * a.cap_g + r0 + t) * f + n];
            }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = ch * 1024 + e * 256 + threadIdx.x;
        const int t = i / f, n = i - t * f;
        if (t < nrows) {
            float g = 0.0f, u = 0.0f;
#pragma unroll
            for (int kk = 0; kk < kMaxKq; ++kk)
                if (kk < a.kq) {
                    g += vg[e][kk];
                    u += vu[e][kk];
                }
            a.hb[(int64_t)(r0 + t) * f + n] = f32_to_bf16_rne(silu(g) * u);
        }
    }
}

template <int FMT, int TG, bool FIN>
__global__ void __launch_bounds__(kDnWaves * 64) gemv_down_kernel(GemvArgs a) {
    constexpr int EPC = WF<FMT>::EPC;
    constexpr int HPT = 4;                 // h elements per thread whose K-part sums load before the weights
    extern __shared__ __attribute__((aligned(16))) uint16_t hs[];   // [TG][f] bf16
    __shared__ float red[kDnWaves][TG][32];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, tid = threadIdx.x;
    const int d = a.d, f = a.f;
    const int Q = d >> 5;
    const int q = blockIdx.x % Q;
    const int ai = blockIdx.x / Q;
    const int n_active = a.meta[0];
    const int slot = a.active_slot[ai];
    const int r0 = a.seg[ai];
    const int r1 = a.seg[ai + 1];
    if (ai >= n_active) return;
    int nrows = r1 - r0;
    nrows = nrows > TG ? TG : nrows;
    const uint8_t* rec = a.pool + (int64_t)slot * a.S;
    const int64_t rowb = WF<FMT>::row_bytes(f);
    const int LB = (int)(rowb >> 5);
    const int jw0 = (wid * LB) / kDnWaves;
    const int jw1 = ((wid + 1) * LB) / kDnWaves;
    const uint8_t* dp = rec + a.off_down + (int64_t)q * 32 * rowb + lane * 16;
    u32x4_t wd[kDnBatch];

    // h (bf16, as the prefill path keeps it) for the slot's rows.  FIN: it was
    // formed by the finalize kernel and is copied in; otherwise it is formed
    // here from the K-part sums, added in order.  Either way its loads are
    // issued before the weights, so building h waits for them only.
    const int nh = TG * f;
    if constexpr (FIN) {
        constexpr int CPT = TG * (8192 / 8) / (kDnWaves * 64);    // 16-byte h chunks per thread, f <= 8192
        u32x4_t hv[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            const int c8 = tid + kDnWaves * 64 * e;
            const int t = (8 * c8) / f;
            hv[e] = u32x4_t{0u, 0u, 0u, 0u};
            if (8 * c8 < nh && t < nrows)
                hv[e] = *reinterpret_cast<const u32x4_t*>(a.hb + (int64_t)(r0 + t) * f + (8 * c8 - t * f));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kDnBatch; ++i)
            if (jw0 + i < jw1) wd[i] = *reinterpret_cast<const u32x4_t*>(dp + (int64_t)(jw0 + i) * 1024);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            const int c8 = tid + kDnWaves * 64 * e;
            if (8 * c8 < nh) *reinterpret_cast<u32x4_t*>(&hs[8 * c8]) = hv[e];
        }
    } else {
        float pg[HPT], pu[HPT];
#pragma unroll
        for (int e = 0; e < HPT; ++e) {
            pg[e] = pu[e] = 0.0f;
            const int i = tid + kDnWaves * 64 * e;
            const int t = i / f, n = i - t * f;
            if (i < nh && t < nrows) {
                // all K-part loads issued together (a runtime-bounded loop would
                // wait for each pair in turn)
                float vg[kMaxKq], vu[kMaxKq];
#pragma unroll
                for (int kk = 0; kk < kMaxKq; ++kk)
                    if (kk < a.kq) {
                        vg[kk] = a.part[((int64_t)kk * a.cap_g + r0 + t) * f + n];
                        vu[kk] = a.part[(((int64_t)a.kq + kk) * a.cap_g + r0 + t) * f + n];
                    }
#pragma unroll
                for (int kk = 0; kk < kMaxKq; ++kk)
                    if (kk < a.kq) {
                        pg[e] += vg[kk];
                        pu[e] += vu[kk];
                    }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kDnBatch; ++i)
            if (jw0 + i < jw1) wd[i] = *reinterpret_cast<const u32x4_t*>(dp + (int64_t)(jw0 + i) * 1024);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < HPT; ++e) {
            const int i = tid + kDnWaves * 64 * e;
            if (i < nh) hs[i] = f32_to_bf16_rne(silu(pg[e]) * pu[e]);
        }
        for (int i = tid + kDnWaves * 64 * HPT; i < nh; i += kDnWaves * 64) {
            const int t = i / f, n = i - t * f;
            float h = 0.0f;
            if (t < nrows) {
                float g = 0.0f, u = 0.0f;
                for (int kk = 0; kk < a.kq; ++kk) {
                    g += a.part[((int64_t)kk * a.cap_g + r0 + t) * f + n];
                    u += a.part[(((int64_t)a.kq + kk) * a.cap_g + r0 + t) * f + n];
                }
                h = silu(g) * u;
            }
            hs[i] = f32_to_bf16_rne(h);
        }
    }
    __syncthreads();

    float acc[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) acc[t] = 0.0f;
    for (int j0 = jw0; j0 < jw1; j0 += kDnBatch) {
        if (j0 != jw0) {
#pragma unroll
            for (int i = 0; i < kDnBatch; ++i)
                if (j0 + i < jw1) wd[i] = *reinterpret_cast<const u32x4_t*>(dp + (int64_t)(j0 + i) * 1024);
        }
#pragma unroll
        for (int i = 0; i < kDnBatch; ++i) {
            const int j = j0 + i;
            if (j < jw1) {
                const float sc = lane_scale<FMT>(rec, a.off_sd, q, j, lane, f);
                const int ko = (2 * j + (lane >> 5)) * EPC;
#pragma unroll
                for (int t = 0; t < TG; ++t) {
                    uint32_t hw[EPC / 2];
#pragma unroll
                    for (int r = 0; r < EPC / 8; ++r) {
                        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&hs[t * f + ko + 8 * r]);
                        hw[4 * r] = v[0];
                        hw[4 * r + 1] = v[1];
                        hw[4 * r + 2] = v[2];
                        hw[4 * r + 3] = v[3];
                    }
                    acc[t] += chunk_dot<FMT>(wd[i], sc, hw);
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TG; ++t) {
        const float v = swap_halves_sum(acc[t]);
        if (lane < 32) red[wid][t][lane] = v;
    }
    __syncthreads();
    if (tid < TG * 32) {
        const int n = tid & 31, t = tid >> 5;
        if (t < nrows) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < kDnWaves; ++w) s += red[w][t][n];
            a.Y[(int64_t)(r0 + t) * d + 32 * q + n] = f32_to_bf16_rne(s);
        }
    }
}

template <int FMT, int TG>
hipError_t launch_fmt(const GemvArgs& a, int max_active, bool fin, Timing* tm, hipStream_t st) {
    const size_t xs_bytes = (size_t)TG * 2 * a.lbq * WF<FMT>::EPC * sizeof(uint16_t);
    const size_t hs_bytes = (size_t)TG * a.f * sizeof(uint16_t);
    const unsigned g1 = (unsigned)(max_active * (a.f / 32) * a.kq);
    const unsigned g2 = (unsigned)(max_active * (a.d / 32));
    TimedLaunch t1 = timing_launch(tm, FT_K_GEMV_GU);
    hipExtLaunchKernelGGL((gemv_gateup_kernel<FMT, TG>), dim3(g1), dim3(kGuWaves * 64), xs_bytes, st, t1.start,
                          t1.stop, 0, a);
    if (fin) {
        TimedLaunch t3 = timing_launch(tm, FT_K_GEMV_DOWN);
        const unsigned g3 = (unsigned)(max_active * ((TG * a.f + 1023) / 1024));
        hipExtLaunchKernelGGL((gemv_swiglu_kernel<TG>), dim3(g3), dim3(256), 0, st, t3.start, t3.stop, 0, a);
        TimedLaunch t2 = timing_launch(tm, FT_K_GEMV_DOWN);
        hipExtLaunchKernelGGL((gemv_down_kernel<FMT, TG, true>), dim3(g2), dim3(kDnWaves * 64), hs_bytes, st,
                              t2.start, t2.stop, 0, a);
    } else {
        TimedLaunch t2 = timing_launch(tm, FT_K_GEMV_DOWN);
        hipExtLaunchKernelGGL((gemv_down_kernel<FMT, TG, false>), dim3(g2), dim3(kDnWaves * 64), hs_bytes, st,
                              t2.start, t2.stop, 0, a);
    }
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
    a.S = c->rl.P;   // slot stride of the pool
    a.off_gate = c->rl.off_gate;
    a.off_up = c->rl.off_up;
    a.off_down = c->rl.off_down;
    a.off_sg = c->rl.off_sg;
    a.off_su = c->rl.off_su;
    a.off_sd = c->rl.off_sd;
    a.part = c->gv_part;
    a.hb = c->H;
    a.Y = c->Y;
    a.cap_g = c->cap_gemv;
    a.kq = c->gv_kq;
    const int64_t rowb = c->sh.fmt == FT_FMT_BF16 ? 2ll * a.d : c->sh.fmt == FT_FMT_FP8_B128 ? a.d : a.d / 2;
    a.lbq = (int)(((rowb >> 5) + a.kq - 1) / a.kq);
    // active slots this call can have: one per route at most, and at most N
    const int64_t R = (int64_t)T * a.k;
    const int max_active = (int)(R < c->N ? R : c->N);
    if (R > a.cap_g) return hipErrorInvalidValue;
    const bool one = T == 1;
    const bool fin = gemv_finalize(c->sh, a.kq);
    switch (c->sh.fmt) {
        case FT_FMT_BF16:
            return one ? launch_fmt<FT_FMT_BF16, 1>(a, max_active, fin, c->timing, st)
                       : launch_fmt<FT_FMT_BF16, kGemvMaxTokens>(a, max_active, fin, c->timing, st);
        case FT_FMT_FP8_B128:
            return one ? launch_fmt<FT_FMT_FP8_B128, 1>(a, max_active, fin, c->timing, st)
                       : launch_fmt<FT_FMT_FP8_B128, kGemvMaxTokens>(a, max_active, fin, c->timing, st);
        case FT_FMT_MXFP4_B32:
            return one ? launch_fmt<FT_FMT_MXFP4_B32, 1>(a, max_active, fin, c->timing, st)
                       : launch_fmt<FT_FMT_MXFP4_B32, kGemvMaxTokens>(a, max_active, fin, c->timing, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ftmoe
