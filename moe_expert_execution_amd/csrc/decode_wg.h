// One-token decode: the routed expert FFN of one GPU route, gate/up, SwiGLU
// and down, in one workgroup per (route, group of NPW neurons), with no
// hand-off between workgroups.
//
// The workgroup streams its group's gate and up panels (32 rows each) over
// the whole K = d, forms h = silu(x Wg) * (x Wu) for its NPW neurons on chip,
// then streams the matching column slice of the down matrix (the NPW
// neurons' chunks of every 32-row panel of WdT) and writes a partial output
// row part[group][route][0..d) (fp32).  The combine adds a route's groups in
// ascending order, so the result does not depend on scheduling.
//
// Records are panel-ordered, so every weight load is a 1 KiB lane block:
// lane l holds row l % 32 at chunk column l / 32.  Weight loads are
// non-temporal: a record is read once per call, and a resident one again
// only after the other layers' experts have streamed through L2 and the
// Infinity Cache; the streaming hint raises what one CU pulls from HBM (a
// plain read of 144 x 384 KiB runs at ~35 GB/s per workgroup, a
// non-temporal one at ~42).  A wave's loads go in two
// register buffers that alternate by step: a step issues the next step's
// loads, then consumes its own; the first down loads are in flight while the
// gate/up sums are reduced across waves.  Step counts are the same in every
// wave (a wave past the end of its range reloads a valid block and ignores
// it), so the one barrier sits at the same step everywhere.
//
// Route-indexed: the workgroup reads the call's rewritten routes (slot ids)
// directly, so it needs no planner output and can run in the same launch as
// the planner and the fill.  `Subset` selects the routes a launch serves: all
// GPU routes, only those whose slot is not being filled by this call, or
// only the filled ones (the expert FFN from one slot record follows "The
// Expert Cache That Follows the Router", section "One logical expert, two
// physical levels of memory"; SwiGLU is this library's activation).
#pragma once
#include "wfmt.h"

namespace ftmoe {

// Neurons per workgroup, chosen so that an expert spreads over many CUs (a
// CU streams ~30 GB/s from HBM, so a launch must keep most of the 256 busy)
// while a down row panel's slice stays whole lane blocks: bf16 16 (half a
// panel: one load covers two K-blocks of 16 rows, four 256-byte runs), FP8 32
// (a panel), MXFP4 64 (two panels).
template <int FMT>
struct DecodeShape {
    static constexpr int NPW = FMT == FT_FMT_MXFP4_B32 ? 64 : 32;
    static constexpr bool HALF = NPW == 16;                               // half-panel gate/up loads
    static constexpr int NP = NPW == 64 ? 2 : 1;                          // gate/up panels
    // down lane blocks per row panel: NPW neurons x element bytes / 32 bytes
    // per lane block row (a lane block is 32 rows x 2 chunks of 16 bytes)
    static constexpr int LBD = NPW * (FMT == FT_FMT_BF16 ? 4 : FMT == FT_FMT_FP8_B128 ? 2 : 1) / 64;
    static_assert(LBD >= 1, "a group's down slice is whole lane blocks");
    // weight loads per register buffer per lane, at 8 waves (up to 256
    // VGPRs) and at 16 waves (up to 128): as many as fit without spilling
    static constexpr int BU8 = FMT == FT_FMT_BF16 ? 16 : 12;
    static constexpr int BU16 = FMT == FT_FMT_BF16 ? 8 : 4;
};

struct DecodeArgs {
    const uint16_t* x;          // [d] bf16, the call's one token
    const int32_t* routes;      // [k] slot ids rewritten by classify (negative: host run, invalid), or expert ids
    const int32_t* wl_counts;   // [4] of the call's classify: q = wl_counts[3]
    const int32_t* wl_slot;     // [>= k] victim slots of the call's fills
    const uint8_t* pool;
    int64_t S;                  // slot stride of the pool (bytes)
    int64_t off_gate, off_up, off_down, off_sg, off_su, off_sd;
    int k, d, f, N;
    int E;
    int slot_base;              // < 0: routes are slot ids (CACHED); else expert ids in buffer slot_base + e (STREAMED)
    float* part;                // [f / NPW][k][d] fp32 partial outputs
};

// The arguments for a cache's pool, x and routes (decode.hip): slot ids
// rewritten by classify (slot_base < 0), or expert ids of the full-layer
// buffer whose first slot is slot_base.
DecodeArgs decode_args(const ft_cache* c, const uint16_t* x, const int32_t* routes, int slot_base = -1);

namespace dec {

__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// dot of one 16-byte weight chunk with EPC bf16 values (v: EPC / 2 packed pairs)
template <int FMT>
__device__ __forceinline__ float chunk_dot(const u32x4_t w, float scale, const uint32_t* v) {
    if constexpr (FMT == FT_FMT_BF16) {
        float s = dot2_bf16(w[0], v[0], 0.0f);
        s = dot2_bf16(w[1], v[1], s);
        s = dot2_bf16(w[2], v[2], s);
        return dot2_bf16(w[3], v[3], s);
    } else if constexpr (FMT == FT_FMT_FP8_B128) {
        float s = 0.0f;        // e4m3 values are exact in bf16; the block scale multiplies the sum
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false);
            const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true);
            s = __builtin_amdgcn_fdot2_f32_bf16(lo, __builtin_bit_cast(bf16x2_t, v[2 * i]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(hi, __builtin_bit_cast(bf16x2_t, v[2 * i + 1]), s, false);
        }
        return s * scale;
    } else {
        float s = 0.0f;        // e2m1 times a power of two is exact in bf16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 0);
            const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 1);
            const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 2);
            const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 3);
            s = __builtin_amdgcn_fdot2_f32_bf16(p0, __builtin_bit_cast(bf16x2_t, v[4 * i]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(p1, __builtin_bit_cast(bf16x2_t, v[4 * i + 1]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(p2, __builtin_bit_cast(bf16x2_t, v[4 * i + 2]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(p3, __builtin_bit_cast(bf16x2_t, v[4 * i + 3]), s, false);
        }
        return s;
    }
}

// a weight scale as stored: fp32 bits (FP8 block scale), e8m0 byte (MXFP4)
template <int FMT>
__device__ __forceinline__ float scale_value(uint32_t raw) {
    if constexpr (FMT == FT_FMT_FP8_B128) return __uint_as_float(raw);
    else if constexpr (FMT == FT_FMT_MXFP4_B32) return e8m0_to_f32(raw);
    else return 1.0f;
}

}  // namespace dec

// Bytes of dynamic LDS the workgroup needs: the token (d bf16).
__host__ __device__ inline size_t decode_lds_bytes(int d) { return (size_t)d * sizeof(uint16_t); }

constexpr int kDecodeMaxD = 8192;      // the token a workgroup stages (larger d: the two-kernel GEMV)

// The workgroup's work for item (route j = item % k, neuron group item / k).
// NW waves; BU weight loads per buffer per lane (two buffers).  `xs` is
// dynamic LDS of decode_lds_bytes(d).
template <int FMT, int NW, int BU, int SUBSET>
__device__ __forceinline__ void decode_route_group(const DecodeArgs& a, int item, uint16_t* xs) {
    using DS = DecodeShape<FMT>;
    constexpr int NPW = DS::NPW, NP = DS::NP, LBD = DS::LBD;
    constexpr int EPC = WF<FMT>::EPC;
    constexpr int NT = NW * 64;
    constexpr int CK = BU / (2 * NP);        // K-blocks per gate/up step
    constexpr int CQ = BU / LBD;             // row panels per down step
    static_assert(CK >= 1 && CQ >= 1, "buffer too small");
    __shared__ float red[NW][2 * NP][32];
    __shared__ __attribute__((aligned(16))) uint16_t hs[NPW];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int k = a.k, d = a.d, f = a.f;
    const int j = item % k, grp = item / k;

    // All independent loads at once: the token's routes and, for a subset,
    // this call's fill victims; the token itself into registers (it goes to
    // LDS once the first weight loads are in flight).
    constexpr int XPT = kDecodeMaxD / 8 / NT;
    const int rl = lane < k ? a.routes[lane] : INT32_MIN;
    int q = 0, ws = -2;
    if constexpr (SUBSET != DEC_ALL) {
        q = a.wl_counts[3];
        ws = lane < k ? a.wl_slot[lane] : -2;
    }
    u32x4_t xr[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int c = tid + i * NT;
        if (c < (d >> 3)) xr[i] = *reinterpret_cast<const u32x4_t*>(a.x + 8 * c);
    }
    const int rj = __shfl(rl, j, 64);
    const int slot = a.slot_base < 0 ? rj : (rj >= 0 && rj < a.E ? a.slot_base + rj : -1);
    // a repeated expert of the token is computed once (the planner drops the repeat)
    bool ok = slot >= 0 && slot < a.N && __ballot(lane < j && rl == rj) == 0;
    if constexpr (SUBSET != DEC_ALL) {
        const bool filled = __ballot(lane < q && ws == slot) != 0;
        ok = ok && (SUBSET == DEC_FILLS ? filled : !filled);
    }
    if (!ok) return;                         // the same in every wave

    const uint8_t* rec = a.pool + (int64_t)slot * a.S;
    const int64_t rowb = WF<FMT>::row_bytes(d);      // gate/up row bytes
    // K-units per panel a load covers: a K-block (lane block), or with half
    // panels two K-blocks
    constexpr int KPU = DS::HALF ? 2 : 1;
    const int LB = (int)(rowb >> 5) / KPU;
    const int nKW = (LB + NW - 1) / NW;              // K-units per wave
    const int kb0 = wid * nKW;
    const int kbn = max(0, min(LB, kb0 + nKW) - kb0);
    const int nGU = (nKW + CK - 1) / CK;             // gate/up steps (every wave)
    const int64_t rowbd = WF<FMT>::row_bytes(f);     // down row bytes
    const int Q = d >> 5;                            // down row panels
    const int nQW = (Q + NW - 1) / NW;
    const int q0 = wid * nQW;
    const int qn = max(0, min(Q, q0 + nQW) - q0);
    const int nD = (nQW + CQ - 1) / CQ;
    const int nsteps = nGU + nD;

    // first gate/up panel of the group; this lane's place in a load
    const int p0 = DS::HALF ? grp >> 1 : grp * NP;
    const int64_t lane_off =
        DS::HALF ? (int64_t)((grp & 1) * 256 + (lane & 15) * 16 + ((lane >> 4) & 1) * 512 + (lane >> 5) * 1024)
                 : (int64_t)lane * 16;
    const uint8_t* gbase = rec + a.off_gate + (int64_t)p0 * 32 * rowb + lane_off;
    const uint8_t* ubase = rec + a.off_up + (int64_t)p0 * 32 * rowb + lane_off;
    const uint8_t* dbase = rec + a.off_down + (int64_t)grp * LBD * 1024 + lane * 16;

    // step s: load its blocks (an index past the wave's range reloads its last
    // block, or the matrix's last one when the wave has none)
    auto issue = [&](int s, u32x4_t (&w)[BU], uint32_t (&sr)[BU]) {
        if (s < nGU) {
#pragma unroll
            for (int c = 0; c < CK; ++c) {
                const int kb = kbn > 0 ? kb0 + min(s * CK + c, kbn - 1) : LB - 1;
#pragma unroll
                for (int i = 0; i < NP; ++i) {
                    w[c * 2 * NP + i] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4_t*>(gbase + (int64_t)i * 32 * rowb + kb * (KPU * 1024)));
                    w[c * 2 * NP + NP + i] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4_t*>(ubase + (int64_t)i * 32 * rowb + kb * (KPU * 1024)));
                    if constexpr (FMT == FT_FMT_FP8_B128) {
                        const uint32_t* sg = reinterpret_cast<const uint32_t*>(rec + a.off_sg);
                        const uint32_t* su = reinterpret_cast<const uint32_t*>(rec + a.off_su);
                        const int idx = ((p0 + i) >> 2) * (d >> 7) + (kb >> 2);
                        sr[c * 2 * NP + i] = sg[idx];
                        sr[c * 2 * NP + NP + i] = su[idx];
                    } else if constexpr (FMT == FT_FMT_MXFP4_B32) {
                        const int64_t o = (int64_t)(p0 + i) * d + kb * 64 + lane;
                        sr[c * 2 * NP + i] = rec[a.off_sg + o];
                        sr[c * 2 * NP + NP + i] = rec[a.off_su + o];
                    }
                }
            }
        } else {
            const int sd = s - nGU;
#pragma unroll
            for (int c = 0; c < CQ; ++c) {
                const int qq = qn > 0 ? q0 + min(sd * CQ + c, qn - 1) : Q - 1;
#pragma unroll
                for (int b = 0; b < LBD; ++b) {
                    w[c * LBD + b] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4_t*>(dbase + (int64_t)qq * 32 * rowbd + b * 1024));
                    if constexpr (FMT == FT_FMT_FP8_B128) {
                        sr[c * LBD + b] = reinterpret_cast<const uint32_t*>(rec + a.off_sd)[(qq >> 2) * (f >> 7) +
                                                                                              ((grp * NPW) >> 7)];
                    } else if constexpr (FMT == FT_FMT_MXFP4_B32) {
                        sr[c * LBD + b] = rec[a.off_sd + (int64_t)qq * f + (grp * LBD + b) * 64 + lane];
                    }
                }
            }
        }
    };

    float ag[NP], au[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) ag[i] = au[i] = 0.0f;
    uint32_t hv[LBD][EPC / 2];               // this lane's h chunks (the same for every row panel)

    auto consume = [&](int s, const u32x4_t (&w)[BU], const uint32_t (&sr)[BU]) {
        if (s < nGU) {
#pragma unroll
            for (int c = 0; c < CK; ++c) {
                const int kl = s * CK + c;
                if (kl < kbn) {
                    const int kb = kb0 + kl;
                    uint32_t xw[EPC / 2];
                    // the lane's chunk along K: (K-block, chunk column)
                    const int xo = DS::HALF ? (4 * kb + 2 * (lane >> 5) + ((lane >> 4) & 1)) * EPC
                                            : (2 * kb + (lane >> 5)) * EPC;
#pragma unroll
                    for (int r = 0; r < EPC / 8; ++r) {
                        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&xs[xo + 8 * r]);
                        xw[4 * r] = v[0];
                        xw[4 * r + 1] = v[1];
                        xw[4 * r + 2] = v[2];
                        xw[4 * r + 3] = v[3];
                    }
#pragma unroll
                    for (int i = 0; i < NP; ++i) {
                        ag[i] += dec::chunk_dot<FMT>(w[c * 2 * NP + i], dec::scale_value<FMT>(sr[c * 2 * NP + i]), xw);
                        au[i] += dec::chunk_dot<FMT>(w[c * 2 * NP + NP + i],
                                                     dec::scale_value<FMT>(sr[c * 2 * NP + NP + i]), xw);
                    }
                }
            }
            if (s == nGU - 1) {
                // g and u of the group's rows: lanes l and l + 32 hold a row's two
                // chunk columns; then the waves' sums in order, SwiGLU, h in bf16
#pragma unroll
                for (int i = 0; i < NP; ++i) {
                    float g = ag[i] + __shfl_xor(ag[i], 32, 64);
                    float u = au[i] + __shfl_xor(au[i], 32, 64);
                    if constexpr (DS::HALF) {      // a half panel's row sits in lanes n, n + 16, n + 32, n + 48
                        g += __shfl_xor(g, 16, 64);
                        u += __shfl_xor(u, 16, 64);
                    }
                    if (lane < (DS::HALF ? 16 : 32)) {
                        red[wid][i][lane] = g;
                        red[wid][NP + i][lane] = u;
                    }
                }
                __syncthreads();
                if (tid < NPW) {
                    const int i = tid >> 5, n = tid & 31;     // (with half panels: i = 0, n < 16)
                    float g = 0.0f, u = 0.0f;
#pragma unroll
                    for (int ww = 0; ww < NW; ++ww) {
                        g += red[ww][i][n];
                        u += red[ww][NP + i][n];
                    }
                    hs[tid] = f32_to_bf16_rne(dec::silu(g) * u);
                }
                __syncthreads();
#pragma unroll
                for (int b = 0; b < LBD; ++b)
#pragma unroll
                    for (int r = 0; r < EPC / 8; ++r) {
                        const u32x4_t v =
                            *reinterpret_cast<const u32x4_t*>(&hs[(2 * b + (lane >> 5)) * EPC + 8 * r]);
                        hv[b][4 * r] = v[0];
                        hv[b][4 * r + 1] = v[1];
                        hv[b][4 * r + 2] = v[2];
                        hv[b][4 * r + 3] = v[3];
                    }
            }
        } else {
            const int sd = s - nGU;
#pragma unroll
            for (int c = 0; c < CQ; ++c) {
                const int ql = sd * CQ + c;
                float acc = 0.0f;
#pragma unroll
                for (int b = 0; b < LBD; ++b)
                    acc += dec::chunk_dot<FMT>(w[c * LBD + b], dec::scale_value<FMT>(sr[c * LBD + b]), hv[b]);
                acc += __shfl_xor(acc, 32, 64);
                if (ql < qn && lane < 32)
                    a.part[((int64_t)grp * k + j) * d + (int64_t)(q0 + ql) * 32 + lane] = acc;
            }
        }
    };

    u32x4_t wa[BU], wb[BU];
    uint32_t sa[BU], sb[BU];
#pragma unroll
    for (int i = 0; i < BU; ++i) sa[i] = sb[i] = 0u;
    issue(0, wa, sa);
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int c = tid + i * NT;
        if (c < (d >> 3)) *reinterpret_cast<u32x4_t*>(&xs[8 * c]) = xr[i];
    }
    __syncthreads();
    for (int s = 0; s < nsteps; s += 2) {
        if (s + 1 < nsteps) issue(s + 1, wb, sb);
        consume(s, wa, sa);
        if (s + 1 < nsteps) {
            if (s + 2 < nsteps) issue(s + 2, wa, sa);
            consume(s + 1, wb, sb);
        }
    }
}

}  // namespace ftmoe
