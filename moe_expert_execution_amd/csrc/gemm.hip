// Prefill expert FFN: grouped GEMMs over the active slots on MFMA.
//
// Rows are the planner's sorted GPU routes; each tile is 128 rows of one slot.
// Gate/up: C[rows x 2*128] = X[rows x d] * [WgT; WuT]^T for 128 neurons at a
// time, the gate and up halves landing in the same lanes, so the epilogue
// writes h = silu(g) * u (bf16) without a shuffle.  Down: Y[rows x 256 cols] =
// H[rows x f] * WdT^T in fp32.  Both operands are K-contiguous and staged
// through LDS (one buffer, next tile prefetched into registers during the MFMA
// loop); block-FP8 and MXFP4 weights are dequantised to bf16 as they are
// written to LDS, so every format issues v_mfma_f32_32x32x16_bf16.
// The expert FFN with its gate/up and down projections read from one slot
// record follows "The Expert Cache That Follows the Router", section "One
// logical expert, two physical levels of memory".
#include "wfmt.h"

namespace ftmoe {

constexpr int kBM = 128, kBN = 256, kBK = 64, kLDK = kBK + 8;
constexpr int kGemmThreads = 256;

int gemm_tile_m() { return kBM; }

struct GemmArgs {
    const uint16_t* x;
    const uint16_t* Hin;   // bf16 [rows x f] (down A)
    uint16_t* Hout;        // bf16 [rows x f] (gate/up C)
    float* Y;              // fp32 [rows x d]
    int k, d, f;
    const int32_t* meta;
    const int32_t* active_slot;
    const int32_t* seg;
    const int32_t* perm;
    const int32_t* tile_active;
    const int32_t* tile_row0;
    const int32_t* tile_first;
    const uint8_t* pool;
    int64_t S;
    int64_t off_gate, off_up, off_down, off_sg, off_su, off_sd;
};

namespace {

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// B loader: a thread owns CPT 16-byte code chunks of the B tile per K-step.
template <int FMT>
struct BLoad {
    static constexpr int EPC = WF<FMT>::EPC;
    static constexpr int CPR = kBK / EPC;                  // chunks per tile row
    static constexpr int CPT = kBN * CPR / kGemmThreads;   // chunks per thread
};

// Global loads of K-step kt into registers: 4 A chunks and CPT B chunks (with
// their block scales for FP8 / MXFP4).
template <int FMT, bool GU>
__device__ __forceinline__ void gemm_gload(const GemmArgs& a, const uint8_t* rec, int K, int nt, int tid, int kt,
                                           const uint16_t* arow0, const uint16_t* arow1, const uint16_t* arow2,
                                           const uint16_t* arow3, int akc, const uint32_t (&boff)[BLoad<FMT>::CPT],
                                           u32x4_t& ra0, u32x4_t& ra1, u32x4_t& ra2, u32x4_t& ra3,
                                           u32x4_t (&rb)[BLoad<FMT>::CPT], float (&rs)[BLoad<FMT>::CPT]) {
    using BL = BLoad<FMT>;
    const int kb = kt * kBK;
    ra0 = *reinterpret_cast<const u32x4_t*>(arow0 + kb + akc);
    ra1 = *reinterpret_cast<const u32x4_t*>(arow1 + kb + akc);
    ra2 = *reinterpret_cast<const u32x4_t*>(arow2 + kb + akc);
    ra3 = *reinterpret_cast<const u32x4_t*>(arow3 + kb + akc);
#pragma unroll
    for (int i = 0; i < BL::CPT; ++i) {
        const int q = tid + kGemmThreads * i;
        const int kk = kb + (q % BL::CPR) * BL::EPC;
        rb[i] = *reinterpret_cast<const u32x4_t*>(rec + boff[i] + WF<FMT>::row_bytes(kk));
        if constexpr (FMT != FT_FMT_BF16) {
            const int br = q / BL::CPR;
            const bool up = GU && br >= kBN / 2;
            const int n = GU ? nt * (kBN / 2) + (up ? br - kBN / 2 : br) : nt * kBN + br;
            const int64_t so = GU ? (up ? a.off_su : a.off_sg) : a.off_sd;
            if constexpr (FMT == FT_FMT_FP8_B128)
                rs[i] = reinterpret_cast<const float*>(rec + so)[(n >> 7) * (K >> 7) + (kk >> 7)];
            else
                rs[i] = e8m0_to_f32(rec[so + (int64_t)n * (K >> 5) + (kk >> 5)]);
        } else {
            rs[i] = 1.0f;
        }
    }
}

// One K-step's registers into the LDS tiles (B dequantised to bf16).
template <int FMT>
__device__ __forceinline__ void gemm_lstore(uint16_t* As, uint16_t* Bs, int tid, int r0, int akc, const u32x4_t& ra0,
                                            const u32x4_t& ra1, const u32x4_t& ra2, const u32x4_t& ra3,
                                            const u32x4_t (&rb)[BLoad<FMT>::CPT], const float (&rs)[BLoad<FMT>::CPT]) {
    using BL = BLoad<FMT>;
    *reinterpret_cast<u32x4_t*>(&As[(r0)*kLDK + akc]) = ra0;
    *reinterpret_cast<u32x4_t*>(&As[(r0 + 32) * kLDK + akc]) = ra1;
    *reinterpret_cast<u32x4_t*>(&As[(r0 + 64) * kLDK + akc]) = ra2;
    *reinterpret_cast<u32x4_t*>(&As[(r0 + 96) * kLDK + akc]) = ra3;
#pragma unroll
    for (int i = 0; i < BL::CPT; ++i) {
        const int q = tid + kGemmThreads * i;
        uint16_t* dst = &Bs[(q / BL::CPR) * kLDK + (q % BL::CPR) * BL::EPC];
        if constexpr (FMT == FT_FMT_BF16) {
            *reinterpret_cast<u32x4_t*>(dst) = rb[i];
        } else if constexpr (FMT == FT_FMT_FP8_B128) {
            float v[16];
            WF<FMT>::to_f32(rb[i], v);
            uint32_t p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                p[j] = (uint32_t)f32_to_bf16_rne(v[2 * j] * rs[i]) |
                       ((uint32_t)f32_to_bf16_rne(v[2 * j + 1] * rs[i]) << 16);
            reinterpret_cast<u32x4_t*>(dst)[0] = u32x4_t{p[0], p[1], p[2], p[3]};
            reinterpret_cast<u32x4_t*>(dst)[1] = u32x4_t{p[4], p[5], p[6], p[7]};
        } else {
            float v[32];
            WF<FMT>::to_f32(rb[i], rs[i], v);
            uint32_t p[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) p[j] = pack_bf16_trunc(v[2 * j], v[2 * j + 1]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                reinterpret_cast<u32x4_t*>(dst)[j] = u32x4_t{p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]};
        }
    }
}

// Tile (kBM rows of one slot) x (kBN columns) per workgroup; 4 waves in 2 x 2,
// each computing 64 x 128 with 2 x 4 v_mfma_f32_32x32x16_bf16 accumulators.
// Gate/up: the kBN columns are 128 gate and the same 128 up neurons; wave
// column wn owns neurons [64 wn, 64 wn + 64) of both, as N-fragments
// (gate0, gate1, up0, up1), so SwiGLU pairs fragment j with j + 2 in-lane.
// Down: wave column wn owns output columns [128 wn, 128 wn + 128).
// Workgroups are renumbered so that each XCD (dispatch round-robin over 8)
// receives a contiguous range of blocks, ordered by slot, then N-tile, then
// M-tile: all blocks of an expert run together in one XCD, where its A rows
// and B tiles are read from HBM about once and then hit that XCD's L2.
template <int FMT, bool GU>
__global__ void __launch_bounds__(kGemmThreads, 2) gemm_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLDK];
    using BL = BLoad<FMT>;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int NT = GU ? a.f / (kBN / 2) : a.d / kBN;
    const int V = a.meta[1] * NT;                 // valid workgroups
    const int b = blockIdx.x;
    if (b >= V) return;
    const int q8 = V >> 3, r8 = V & 7, x8 = b & 7;
    const int lb = x8 * q8 + (x8 < r8 ? x8 : r8) + (b >> 3);
    // within one slot's blocks [t0 NT, (t0 + mt) NT): N-tile major, M-tile minor,
    // so the M-tiles sharing a B tile run side by side
    const int ai = a.tile_active[lb / NT];
    const int t0 = a.tile_first[ai], mt = a.tile_first[ai + 1] - t0;
    const int local = lb - t0 * NT;
    const int nt = local / mt;
    const int tile = t0 + (local - nt * mt);
    const int row0 = a.tile_row0[tile];
    const int seg_end = a.seg[ai + 1];
    const int slot = a.active_slot[ai];
    int rows_valid = seg_end - row0;
    rows_valid = rows_valid > kBM ? kBM : rows_valid;
    const int K = GU ? a.d : a.f;
    const uint8_t* rec = a.pool + (int64_t)slot * a.S;
    const int64_t rowb = WF<FMT>::row_bytes(K);

    // A: 4 chunks of 8 bf16 per thread per K-step (row q >> 3, chunk q & 7)
    const uint16_t* arow0;
    const uint16_t* arow1;
    const uint16_t* arow2;
    const uint16_t* arow3;
    {
        // rows past the tile's end repeat its last row: their outputs are never stored
        const uint16_t* ap[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int r = (tid + kGemmThreads * i) >> 3;
            r = r < rows_valid ? r : rows_valid - 1;
            const int p = row0 + r;
            ap[i] = GU ? a.x + (int64_t)(a.perm[p] / a.k) * a.d : a.Hin + (int64_t)p * a.f;
        }
        arow0 = ap[0];
        arow1 = ap[1];
        arow2 = ap[2];
        arow3 = ap[3];
    }
    const int akc = (tid & 7) * 8;
    // B: chunk i of this thread is tile row (tid + 256 i) / CPR; its record
    // offset fits 32 bits (a record is at most a few tens of MB)
    uint32_t boff[BL::CPT];
#pragma unroll
    for (int i = 0; i < BL::CPT; ++i) {
        const int br = (tid + kGemmThreads * i) / BL::CPR;
        if (GU) {
            const bool up = br >= kBN / 2;
            const int n = nt * (kBN / 2) + (up ? br - kBN / 2 : br);
            boff[i] = (uint32_t)((up ? a.off_up : a.off_gate) + (int64_t)n * rowb);
        } else {
            boff[i] = (uint32_t)(a.off_down + (int64_t)(nt * kBN + br) * rowb);
        }
    }

    f32x16_t acc[2][4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

#define FT_BBASE(ni) (GU ? (((ni) >> 1) * (kBN / 2) + 64 * wn + 32 * ((ni) & 1)) : (128 * wn + 32 * (ni)))

    const int KT = K / kBK;
    const int r0 = tid >> 3;

    {
        u32x4_t ra0, ra1, ra2, ra3, rb[BL::CPT];
        float rs[BL::CPT];
        gemm_gload<FMT, GU>(a, rec, K, nt, tid, 0, arow0, arow1, arow2, arow3, akc, boff, ra0, ra1, ra2, ra3, rb, rs);
        gemm_lstore<FMT>(As, Bs, tid, r0, akc, ra0, ra1, ra2, ra3, rb, rs);
    }
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const bool more = kt + 1 < KT;
        u32x4_t ra0, ra1, ra2, ra3, rb[BL::CPT];
        float rs[BL::CPT];
        if (more)
            gemm_gload<FMT, GU>(a, rec, K, nt, tid, kt + 1, arow0, arow1, arow2, arow3, akc, boff, ra0, ra1, ra2,
                                ra3, rb, rs);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int kof = ks * 16 + (lane >> 5) * 8;
            bf16x8_t af[2], bfr[4];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8_t*>(&As[(wm * 64 + mi * 32 + (lane & 31)) * kLDK + kof]);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                bfr[ni] = *reinterpret_cast<const bf16x8_t*>(&Bs[(FT_BBASE(ni) + (lane & 31)) * kLDK + kof]);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
        }
        __syncthreads();
        if (more) {
            gemm_lstore<FMT>(As, Bs, tid, r0, akc, ra0, ra1, ra2, ra3, rb, rs);
            __syncthreads();
        }
    }

    // epilogue
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (r < rows_valid) {
                const int64_t p = row0 + r;
                if (GU) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int n = nt * (kBN / 2) + 64 * wn + 32 * j + (lane & 31);
                        a.Hout[p * a.f + n] = f32_to_bf16_rne(silu(acc[mi][j][v]) * acc[mi][j + 2][v]);
                    }
                } else {
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        const int c = nt * kBN + FT_BBASE(ni) + (lane & 31);
                        a.Y[p * a.d + c] = acc[mi][ni][v];
                    }
                }
            }
        }
    }
#undef FT_BBASE
}

template <int FMT>
hipError_t launch_fmt(const GemmArgs& a, int64_t max_tiles, Timing* tm, hipStream_t st) {
    const int64_t g1 = max_tiles * (a.f / (kBN / 2)), g2 = max_tiles * (a.d / kBN);
    TimedLaunch t1 = timing_launch(tm, FT_K_GEMM_GU);
    hipExtLaunchKernelGGL((gemm_kernel<FMT, true>), dim3((unsigned)g1), dim3(kGemmThreads), 0, st, t1.start, t1.stop,
                          0, a);
    TimedLaunch t2 = timing_launch(tm, FT_K_GEMM_DOWN);
    hipExtLaunchKernelGGL((gemm_kernel<FMT, false>), dim3((unsigned)g2), dim3(kGemmThreads), 0, st, t2.start,
                          t2.stop, 0, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(ft_cache* c, const uint16_t* x, int T, hipStream_t st) {
    GemmArgs a;
    a.x = x;
    a.Hin = c->H;
    a.Hout = c->H;
    a.Y = c->Y;
    a.k = c->sh.top_k;
    a.d = c->sh.d_model;
    a.f = c->sh.d_ff;
    a.meta = c->plan.meta;
    a.active_slot = c->plan.active_slot;
    a.seg = c->plan.seg;
    a.perm = c->plan.perm;
    a.tile_active = c->plan.tile_active;
    a.tile_row0 = c->plan.tile_row0;
    a.tile_first = c->plan.tile_first;
    a.pool = c->pool;
    a.S = c->rl.S;
    a.off_gate = c->rl.off_gate;
    a.off_up = c->rl.off_up;
    a.off_down = c->rl.off_down;
    a.off_sg = c->rl.off_sg;
    a.off_su = c->rl.off_su;
    a.off_sd = c->rl.off_sd;
    // tiles possible for T tokens: rows / BM + active slots
    const int64_t R = (int64_t)T * a.k;
    int64_t act = R < c->N ? R : c->N;
    const int64_t max_tiles = (R + kBM - 1) / kBM + act;
    if (max_tiles > c->plan.max_tiles) return hipErrorInvalidValue;
    switch (c->sh.fmt) {
        case FT_FMT_BF16: return launch_fmt<FT_FMT_BF16>(a, max_tiles, c->timing, st);
        case FT_FMT_FP8_B128: return launch_fmt<FT_FMT_FP8_B128>(a, max_tiles, c->timing, st);
        case FT_FMT_MXFP4_B32: return launch_fmt<FT_FMT_MXFP4_B32>(a, max_tiles, c->timing, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ftmoe
