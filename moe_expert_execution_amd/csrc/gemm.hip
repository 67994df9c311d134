// Prefill expert FFN: grouped GEMMs over the active slots on MFMA.
//
// Rows are the planner's sorted GPU routes; each tile is BM rows of one slot.
// Gate/up: C[rows x 2*64] = X[rows x d] * [WgT; WuT]^T for 64 neurons at a
// time, the gate and up halves landing in the same lanes, so the epilogue
// writes h = silu(g) * u (bf16) without a shuffle.  Down: Y[rows x 128 cols] =
// H[rows x f] * WdT^T in fp32.  Both operands are K-contiguous and staged
// through LDS (one buffer, next tile prefetched into registers during the MFMA
// loop); block-FP8 and MXFP4 weights are dequantised to bf16 as they are
// written to LDS, so every format issues v_mfma_f32_32x32x16_bf16.
// The expert FFN with its gate/up and down projections read from one slot
// record follows "The Expert Cache That Follows the Router", section "One
// logical expert, two physical levels of memory".
#include "wfmt.h"

namespace ftmoe {

constexpr int kBM = 128, kBN = 128, kBK = 64, kLDK = kBK + 8;
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

template <int FMT, bool GU>
__global__ void __launch_bounds__(kGemmThreads) gemm_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLDK];
    using BL = BLoad<FMT>;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int NT = GU ? a.f / 64 : a.d / kBN;
    const int tile = blockIdx.x / NT, nt = blockIdx.x - (blockIdx.x / NT) * NT;
    if (tile >= a.meta[1]) return;
    const int ai = a.tile_active[tile];
    const int row0 = a.tile_row0[tile];
    const int seg_end = a.seg[ai + 1];
    const int slot = a.active_slot[ai];
    int rows_valid = seg_end - row0;
    rows_valid = rows_valid > kBM ? kBM : rows_valid;
    const int K = GU ? a.d : a.f;
    const uint8_t* rec = a.pool + (int64_t)slot * a.S;
    const int64_t rowb = WF<FMT>::row_bytes(K);

    // A rows (4 chunks of 8 bf16 per thread per K-step)
    const uint16_t* arow[4];
    int akc[4], ar[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + kGemmThreads * i;
        ar[i] = q >> 3;
        akc[i] = q & 7;
        arow[i] = nullptr;
        if (ar[i] < rows_valid) {
            const int p = row0 + ar[i];
            arow[i] = GU ? a.x + (int64_t)(a.perm[p] / a.k) * a.d : a.Hin + (int64_t)p * a.f;
        }
    }
    // B rows
    const uint8_t* brow[BL::CPT];
    int bkc[BL::CPT], br[BL::CPT], bn[BL::CPT];
    int64_t bso[BL::CPT];
#pragma unroll
    for (int i = 0; i < BL::CPT; ++i) {
        const int q = tid + kGemmThreads * i;
        br[i] = q / BL::CPR;
        bkc[i] = q - br[i] * BL::CPR;
        int n;
        int64_t off, soff;
        if (GU) {
            const bool up = br[i] >= 64;
            n = nt * 64 + (up ? br[i] - 64 : br[i]);
            off = up ? a.off_up : a.off_gate;
            soff = up ? a.off_su : a.off_sg;
        } else {
            n = nt * kBN + br[i];
            off = a.off_down;
            soff = a.off_sd;
        }
        bn[i] = n;
        brow[i] = rec + off + (int64_t)n * rowb;
        bso[i] = soff;
    }

    f32x16_t acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

    uint4 ra[4], rb[BL::CPT];
    float rs[BL::CPT];
    const int KT = K / kBK;
    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ra[i] = arow[i] ? *reinterpret_cast<const uint4*>(arow[i] + kt * kBK + akc[i] * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < BL::CPT; ++i) {
            const int kk = kt * kBK + bkc[i] * BL::EPC;
            rb[i] = *reinterpret_cast<const uint4*>(brow[i] + WF<FMT>::row_bytes(kk));
            if constexpr (FMT == FT_FMT_FP8_B128) {
                rs[i] = reinterpret_cast<const float*>(rec + bso[i])[(bn[i] >> 7) * (K >> 7) + (kk >> 7)];
            } else if constexpr (FMT == FT_FMT_MXFP4_B32) {
                rs[i] = e8m0_to_f32(rec[bso[i] + (int64_t)bn[i] * (K >> 5) + (kk >> 5)]);
            } else {
                rs[i] = 1.0f;
            }
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&As[ar[i] * kLDK + akc[i] * 8]) = ra[i];
#pragma unroll
        for (int i = 0; i < BL::CPT; ++i) {
            uint16_t* dst = &Bs[br[i] * kLDK + bkc[i] * BL::EPC];
            if constexpr (FMT == FT_FMT_BF16) {
                *reinterpret_cast<uint4*>(dst) = rb[i];
            } else if constexpr (FMT == FT_FMT_FP8_B128) {
                float v[16];
                WF<FMT>::to_f32(rb[i], v);
                uint32_t p[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    p[j] = (uint32_t)f32_to_bf16_rne(v[2 * j] * rs[i]) |
                           ((uint32_t)f32_to_bf16_rne(v[2 * j + 1] * rs[i]) << 16);
                reinterpret_cast<uint4*>(dst)[0] = make_uint4(p[0], p[1], p[2], p[3]);
                reinterpret_cast<uint4*>(dst)[1] = make_uint4(p[4], p[5], p[6], p[7]);
            } else {
                float v[32];
                WF<FMT>::to_f32(rb[i], rs[i], v);
                uint32_t p[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) p[j] = pack_bf16_trunc(v[2 * j], v[2 * j + 1]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    reinterpret_cast<uint4*>(dst)[j] = make_uint4(p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]);
            }
        }
    };

    int bbase[2];
    if (GU) {
        bbase[0] = 32 * wn;
        bbase[1] = 64 + 32 * wn;
    } else {
        bbase[0] = 64 * wn;
        bbase[1] = 64 * wn + 32;
    }

    gload(0);
    for (int kt = 0; kt < KT; ++kt) {
        __syncthreads();
        lstore();
        __syncthreads();
        if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int kof = ks * 16 + (lane >> 5) * 8;
            bf16x8_t af[2], bfr[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8_t*>(&As[(wm * 64 + mi * 32 + (lane & 31)) * kLDK + kof]);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                bfr[ni] = *reinterpret_cast<const bf16x8_t*>(&Bs[(bbase[ni] + (lane & 31)) * kLDK + kof]);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
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
                    const int n = nt * 64 + 32 * wn + (lane & 31);
                    a.Hout[p * a.f + n] = f32_to_bf16_rne(silu(acc[mi][0][v]) * acc[mi][1][v]);
                } else {
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        const int c = nt * kBN + bbase[ni] + (lane & 31);
                        a.Y[p * a.d + c] = acc[mi][ni][v];
                    }
                }
            }
        }
    }
}

template <int FMT>
hipError_t launch_fmt(const GemmArgs& a, int64_t max_tiles, Timing* tm, hipStream_t st) {
    const int64_t g1 = max_tiles * (a.f / 64), g2 = max_tiles * (a.d / kBN);
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
