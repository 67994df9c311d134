// One-token decode expert FFN as one launch (decode_wg.h): one workgroup per
// (GPU route, neuron group); its partial output rows are summed by the
// combine (combine.hip, combine_part_kernel).
#include "decode_wg.h"

namespace ftmoe {
namespace {

constexpr int kDecWaves = 8;       // waves per workgroup of the standalone launch

template <int FMT, int SUBSET>
__global__ void __launch_bounds__(kDecWaves * 64) decode_kernel(DecodeArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
    decode_route_group<FMT, kDecWaves, DecodeShape<FMT>::BU8, SUBSET>(a, blockIdx.x, xs);
}

template <int FMT>
hipError_t launch_fmt(const DecodeArgs& a, int subset, Timing* tm, hipStream_t st) {
    const unsigned grid = (unsigned)(a.k * (a.f / DecodeShape<FMT>::NPW));
    const size_t lds = decode_lds_bytes(a.d);
    TimedLaunch t = timing_launch(tm, FT_K_GEMV_GU);
    if (subset == DEC_FILLS)
        hipExtLaunchKernelGGL((decode_kernel<FMT, DEC_FILLS>), dim3(grid), dim3(kDecWaves * 64), lds, st, t.start,
                              t.stop, 0, a);
    else if (subset == DEC_HITS)
        hipExtLaunchKernelGGL((decode_kernel<FMT, DEC_HITS>), dim3(grid), dim3(kDecWaves * 64), lds, st, t.start,
                              t.stop, 0, a);
    else
        hipExtLaunchKernelGGL((decode_kernel<FMT, DEC_ALL>), dim3(grid), dim3(kDecWaves * 64), lds, st, t.start,
                              t.stop, 0, a);
    return hipGetLastError();
}

}  // namespace

int decode_groups(const ft_shape& s) {
    switch (s.fmt) {
        case FT_FMT_BF16: return s.d_ff / DecodeShape<FT_FMT_BF16>::NPW;
        case FT_FMT_FP8_B128: return s.d_ff / DecodeShape<FT_FMT_FP8_B128>::NPW;
        default: return s.d_ff / DecodeShape<FT_FMT_MXFP4_B32>::NPW;
    }
}

bool decode_fits(const ft_shape& s) { return s.d_model <= kDecodeMaxD; }

DecodeArgs decode_args(const ft_cache* c, const uint16_t* x, const int32_t* routes, int slot_base) {
    DecodeArgs a;
    a.slot_base = slot_base;
    a.E = c->sh.experts;
    a.x = x;
    a.routes = routes;
    a.wl_counts = c->wl_counts;
    a.wl_slot = c->wl_slot;
    a.pool = c->pool;
    a.S = c->rl.P;      // slot stride of the pool
    a.off_gate = c->rl.off_gate;
    a.off_up = c->rl.off_up;
    a.off_down = c->rl.off_down;
    a.off_sg = c->rl.off_sg;
    a.off_su = c->rl.off_su;
    a.off_sd = c->rl.off_sd;
    a.k = c->sh.top_k;
    a.d = c->sh.d_model;
    a.f = c->sh.d_ff;
    a.N = (int)c->N;
    a.part = c->dpart;
    return a;
}

hipError_t launch_decode(ft_cache* c, const uint16_t* x, const int32_t* routes, int subset, hipStream_t st,
                         int slot_base) {
    const DecodeArgs a = decode_args(c, x, routes, slot_base);
    switch (c->sh.fmt) {
        case FT_FMT_BF16: return launch_fmt<FT_FMT_BF16>(a, subset, c->timing, st);
        case FT_FMT_FP8_B128: return launch_fmt<FT_FMT_FP8_B128>(a, subset, c->timing, st);
        case FT_FMT_MXFP4_B32: return launch_fmt<FT_FMT_MXFP4_B32>(a, subset, c->timing, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ftmoe
