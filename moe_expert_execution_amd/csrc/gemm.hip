// Prefill expert FFN: grouped GEMMs over the active slots on MFMA.
//
// Rows are the planner's sorted GPU routes; each tile is 128 rows of one slot.
// Gate/up: C[rows x 2*128] = X[rows x d] * [WgT; WuT]^T for 128 neurons at a
// time, the gate and up halves landing in the same lanes, so the epilogue
// writes h = silu(g) * u (bf16) without a shuffle.  Down: Y[rows x 256 cols] =
// H[rows x f] * WdT^T, accumulated in fp32 and stored as bf16.
//
// Weights are panel-ordered in the slot record: one 16-byte load per lane at
// consecutive addresses delivers a 32-column x (two 16-byte chunk columns)
// operand tile, which is exactly an operand layout of
// v_mfma_f32_32x32x16_bf16 (lane l: row l % 32, chunk column l / 32).  So
// the weights go from memory straight into registers — no LDS staging, no
// shuffles — two K-steps ahead of their use; only the activation tile (shared
// by the four waves) is staged through LDS, loaded straight into a 4-deep
// ring of buffers, one barrier per K-step.  Block-FP8 and MXFP4 weights are
// converted to bf16 in registers right before their MFMA, so every format
// issues the bf16 MFMA.  The expert FFN with its gate/up and down projections
// read from one slot record follows "The Expert Cache That Follows the
// Router", section "One logical expert, two physical levels of memory".
#include <type_traits>

#include "wfmt.h"

namespace ftmoe {

constexpr int kBM = 128, kBN = 256, kBK = 64, kStages = 4;
constexpr int kGemmThreads = 256;

int gemm_tile_m() { return kBM; }

struct GemmArgs {
    const uint16_t* x;
    const uint16_t* Hin;   // bf16 [rows x f] (down A)
    uint16_t* Hout;        // bf16 [rows x f] (gate/up C)
    uint16_t* Y;           // bf16 [rows x d]
    int k, d, f;
    uint32_t x_bytes, h_bytes;   // extents of x and H (their rows are reached by 32-bit offsets)
    const int32_t* meta;
    const int32_t* active_slot;
    const int32_t* seg;
    const int32_t* perm;
    const int32_t* tile_active;
    const int32_t* tile_row0;
    const int32_t* tile_first;
    const uint8_t* pool;
    int64_t S;          // slot stride of the pool (bytes)
    int64_t off_gate, off_up, off_down, off_sg, off_su, off_sd;
};

namespace {

// silu with a hardware reciprocal (1 ulp): z / (1 + e^-z)
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Per format: lane blocks (1 KiB panel runs) per K-step, and where the lane's
// 8 bf16 of MFMA step ks sit inside the 64-wide K-step (the A side must read
// the same K positions).
template <int FMT>
struct Frag {
    static constexpr int LBK = 64 / (2 * WF<FMT>::EPC);    // lane blocks per K-step: 4, 2, 1
    // a weight scale as stored: fp32 bits (FP8), an e8m0 byte (MXFP4)
    using SRaw = std::conditional_t<FMT == FT_FMT_MXFP4_B32, uint8_t, uint32_t>;
    __device__ static int a_koff(int ks, int g) {
        if constexpr (FMT == FT_FMT_BF16) return ks * 16 + g * 8;
        else if constexpr (FMT == FT_FMT_FP8_B128) return (ks >> 1) * 32 + g * 16 + (ks & 1) * 8;
        else return g * 32 + ks * 8;
    }
};

// B operand of MFMA step ks from the K-step's lane-block registers; `sraw` is
// the scale as loaded (FP8: fp32 bits, MXFP4: the e8m0 byte), decoded here so
// that its load is waited for only where it is used.
template <int FMT>
__device__ __forceinline__ bf16x8_t b_frag(const u32x4_t (&r)[Frag<FMT>::LBK], int ks, typename Frag<FMT>::SRaw sraw) {
    if constexpr (FMT == FT_FMT_BF16) {
        return __builtin_bit_cast(bf16x8_t, r[ks]);
    } else if constexpr (FMT == FT_FMT_FP8_B128) {
        const float scale = __uint_as_float(sraw);
        const u32x4_t w = r[ks >> 1];
        const uint32_t w0 = (ks & 1) ? w[2] : w[0];
        const uint32_t w1 = (ks & 1) ? w[3] : w[1];
        const f32x2_t p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false);
        const f32x2_t p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
        const f32x2_t p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false);
        const f32x2_t p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
        const bf16x2_t q0 = __builtin_convertvector(p0 * scale, bf16x2_t);
        const bf16x2_t q1 = __builtin_convertvector(p1 * scale, bf16x2_t);
        const bf16x2_t q2 = __builtin_convertvector(p2 * scale, bf16x2_t);
        const bf16x2_t q3 = __builtin_convertvector(p3 * scale, bf16x2_t);
        return bf16x8_t{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
    } else {
        const float scale = e8m0_to_f32(sraw);
        const uint32_t w = r[0][ks];
        const bf16x2_t q0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
        const bf16x2_t q1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
        const bf16x2_t q2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
        const bf16x2_t q3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
        return bf16x8_t{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
    }
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (they complete in issue order); the other counters are left alone.
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Tile (kBM rows of one slot) x (kBN columns) per workgroup; 4 waves side by
// side along N, each computing 128 x 64 with 4 x 2 v_mfma_f32_32x32x16_bf16
// accumulators.  Gate/up: the kBN columns are 128 gate and the same 128 up
// neurons; wave w owns neurons [32 w, 32 w + 32) of both (B panel 0 gate,
// panel 1 up), so SwiGLU pairs accumulator 0 with 1 in-lane.  Down: wave w
// owns output columns [64 w, 64 w + 64), two panels.
// Workgroups are renumbered so that each XCD (dispatch round-robin over 8)
// receives a contiguous range of blocks, ordered by slot, then N-tile, then
// M-tile: all blocks of an expert run together in one XCD, where its A rows
// and weight panels are read from HBM about once and then hit that XCD's L2.
//
// The activation tile goes from memory straight into LDS (buffer_load_dwordx4
// with the lds modifier: each lane's 16 bytes land at the wave's base + 16 x
// lane) through a ring of kStages K-step buffers, kStages - 1 steps ahead of
// its use.  The buffer form, not global_load_lds: the compiler treats the
// latter as a FLAT access to both memory kinds and then turns every register
// wait into vmcnt(0), draining the weight prefetch.  A buffer is 128 rows x 128 bytes; 16-byte chunk c of row r sits
// at position c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1), so that the 16 (or 8)
// rows one ds_read_b128 serves per cycle fall in distinct banks.  Waits are
// explicit (vmcnt + s_barrier): a __syncthreads would also drain the weight
// loads that are in flight for later steps.
template <int FMT, bool GU>
__global__ void __launch_bounds__(kGemmThreads, 2) gemm_kernel(GemmArgs a) {
    using FR = Frag<FMT>;
    constexpr int LBK = FR::LBK;
    constexpr int NB = 2 * LBK;                   // weight loads per wave per K-step
    __shared__ __attribute__((aligned(1024))) uint16_t As[kStages][kBM * kBK];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // d (a multiple of 128) may end in a half N-tile of the down product: its
    // waves 2 and 3 have no columns, re-read the last panel and store nothing
    const int NT = GU ? a.f / (kBN / 2) : (a.d + kBN - 1) / kBN;
    const int V = a.meta[1] * NT;                 // valid workgroups
    const int b = blockIdx.x;
    if (b >= V) return;
    const int q8 = V >> 3, r8 = V & 7, x8 = b & 7;
    const int lb = x8 * q8 + (x8 < r8 ? x8 : r8) + (b >> 3);
    // within one slot's blocks [t0 NT, (t0 + mt) NT): N-tile major, M-tile minor,
    // so the M-tiles sharing a weight panel run side by side
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
    const int64_t panel_bytes = 32 * rowb;

    // this wave's two weight panels (+ lane offset); their scale locations
    const uint8_t* bp[2];
    int64_t soff[2];
    int pn[2];
    if (GU) {
        pn[0] = pn[1] = nt * 4 + w;
        bp[0] = rec + a.off_gate + pn[0] * panel_bytes + lane * 16;
        bp[1] = rec + a.off_up + pn[1] * panel_bytes + lane * 16;
        soff[0] = a.off_sg;
        soff[1] = a.off_su;
    } else {
        const int last = a.d / 32 - 1;
        pn[0] = min(nt * 8 + 2 * w, last);
        pn[1] = min(nt * 8 + 2 * w + 1, last);
        bp[0] = rec + a.off_down + pn[0] * panel_bytes + lane * 16;
        bp[1] = rec + a.off_down + pn[1] * panel_bytes + lane * 16;
        soff[0] = soff[1] = a.off_sd;
    }
    // per-K-step weight scale of panel i, as stored: FP8 — the 128 x 128
    // block's fp32 (uniform over the panel); MXFP4 — the lane's e8m0 byte for
    // its chunk
    auto scale_of = [&](int i, int kt) -> typename FR::SRaw {
        if constexpr (FMT == FT_FMT_FP8_B128) {
            return reinterpret_cast<const uint32_t*>(rec + soff[i])[(pn[i] >> 2) * (K >> 7) + (kt >> 1)];
        } else if constexpr (FMT == FT_FMT_MXFP4_B32) {
            return rec[soff[i] + (int64_t)pn[i] * K + kt * 64 + lane];
        } else {
            return 0;
        }
    };

    // A: wave w fills rows [32 w, 32 w + 32) of a buffer with 4 loads, load i
    // covering the 1 KiB of rows 32 w + 8 i .. + 7: lane l takes row
    // 32 w + 8 i + l / 8 at physical chunk l % 8, i.e. logical chunk
    // (l % 8) ^ (l / 8) ^ (i & 1).  Rows past the tile's end repeat its last
    // row: their outputs are never stored.  The loads are buffer loads (byte
    // offsets from x or H, the K-step in the scalar offset); the hardware
    // returns zeros for any offset past the buffer's extent.
    const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(GU ? a.x : a.Hin), 0, (int)(GU ? a.x_bytes : a.h_bytes), 0x00020000);
    uint32_t avo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int r = 32 * w + 8 * i + (lane >> 3);
        r = r < rows_valid ? r : rows_valid - 1;
        const int p = row0 + r;
        const int c = (lane & 7) ^ (lane >> 3) ^ (i & 1);
        const uint32_t row = GU ? (uint32_t)(a.perm[p] / a.k) * (uint32_t)a.d : (uint32_t)p * (uint32_t)a.f;
        avo[i] = (row + (uint32_t)c * 8u) * 2u;
    }
    const int KT = K / kBK;        // even: K is a multiple of 128
    auto load_a = [&](int kt, int stage) {
        const int ks = kt < KT ? kt : KT - 1;       // past the end: reload the last step (never read)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                arsrc, (__attribute__((address_space(3))) void*)(&As[stage][(4 * w + i) * 512]), 16, avo[i],
                ks * kBK * 2, 0, 0);
    };

    // The tile's MI = ceil(rows_valid / 32) row blocks are all that is
    // computed: a short last tile of an expert (its few leftover rows) costs
    // MI / 4 of a full tile's MFMAs.
    auto body = [&](auto mi_count) {
        constexpr int MI = decltype(mi_count)::value;
        f32x16_t acc[MI][2];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

        // Two sets of weight registers, for even and odd K-steps: step kt reads
        // set kt % 2 and then refills it with K-step kt + 2, so every weight load
        // has two K-steps to arrive and lands in the registers its consumer reads.
        u32x4_t br[2][2][LBK];
        typename FR::SRaw bs[2][2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int j = 0; j < LBK; ++j)
                    br[s2][i][j] = *reinterpret_cast<const u32x4_t*>(bp[i] + (int64_t)(s2 * LBK + j) * 1024);
                bs[s2][i] = scale_of(i, s2);
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < kStages - 1; ++s) load_a(s, s);
        __builtin_amdgcn_sched_barrier(0);

        // A operand of MFMA step ks for the MI row blocks, from buffer `stage`
        const int m = lane & 31;
        const int fm = (m & 7) ^ ((m >> 3) & 1);
        auto read_a = [&](bf16x8_t (&af)[MI], int stage, int ks) {
            const int c = FR::a_koff(ks, g) >> 3;
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8_t*>(&As[stage][(mi * 32 + m) * kBK + ((c ^ fm) << 3)]);
        };
        bf16x8_t af[2][MI];
        // A(0) has landed once only A(1) and A(2) may be outstanding
        vm_wait<8>();
        __builtin_amdgcn_s_barrier();
        read_a(af[0], 0, 0);

        // One K-step.  Vector-memory operations of a wave complete in issue order,
        // so "A of step kt + 1 has landed" is a count of the loads issued after
        // it.  A step issues RP weight refills, then (before its last MFMA
        // group) A(kt + 3), then the last NB - RP refills (scale loads come after
        // them and only make the count conservative); the prologue issued B(0),
        // B(1), A(0), A(1), A(2).  After every wave has seen its own loads land,
        // one barrier publishes buffer kt + 1; it also tells that every wave has
        // finished step kt - 1, the last reader of the buffer A(kt + 3) refills.
        // Putting it before the last MFMA group lets the next step's first LDS
        // reads overlap this step's last MFMAs.  Instruction order is pinned with
        // scheduling barriers: the compiler would otherwise sink every prefetch
        // below the last MFMA.
        constexpr int RP = 2 * (LBK - 1);             // refills issued before A(kt + 3)
        auto kstep = [&](int kt, int stage, u32x4_t (&brs)[2][LBK], typename FR::SRaw (&bss)[2]) {
            const int kw = kt + 2 < KT ? kt + 2 : KT - 1;     // weights refilled for two steps ahead
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (ks < 3) {
                    read_a(af[(ks + 1) & 1], stage, ks + 1);
                } else {
                    if (kt >= 2) vm_wait<2 * NB + 4>();
                    else if (kt == 1) vm_wait<NB + 4 + RP>();
                    else vm_wait<4 + RP>();
                    __builtin_amdgcn_s_barrier();
                    __builtin_amdgcn_sched_barrier(0);
                    load_a(kt + 3, (stage + 3) % kStages);
                    __builtin_amdgcn_sched_barrier(0);
                    read_a(af[0], (stage + 1) % kStages, 0);
                }
                const bf16x8_t b0 = b_frag<FMT>(brs[0], ks, bss[0]);
                const bf16x8_t b1 = b_frag<FMT>(brs[1], ks, bss[1]);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    acc[mi][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, af[ks & 1][mi], acc[mi][0], 0, 0, 0);
                    acc[mi][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, af[ks & 1][mi], acc[mi][1], 0, 0, 0);
                }
                constexpr int kDone = 4 / LBK;                // MFMA steps per lane block
                if ((ks % kDone) == kDone - 1) {
                    const int j = ks / kDone;
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        brs[i][j] = *reinterpret_cast<const u32x4_t*>(bp[i] + (int64_t)(kw * LBK + j) * 1024);
                }
                // order inside the group: the next group's LDS reads interleaved
                // with the first MFMAs, then the rest, then the refill loads
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, MI, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);       // global loads
                __builtin_amdgcn_sched_barrier(0);
            }
            // the refilled set's scales, loaded straight into the registers that
            // step kw reads (a copy would have to wait for the load)
#pragma unroll
            for (int i = 0; i < 2; ++i) bss[i] = scale_of(i, kw);
        };
        static_assert(kStages == 4, "the step unrolling below pairs stages with weight register sets");
        for (int kt = 0; kt < KT; kt += 4) {
            kstep(kt, 0, br[0], bs[0]);
            kstep(kt + 1, 1, br[1], bs[1]);
            if (kt + 2 < KT) {
                kstep(kt + 2, 2, br[0], bs[0]);
                kstep(kt + 3, 3, br[1], bs[1]);
            }
        }
        // the ring's last (unused) loads must land before the buffers are reused
        vm_wait<0>();
        __builtin_amdgcn_s_barrier();

        // Epilogue.  The MFMAs compute C^T (weights as the A operand), so lane l
        // holds row mi*32 + l%32 and, per group q, the four consecutive columns
        // 8q + 4(l/32) .. +3 of each 32-column panel.  The tile goes through LDS
        // (free once the ring has drained) so that every global store
        // instruction writes whole contiguous row segments.
        if (GU) {
            // h = silu(g) * u, the whole 128 x 128 bf16 tile, rows padded by 16 bytes
            constexpr int LDH = kBN / 2 + 8;
            uint16_t* Hs = &As[0][0];
            static_assert(kBM * LDH <= kStages * kBM * kBK, "h tile must fit the A buffers");
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float h[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) h[j] = silu(acc[mi][0][4 * q + j]) * acc[mi][1][4 * q + j];
                    uint2 o;
                    o.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{h[0], h[1]}, bf16x2_t));
                    o.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{h[2], h[3]}, bf16x2_t));
                    *reinterpret_cast<uint2*>(&Hs[(mi * 32 + m) * LDH + 32 * w + 8 * q + 4 * g]) = o;
                }
            __syncthreads();
            // 16 lanes per 256-byte row, 16 rows per pass
#pragma unroll
            for (int it = 0; it < MI * 2; ++it) {
                const int r = it * 16 + (tid >> 4), c = (tid & 15) * 8;
                if (r < rows_valid)
                    *reinterpret_cast<u32x4_t*>(a.Hout + (int64_t)(row0 + r) * a.f + nt * (kBN / 2) + c) =
                        *reinterpret_cast<const u32x4_t*>(&Hs[r * LDH + c]);
            }
        } else {
            // per wave: 32 rows x 64 bf16 columns at a time, rows padded by 16 bytes
            constexpr int LDY = 64 + 8;
            uint16_t* Ys = &As[0][0] + w * 32 * LDY;
            const bool col_ok = nt * kBN + 64 * w < a.d;
            static_assert(4 * 32 * LDY <= kStages * kBM * kBK, "y tiles must fit the A buffers");
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        uint2 o;
                        o.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                  f32x2_t{acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1]}, bf16x2_t));
                        o.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                  f32x2_t{acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]}, bf16x2_t));
                        *reinterpret_cast<uint2*>(&Ys[m * LDY + 32 * ni + 8 * q + 4 * g]) = o;
                    }
                // the wave reads back what it wrote (LDS operations of a wave stay in order)
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                // 8 lanes per 128-byte row, 8 rows per pass
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int rr = it * 8 + (lane >> 3), c = (lane & 7) * 8;
                    const int r = mi * 32 + rr;
                    if (r < rows_valid && col_ok)
                        *reinterpret_cast<u32x4_t*>(a.Y + (int64_t)(row0 + r) * a.d + nt * kBN + 64 * w + c) =
                            *reinterpret_cast<const u32x4_t*>(&Ys[rr * LDY + c]);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        }
    };
    const int nmi = (rows_valid + 31) >> 5;
    if (nmi >= 4) body(std::integral_constant<int, 4>{});
    else if (nmi == 3) body(std::integral_constant<int, 3>{});
    else if (nmi == 2) body(std::integral_constant<int, 2>{});
    else body(std::integral_constant<int, 1>{});
}

template <int FMT>
hipError_t launch_fmt(const GemmArgs& a, int64_t max_tiles, Timing* tm, hipStream_t st) {
    const int64_t g1 = max_tiles * (a.f / (kBN / 2)), g2 = max_tiles * ((a.d + kBN - 1) / kBN);
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
    // creation keeps both below 4 GiB
    a.x_bytes = (uint32_t)((int64_t)T * a.d * 2);
    a.h_bytes = (uint32_t)((int64_t)c->cap * a.f * 2);
    a.meta = c->plan.meta;
    a.active_slot = c->plan.active_slot;
    a.seg = c->plan.seg;
    a.perm = c->plan.perm;
    a.tile_active = c->plan.tile_active;
    a.tile_row0 = c->plan.tile_row0;
    a.tile_first = c->plan.tile_first;
    a.pool = c->pool;
    a.S = c->rl.P;   // slot stride of the pool
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
