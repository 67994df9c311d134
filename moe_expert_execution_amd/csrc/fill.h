// Device-initiated pull of whole expert records from the pinned host bank
// into slots: the decode fill of "The Expert Cache That Follows the Router",
// section "One logical expert, two physical levels of memory" (a miss admitted
// to the cache brings its whole record to the device).
#pragma once

#include "common.h"

namespace ftmoe {

constexpr int64_t kFillChunk = 64 * 1024;
typedef uint32_t fill_vec_t __attribute__((ext_vector_type(4)));   // 16 bytes

// Record wl_src[i] (a flat id: layer wl_src[i] / E, expert wl_src[i] % E) of
// the host bank -> slot wl_slot[i] of the pool (slots P bytes apart, P a
// multiple of 256), for i < q =
// wl_counts[3] (device data, so the grid is fixed).  Workgroup `blk` of
// `nblk`, NT threads, walks 64 KiB chunks of the q records, one 16-byte load
// in flight per thread; a record size that is not a multiple of 16 bytes
// (block-FP8 at small d, f; always a multiple of 4) is copied in 4-byte
// words, whose bank addresses are then only 4-byte aligned.  Measured on the MI355X host link, 9.44 MB records, 512
// workgroups: a workgroup's host reads in flight set the rate — 4 KiB
// (256 threads x 1 load) 55.6-56.5 GB/s, 16 KiB 52.4-53.5, 32 KiB 49.8-52.2.
template <int NT>
__device__ __forceinline__ void fill_records(const int32_t* wl_counts, const int32_t* wl_slot,
                                             const int32_t* wl_src, const uint8_t* const* __restrict__ banks,
                                             int E, uint8_t* __restrict__ pool, int64_t S, int64_t P, int blk,
                                             int nblk) {
    const int q = wl_counts[3];
    const int64_t cpr = (S + kFillChunk - 1) / kFillChunk;
    const int64_t total = (int64_t)q * cpr;
    for (int64_t c = blk; c < total; c += nblk) {
        const int64_t i = c / cpr;
        const int64_t off = (c - i * cpr) * kFillChunk;
        const int64_t len = (S - off) < kFillChunk ? (S - off) : kFillChunk;
        const int flat = wl_src[i];
        const uint8_t* s8 = banks[flat / E] + (int64_t)(flat % E) * S + off;
        uint8_t* d8 = pool + (int64_t)wl_slot[i] * P + off;
        // streaming (nontemporal) stores: the records go to HBM without
        // leaving dirty L2 lines whose write-back would delay the expert
        // kernels that read them next
        if ((S & 15) == 0) {
            const fill_vec_t* src = reinterpret_cast<const fill_vec_t*>(s8);
            fill_vec_t* dst = reinterpret_cast<fill_vec_t*>(d8);
            for (int64_t b = threadIdx.x; b < len / 16; b += NT) __builtin_nontemporal_store(src[b], dst + b);
        } else {
            const uint32_t* src = reinterpret_cast<const uint32_t*>(s8);
            uint32_t* dst = reinterpret_cast<uint32_t*>(d8);
            for (int64_t b = threadIdx.x; b < len / 4; b += NT) __builtin_nontemporal_store(src[b], dst + b);
        }
    }
}

}  // namespace ftmoe
