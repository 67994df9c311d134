// Dot products of the host branch over panel-ordered expert records (AVX-512,
// plain C++: no HIP).  A host-run expert reads its record straight from the
// pinned host bank ("The Expert Cache That Follows the Router": a host-run
// miss reads the source without changing residency).
//
// Panel order: rows 32p..32p+31 of a [rows x K] matrix form one contiguous
// block; inside it the 16-byte unit c of row r sits at unit (c/2)*64 +
// (c%2)*32 + r%32.  So the 16 rows [32p + 16h, +16) at chunk column c are
// 256 contiguous bytes, and a panel's lane block (chunk columns 2i, 2i + 1)
// is 1 KiB.
#pragma once
#include <immintrin.h>
#include <stdint.h>

#include <cmath>

namespace ftmoe {
namespace hostk {

enum { FMT_BF16 = 0, FMT_FP8_B128 = 1, FMT_MXFP4_B32 = 2 };   // the ft_shape formats

inline const float* e2m1_table() {
    alignas(64) static const float t[16] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f,
                                            -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};
    return t;
}

// 16 e4m3 codes -> fp32 / 256.  OCP E4M3 (bias 7): normal (1 + m/8) 2^(e-7),
// subnormal m 2^-9.  The code's 7 magnitude bits shifted left by 7 are an
// fp16 bit pattern (bias 15) with the same exponent and mantissa fields:
// normal (1 + m/8) 2^(e-15), subnormal m 2^-17, i.e. exactly 2^-8 times the
// e4m3 value in both cases, so the hardware fp16 -> fp32 conversion decodes
// it and the caller folds the 2^8 into its scale.  (NaN codes are not
// produced by the encoder and decode as finite values here.)  The byte is
// sign-extended to 16 bits, so one shift by 7 puts the magnitude at bits
// 7..13 and a copy of the sign at bits 14 and 15; clearing bit 14 leaves
// the fp16 pattern.
constexpr float kE4M3Fp16Scale = 256.0f;
inline __m512 e4m3x16_div256(const uint8_t* p) {
    const __m256i v = _mm256_cvtepi8_epi16(_mm_loadu_si128(reinterpret_cast<const __m128i*>(p)));
    return _mm512_cvtph_ps(_mm256_and_si256(_mm256_slli_epi16(v, 7), _mm256_set1_epi16((short)0xBF80)));
}

// e8m0 scale byte -> 2^(e - 127) as fp32 bits (e = 0 gives the subnormal
// 2^-127; 255, the NaN code, is not produced by the encoder)
inline float e8m0(uint32_t e) {
    const uint32_t bits = e ? e << 23 : 0x00400000u;
    float f;
    __builtin_memcpy(&f, &bits, 4);
    return f;
}

// 8 bytes of packed e2m1 (low nibble first) -> 16 fp32 values
inline __m512 e2m1x16(const uint8_t* p, __m512 lut) {
    const __m128i b = _mm_loadl_epi64(reinterpret_cast<const __m128i*>(p));
    const __m512i v = _mm512_cvtepu8_epi32(_mm_unpacklo_epi8(b, b));      // b0 b0 b1 b1 ...
    const __m512i sh = _mm512_set_epi32(4, 0, 4, 0, 4, 0, 4, 0, 4, 0, 4, 0, 4, 0, 4, 0);
    const __m512i idx = _mm512_and_si512(_mm512_srlv_epi32(v, sh), _mm512_set1_epi32(0xF));
    return _mm512_permutexvar_ps(idx, lut);
}

// Where the half panel (p, h) of a [rows x K] code matrix at `off` starts.
inline const uint8_t* half_panel_base(int fmt, const uint8_t* rec, int64_t off, int p, int h, int K) {
    const int64_t row_bytes = fmt == FMT_BF16 ? 2ll * K : fmt == FMT_FP8_B128 ? (int64_t)K : (int64_t)K / 2;
    return rec + off + (int64_t)p * 32 * row_bytes + h * 256;
}

// Software prefetch distance of the dot loops, in 16-byte row units: each
// loop touches the panel lines it will read this many units on (8 KiB of the
// panel ahead).  One core's own demand misses leave it waiting on memory:
// block-FP8, one vector, 12 cores of a 16-core EPYC host read 103 GB/s of
// codes without it and 180 GB/s with it, against 366 GB/s from L2.
constexpr int kPrefetchUnits = 16;

// Prefetch the first `bytes` bytes (a multiple of 16, at most 512) of unit
// column c of the rows that start at `base`, if c < nunits.
inline void prefetch_unit(const uint8_t* base, int c, int nunits, int bytes) {
    if (c >= nunits) return;
    const char* q = reinterpret_cast<const char*>(base + (int64_t)(c >> 1) * 1024 + (c & 1) * 512);
    for (int o = 0; o < bytes; o += 64) _mm_prefetch(q + o, _MM_HINT_T0);
}

// Most vectors the streaming pass below takes for a format; with more, the
// half panel is decoded once into bf16 and dotted by register-blocked tiles.
// One core streams the codes once per pass, so below these counts the record's
// bytes set the pace and the pass beats decoding (block-FP8, 12 cores, codes in
// L2: 4 vectors 249 against 91 GB/s, 6 vectors 187 against 83).
inline int stream_max_vectors(int fmt) { return fmt == FMT_MXFP4_B32 ? 3 : 8; }

// One pass over the half panel for NT vectors: each unit of codes is decoded
// once and dotted with the NT vectors; the 16 rows go in passes of R rows, R
// set so that the R x NT accumulators and the NT vector chunks stay in
// registers.  A row's multiply-adds run in the same order for every R.
template <int NT>
inline void half_panel_dots_stream(int fmt, const uint8_t* rec, int64_t off, int64_t soff, int p, int h, int K,
                                   const float* const* vec, float* out) {
    const uint8_t* base = half_panel_base(fmt, rec, off, p, h, K);
    if (fmt == FMT_BF16) {
        // a zmm holds rows (r0 + 2q, r0 + 2q + 1) x 8 values, the two halves
        // reduced separately
        constexpr int R = NT <= 6 ? 8 : 4, Q = R / 2;
        for (int r0 = 0; r0 < 16; r0 += R) {
            const uint8_t* b0 = base + 16 * r0;
            __m512 a[Q][NT];
            for (int q = 0; q < Q; ++q)
                for (int i = 0; i < NT; ++i) a[q][i] = _mm512_setzero_ps();
            for (int c = 0; c < K / 8; ++c) {
                prefetch_unit(b0, c + kPrefetchUnits, K / 8, 16 * R);
                const uint8_t* u = b0 + (int64_t)(c >> 1) * 1024 + (c & 1) * 512;
                __m512 x[NT];
                for (int i = 0; i < NT; ++i) x[i] = _mm512_broadcast_f32x8(_mm256_loadu_ps(vec[i] + 8 * c));
                for (int q = 0; q < Q; ++q) {
                    const __m256i w16 = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(u + 32 * q));
                    const __m512 w = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(w16), 16));
                    for (int i = 0; i < NT; ++i) a[q][i] = _mm512_fmadd_ps(w, x[i], a[q][i]);
                }
            }
            for (int i = 0; i < NT; ++i)
                for (int q = 0; q < Q; ++q) {
                    out[i * 16 + r0 + 2 * q] = _mm512_mask_reduce_add_ps(0x00FF, a[q][i]);
                    out[i * 16 + r0 + 2 * q + 1] = _mm512_mask_reduce_add_ps(0xFF00, a[q][i]);
                }
        }
        return;
    }
    if (fmt == FMT_FP8_B128) {
        // the block scale is one number for the unit's rows: it multiplies the
        // NT vector chunks, not the rows' codes
        constexpr int R = NT <= 3 ? 8 : NT <= 6 ? 4 : 2;
        const float* sc = reinterpret_cast<const float*>(rec + soff) + (int64_t)(p >> 2) * (K >> 7);
        for (int r0 = 0; r0 < 16; r0 += R) {
            const uint8_t* b0 = base + 16 * r0;
            __m512 a[R][NT];
            for (int j = 0; j < R; ++j)
                for (int i = 0; i < NT; ++i) a[j][i] = _mm512_setzero_ps();
            for (int c = 0; c < K / 16; ++c) {
                prefetch_unit(b0, c + kPrefetchUnits, K / 16, 16 * R);
                const uint8_t* u = b0 + (int64_t)(c >> 1) * 1024 + (c & 1) * 512;
                const __m512 s = _mm512_set1_ps(sc[(16 * c) >> 7] * kE4M3Fp16Scale);
                __m512 x[NT];
                for (int i = 0; i < NT; ++i) x[i] = _mm512_mul_ps(_mm512_loadu_ps(vec[i] + 16 * c), s);
                for (int j = 0; j < R; ++j) {
                    const __m512 w = e4m3x16_div256(u + 16 * j);
                    for (int i = 0; i < NT; ++i) a[j][i] = _mm512_fmadd_ps(w, x[i], a[j][i]);
                }
            }
            for (int i = 0; i < NT; ++i)
                for (int j = 0; j < R; ++j) out[i * 16 + r0 + j] = _mm512_reduce_add_ps(a[j][i]);
        }
        return;
    }
    constexpr int R = NT <= 3 ? 8 : NT <= 6 ? 2 : 1;
    const __m512 lut = _mm512_load_ps(e2m1_table());
    for (int r0 = 0; r0 < 16; r0 += R) {
        const uint8_t* b0 = base + 16 * r0;
        const uint8_t* sb = rec + soff + (int64_t)p * K + 16 * h + r0;     // scale panel: 32 x K/32 bytes
        __m512 a[R][NT];
        for (int j = 0; j < R; ++j)
            for (int i = 0; i < NT; ++i) a[j][i] = _mm512_setzero_ps();
        for (int c = 0; c < K / 32; ++c) {
            prefetch_unit(b0, c + kPrefetchUnits, K / 32, 16 * R);
            const uint8_t* u = b0 + (int64_t)(c >> 1) * 1024 + (c & 1) * 512;
            const uint8_t* su = sb + (c >> 1) * 64 + (c & 1) * 32;
            __m512 x0[NT], x1[NT];
            for (int i = 0; i < NT; ++i) {
                x0[i] = _mm512_loadu_ps(vec[i] + 32 * c);
                x1[i] = _mm512_loadu_ps(vec[i] + 32 * c + 16);
            }
            for (int j = 0; j < R; ++j) {
                const __m512 s = _mm512_set1_ps(e8m0(su[j]));
                const __m512 w0 = _mm512_mul_ps(e2m1x16(u + 16 * j, lut), s);
                const __m512 w1 = _mm512_mul_ps(e2m1x16(u + 16 * j + 8, lut), s);
                for (int i = 0; i < NT; ++i)
                    a[j][i] = _mm512_fmadd_ps(w1, x1[i], _mm512_fmadd_ps(w0, x0[i], a[j][i]));
            }
        }
        for (int i = 0; i < NT; ++i)
            for (int j = 0; j < R; ++j) out[i * 16 + r0 + j] = _mm512_reduce_add_ps(a[j][i]);
    }
}

// One vector, a whole panel: out[r] = row 32p + r of the matrix dotted with
// x, r < 32.  Every lane block is read front to back: bf16 in one pass with
// two rows per accumulator (16 of them), block-FP8 and MXFP4 in two passes
// of 16 rows (the halves), one row per accumulator, so a 1 KiB lane block is
// read in one or two passes instead of four.  For bf16 and block-FP8 each
// row's multiply-adds run in the order of half_panel_dots_stream<1> (the
// same numbers); MXFP4 sums each chunk before applying its scale (fp32
// rounding of the same products).
inline void panel_dots_1(int fmt, const uint8_t* rec, int64_t off, int64_t soff, int p, int K, const float* x,
                         float* out) {
    if (fmt == FMT_BF16) {
        const uint8_t* base = half_panel_base(fmt, rec, off, p, 0, K);
        __m512 a[16];
        for (int q = 0; q < 16; ++q) a[q] = _mm512_setzero_ps();
        for (int c = 0; c < K / 8; ++c) {
            prefetch_unit(base, c + kPrefetchUnits, K / 8, 512);
            const uint8_t* u = base + (int64_t)(c >> 1) * 1024 + (c & 1) * 512;
            const __m512 xv = _mm512_broadcast_f32x8(_mm256_loadu_ps(x + 8 * c));
            for (int q = 0; q < 16; ++q) {      // rows 2q, 2q + 1
                const __m256i w16 = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(u + 32 * q));
                const __m512 w = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(w16), 16));
                a[q] = _mm512_fmadd_ps(w, xv, a[q]);
            }
        }
        for (int q = 0; q < 16; ++q) {
            out[2 * q] = _mm512_mask_reduce_add_ps(0x00FF, a[q]);
            out[2 * q + 1] = _mm512_mask_reduce_add_ps(0xFF00, a[q]);
        }
        return;
    }
    for (int h = 0; h < 2; ++h) {
        const uint8_t* base = half_panel_base(fmt, rec, off, p, h, K);
        __m512 a[16];
        for (int j = 0; j < 16; ++j) a[j] = _mm512_setzero_ps();
        if (fmt == FMT_FP8_B128) {
            const float* sc = reinterpret_cast<const float*>(rec + soff) + (int64_t)(p >> 2) * (K >> 7);
            for (int c = 0; c < K / 16; ++c) {
                prefetch_unit(base, c + kPrefetchUnits, K / 16, 256);
                const uint8_t* u = base + (int64_t)(c >> 1) * 1024 + (c & 1) * 512;
                const __m512 xv = _mm512_mul_ps(_mm512_loadu_ps(x + 16 * c),
                                                _mm512_set1_ps(sc[(16 * c) >> 7] * kE4M3Fp16Scale));
                for (int j = 0; j < 16; ++j) a[j] = _mm512_fmadd_ps(e4m3x16_div256(u + 16 * j), xv, a[j]);
            }
        } else {
            // A row's 16 code bytes hold its 32 values of the chunk: the low
            // nibbles are the even elements, the high nibbles the odd ones, so
            // each half converts with one table permute against the even or the
            // odd half of x (de-interleaved once per chunk for all 16 rows).  The
            // row's block scale (a power of two) multiplies the chunk's sum once;
            // the 16 rows' scale bytes are one 16-byte load.
            const __m512 lut = _mm512_load_ps(e2m1_table());
            const __m512i even = _mm512_set_epi32(30, 28, 26, 24, 22, 20, 18, 16, 14, 12, 10, 8, 6, 4, 2, 0);
            const __m512i odd = _mm512_add_epi32(even, _mm512_set1_epi32(1));
            const uint8_t* sb = rec + soff + (int64_t)p * K + 16 * h;     // scale panel: 32 x K/32 bytes
            for (int c = 0; c < K / 32; ++c) {
                prefetch_unit(base, c + kPrefetchUnits, K / 32, 256);
                const uint8_t* u = base + (int64_t)(c >> 1) * 1024 + (c & 1) * 512;
                const uint8_t* su = sb + (c >> 1) * 64 + (c & 1) * 32;
                const __m512 x0 = _mm512_loadu_ps(x + 32 * c);
                const __m512 x1 = _mm512_loadu_ps(x + 32 * c + 16);
                const __m512 xe = _mm512_permutex2var_ps(x0, even, x1);
                const __m512 xo = _mm512_permutex2var_ps(x0, odd, x1);
                // e8m0 -> 2^(e - 127): e << 23, and the subnormal 2^-127 for e = 0
                const __m512i e = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(su)));
                const __m512 sv = _mm512_castsi512_ps(_mm512_mask_blend_epi32(
                    _mm512_cmpeq_epi32_mask(e, _mm512_setzero_si512()), _mm512_slli_epi32(e, 23),
                    _mm512_set1_epi32(0x00400000)));
                for (int j = 0; j < 16; ++j) {
                    const __m512i b = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(u + 16 * j)));
                    const __m512 we = _mm512_permutexvar_ps(_mm512_and_si512(b, _mm512_set1_epi32(0xF)), lut);
                    const __m512 wo = _mm512_permutexvar_ps(_mm512_srli_epi32(b, 4), lut);
                    const __m512 t = _mm512_fmadd_ps(wo, xo, _mm512_mul_ps(we, xe));
                    a[j] = _mm512_fmadd_ps(t, _mm512_permutexvar_ps(_mm512_set1_epi32(j), sv), a[j]);
                }
            }
        }
        for (int j = 0; j < 16; ++j) out[16 * h + j] = _mm512_reduce_add_ps(a[j]);
    }
}

// Decode the half panel (p, h) into w[r * K + k], r < 16 (fp32, row-major).
inline void half_panel_decode(int fmt, const uint8_t* rec, int64_t off, int64_t soff, int p, int h, int K, float* w) {
    const uint8_t* base = half_panel_base(fmt, rec, off, p, h, K);
    switch (fmt) {
        case FMT_BF16:
            for (int c = 0; c < K / 8; ++c) {
                const uint8_t* u = base + (int64_t)(c >> 1) * 1024 + (c & 1) * 512;
                for (int r = 0; r < 16; r += 2) {
                    const __m256i w16 = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(u + 16 * r));
                    const __m512 v = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(w16), 16));
                    _mm256_storeu_ps(w + (int64_t)r * K + 8 * c, _mm512_castps512_ps256(v));
                    _mm256_storeu_ps(w + (int64_t)(r + 1) * K + 8 * c,
                                     _mm256_castpd_ps(_mm512_extractf64x4_pd(_mm512_castps_pd(v), 1)));
                }
            }
            return;
        case FMT_FP8_B128: {
            const float* sc = reinterpret_cast<const float*>(rec + soff) + (int64_t)(p >> 2) * (K >> 7);
            for (int c = 0; c < K / 16; ++c) {
                const uint8_t* u = base + (int64_t)(c >> 1) * 1024 + (c & 1) * 512;
                const __m512 s = _mm512_set1_ps(sc[(16 * c) >> 7] * kE4M3Fp16Scale);
                for (int r = 0; r < 16; ++r)
                    _mm512_storeu_ps(w + (int64_t)r * K + 16 * c, _mm512_mul_ps(e4m3x16_div256(u + 16 * r), s));
            }
            return;
        }
        default: {
            const __m512 lut = _mm512_load_ps(e2m1_table());
            const uint8_t* sb = rec + soff + (int64_t)p * K + 16 * h;
            for (int c = 0; c < K / 32; ++c) {
                const uint8_t* u = base + (int64_t)(c >> 1) * 1024 + (c & 1) * 512;
                const uint8_t* su = sb + (c >> 1) * 64 + (c & 1) * 32;
                for (int r = 0; r < 16; ++r) {
                    const __m512 s = _mm512_set1_ps(e8m0(su[r]));
                    _mm512_storeu_ps(w + (int64_t)r * K + 32 * c, _mm512_mul_ps(e2m1x16(u + 16 * r, lut), s));
                    _mm512_storeu_ps(w + (int64_t)r * K + 32 * c + 16,
                                     _mm512_mul_ps(e2m1x16(u + 16 * r + 8, lut), s));
                }
            }
            return;
        }
    }
}

// out[i * 16 + r0 + j] = sum_k w[(r0 + j) * K + k] * vec[t0 + i][k] for
// j < 4, i < TB: 4 rows x TB vectors of accumulators in registers, each
// K-step of 16 loads 4 + TB vectors for 4 * TB multiply-adds.
template <int TB>
inline void dots_4xTB(const float* w, int K, const float* const* vec, int t0, int r0, float* out) {
    __m512 a[4][TB];
    for (int j = 0; j < 4; ++j)
        for (int i = 0; i < TB; ++i) a[j][i] = _mm512_setzero_ps();
    const float* w0 = w + (int64_t)r0 * K;
    for (int k = 0; k < K; k += 16) {
        const __m512 wv0 = _mm512_loadu_ps(w0 + k);
        const __m512 wv1 = _mm512_loadu_ps(w0 + K + k);
        const __m512 wv2 = _mm512_loadu_ps(w0 + 2 * (int64_t)K + k);
        const __m512 wv3 = _mm512_loadu_ps(w0 + 3 * (int64_t)K + k);
        for (int i = 0; i < TB; ++i) {
            const __m512 x = _mm512_loadu_ps(vec[t0 + i] + k);
            a[0][i] = _mm512_fmadd_ps(wv0, x, a[0][i]);
            a[1][i] = _mm512_fmadd_ps(wv1, x, a[1][i]);
            a[2][i] = _mm512_fmadd_ps(wv2, x, a[2][i]);
            a[3][i] = _mm512_fmadd_ps(wv3, x, a[3][i]);
        }
    }
    for (int i = 0; i < TB; ++i)
        for (int j = 0; j < 4; ++j) out[(t0 + i) * 16 + r0 + j] = _mm512_reduce_add_ps(a[j][i]);
}

// Dots of 16 decoded rows w [16 x K] with nt vectors: out[i * 16 + r].
inline void dots_16xT(const float* w, int K, const float* const* vec, int nt, float* out) {
    for (int r0 = 0; r0 < 16; r0 += 4) {
        int t0 = 0;
        for (; t0 + 6 <= nt; t0 += 6) dots_4xTB<6>(w, K, vec, t0, r0, out);
        switch (nt - t0) {
            case 5: dots_4xTB<5>(w, K, vec, t0, r0, out); break;
            case 4: dots_4xTB<4>(w, K, vec, t0, r0, out); break;
            case 3: dots_4xTB<3>(w, K, vec, t0, r0, out); break;
            case 2: dots_4xTB<2>(w, K, vec, t0, r0, out); break;
            case 1: dots_4xTB<1>(w, K, vec, t0, r0, out); break;
            default: break;
        }
    }
}

// ---- many vectors in bf16 (AVX512-BF16) ------------------------------------
// With many vectors the multiply-adds set the pace: the half panel is decoded
// once into bf16 rows and dotted by 4-row x 6-vector register tiles over
// column slices that stay in L1; bf16 operands halve the bytes and VDPBF16PS
// does two multiply-adds a lane.  Products of bf16 values are exact in fp32;
// the sums are fp32.

// Row stride of decoded bf16 rows: K plus one cache line, so that rows of a
// power-of-two K do not all fall in one L1 set (16 rows 8 KiB apart thrash a
// 12-way set on every unit).  FP8 configuration, 16 tokens an expert, 12
// cores of one host: decode and dots 38 -> 67 GB/s of codes.
inline int64_t decoded_ld(int K) { return (int64_t)K + 32; }

// Decode the half panel (p, h) into bf16 rows w[r * ld + k], r < 16, k < K:
// bf16 codes as they are; e4m3 times its block scale rounded to bf16 (as the
// GPU grouped GEMM does); e2m1 times its power-of-two scale, exact.
inline void half_panel_decode_bf16(int fmt, const uint8_t* rec, int64_t off, int64_t soff, int p, int h, int K,
                                   uint16_t* w, int64_t ld) {
    const uint8_t* base = half_panel_base(fmt, rec, off, p, h, K);
    switch (fmt) {
        case FMT_BF16:
            for (int c = 0; c < K / 8; ++c) {
                prefetch_unit(base, c + kPrefetchUnits, K / 8, 256);
                const uint8_t* u = base + (int64_t)(c >> 1) * 1024 + (c & 1) * 512;
                for (int r = 0; r < 16; ++r)
                    _mm_storeu_si128(reinterpret_cast<__m128i*>(w + r * ld + 8 * c),
                                     _mm_loadu_si128(reinterpret_cast<const __m128i*>(u + 16 * r)));
            }
            return;
        case FMT_FP8_B128: {
            const float* sc = reinterpret_cast<const float*>(rec + soff) + (int64_t)(p >> 2) * (K >> 7);
            for (int c = 0; c < K / 16; ++c) {
                prefetch_unit(base, c + kPrefetchUnits, K / 16, 256);
                const uint8_t* u = base + (int64_t)(c >> 1) * 1024 + (c & 1) * 512;
                const __m512 s = _mm512_set1_ps(sc[(16 * c) >> 7] * kE4M3Fp16Scale);
                for (int r = 0; r < 16; ++r) {
                    const __m256bh v = _mm512_cvtneps_pbh(_mm512_mul_ps(e4m3x16_div256(u + 16 * r), s));
                    _mm256_storeu_si256(reinterpret_cast<__m256i*>(w + r * ld + 16 * c), (__m256i)v);
                }
            }
            return;
        }
        default: {
            const __m512 lut = _mm512_load_ps(e2m1_table());
            const uint8_t* sb = rec + soff + (int64_t)p * K + 16 * h;
            for (int c = 0; c < K / 32; ++c) {
                prefetch_unit(base, c + kPrefetchUnits, K / 32, 256);
                const uint8_t* u = base + (int64_t)(c >> 1) * 1024 + (c & 1) * 512;
                const uint8_t* su = sb + (c >> 1) * 64 + (c & 1) * 32;
                for (int r = 0; r < 16; ++r) {
                    const __m512 s = _mm512_set1_ps(e8m0(su[r]));
                    const __m512bh v = _mm512_cvtne2ps_pbh(_mm512_mul_ps(e2m1x16(u + 16 * r + 8, lut), s),
                                                            _mm512_mul_ps(e2m1x16(u + 16 * r, lut), s));
                    _mm512_storeu_si512(reinterpret_cast<__m512i*>(w + r * ld + 32 * c), (__m512i)v);
                }
            }
            return;
        }
    }
}

// Columns per slice of the many-vector dots: a tile's 6 vector slices (12 KiB)
// stay in L1 while the 4 row groups pass over them.
constexpr int kDotSlice = 1024;

// acc[j * TB + i] += the lanes of sum_{k0 <= k < k1} w[(r0 + j) * ld + k] *
// vec[t0 + i][k] (bf16 rows and vectors, fp32 lanes) for j < 4, i < TB; the
// accumulators start at zero when `first`.  A lane's multiply-adds run in k
// order whatever the slices, so the sums do not depend on the slicing.
template <int TB>
inline void dots_4xTB_bf16(const uint16_t* w, int64_t ld, const uint16_t* const* vec, int t0, int r0, int k0,
                           int k1, __m512* acc, bool first) {
    __m512 a[4][TB];
    for (int j = 0; j < 4; ++j)
        for (int i = 0; i < TB; ++i) a[j][i] = first ? _mm512_setzero_ps() : acc[j * TB + i];
    const uint16_t* w0 = w + r0 * ld;
    for (int k = k0; k < k1; k += 32) {
        __m512bh wv[4];
        for (int j = 0; j < 4; ++j)
            wv[j] = (__m512bh)_mm512_loadu_si512(reinterpret_cast<const void*>(w0 + j * ld + k));
        for (int i = 0; i < TB; ++i) {
            const __m512bh x = (__m512bh)_mm512_loadu_si512(reinterpret_cast<const void*>(vec[t0 + i] + k));
            for (int j = 0; j < 4; ++j) a[j][i] = _mm512_dpbf16_ps(a[j][i], wv[j], x);
        }
    }
    for (int j = 0; j < 4; ++j)
        for (int i = 0; i < TB; ++i) acc[j * TB + i] = a[j][i];
}

// out[(t0 + i) * 16 + r] = row r of w dotted with vec[t0 + i], r < 16, i < TB:
// slice by slice, the four 4-row groups over the same vector slices.
template <int TB>
inline void dots_16xTB_bf16(const uint16_t* w, int64_t ld, int K, const uint16_t* const* vec, int t0, float* out) {
    __m512 acc[4][4 * TB];
    for (int k0 = 0; k0 < K; k0 += kDotSlice) {
        const int k1 = k0 + kDotSlice < K ? k0 + kDotSlice : K;
        for (int g = 0; g < 4; ++g) dots_4xTB_bf16<TB>(w, ld, vec, t0, 4 * g, k0, k1, acc[g], k0 == 0);
    }
    for (int g = 0; g < 4; ++g)
        for (int j = 0; j < 4; ++j)
            for (int i = 0; i < TB; ++i) out[(t0 + i) * 16 + 4 * g + j] = _mm512_reduce_add_ps(acc[g][j * TB + i]);
}

// Dots of 16 bf16 rows (row r at w + r * ld, K values) with nt bf16 vectors:
// out[i * 16 + r].
inline void dots_16xT_bf16(const uint16_t* w, int64_t ld, int K, const uint16_t* const* vec, int nt, float* out) {
    int t0 = 0;
    for (; t0 + 6 <= nt; t0 += 6) dots_16xTB_bf16<6>(w, ld, K, vec, t0, out);
    switch (nt - t0) {
        case 5: dots_16xTB_bf16<5>(w, ld, K, vec, t0, out); break;
        case 4: dots_16xTB_bf16<4>(w, ld, K, vec, t0, out); break;
        case 3: dots_16xTB_bf16<3>(w, ld, K, vec, t0, out); break;
        case 2: dots_16xTB_bf16<2>(w, ld, K, vec, t0, out); break;
        case 1: dots_16xTB_bf16<1>(w, ld, K, vec, t0, out); break;
        default: break;
    }
}

// Dots of the 16 rows [32p + 16h, +16) of a panel-ordered [rows x K] matrix
// (codes at `off`, scales at `soff`) with nt >= 1 fp32 vectors vec[i] (length
// K): out[i * 16 + r].  Up to stream_max_vectors(fmt) vectors one streaming
// pass; more, the half panel decoded to fp32 once (wdec: scratch of 16 * K
// floats) and dotted by register-blocked tiles.  (The host branch takes the
// bf16 form above for such counts: T = 2,048 calls of the FP8 configuration
// ran 80% faster with it on one box.)
inline void half_panel_dots(int fmt, const uint8_t* rec, int64_t off, int64_t soff, int p, int h, int K,
                            const float* const* vec, int nt, float* wdec, float* out) {
    if (nt <= stream_max_vectors(fmt)) {
        switch (nt) {
            case 1: half_panel_dots_stream<1>(fmt, rec, off, soff, p, h, K, vec, out); return;
            case 2: half_panel_dots_stream<2>(fmt, rec, off, soff, p, h, K, vec, out); return;
            case 3: half_panel_dots_stream<3>(fmt, rec, off, soff, p, h, K, vec, out); return;
            case 4: half_panel_dots_stream<4>(fmt, rec, off, soff, p, h, K, vec, out); return;
            case 5: half_panel_dots_stream<5>(fmt, rec, off, soff, p, h, K, vec, out); return;
            case 6: half_panel_dots_stream<6>(fmt, rec, off, soff, p, h, K, vec, out); return;
            case 7: half_panel_dots_stream<7>(fmt, rec, off, soff, p, h, K, vec, out); return;
            case 8: half_panel_dots_stream<8>(fmt, rec, off, soff, p, h, K, vec, out); return;
            default: break;
        }
    }
    half_panel_decode(fmt, rec, off, soff, p, h, K, wdec);
    dots_16xT(wdec, K, vec, nt, out);
}

}  // namespace hostk
}  // namespace ftmoe
