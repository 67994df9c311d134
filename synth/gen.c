/* Seeded synthetic input generator (weights, router matrices, activations).
 *
 * This file draws inputs only; it holds none of the MoE layer's arithmetic.
 * Randomness comes from a counter-based generator: element i of a stream with
 * key K is a 16-bit lane of SplitMix64's output function applied to
 * K + (i/4 + 1) * 0x9e3779b97f4a7c15 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  Because every element is a
 * pure function of (key, index), records can be generated in any order and by
 * any number of threads with identical bytes.
 *
 * Distributions are produced by table lookup: the caller passes a 65536-entry
 * table (for example bf16 values of sigma * Phi^-1((i + 0.5) / 65536)) and the
 * 16-bit lane selects an entry.
 *
 * Record layout written here (bytes of one layer-expert record), matching the
 * library header:
 *   bf16 : WgT [f x d] | WuT [f x d] | WdT [d x f]                (bf16)
 *   fp8  : WgT | WuT | WdT codes (e4m3fn, u8) | sg [f/128 x d/128] | su | sd [d/128 x f/128] (f32)
 *   mxfp4: WgT [f x d/2] | WuT | WdT [d x f/2] codes (two e2m1 per byte, low nibble = even k)
 *          | sg [f x d/32] | su | sd [d x f/32] (e8m0, u8)
 * Every code matrix and every e8m0 scale matrix [rows x K] is stored in
 * 32-row panels: panel p (rows 32p .. 32p+31) occupies one contiguous block,
 * and inside it unit c of row r (a unit is 16 bytes of codes, or one scale
 * byte; c counts along K) sits at unit index (c/2)*64 + (c%2)*32 + (r%32).
 * The fp8 block scales stay row-major.  The logical matrices (the streams
 * below, read row-major) do not depend on this layout.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <pthread.h>
#include <stdlib.h>

#define GOLDEN 0x9e3779b97f4a7c15ULL

static inline uint64_t sx_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* Stream key from a seed and a tuple of integers (config, tensor, layer, expert, ...). */
uint64_t sx_key(uint64_t seed, const int64_t* parts, int n) {
    uint64_t k = sx_mix(seed + GOLDEN);
    for (int i = 0; i < n; ++i) k = sx_mix(k + (uint64_t)parts[i] * GOLDEN + 0x632be59bd9b4e019ULL);
    return k;
}

static inline uint16_t lane16(uint64_t key, int64_t i) {
    uint64_t h = sx_mix(key + (uint64_t)(i / 4 + 1) * GOLDEN);
    return (uint16_t)(h >> (16 * (i & 3)));
}

/* Elements [i0, i0 + n) of a stream. */
void sx_fill_u16_at(uint16_t* out, int64_t i0, int64_t n, uint64_t key, const uint16_t* table) {
    int64_t i = i0, end = i0 + n;
    for (; i < end && (i & 3); ++i) out[i - i0] = table[lane16(key, i)];
    for (; i + 4 <= end; i += 4) {
        uint64_t h = sx_mix(key + (uint64_t)(i / 4 + 1) * GOLDEN);
        out[i - i0] = table[h & 0xFFFF];
        out[i - i0 + 1] = table[(h >> 16) & 0xFFFF];
        out[i - i0 + 2] = table[(h >> 32) & 0xFFFF];
        out[i - i0 + 3] = table[(h >> 48) & 0xFFFF];
    }
    for (; i < end; ++i) out[i - i0] = table[lane16(key, i)];
}

void sx_fill_u16(uint16_t* out, int64_t n, uint64_t key, const uint16_t* table) {
    sx_fill_u16_at(out, 0, n, key, table);
}

void sx_fill_u8_at(uint8_t* out, int64_t i0, int64_t n, uint64_t key, const uint8_t* table) {
    for (int64_t i = 0; i < n; ++i) out[i] = table[lane16(key, i0 + i)];
}

void sx_fill_u8(uint8_t* out, int64_t n, uint64_t key, const uint8_t* table) {
    sx_fill_u8_at(out, 0, n, key, table);
}

void sx_fill_f32_at(float* out, int64_t i0, int64_t n, uint64_t key, const float* table) {
    for (int64_t i = 0; i < n; ++i) out[i] = table[lane16(key, i0 + i)];
}

void sx_fill_f32(float* out, int64_t n, uint64_t key, const float* table) {
    sx_fill_f32_at(out, 0, n, key, table);
}

/* Uniform random bytes [b0, b0 + n) of a stream (each byte = two uniform e2m1 codes). */
void sx_fill_bytes_at(uint8_t* out, int64_t b0, int64_t n, uint64_t key) {
    int64_t i = b0, end = b0 + n;
    while (i < end) {
        uint64_t h = sx_mix(key + (uint64_t)(i / 8 + 1) * GOLDEN);
        uint8_t b[8];
        memcpy(b, &h, 8);
        int64_t stop = (i / 8 + 1) * 8;
        if (stop > end) stop = end;
        for (; i < stop; ++i) out[i - b0] = b[i & 7];
    }
}

void sx_fill_bytes(uint8_t* out, int64_t n, uint64_t key) {
    sx_fill_bytes_at(out, 0, n, key);
}

/* Store 32 logical rows (row-major, `units` units of `unit` bytes per row,
 * `units` even) as one panel: unit c of row r goes to unit index
 * (c/2)*64 + (c%2)*32 + r. */
static void panel_store(const uint8_t* src, uint8_t* dst, int64_t units, int unit) {
    for (int r = 0; r < 32; ++r)
        for (int64_t c = 0; c < units; ++c)
            memcpy(dst + ((c >> 1) * 64 + (c & 1) * 32 + r) * unit, src + (r * units + c) * unit, (size_t)unit);
}

/* Harness-side e4m3fn encoder (OCP 8-bit floating point, E4M3 with no infinities,
 * max finite 448): round to nearest even, saturating to +-448. */
static uint8_t enc_e4m3(float v) {
    uint8_t sign = 0;
    if (v < 0) { sign = 0x80; v = -v; }
    if (!(v == v)) return 0x7F;
    if (v >= 448.0f) return sign | 0x7E;
    if (v == 0.0f) return sign;
    int e;
    frexpf(v, &e);            /* v = m * 2^e, m in [0.5, 1) -> unbiased exponent e-1 */
    int ue = e - 1;
    if (ue < -6) ue = -6;     /* subnormal range shares the 2^-6 exponent, step 2^-9 */
    float step = ldexpf(1.0f, ue - 3);
    float q = v / step;       /* exact: step is a power of two */
    float r = nearbyintf(q);  /* default rounding mode: nearest-even */
    float val = r * step;
    if (val >= 448.0f) return sign | 0x7E;
    if (r == 0.0f) return sign;
    int e2;
    frexpf(val, &e2);
    int ue2 = e2 - 1;
    if (ue2 < -6) {           /* subnormal: exponent field 0, mantissa = val / 2^-9 */
        return sign | (uint8_t)(int)(val / ldexpf(1.0f, -9));
    }
    int man = (int)(val / ldexpf(1.0f, ue2) * 8.0f) - 8;
    return sign | (uint8_t)(((ue2 + 7) << 3) | man);
}

/* Quantise a [rows x cols] fp32 matrix in 128x128 blocks: scale = amax / 448,
 * code = e4m3(w / scale).  scales is [rows/128 x cols/128]. */
void sx_quant_e4m3_128(const float* w, int64_t rows, int64_t cols, uint8_t* codes, float* scales) {
    int64_t br = rows / 128, bc = cols / 128;
    for (int64_t bi = 0; bi < br; ++bi)
        for (int64_t bj = 0; bj < bc; ++bj) {
            float amax = 0.0f;
            for (int64_t r = 0; r < 128; ++r)
                for (int64_t c = 0; c < 128; ++c) {
                    float a = fabsf(w[(bi * 128 + r) * cols + bj * 128 + c]);
                    if (a > amax) amax = a;
                }
            float s = amax > 0.0f ? amax / 448.0f : 1.0f;
            scales[bi * bc + bj] = s;
            for (int64_t r = 0; r < 128; ++r)
                for (int64_t c = 0; c < 128; ++c) {
                    int64_t o = (bi * 128 + r) * cols + bj * 128 + c;
                    codes[o] = enc_e4m3(w[o] / s);
                }
        }
}

enum { FMT_BF16 = 0, FMT_FP8 = 1, FMT_MXFP4 = 2 };

int64_t sx_record_bytes(int fmt, int64_t d, int64_t f) {
    if (fmt == FMT_BF16) return 3 * d * f * 2;
    if (fmt == FMT_FP8) return 3 * d * f + 3 * (d / 128) * (f / 128) * 4;
    if (fmt == FMT_MXFP4) return 3 * d * f / 2 + 3 * d * f / 32;
    return -1;
}

typedef struct {
    int fmt; int64_t d, f; uint64_t seed; int64_t cfg, E, rec0, rec1, layer_alias, layer_offset;
    uint8_t* out; int64_t stride;
    const uint16_t* t_bf16; const float* t_f32; const uint8_t* t_e8m0;
    int64_t next; pthread_mutex_t mu;
} bank_job;

/* One record.  Tensor ids: 1 gate, 2 up, 3 down; 11, 12, 13 their MX scales.
 * scratch: 128 * max(d, f) floats; codes: 128 * max(d, f) bytes. */
static void gen_record(const bank_job* j, int64_t rec, uint8_t* dst, float* scratch, uint8_t* codes) {
    int64_t layer = (rec / j->E) + j->layer_offset, expert = rec % j->E;
    if (j->layer_alias > 0) layer %= j->layer_alias;
    int64_t d = j->d, f = j->f, fd = f * d;
    for (int t = 0; t < 3; ++t) {
        int64_t parts[4] = {j->cfg, t + 1, layer, expert};
        uint64_t key = sx_key(j->seed, parts, 4);
        int64_t rows = (t < 2) ? f : d, K = (t < 2) ? d : f;
        if (j->fmt == FMT_BF16) {
            uint8_t* m = dst + 2 * fd * t;
            for (int64_t p = 0; p < rows / 32; ++p) {
                sx_fill_u16_at((uint16_t*)codes, 32 * p * K, 32 * K, key, j->t_bf16);
                panel_store(codes, m + p * 32 * K * 2, K / 8, 16);
            }
        } else if (j->fmt == FMT_FP8) {
            uint8_t* m = dst + fd * t;
            float* sc = (float*)(dst + 3 * fd + 4 * (fd / 16384) * t);
            for (int64_t b = 0; b < rows / 128; ++b) {
                sx_fill_f32_at(scratch, 128 * b * K, 128 * K, key, j->t_f32);
                sx_quant_e4m3_128(scratch, 128, K, codes, sc + b * (K / 128));
                for (int q = 0; q < 4; ++q) panel_store(codes + q * 32 * K, m + (4 * b + q) * 32 * K, K / 16, 16);
            }
        } else {
            uint8_t* m = dst + (fd / 2) * t;
            int64_t sparts[4] = {j->cfg, t + 11, layer, expert};
            uint64_t skey = sx_key(j->seed, sparts, 4);
            uint8_t* s = dst + 3 * fd / 2 + (fd / 32) * t;
            for (int64_t p = 0; p < rows / 32; ++p) {
                sx_fill_bytes_at(codes, 32 * p * (K / 2), 32 * (K / 2), key);
                panel_store(codes, m + p * 32 * (K / 2), K / 32, 16);
                sx_fill_u8_at(codes, 32 * p * (K / 32), 32 * (K / 32), skey, j->t_e8m0);
                panel_store(codes, s + p * 32 * (K / 32), K / 32, 1);
            }
        }
    }
}

static void* bank_worker(void* arg) {
    bank_job* j = (bank_job*)arg;
    int64_t kmax = j->d > j->f ? j->d : j->f;
    float* scratch = (float*)malloc(sizeof(float) * 128 * kmax);
    uint8_t* codes = (uint8_t*)malloc((size_t)(128 * kmax));
    for (;;) {
        pthread_mutex_lock(&j->mu);
        int64_t r = j->next++;
        pthread_mutex_unlock(&j->mu);
        if (r >= j->rec1) break;
        gen_record(j, r, j->out + (r - j->rec0) * j->stride, scratch, codes);
    }
    free(scratch);
    free(codes);
    return NULL;
}

/* Generate records [rec0, rec1) (flat id = layer * E + expert, layer counted
 * from layer_offset) into out, one record every `stride` bytes.  With
 * layer_alias > 0 the weights of layer l are those of layer l mod layer_alias. */
int sx_gen_bank(int fmt, int64_t d, int64_t f, uint64_t seed, int64_t cfg, int64_t E,
                int64_t rec0, int64_t rec1, int64_t layer_offset, int64_t layer_alias,
                uint8_t* out, int64_t stride, const uint16_t* t_bf16, const float* t_f32,
                const uint8_t* t_e8m0, int nthreads) {
    if (sx_record_bytes(fmt, d, f) < 0 || stride < sx_record_bytes(fmt, d, f)) return -1;
    if (d % 128 || f % 128) return -1;
    bank_job j = {fmt, d, f, seed, cfg, E, rec0, rec1, layer_alias, layer_offset, out, stride,
                  t_bf16, t_f32, t_e8m0, rec0};
    pthread_mutex_init(&j.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, bank_worker, &j);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&j.mu);
    return 0;
}
