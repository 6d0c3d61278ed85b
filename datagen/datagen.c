/*
 * Seeded synthetic inputs for the attention library's tests and benchmark.
 *
 * This module holds NONE of the attention arithmetic. It only draws numbers
 * and stores them in the storage formats the library reads (fp32, bf16 bit
 * patterns, OCP fp8-e4m3 codes with a per-head fp32 scale, OCP MX fp4 codes
 * with one power-of-two scale per 32 elements). Both the HIP path
 * and the double-precision oracle consume its output; neither shares any other
 * code with the other.
 *
 * Generator (counter based, so every element can be drawn independently and
 * the result does not depend on the number of threads):
 *   key      = mix(mix(seed) ^ (tensor_id + 1) * GOLDEN)
 *   word(c)  = mix(key + (c + 1) * GOLDEN)            -- the SplitMix64 stream
 *              (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
 *              number generators", OOPSLA 2014) started at state `key`
 *   u1       = ((word(2i) >> 11) + 1) * 2^-53         in (0, 1]
 *   u2       =  (word(2i+1) >> 11)    * 2^-53         in [0, 1)
 *   normal i = sqrt(-2 ln u1) * cos(2 pi u2)          (Box & Muller, 1958)
 * A value is normal * mul computed in double, rounded once to fp32 (RNE), and
 * from there to the storage format.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static uint64_t mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static uint64_t stream_key(uint64_t seed, uint64_t tensor_id) {
    return mix(mix(seed) ^ ((tensor_id + 1) * GOLDEN));
}

static uint64_t word_at(uint64_t key, uint64_t c) { return mix(key + (c + 1) * GOLDEN); }

static double normal_at(uint64_t key, uint64_t i) {
    const double two_m53 = 1.0 / 9007199254740992.0;
    double u1 = (double)((word_at(key, 2 * i) >> 11) + 1) * two_m53;
    double u2 = (double)(word_at(key, 2 * i + 1) >> 11) * two_m53;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

/* ---- storage-format encoders (round to nearest, ties to even) ---------- */

uint16_t dg_f32_to_bf16(float x) {
    uint32_t b;
    memcpy(&b, &x, 4);
    if ((b & 0x7f800000u) == 0x7f800000u && (b & 0x007fffffu)) return 0x7fc0; /* NaN */
    uint32_t lsb = (b >> 16) & 1u;
    return (uint16_t)((b + 0x7fffu + lsb) >> 16);
}

/* OCP FP8 E4M3 ("e4m3fn"): bias 7, no infinities, max finite 448,
 * subnormals m * 2^-9. Out-of-range magnitudes saturate to +-448. */
uint8_t dg_f32_to_e4m3(float xf) {
    double x = (double)xf;
    uint8_t sign = 0;
    if (x != x) return 0x7f;
    if (x < 0 || (x == 0 && signbit(x))) { sign = 0x80; x = -x; }
    if (x >= 464.0) return sign | 0x7e; /* would round past 448: saturate */
    if (x < 0.015625) {                 /* below 2^-6: subnormal grid step 2^-9 */
        double m = rint(x * 512.0);     /* 0..8; 8 is the smallest normal */
        return sign | (uint8_t)m;
    }
    int e;
    double fr = frexp(x, &e); /* x = fr * 2^e, fr in [0.5, 1) */
    e -= 1;                   /* x = (2 fr) * 2^e, 2fr in [1, 2) */
    double m = rint((2.0 * fr - 1.0) * 8.0);
    if (m == 8.0) { m = 0.0; e += 1; }
    if (e > 8 || (e == 8 && m > 6.0)) return sign | 0x7e;
    return sign | (uint8_t)(((e + 7) << 3) | (int)m);
}

/* ---- threaded fills -------------------------------------------------------- */

typedef struct {
    uint64_t key;
    uint64_t begin, end;
    double mul;
    int kind; /* 0: f32, 1: bf16, 2: f64 raw */
    void* out;
} fill_job;

static void* fill_worker(void* arg) {
    fill_job* j = (fill_job*)arg;
    for (uint64_t i = j->begin; i < j->end; ++i) {
        double v = normal_at(j->key, i) * j->mul;
        if (j->kind == 2) {
            ((double*)j->out)[i] = v;
        } else {
            float f = (float)v;
            if (j->kind == 0) ((float*)j->out)[i] = f;
            else ((uint16_t*)j->out)[i] = dg_f32_to_bf16(f);
        }
    }
    return NULL;
}

static void run_fill(uint64_t seed, uint64_t tensor_id, uint64_t n, double mul, int kind, void* out,
                     int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((uint64_t)nthreads > n / 4096 + 1) nthreads = (int)(n / 4096 + 1);
    pthread_t th[256];
    fill_job jobs[256];
    uint64_t key = stream_key(seed, tensor_id);
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].key = key;
        jobs[t].begin = n * (uint64_t)t / (uint64_t)nthreads;
        jobs[t].end = n * (uint64_t)(t + 1) / (uint64_t)nthreads;
        jobs[t].mul = mul;
        jobs[t].kind = kind;
        jobs[t].out = out;
        pthread_create(&th[t], NULL, fill_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

void dg_normal_f64(uint64_t seed, uint64_t tensor_id, uint64_t n, double mul, double* out, int nthreads) {
    run_fill(seed, tensor_id, n, mul, 2, out, nthreads);
}

void dg_fill_f32(uint64_t seed, uint64_t tensor_id, uint64_t n, double mul, float* out, int nthreads) {
    run_fill(seed, tensor_id, n, mul, 0, out, nthreads);
}

void dg_fill_bf16(uint64_t seed, uint64_t tensor_id, uint64_t n, double mul, uint16_t* out, int nthreads) {
    run_fill(seed, tensor_id, n, mul, 1, out, nthreads);
}

/* fp8 e4m3 with one fp32 scale per group of `per_group` consecutive elements
 * (one group = one (batch, kv head) slice of the cache):
 *   scale = amax(|x|) / 448 (fp32), code = e4m3(x / scale) (fp32 division).
 * An all-zero group gets scale 1. */
typedef struct {
    uint64_t key, per_group, g0, g1;
    double mul;
    uint8_t* out;
    float* scales;
} e4m3_job;

static void* e4m3_worker(void* arg) {
    e4m3_job* j = (e4m3_job*)arg;
    float* tmp = (float*)malloc(sizeof(float) * j->per_group);
    for (uint64_t g = j->g0; g < j->g1; ++g) {
        float amax = 0.0f;
        for (uint64_t i = 0; i < j->per_group; ++i) {
            float f = (float)(normal_at(j->key, g * j->per_group + i) * j->mul);
            tmp[i] = f;
            float a = fabsf(f);
            if (a > amax) amax = a;
        }
        float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
        j->scales[g] = scale;
        uint8_t* o = j->out + g * j->per_group;
        for (uint64_t i = 0; i < j->per_group; ++i) o[i] = dg_f32_to_e4m3(tmp[i] / scale);
    }
    free(tmp);
    return NULL;
}

void dg_fill_e4m3(uint64_t seed, uint64_t tensor_id, uint64_t groups, uint64_t per_group, double mul,
                  uint8_t* out, float* scales, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((uint64_t)nthreads > groups) nthreads = (int)groups;
    pthread_t th[256];
    e4m3_job jobs[256];
    uint64_t key = stream_key(seed, tensor_id);
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].key = key;
        jobs[t].per_group = per_group;
        jobs[t].g0 = groups * (uint64_t)t / (uint64_t)nthreads;
        jobs[t].g1 = groups * (uint64_t)(t + 1) / (uint64_t)nthreads;
        jobs[t].mul = mul;
        jobs[t].out = out;
        jobs[t].scales = scales;
        pthread_create(&th[t], NULL, e4m3_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* OCP MX FP4 element (E2M1): sign bit, 2-bit exponent (bias 1), 1-bit
 * mantissa; code c = eem holds the magnitude 0, 0.5, 1, 1.5, 2, 3, 4, 6 for
 * c = 0 .. 7. Round to nearest, ties to the even code (mantissa bit 0),
 * saturating to +-6. */
uint8_t dg_f32_to_e2m1(float xf) {
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double x = (double)xf;
    uint8_t sign = 0;
    if (x != x) return 0;
    if (x < 0 || (x == 0 && signbit(x))) { sign = 0x8; x = -x; }
    if (x >= 6.0) return sign | 7;
    int c = 0;
    while (grid[c + 1] <= x) ++c; /* grid[c] <= x < grid[c + 1], c < 7 */
    const double mid = 0.5 * (grid[c] + grid[c + 1]);
    if (x > mid || (x == mid && (c & 1))) ++c;
    return sign | (uint8_t)c;
}

/* OCP MX FP4 with block size 32 along the last dimension: per block of 32
 * consecutive values, the shared scale is 2^X with X = floor(log2(amax)) - 2
 * (2 = the largest E2M1 exponent), stored as the E8M0 byte X + 127 (X held
 * in [-127, 127]; an all-zero block stores 127), and each element is
 * e2m1(x / 2^X). Codes pack two per byte, element 2i in the low nibble of
 * byte i of its row. `d` must be a multiple of 32. */
typedef struct {
    uint64_t key, d, r0, r1;
    double mul;
    uint8_t* codes;
    uint8_t* scales;
} mx_job;

static void* mx_worker(void* arg) {
    mx_job* j = (mx_job*)arg;
    for (uint64_t r = j->r0; r < j->r1; ++r) {
        for (uint64_t b0 = 0; b0 < j->d; b0 += 32) {
            float v[32];
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                v[i] = (float)(normal_at(j->key, r * j->d + b0 + i) * j->mul);
                if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
            }
            int X = 0;
            if (amax > 0.0f) {
                int e;
                frexp((double)amax, &e); /* amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
                X = (e - 1) - 2;
                if (X < -127) X = -127;
                if (X > 127) X = 127;
            }
            j->scales[r * (j->d / 32) + b0 / 32] = (uint8_t)(X + 127);
            uint8_t* o = j->codes + r * (j->d / 2) + b0 / 2;
            for (int i = 0; i < 32; i += 2) {
                const uint8_t lo = dg_f32_to_e2m1((float)ldexp((double)v[i], -X));
                const uint8_t hi = dg_f32_to_e2m1((float)ldexp((double)v[i + 1], -X));
                o[i / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
    return NULL;
}

void dg_fill_mxfp4(uint64_t seed, uint64_t tensor_id, uint64_t rows, uint64_t d, double mul, uint8_t* codes,
                   uint8_t* scales, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((uint64_t)nthreads > rows) nthreads = (int)rows;
    if (nthreads < 1) return;
    pthread_t th[256];
    mx_job jobs[256];
    uint64_t key = stream_key(seed, tensor_id);
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].key = key;
        jobs[t].d = d;
        jobs[t].r0 = rows * (uint64_t)t / (uint64_t)nthreads;
        jobs[t].r1 = rows * (uint64_t)(t + 1) / (uint64_t)nthreads;
        jobs[t].mul = mul;
        jobs[t].codes = codes;
        jobs[t].scales = scales;
        pthread_create(&th[t], NULL, mx_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* Integers uniform on [lo, hi] inclusive: lo + word(i) mod (hi - lo + 1).
 * (The modulo bias is below 2^-40 for the ranges used here.) */
void dg_uniform_int(uint64_t seed, uint64_t tensor_id, uint64_t n, int32_t lo, int32_t hi, int32_t* out) {
    uint64_t key = stream_key(seed, tensor_id);
    uint64_t span = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
    for (uint64_t i = 0; i < n; ++i) out[i] = (int32_t)((int64_t)lo + (int64_t)(word_at(key, i) % span));
}

/* Raw generator words, for reproducibility tests. */
void dg_words(uint64_t seed, uint64_t tensor_id, uint64_t n, uint64_t* out) {
    uint64_t key = stream_key(seed, tensor_id);
    for (uint64_t i = 0; i < n; ++i) out[i] = word_at(key, i);
}
