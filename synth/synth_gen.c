/*
 * synth_gen.c - seeded synthetic inputs for the SCAPE optimizer step.
 *
 * This module produces the gradients and initial parameters that both the
 * GPU path and the oracle consume.  It holds none of the optimizer's
 * arithmetic: it only turns a (seed, purpose, tensor, step, worker, element)
 * counter into numbers with a stated distribution.
 *
 * Generator: Philox4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11),
 * written here from its published round function.  One call maps a 128-bit
 * counter and a 64-bit key to four 32-bit words.
 *
 * Distributions (all produced with IEEE operations that round to nearest
 * even, so the output bits are a pure function of the counter):
 *   normal   : Irwin-Hall sum of the eight 16-bit halves of one Philox call,
 *              centred and scaled to unit variance (support +-4.9 sigma).
 *   student2 : Student-t with two degrees of freedom by inversion of its
 *              CDF, t = (2u-1)/sqrt(2u(1-u)), in fp32 with u on a 2^-24 grid
 *              (u = (2*(w>>9)+1) * 2^-24, so 2u-1 and 1-u are exact).
 *   quantised: a value v snapped to Delta*clamp(rne(v/Delta), -8, 7) with
 *              Delta = 2^-12, i.e. 16 levels, all exact in bfloat16.
 * Gradients are rounded to bfloat16 (round to nearest even) from fp32.
 *
 * Built with gcc -O2 -fopenmp -ffp-contract=off; elements are independent,
 * so the OpenMP split does not change any output bit.  synth_gen.hip is the
 * same generator for the GPU; both use only integer operations and
 * correctly rounded fp32 operations (add, multiply, divide, sqrt, rint), so
 * they agree bit for bit.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k[0];
    uint32_t n2 = hi0 ^ c[3] ^ k[1];
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
}

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k[0] += PHILOX_W0;
            k[1] += PHILOX_W1;
        }
        philox_round(c, k);
    }
    out[0] = c[0];
    out[1] = c[1];
    out[2] = c[2];
    out[3] = c[3];
}

/* Purposes: separate key streams so that no two uses share a counter. */
enum { PURPOSE_GRAD = 1, PURPOSE_PARAM = 2, PURPOSE_SIGMA = 3 };

/* bfloat16 from fp32, round to nearest even (inputs are finite). */
static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

/* Unit-variance Irwin-Hall(8) value in fp32 (exact: 19-bit integer / 2^16). */
static inline float irwin_hall8(const uint32_t w[4]) {
    int32_t s = 0;
    for (int i = 0; i < 4; ++i) s += (int32_t)(w[i] & 0xFFFFu) + (int32_t)(w[i] >> 16);
    /* mean of eight uniform 16-bit halves is 8 * 32767.5 = 262140 */
    return (float)(s - 262140) * (1.0f / 65536.0f);
}

/* fp32 scale that turns irwin_hall8 (variance 2/3) into standard deviation sigma. */
float synth_normal_scale(double sigma) { return (float)(sigma * sqrt(1.5)); }

/* Per-tensor sigma, log-uniform in [1e-5, 1e-2]: 10^(-5 + 3u). */
double synth_tensor_sigma(uint32_t seed, uint32_t tensor) {
    uint32_t ctr[4] = {tensor, 0u, 0u, 0u}, key[2] = {seed, PURPOSE_SIGMA}, o[4];
    synth_philox4x32_10(ctr, key, o);
    double u = ((double)o[0] + 0.5) * (1.0 / 4294967296.0);
    return pow(10.0, -5.0 + 3.0 * u);
}

static inline float quantise16(float v) {
    const float delta = 1.0f / 4096.0f;
    float q = rintf(v / delta);
    if (q < -8.0f) q = -8.0f;
    if (q > 7.0f) q = 7.0f;
    return q * delta;
}

static inline float student2(uint32_t w) {
    const float u = (float)(2u * (w >> 9) + 1u) * (1.0f / 16777216.0f);
    return (2.0f * u - 1.0f) / sqrtf(2.0f * u * (1.0f - u));
}

/*
 * Gradient values for elements [e0, e0+n) of one tensor, as bfloat16 bits.
 * kind 0: normal with fp32 scale `scale` (from synth_normal_scale(sigma)).
 * kind 1: Student-t(2) times `scale`.
 * quantise != 0 snaps the fp32 value to the 16-level grid before rounding.
 */
void synth_grad_bf16(uint32_t seed, uint32_t tensor, uint32_t step, uint32_t worker, int kind,
                     float scale, int quantise, uint64_t e0, uint64_t n, uint16_t* out) {
    const uint32_t key[2] = {seed, PURPOSE_GRAD};
#pragma omp parallel for schedule(static, 65536)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint32_t ctr[4] = {(uint32_t)(e0 + (uint64_t)i), tensor, step, worker}, w[4];
        synth_philox4x32_10(ctr, key, w);
        const float v0 = kind == 0 ? irwin_hall8(w) : student2(w[0]);
        float v = v0 * scale;
        if (quantise) v = quantise16(v);
        out[i] = f32_to_bf16_rne(v);
    }
}

/* Initial parameters in fp32: normal with fp32 scale `scale`. */
void synth_param_f32(uint32_t seed, uint32_t tensor, float scale, uint64_t e0, uint64_t n, float* out) {
    const uint32_t key[2] = {seed, PURPOSE_PARAM};
#pragma omp parallel for schedule(static, 65536)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint32_t ctr[4] = {(uint32_t)(e0 + (uint64_t)i), tensor, 0u, 0u}, w[4];
        synth_philox4x32_10(ctr, key, w);
        out[i] = irwin_hall8(w) * scale;
    }
}

/* Uniform u32 words for elements [e0, e0+n): first Philox word of each counter. */
void synth_u32(uint32_t seed, uint32_t purpose, uint32_t tensor, uint32_t step, uint32_t worker,
               uint64_t e0, uint64_t n, uint32_t* out) {
    const uint32_t key[2] = {seed, purpose};
#pragma omp parallel for schedule(static, 65536)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint32_t ctr[4] = {(uint32_t)(e0 + (uint64_t)i), tensor, step, worker}, w[4];
        synth_philox4x32_10(ctr, key, w);
        out[i] = w[0];
    }
}
