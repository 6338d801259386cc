/*
 * synth.c - bulk fill for the seeded synthetic KV-cache workloads.
 *
 * This is input generation only: it holds none of the attention method's
 * arithmetic. Both the CPU oracle and the GPU library are fed from it (the
 * GPU side receives the same bytes by an upload), so the two never disagree
 * about their inputs.
 *
 * Random numbers: element n of a stream with 64-bit key `key` is the n-th
 * output of SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) started at state `key`: the state is
 * advanced by the golden-ratio increment and passed through the 64-bit
 * finalizer with the multipliers 0xBF58476D1CE4E5B9 and 0x94D049BB133111EB
 * (Stafford's "Mix13" variant, as used by the public splitmix64 reference).
 *
 * Gaussian values come from a 65536-entry table of normal quantiles that the
 * caller supplies (built once in fp64 and rounded to fp32); the top 16 bits
 * of the random word index the table.
 *
 * Compile with -ffp-contract=off so that `a + b * c` rounds twice, exactly as
 * the numpy twin in synth/__init__.py does.
 */
#include <stdint.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64(uint64_t key, uint64_t n)
{
    uint64_t z = key + (n + 1ULL) * SM64_GAMMA;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* fp32 -> bf16 bits, round to nearest even (inputs are finite). */
static inline uint16_t f32_to_bf16(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

static inline void store(void *dst, int dtype, int64_t idx, float v)
{
    if (dtype == 0)
        ((uint16_t *)dst)[idx] = f32_to_bf16(v);
    else
        ((float *)dst)[idx] = v;
}

uint64_t synth_sm64(uint64_t key, uint64_t n) { return sm64(key, n); }

/*
 * Gaussian block: for heads [h0,h1) and tokens [t0,t1) of a tensor laid out
 * logically as [n_heads][n_tok][d], element (h,t,c) has counter
 * (h*n_tok + t)*d + c and value  nq[u >> 48] * scale[h*d + c]  (fp32 product,
 * scale may be NULL meaning 1), stored as bf16 (dtype 0) or fp32 (dtype 1) at
 * dst[(h-h0)*head_stride + (t-t0)*row_stride + c]  (strides in elements).
 */
void synth_normal(void *dst, int dtype, int64_t head_stride, int64_t row_stride,
                  uint64_t key, int64_t n_tok, int32_t d,
                  int32_t h0, int32_t h1, int64_t t0, int64_t t1,
                  const float *nq, const float *scale, int n_threads)
{
    int64_t rows = (int64_t)(h1 - h0) * (t1 - t0);
    int64_t nt = t1 - t0;
#pragma omp parallel for schedule(static) num_threads(n_threads)
    for (int64_t r = 0; r < rows; ++r) {
        int32_t h = h0 + (int32_t)(r / nt);
        int64_t t = t0 + r % nt;
        int64_t base = (int64_t)(h - h0) * head_stride + (t - t0) * row_stride;
        uint64_t ctr = ((uint64_t)h * (uint64_t)n_tok + (uint64_t)t) * (uint64_t)d;
        for (int32_t c = 0; c < d; ++c) {
            uint64_t u = sm64(key, ctr + (uint64_t)c);
            float x = nq[u >> 48];
            if (scale) x = x * scale[(int64_t)h * d + c];
            store(dst, dtype, base + c, x);
        }
    }
}

/*
 * Needle rows: for every listed needle (head nh[i], tokens [nt0[i], nt0[i]+len)),
 * element (h,t,c) inside the block [h0,h1) x [t0,t1) is overwritten with
 *     centre[h*d + c] + noise * nq[u >> 48]
 * (fp32 multiply, then fp32 add), u drawn from `key` at counter (h*n_tok+t)*d+c.
 */
void synth_needles(void *dst, int dtype, int64_t head_stride, int64_t row_stride,
                   uint64_t key, int64_t n_tok, int32_t d,
                   int32_t h0, int32_t h1, int64_t t0, int64_t t1,
                   const int32_t *nh, const int64_t *nt0, int32_t len, int32_t n_needles,
                   const float *centre, float noise, const float *nq)
{
    for (int32_t i = 0; i < n_needles; ++i) {
        int32_t h = nh[i];
        if (h < h0 || h >= h1) continue;
        int64_t a = nt0[i] > t0 ? nt0[i] : t0;
        int64_t b = nt0[i] + len < t1 ? nt0[i] + len : t1;
        for (int64_t t = a; t < b; ++t) {
            int64_t base = (int64_t)(h - h0) * head_stride + (t - t0) * row_stride;
            uint64_t ctr = ((uint64_t)h * (uint64_t)n_tok + (uint64_t)t) * (uint64_t)d;
            for (int32_t c = 0; c < d; ++c) {
                uint64_t u = sm64(key, ctr + (uint64_t)c);
                float n = noise * nq[u >> 48];
                float x = centre[(int64_t)h * d + c] + n;
                store(dst, dtype, base + c, x);
            }
        }
    }
}
