// score.hip - step 1a: position-agnostic token scoring with span max-reduce.
//
// For KV head h, the middle cache [G', T-L') is cut into spans of S tokens.
// The score of token t for query i is the dot product of the UN-rotated query
// with the PRE-RoPE key, summed over the query heads of h's GQA group
// (ReAttention research-map summary, "Approach": segments are chosen by the
// query/un-positioned-key dot product; OpenReview discussion, "Decoding Phase"
// pseudocode: score = query @ key[G:-L]^T).  A span's score is the maximum of
// its token scores; a block of queries sums its queries' maxima.  Token scores
// are never written out: only span scores leave the kernel.
//
// Arithmetic: the group-summed query is formed in fp64 (exact for bf16 and,
// in practice, fp32 inputs), every product bf16/fp32 x fp64 is exact in fp64,
// and sums are fp64, so span scores agree with the exact ones to ~1e-16
// relative and the top-k decision downstream matches an exact evaluation
// except for gaps below that.
//
// Memory: decoding streams the whole middle K once (2.14 GB per layer at 1M
// tokens, d=128, 8 KV heads).  Four lanes share one key row; each lane issues
// 16-byte loads so that one wave instruction reads 16 rows x 64 contiguous
// bytes.  Two rounds (32 tokens = 8 KB per wave for d=128 bf16) are loaded
// before any arithmetic to keep enough bytes in flight.  The grid gives every
// (block, KV head) P workgroups, each streaming a contiguous run of spans.
#include "rea_internal.h"

#include <math.h>

namespace rea {
namespace {

constexpr int kThreads = 256;   // 4 waves
constexpr int kWaves = kThreads / 64;

struct ScoreArgs {
    const void *q;
    const unsigned char *k;
    double *out;
    int64_t sh_bytes, st_bytes;
    int64_t mid_lo, mid_hi, n_spans;
    int S, Hq, Hkv, g, block_q, P;
};

template <typename TIn> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int EPV = 8; };   // bf16 per 16 B
template <> struct Elem<float> { static constexpr int EPV = 4; };

__device__ __forceinline__ double load_f64(const uint16_t *p, int64_t i) {
    return (double)__uint_as_float(((uint32_t)p[i]) << 16);
}
__device__ __forceinline__ double load_f64(const float *p, int64_t i) {
    return (double)p[i];
}

__device__ __forceinline__ void unpack(const uint4 &x, double (&o)[8]) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = (double)__uint_as_float(w[i] << 16);
        o[2 * i + 1] = (double)__uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack(const uint4 &x, double (&o)[4]) {
    o[0] = (double)__uint_as_float(x.x);
    o[1] = (double)__uint_as_float(x.y);
    o[2] = (double)__uint_as_float(x.z);
    o[3] = (double)__uint_as_float(x.w);
}

__device__ __forceinline__ double wave_max(double v) {
    v = fmax(v, __shfl_xor(v, 4));
    v = fmax(v, __shfl_xor(v, 8));
    v = fmax(v, __shfl_xor(v, 16));
    v = fmax(v, __shfl_xor(v, 32));
    return v;
}

// Decode: one query per block; the group-summed query lives in registers.
template <typename TIn, int D, int R>
__global__ __launch_bounds__(kThreads) void k_score_decode(ScoreArgs a) {
    constexpr int EPV = Elem<TIn>::EPV;
    constexpr int NV = D / (4 * EPV);            // 16-byte vectors per lane per token
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int quad = lane >> 2, c4 = lane & 3;
    const int bh = blockIdx.x / a.P, p = blockIdx.x % a.P;
    const int b = bh / a.Hkv, h = bh % a.Hkv;
    const int64_t j0 = (int64_t)p * a.n_spans / a.P;
    const int64_t j1 = (int64_t)(p + 1) * a.n_spans / a.P;

    double qr[NV][EPV];
    {
        const TIn *qb = (const TIn *)a.q + (int64_t)b * a.Hq * D + (int64_t)h * a.g * D;
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const int c = v * 4 * EPV + c4 * EPV + e;
                double s = 0.0;
                for (int gg = 0; gg < a.g; ++gg) s += load_f64(qb, (int64_t)gg * D + c);
                qr[v][e] = s;
            }
    }

    const unsigned char *kh = a.k + (int64_t)h * a.sh_bytes;
    for (int64_t j = j0 + wave; j < j1; j += kWaves) {
        const int64_t t_beg = a.mid_lo + j * a.S;
        const int64_t t_end = min(t_beg + (int64_t)a.S, a.mid_hi);
        double best = -INFINITY;
        for (int64_t r0 = t_beg; r0 < t_end; r0 += 16 * R) {
            uint4 buf[R][NV];
            bool ok[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t t = r0 + r * 16 + quad;
                ok[r] = t < t_end;
                const uint4 *src = (const uint4 *)(kh + t * a.st_bytes) + c4;
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    buf[r][v] = ok[r] ? src[v * 4] : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                double acc = 0.0;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    double x[EPV];
                    unpack(buf[r][v], x);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) acc = fma(qr[v][e], x[e], acc);
                }
                acc += __shfl_xor(acc, 1);
                acc += __shfl_xor(acc, 2);
                if (ok[r]) best = fmax(best, acc);
            }
        }
        best = wave_max(best);
        if (lane == 0) a.out[(int64_t)bh * a.n_spans + j] = best + 0.0;   // -0 -> +0
    }
}

// Blocks of several queries (chunked prefill on the VALU): the group-summed
// queries of the block sit in LDS; span score = sum over queries of the max.
template <typename TIn, int D>
__global__ __launch_bounds__(kThreads) void k_score_block(ScoreArgs a) {
    constexpr int EPV = Elem<TIn>::EPV;
    constexpr int NV = D / (4 * EPV);
    extern __shared__ double qe[];                // [block_q][D]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int quad = lane >> 2, c4 = lane & 3;
    const int bh = blockIdx.x / a.P, p = blockIdx.x % a.P;
    const int b = bh / a.Hkv, h = bh % a.Hkv;
    const int64_t j0 = (int64_t)p * a.n_spans / a.P;
    const int64_t j1 = (int64_t)(p + 1) * a.n_spans / a.P;

    const TIn *qb = (const TIn *)a.q;
    for (int idx = threadIdx.x; idx < a.block_q * D; idx += kThreads) {
        const int i = idx / D, c = idx % D;
        const int64_t row = ((int64_t)b * a.block_q + i) * a.Hq + (int64_t)h * a.g;
        double s = 0.0;
        for (int gg = 0; gg < a.g; ++gg) s += load_f64(qb, (row + gg) * D + c);
        qe[idx] = s;
    }
    __syncthreads();

    const unsigned char *kh = a.k + (int64_t)h * a.sh_bytes;
    for (int64_t j = j0 + wave; j < j1; j += kWaves) {
        const int64_t t_beg = a.mid_lo + j * a.S;
        const int64_t t_end = min(t_beg + (int64_t)a.S, a.mid_hi);
        double total = 0.0;
        for (int i = 0; i < a.block_q; ++i) {
            const double *qi = qe + (int64_t)i * D;
            double best = -INFINITY;
            for (int64_t r0 = t_beg; r0 < t_end; r0 += 16) {
                const int64_t t = r0 + quad;
                const bool ok = t < t_end;
                const uint4 *src = (const uint4 *)(kh + t * a.st_bytes) + c4;
                double acc = 0.0;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const uint4 raw = ok ? src[v * 4] : make_uint4(0u, 0u, 0u, 0u);
                    double x[EPV];
                    unpack(raw, x);
#pragma unroll
                    for (int e = 0; e < EPV; ++e)
                        acc = fma(qi[v * 4 * EPV + c4 * EPV + e], x[e], acc);
                }
                acc += __shfl_xor(acc, 1);
                acc += __shfl_xor(acc, 2);
                if (ok) best = fmax(best, acc);
            }
            total += wave_max(best);
        }
        if (lane == 0) a.out[(int64_t)bh * a.n_spans + j] = total + 0.0;
    }
}

template <typename TIn, int D>
hipError_t launch_typed(const Geom &g, const ScoreArgs &a, int nblocks, hipStream_t s) {
    if (g.block_q == 1) {
        if (g.S <= 16)
            hipLaunchKernelGGL((k_score_decode<TIn, D, 1>), dim3(nblocks), dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL((k_score_decode<TIn, D, 2>), dim3(nblocks), dim3(kThreads), 0, s, a);
    } else {
        const size_t lds = (size_t)g.block_q * D * sizeof(double);
        hipLaunchKernelGGL((k_score_block<TIn, D>), dim3(nblocks), dim3(kThreads), lds, s, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const Geom &g, const void *q, const void *k, double *span_scores,
                        int num_cu, hipStream_t s) {
    if (g.n_spans == 0) return hipSuccess;
    ScoreArgs a;
    a.q = q;
    a.k = (const unsigned char *)k;
    a.out = span_scores;
    a.sh_bytes = g.sh * g.esize;
    a.st_bytes = g.st * g.esize;
    a.mid_lo = g.mid_lo;
    a.mid_hi = g.mid_hi;
    a.n_spans = g.n_spans;
    a.S = g.S;
    a.Hq = g.Hq;
    a.Hkv = g.Hkv;
    a.g = g.g;
    a.block_q = g.block_q;
    const int64_t units = (int64_t)g.n_blk * g.Hkv;
    const int64_t target = (int64_t)(num_cu > 0 ? num_cu : 256) * 4;
    int64_t P = (target + units - 1) / units;
    const int64_t maxP = (g.n_spans + kWaves - 1) / kWaves;
    if (P > maxP) P = maxP;
    if (P < 1) P = 1;
    a.P = (int)P;
    const int nblocks = (int)(units * P);
    if (g.dtype == 0)
        return g.d == 128 ? launch_typed<uint16_t, 128>(g, a, nblocks, s)
                          : launch_typed<uint16_t, 64>(g, a, nblocks, s);
    return g.d == 128 ? launch_typed<float, 128>(g, a, nblocks, s)
                      : launch_typed<float, 64>(g, a, nblocks, s);
}

}  // namespace rea
