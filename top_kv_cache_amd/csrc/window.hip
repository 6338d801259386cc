// window.hip - steps 2-3: gather the compact window and apply RoPE at fresh
// positions.
//
// Window of (block b, KV head h) = global [0, G') ++ the selected spans in
// ascending order ++ local [T-L', T)  (OpenReview discussion, "Decoding
// Phase" pseudocode: key_recall / value_recall concatenations).  Window row w
// is rotated to position w, so positions stay below the window length however
// long the cache is (research-map summary, "Approach": positional embeddings
// are applied only after concatenation).  Keys are written rotated in fp32;
// values are exact copies.  Each query is rotated to the row that holds its
// own key, W - n_q + i.
//
// RoPE is rotate-half: channel c pairs with c + d/2 and turns by angle
// w * theta^(-2c/d).  The inverse frequencies come from the host in fp64; the
// angle, its sine/cosine and the rotation are evaluated in fp64 and the result
// is rounded once to fp32.
//
// Layout: one workgroup handles 16 window rows of one block for every KV
// head, so each (row, channel-pair) angle is evaluated once and reused across
// heads.  16 threads share a row; each owns d/32 contiguous channel pairs.
#include "rea_internal.h"

#include <math.h>

namespace rea {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;

struct GatherArgs {
    const unsigned char *k, *v;
    const void *q;
    const int32_t *sel, *n_sel;
    float *k_win;
    void *v_win;
    float *q_rot;
    int32_t *W;
    int64_t sh, st;         // elements
    int64_t T, Gp, Lp, mid_lo, n_spans, W_cap;
    int S, last_len, topk, Hkv, Hq, g, n_q, block_q;
    double inv_freq[kMaxHalfDim];
};

template <typename TIn> __device__ __forceinline__ double ld(const TIn *p, int64_t i);
template <> __device__ __forceinline__ double ld<uint16_t>(const uint16_t *p, int64_t i) {
    return (double)__uint_as_float(((uint32_t)p[i]) << 16);
}
template <> __device__ __forceinline__ double ld<float>(const float *p, int64_t i) {
    return (double)p[i];
}

// Window length of (b, h) from its selection.  Only span n_spans-1 can be
// short, and a sorted selection holds it last.
__device__ __forceinline__ int64_t window_len(const GatherArgs &a, const int32_t *selp, int ns,
                                              int64_t *sel_len) {
    int64_t len = (int64_t)ns * a.S;
    if (ns > 0 && selp[ns - 1] == a.n_spans - 1) len -= a.S - a.last_len;
    *sel_len = len;
    return a.Gp + len + a.Lp;
}

template <typename TIn, int D>
__global__ __launch_bounds__(kThreads) void k_gather_rope(GatherArgs a) {
    constexpr int HALF = D / 2;
    constexpr int NP = HALF / 16;           // channel pairs per thread
    const int r = threadIdx.x / 16, l16 = threadIdx.x % 16;
    const int64_t w = (int64_t)blockIdx.x * kRows + r;
    const int b = blockIdx.y;
    const int c0 = l16 * NP;

    if (blockIdx.x == 0) {
        for (int h = threadIdx.x; h < a.Hkv; h += kThreads) {
            const int32_t *selp = a.sel + ((int64_t)b * a.Hkv + h) * a.topk;
            int64_t sl;
            a.W[(int64_t)b * a.Hkv + h] =
                (int32_t)window_len(a, selp, a.n_sel[(int64_t)b * a.Hkv + h], &sl);
        }
    }
    if (w >= a.W_cap) return;

    double cs[NP], sn[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) sincos((double)w * a.inv_freq[c0 + p], &sn[p], &cs[p]);

    for (int h = 0; h < a.Hkv; ++h) {
        const int64_t bh = (int64_t)b * a.Hkv + h;
        const int32_t *selp = a.sel + bh * a.topk;
        const int ns = a.n_sel[bh];
        int64_t sel_len;
        const int64_t Wbh = window_len(a, selp, ns, &sel_len);
        if (w >= Wbh) continue;
        int64_t src;
        if (w < a.Gp) {
            src = w;
        } else if (w < a.Gp + sel_len) {
            const int64_t o = w - a.Gp;
            src = a.mid_lo + (int64_t)selp[o / a.S] * a.S + o % a.S;
        } else {
            src = a.T - a.Lp + (w - a.Gp - sel_len);
        }
        const TIn *krow = (const TIn *)a.k + h * a.sh + src * a.st;
        const TIn *vrow = (const TIn *)a.v + h * a.sh + src * a.st;
        float *kout = a.k_win + (bh * a.W_cap + w) * D;
        TIn *vout = (TIn *)a.v_win + (bh * a.W_cap + w) * D;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int c = c0 + p;
            const double x1 = ld(krow, c), x2 = ld(krow, c + HALF);
            kout[c] = (float)(x1 * cs[p] - x2 * sn[p]);
            kout[c + HALF] = (float)(x2 * cs[p] + x1 * sn[p]);
            vout[c] = vrow[c];
            vout[c + HALF] = vrow[c + HALF];
        }
    }
}

// q_rot[i][hq] = RoPE(q[i][hq], W[b][hq/g] - n_q + i), one workgroup per query.
template <typename TIn, int D>
__global__ __launch_bounds__(kThreads) void k_rope_query(GatherArgs a) {
    constexpr int HALF = D / 2;
    const int i = blockIdx.x;
    const int b = i / a.block_q;
    const TIn *q = (const TIn *)a.q;
    for (int idx = threadIdx.x; idx < a.Hq * HALF; idx += kThreads) {
        const int hq = idx / HALF, c = idx % HALF;
        const int h = hq / a.g;
        const int64_t pos = (int64_t)a.W[(int64_t)b * a.Hkv + h] - a.n_q + i;
        double s, co;
        sincos((double)pos * a.inv_freq[c], &s, &co);
        const int64_t base = ((int64_t)i * a.Hq + hq) * D;
        const double x1 = ld(q, base + c), x2 = ld(q, base + c + HALF);
        a.q_rot[base + c] = (float)(x1 * co - x2 * s);
        a.q_rot[base + c + HALF] = (float)(x2 * co + x1 * s);
    }
}

template <typename TIn, int D>
hipError_t launch_typed(const GatherArgs &a, int n_blk, hipStream_t s) {
    const unsigned gx = (unsigned)((a.W_cap + kRows - 1) / kRows);
    hipLaunchKernelGGL((k_gather_rope<TIn, D>), dim3(gx, n_blk), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_rope_query<TIn, D>), dim3(a.n_q), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_rope(const Geom &g, const void *k, const void *v, const void *q,
                              const int32_t *sel, const int32_t *n_sel, float *k_win,
                              void *v_win, float *q_rot, int32_t *W, int64_t W_cap,
                              hipStream_t s) {
    GatherArgs a;
    a.k = (const unsigned char *)k;
    a.v = (const unsigned char *)v;
    a.q = q;
    a.sel = sel;
    a.n_sel = n_sel;
    a.k_win = k_win;
    a.v_win = v_win;
    a.q_rot = q_rot;
    a.W = W;
    a.sh = g.sh;
    a.st = g.st;
    a.T = g.T;
    a.Gp = g.Gp;
    a.Lp = g.Lp;
    a.mid_lo = g.mid_lo;
    a.n_spans = g.n_spans;
    a.W_cap = W_cap;
    a.S = g.S;
    a.last_len = g.last_len;
    a.topk = g.topk;
    a.Hkv = g.Hkv;
    a.Hq = g.Hq;
    a.g = g.g;
    a.n_q = g.n_q;
    a.block_q = g.block_q;
    for (int c = 0; c < kMaxHalfDim; ++c)
        a.inv_freq[c] = c < g.d / 2 ? pow(g.theta, -2.0 * (double)c / (double)g.d) : 0.0;
    if (g.dtype == 0)
        return g.d == 128 ? launch_typed<uint16_t, 128>(a, g.n_blk, s)
                          : launch_typed<uint16_t, 64>(a, g.n_blk, s);
    return g.d == 128 ? launch_typed<float, 128>(a, g.n_blk, s)
                      : launch_typed<float, 64>(a, g.n_blk, s);
}

}  // namespace rea
