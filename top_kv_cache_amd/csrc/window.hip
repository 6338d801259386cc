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
// Layout: a workgroup handles a tile of window rows of one block for every KV
// head, so each (row, channel-pair) angle is evaluated once and reused across
// heads.  A thread owns 8 channel pairs of a row (16-byte loads and stores);
// the source rows of several heads are resolved and loaded before any of them
// is rotated, to keep their latencies overlapped.  The same launch rotates
// the block's queries.
#include "rea_internal.h"

#include <math.h>

namespace rea {
namespace {

constexpr int kThreads = 256;
constexpr int kPairs = 8;           // channel pairs per thread

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
    int S, last_len, topk, Hkv, Hq, g, n_q, block_q, rep;
    double inv_freq[kMaxHalfDim];
};

// 8 consecutive stored elements as raw 16-byte vectors.
template <typename TIn> struct Raw8;
template <> struct Raw8<uint16_t> {
    uint4 a;
    __device__ void load(const uint16_t *p) { a = *(const uint4 *)p; }
    __device__ void store(uint16_t *p) const { *(uint4 *)p = a; }
    __device__ void to_f64(double (&x)[8]) const {
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = (double)__uint_as_float(w[i] << 16);
            x[2 * i + 1] = (double)__uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct Raw8<float> {
    float4 a, b;
    __device__ void load(const float *p) {
        a = ((const float4 *)p)[0];
        b = ((const float4 *)p)[1];
    }
    __device__ void store(float *p) const {
        ((float4 *)p)[0] = a;
        ((float4 *)p)[1] = b;
    }
    __device__ void to_f64(double (&x)[8]) const {
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
};

__device__ __forceinline__ void store8(float *p, const double (&x)[8]) {
    ((float4 *)p)[0] = make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
    ((float4 *)p)[1] = make_float4((float)x[4], (float)x[5], (float)x[6], (float)x[7]);
}

// Window length of (b, h) from its selection.  Only span n_spans-1 can be
// short, and a sorted selection holds it last.
__device__ __forceinline__ int64_t window_len(const GatherArgs &a, int64_t bh, int64_t *sel_len) {
    const int ns = a.n_sel[bh];
    int64_t len = (int64_t)ns * a.S;
    if (ns > 0 && a.sel[bh * a.topk + ns - 1] == a.n_spans - 1) len -= a.S - a.last_len;
    *sel_len = len;
    return a.Gp + len + a.Lp;
}

template <typename TIn, int D>
__global__ __launch_bounds__(kThreads) void k_gather_rope(GatherArgs a) {
    constexpr int HALF = D / 2;
    constexpr int TPR = HALF / kPairs;          // threads per window row
    constexpr int RPB = kThreads / TPR;         // window rows per workgroup
    constexpr int HB = sizeof(TIn) == 2 ? 4 : 2;   // heads in flight together
    const int tid = threadIdx.x;
    const int b = blockIdx.y;

    if (blockIdx.x == 0) {
        for (int h = tid; h < a.Hkv; h += kThreads) {
            int64_t sl;
            a.W[(int64_t)b * a.Hkv + h] = (int32_t)window_len(a, (int64_t)b * a.Hkv + h, &sl);
        }
    }

    // the block's queries: item = (query, q head, 8-pair slice)
    {
        const int64_t items = (int64_t)a.block_q * a.Hq * TPR;
        const TIn *q = (const TIn *)a.q;
        for (int64_t it = (int64_t)blockIdx.x * kThreads + tid; it < items;
             it += (int64_t)gridDim.x * kThreads) {
            const int64_t il = it / (a.Hq * TPR);
            const int rem = (int)(it % (a.Hq * TPR));
            const int hq = rem / TPR, c = (rem % TPR) * kPairs;
            const int64_t i = (int64_t)b * a.block_q + il;
            int64_t sl;
            const int64_t Wbh = window_len(a, (int64_t)b * a.Hkv + hq / a.g, &sl);
            const double pos = (double)(Wbh - a.n_q + i);
            const int64_t base = (i * a.Hq + hq) * D;
            Raw8<TIn> r1, r2;
            r1.load(q + base + c);
            r2.load(q + base + c + HALF);
            double x1[8], x2[8], y1[8], y2[8];
            r1.to_f64(x1);
            r2.to_f64(x2);
#pragma unroll
            for (int p = 0; p < kPairs; ++p) {
                double s, co;
                sincos(pos * a.inv_freq[c + p], &s, &co);
                y1[p] = x1[p] * co - x2[p] * s;
                y2[p] = x2[p] * co + x1[p] * s;
            }
            store8(a.q_rot + base + c, y1);
            store8(a.q_rot + base + c + HALF, y2);
        }
    }

    const int r = tid / TPR, c0 = (tid % TPR) * kPairs;
    const int64_t w = (int64_t)blockIdx.x * RPB + r;
    if (w >= a.W_cap) return;

    double cs[kPairs], sn[kPairs];
#pragma unroll
    for (int p = 0; p < kPairs; ++p) sincos((double)w * a.inv_freq[c0 + p], &sn[p], &cs[p]);

    const TIn *kb = (const TIn *)a.k;
    const TIn *vb = (const TIn *)a.v;
    for (int h0 = 0; h0 < a.Hkv; h0 += HB) {
        int64_t src[HB];
        bool ok[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const int h = h0 + hb;
            ok[hb] = false;
            src[hb] = 0;
            if (h < a.Hkv) {
                const int64_t bh = (int64_t)b * a.Hkv + h;
                int64_t sel_len;
                const int64_t Wbh = window_len(a, bh, &sel_len);
                if (w < Wbh) {
                    ok[hb] = true;
                    if (w < a.Gp) {
                        src[hb] = w;
                    } else if (w < a.Gp + sel_len) {
                        const int64_t o = w - a.Gp;
                        src[hb] = a.mid_lo + (int64_t)a.sel[bh * a.topk + o / a.S] * a.S + o % a.S;
                    } else {
                        src[hb] = a.T - a.Lp + (w - a.Gp - sel_len);
                    }
                }
            }
        }
        Raw8<TIn> k1[HB], k2[HB], v1[HB], v2[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            if (ok[hb]) {
                const int64_t row = (int64_t)((h0 + hb) / a.rep) * a.sh + src[hb] * a.st;
                k1[hb].load(kb + row + c0);
                k2[hb].load(kb + row + c0 + HALF);
                v1[hb].load(vb + row + c0);
                v2[hb].load(vb + row + c0 + HALF);
            }
        }
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            if (!ok[hb]) continue;
            const int64_t out_row = (((int64_t)b * a.Hkv + h0 + hb) * a.W_cap + w) * D;
            double x1[8], x2[8], y1[8], y2[8];
            k1[hb].to_f64(x1);
            k2[hb].to_f64(x2);
#pragma unroll
            for (int p = 0; p < kPairs; ++p) {
                y1[p] = x1[p] * cs[p] - x2[p] * sn[p];
                y2[p] = x2[p] * cs[p] + x1[p] * sn[p];
            }
            store8(a.k_win + out_row + c0, y1);
            store8(a.k_win + out_row + c0 + HALF, y2);
            TIn *vo = (TIn *)a.v_win + out_row;
            v1[hb].store(vo + c0);
            v2[hb].store(vo + c0 + HALF);
        }
    }
}

template <typename TIn, int D>
hipError_t launch_typed(const GatherArgs &a, int n_blk, hipStream_t s) {
    constexpr int RPB = kThreads / (D / 2 / kPairs);
    const unsigned gx = (unsigned)((a.W_cap + RPB - 1) / RPB);
    hipLaunchKernelGGL((k_gather_rope<TIn, D>), dim3(gx, n_blk), dim3(kThreads), 0, s, a);
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
    a.rep = g.rep;
    for (int c = 0; c < kMaxHalfDim; ++c)
        a.inv_freq[c] = c < g.d / 2 ? pow(g.theta, -2.0 * (double)c / (double)g.d) : 0.0;
    if (g.dtype == 0)
        return g.d == 128 ? launch_typed<uint16_t, 128>(a, g.n_blk, s)
                          : launch_typed<uint16_t, 64>(a, g.n_blk, s);
    return g.d == 128 ? launch_typed<float, 128>(a, g.n_blk, s)
                      : launch_typed<float, 64>(a, g.n_blk, s);
}

}  // namespace rea
