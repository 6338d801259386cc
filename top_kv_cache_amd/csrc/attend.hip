// attend.hip - step 4: ordinary causal softmax attention over the window.
//
// The window's keys are already rotated (step 3), so this is plain attention
// (OpenReview discussion, "Decoding Phase" pseudocode:
// flash_attention(query, key_recall, value_recall)).  Query row r of a block
// is (query i = r / g, head hq = h*g + r % g); it sees window rows w <= its
// own position W - n_q + i.
//
// Split-window ("flash-decoding") scheme on the VALU, fp32 throughout:
//   k_attend_split   one workgroup per (split of 256 window rows, KV head,
//                    block).  For groups of 4 query rows: logits into LDS
//                    (16 lanes per key row), softmax statistics per row (one
//                    wave per row), then P.V with one wave per row.  Writes
//                    the partial (max m, sum l, unnormalised acc[d]).
//   k_attend_combine one workgroup per (query row, KV head, block) merges the
//                    splits: out = sum_s e^(m_s-M) acc_s / sum_s e^(m_s-M) l_s.
// The g query heads of a KV head share every K/V row they read.
#include "rea_internal.h"

#include <math.h>

namespace rea {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 256;     // window rows per split
constexpr int kQG = 4;          // query rows per pass (one wave each in softmax / PV)

struct AttendArgs {
    const float *q_rot;
    const float *k_win;
    const void *v_win;
    const int32_t *W;
    float *part_acc;    // [n_blk][Hkv][n_split][QR][D]
    float *part_ml;     // [n_blk][Hkv][n_split][QR][2]
    float *out;         // [n_q][Hq][D]
    int64_t W_cap;
    int n_split, QR, Hq, Hkv, g, n_q, block_q;
    float scale;
};

__device__ __forceinline__ float ldv(const uint16_t *p, int64_t i) {
    return __uint_as_float(((uint32_t)p[i]) << 16);
}
__device__ __forceinline__ float ldv(const float *p, int64_t i) { return p[i]; }

template <typename TV, int D>
__global__ __launch_bounds__(kThreads) void k_attend_split(AttendArgs a) {
    constexpr int CPL = D / 16;     // channels per lane in the logit phase
    constexpr int CPT = D / 64;     // channels per thread in the P.V phase
    __shared__ float qs[kQG][D];
    __shared__ float ps[kQG][kChunk];
    __shared__ float ml[kQG][2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int64_t bh = (int64_t)b * a.Hkv + h;
    const int64_t Wbh = a.W[bh];
    const int64_t w0 = (int64_t)s * kChunk;
    const int64_t w1 = min(w0 + (int64_t)kChunk, Wbh);
    const float *kb = a.k_win + bh * a.W_cap * D;
    const TV *vb = (const TV *)a.v_win + bh * a.W_cap * D;

    for (int r0 = 0; r0 < a.QR; r0 += kQG) {
        for (int idx = tid; idx < kQG * D; idx += kThreads) {
            const int rr = idx / D, c = idx % D, r = r0 + rr;
            float v = 0.f;
            if (r < a.QR) {
                const int64_t i = (int64_t)b * a.block_q + r / a.g;
                const int hq = h * a.g + r % a.g;
                v = a.q_rot[(i * a.Hq + hq) * D + c];
            }
            qs[rr][c] = v;
        }
        __syncthreads();

        // logits
        const int l16 = tid & 15, rsub = tid >> 4;
        for (int base = 0; base < kChunk; base += kThreads / 16) {
            const int64_t w = w0 + base + rsub;
            float part[kQG];
#pragma unroll
            for (int rr = 0; rr < kQG; ++rr) part[rr] = 0.f;
            if (w < w1) {
#pragma unroll
                for (int e = 0; e < CPL; ++e) {
                    const int c = l16 * CPL + e;
                    const float kv = kb[w * D + c];
#pragma unroll
                    for (int rr = 0; rr < kQG; ++rr) part[rr] = fmaf(qs[rr][c], kv, part[rr]);
                }
            }
#pragma unroll
            for (int rr = 0; rr < kQG; ++rr) {
                float v = part[rr];
                v += __shfl_xor(v, 1);
                v += __shfl_xor(v, 2);
                v += __shfl_xor(v, 4);
                v += __shfl_xor(v, 8);
                part[rr] = v;
            }
            if (l16 == 0) {
#pragma unroll
                for (int rr = 0; rr < kQG; ++rr) {
                    const int r = r0 + rr;
                    const int64_t pos = Wbh - a.n_q + ((int64_t)b * a.block_q + r / a.g);
                    const bool ok = r < a.QR && w < w1 && w <= pos;
                    ps[rr][base + rsub] = ok ? part[rr] * a.scale : -INFINITY;
                }
            }
        }
        __syncthreads();

        // softmax statistics, wave `wave` owns query row r0 + wave
        {
            float m = -INFINITY;
            for (int j = lane; j < kChunk; j += 64) m = fmaxf(m, ps[wave][j]);
            for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
            float l = 0.f;
            for (int j = lane; j < kChunk; j += 64) {
                const float x = ps[wave][j];
                const float p = (m == -INFINITY) ? 0.f : expf(x - m);
                ps[wave][j] = p;
                l += p;
            }
            for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
            if (lane == 0) {
                ml[wave][0] = m;
                ml[wave][1] = l;
            }
        }
        __syncthreads();

        // P.V, wave `wave` owns query row r0 + wave
        {
            float acc[CPT];
#pragma unroll
            for (int e = 0; e < CPT; ++e) acc[e] = 0.f;
            for (int64_t w = w0; w < w1; ++w) {
                const float p = ps[wave][w - w0];
#pragma unroll
                for (int e = 0; e < CPT; ++e) acc[e] = fmaf(p, ldv(vb, w * D + lane * CPT + e), acc[e]);
            }
            const int r = r0 + wave;
            if (r < a.QR) {
                const int64_t slot = (bh * a.n_split + s) * a.QR + r;
#pragma unroll
                for (int e = 0; e < CPT; ++e) a.part_acc[slot * D + lane * CPT + e] = acc[e];
                if (lane == 0) {
                    a.part_ml[slot * 2] = ml[wave][0];
                    a.part_ml[slot * 2 + 1] = ml[wave][1];
                }
            }
        }
        __syncthreads();
    }
}

template <int D>
__global__ __launch_bounds__(D) void k_attend_combine(AttendArgs a) {
    const int r = blockIdx.x, h = blockIdx.y, b = blockIdx.z, c = threadIdx.x;
    const int64_t bh = (int64_t)b * a.Hkv + h;
    const int64_t base = bh * a.n_split * a.QR + r;
    float M = -INFINITY;
    for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, a.part_ml[(base + (int64_t)s * a.QR) * 2]);
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < a.n_split; ++s) {
        const int64_t slot = base + (int64_t)s * a.QR;
        const float m = a.part_ml[slot * 2];
        if (m == -INFINITY) continue;
        const float f = expf(m - M);
        L = fmaf(a.part_ml[slot * 2 + 1], f, L);
        acc = fmaf(a.part_acc[slot * D + c], f, acc);
    }
    const int64_t i = (int64_t)b * a.block_q + r / a.g;
    const int hq = h * a.g + r % a.g;
    a.out[(i * a.Hq + hq) * D + c] = acc / L;
}

template <typename TV, int D>
hipError_t launch_typed(const Geom &g, const AttendArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((k_attend_split<TV, D>), dim3(a.n_split, g.Hkv, g.n_blk), dim3(kThreads),
                       0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_attend_combine<D>), dim3(a.QR, g.Hkv, g.n_blk), dim3(D), 0, s, a);
    return hipGetLastError();
}

int n_split_of(int64_t W_cap) { return (int)((W_cap + kChunk - 1) / kChunk); }

}  // namespace

size_t attend_ws_bytes(const Geom &g, int64_t W_cap) {
    const size_t rows = (size_t)g.n_blk * g.Hkv * n_split_of(W_cap) * (size_t)(g.block_q * g.g);
    const size_t acc = rows * g.d * sizeof(float);
    const size_t ml = rows * 2 * sizeof(float);
    return ((acc + 255) & ~(size_t)255) + ((ml + 255) & ~(size_t)255);
}

hipError_t launch_attend(const Geom &g, const float *q_rot, const float *k_win,
                         const void *v_win, const int32_t *W, int64_t W_cap, float *out,
                         void *ws, hipStream_t s) {
    AttendArgs a;
    a.q_rot = q_rot;
    a.k_win = k_win;
    a.v_win = v_win;
    a.W = W;
    a.W_cap = W_cap;
    a.n_split = n_split_of(W_cap);
    a.QR = g.block_q * g.g;
    a.Hq = g.Hq;
    a.Hkv = g.Hkv;
    a.g = g.g;
    a.n_q = g.n_q;
    a.block_q = g.block_q;
    a.scale = g.scale;
    a.out = out;
    const size_t rows = (size_t)g.n_blk * g.Hkv * a.n_split * (size_t)a.QR;
    const size_t acc = rows * g.d * sizeof(float);
    a.part_acc = (float *)ws;
    a.part_ml = (float *)((char *)ws + ((acc + 255) & ~(size_t)255));
    if (g.dtype == 0)
        return g.d == 128 ? launch_typed<uint16_t, 128>(g, a, s) : launch_typed<uint16_t, 64>(g, a, s);
    return g.d == 128 ? launch_typed<float, 128>(g, a, s) : launch_typed<float, 64>(g, a, s);
}

}  // namespace rea
