// attend.hip - step 4: ordinary causal softmax attention over the window.
//
// The window's keys are already rotated (step 3), so this is plain attention
// (OpenReview discussion, "Decoding Phase" pseudocode:
// flash_attention(query, key_recall, value_recall)).  Query row r of a block
// is (query i = r / g, head hq = h*g + r % g); it sees window rows w <= its
// own position W - n_q + i.  Everything is fp32 on the VALU.
//
//   k_attend_split   one workgroup per (split of the window, KV head, block).
//                    The split's rows are walked in sub-chunks of 64: K (fp32)
//                    and V are staged in LDS with 16-byte loads, then for up
//                    to 16 query rows at a time the logits, an online softmax
//                    (running max / sum carried across sub-chunks) and P.V are
//                    computed from LDS.  Writes the partial (m, l, acc[d]).
//   k_attend_combine one wave per query row merges the splits:
//                    out = sum_s e^(m_s-M) acc_s / sum_s e^(m_s-M) l_s.
// The number of splits is chosen so that about two workgroups per compute
// unit run; the g query heads of a KV head share every K/V row they read.
#include "rea_internal.h"

#include <math.h>

namespace rea {
namespace {

constexpr int kThreads = 256;
constexpr int kSub = 64;        // window rows staged per sub-chunk
constexpr int kQG = 16;         // query rows per pass
constexpr int kPad = 4;         // LDS row padding (floats) for K

struct AttendArgs {
    const float *q_rot;
    const float *k_win;
    const void *v_win;
    const int32_t *W;
    float *part_acc;    // [n_blk][Hkv][n_split][QR][D]
    float *part_ml;     // [n_blk][Hkv][n_split][QR][2]
    float *out;         // [n_q][Hq][D]
    int64_t W_cap;
    int64_t rows_per_split;
    int n_split, QR, Hq, Hkv, g, n_q, block_q;
    float scale;
};

template <typename TV> struct VLoad;
template <> struct VLoad<uint16_t> {          // 8 bf16 -> 8 fp32
    static constexpr int N = 8;
    __device__ static void get(const uint16_t *p, float *o) {
        const uint4 u = *(const uint4 *)p;
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct VLoad<float> {
    static constexpr int N = 4;
    __device__ static void get(const float *p, float *o) {
        const float4 u = *(const float4 *)p;
        o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w;
    }
};

template <typename TV, int D>
__global__ __launch_bounds__(kThreads) void k_attend_split(AttendArgs a) {
    constexpr int TPQ = kThreads / kQG;       // threads per query row in P.V (16)
    constexpr int CPT = D / TPQ;              // channels per thread in P.V
    __shared__ __align__(16) float ks[kSub][D + kPad];
    __shared__ __align__(16) float vs[kSub][D];
    __shared__ __align__(16) float qs[kQG][D];
    __shared__ float ps[kQG][kSub];
    __shared__ float m_run[kQG], l_run[kQG], fac[kQG];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int64_t bh = (int64_t)b * a.Hkv + h;
    const int64_t Wbh = a.W[bh];
    const int64_t w0 = (int64_t)s * a.rows_per_split;
    const int64_t w1 = min(w0 + a.rows_per_split, Wbh);
    const float *kb = a.k_win + bh * a.W_cap * D;
    const TV *vb = (const TV *)a.v_win + bh * a.W_cap * D;
    const int pr = tid / TPQ, pc = (tid % TPQ) * CPT;      // P.V ownership

    for (int r0 = 0; r0 < a.QR; r0 += kQG) {
        for (int idx = tid; idx < kQG * D / 4; idx += kThreads) {
            const int rr = idx / (D / 4), c = (idx % (D / 4)) * 4, r = r0 + rr;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < a.QR) {
                const int64_t i = (int64_t)b * a.block_q + r / a.g;
                const int hq = h * a.g + r % a.g;
                v = *(const float4 *)(a.q_rot + (i * a.Hq + hq) * D + c);
            }
            *(float4 *)&qs[rr][c] = v;
        }
        if (tid < kQG) {
            m_run[tid] = -INFINITY;
            l_run[tid] = 0.f;
        }
        float acc[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) acc[e] = 0.f;

        for (int64_t c0 = w0; c0 < w1; c0 += kSub) {
            const int nrows = (int)min((int64_t)kSub, w1 - c0);
            __syncthreads();    // previous sub-chunk fully consumed
            for (int idx = tid; idx < nrows * (D / 4); idx += kThreads) {
                const int row = idx / (D / 4), c = (idx % (D / 4)) * 4;
                *(float4 *)&ks[row][c] = *(const float4 *)(kb + (c0 + row) * D + c);
            }
            constexpr int VN = VLoad<TV>::N;
            for (int idx = tid; idx < nrows * (D / VN); idx += kThreads) {
                const int row = idx / (D / VN), c = (idx % (D / VN)) * VN;
                VLoad<TV>::get(vb + (c0 + row) * D + c, &vs[row][c]);
            }
            __syncthreads();
            // logits
            for (int pidx = tid; pidx < kQG * kSub; pidx += kThreads) {
                const int rr = pidx / kSub, wl = pidx % kSub, r = r0 + rr;
                float v = -INFINITY;
                if (r < a.QR && wl < nrows) {
                    const int64_t pos = Wbh - a.n_q + ((int64_t)b * a.block_q + r / a.g);
                    if (c0 + wl <= pos) {
                        float d = 0.f;
#pragma unroll 8
                        for (int c = 0; c < D; c += 4) {
                            const float4 x = *(const float4 *)&qs[rr][c];
                            const float4 y = *(const float4 *)&ks[wl][c];
                            d = fmaf(x.x, y.x, d);
                            d = fmaf(x.y, y.y, d);
                            d = fmaf(x.z, y.z, d);
                            d = fmaf(x.w, y.w, d);
                        }
                        v = d * a.scale;
                    }
                }
                ps[rr][wl] = v;
            }
            __syncthreads();
            // online softmax statistics: wave `wave` owns rows wave, wave+4, ...
            for (int rr = wave; rr < kQG; rr += kThreads / 64) {
                const float x = ps[rr][lane];
                float mc = x;
                for (int o = 32; o > 0; o >>= 1) mc = fmaxf(mc, __shfl_xor(mc, o));
                const float mo = m_run[rr];
                const float mn = fmaxf(mo, mc);
                const float p = (mn == -INFINITY) ? 0.f : expf(x - mn);
                ps[rr][lane] = p;
                float lc = p;
                for (int o = 32; o > 0; o >>= 1) lc += __shfl_xor(lc, o);
                if (lane == 0) {
                    const float f = (mo == -INFINITY) ? 0.f : expf(mo - mn);
                    fac[rr] = f;
                    m_run[rr] = mn;
                    l_run[rr] = l_run[rr] * f + lc;
                }
            }
            __syncthreads();
            // P.V
            {
                const float f = fac[pr];
#pragma unroll
                for (int e = 0; e < CPT; ++e) acc[e] *= f;
                for (int wl = 0; wl < nrows; ++wl) {
                    const float p = ps[pr][wl];
#pragma unroll
                    for (int e = 0; e < CPT; e += 4) {
                        const float4 v = *(const float4 *)&vs[wl][pc + e];
                        acc[e] = fmaf(p, v.x, acc[e]);
                        acc[e + 1] = fmaf(p, v.y, acc[e + 1]);
                        acc[e + 2] = fmaf(p, v.z, acc[e + 2]);
                        acc[e + 3] = fmaf(p, v.w, acc[e + 3]);
                    }
                }
            }
        }
        __syncthreads();
        const int r = r0 + pr;
        if (r < a.QR) {
            const int64_t slot = (bh * a.n_split + s) * a.QR + r;
#pragma unroll
            for (int e = 0; e < CPT; e += 4)
                *(float4 *)(a.part_acc + slot * D + pc + e) =
                    make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
            if (pc == 0) {
                a.part_ml[slot * 2] = m_run[pr];
                a.part_ml[slot * 2 + 1] = l_run[pr];
            }
        }
        __syncthreads();
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_attend_combine(AttendArgs a) {
    constexpr int CPL = D / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = blockIdx.x * (kThreads / 64) + wave;
    const int h = blockIdx.y, b = blockIdx.z;
    if (r >= a.QR) return;
    const int64_t bh = (int64_t)b * a.Hkv + h;
    const int64_t base = bh * a.n_split * a.QR + r;
    float M = -INFINITY;
    for (int s = lane; s < a.n_split; s += 64) M = fmaxf(M, a.part_ml[(base + (int64_t)s * a.QR) * 2]);
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.f;
    for (int s = lane; s < a.n_split; s += 64) {
        const int64_t slot = base + (int64_t)s * a.QR;
        const float m = a.part_ml[slot * 2];
        if (m != -INFINITY) L += a.part_ml[slot * 2 + 1] * expf(m - M);
    }
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
    float acc[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[e] = 0.f;
#pragma unroll 4
    for (int s = 0; s < a.n_split; ++s) {
        const int64_t slot = base + (int64_t)s * a.QR;
        const float m = a.part_ml[slot * 2];
        const float f = (m == -INFINITY) ? 0.f : expf(m - M);
#pragma unroll
        for (int e = 0; e < CPL; ++e) acc[e] = fmaf(f, a.part_acc[slot * D + lane * CPL + e], acc[e]);
    }
    const int64_t i = (int64_t)b * a.block_q + r / a.g;
    const int hq = h * a.g + r % a.g;
#pragma unroll
    for (int e = 0; e < CPL; ++e) a.out[(i * a.Hq + hq) * D + lane * CPL + e] = acc[e] / L;
}

template <typename TV, int D>
hipError_t launch_typed(const Geom &g, const AttendArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((k_attend_split<TV, D>), dim3(a.n_split, g.Hkv, g.n_blk), dim3(kThreads),
                       0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_attend_combine<D>), dim3((a.QR + 3) / 4, g.Hkv, g.n_blk),
                       dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

// Rows per split: whole sub-chunks, about 512 workgroups in total.
int64_t rows_per_split(const Geom &g, int64_t W_cap) {
    const int64_t subs = (W_cap + kSub - 1) / kSub;
    const int64_t units = (int64_t)g.Hkv * g.n_blk;
    int64_t want = (512 + units - 1) / units;        // splits per (block, KV head)
    if (want < 1) want = 1;
    const int64_t subs_per = (subs + want - 1) / want;
    return (subs_per < 1 ? 1 : subs_per) * kSub;
}

int n_split_of(const Geom &g, int64_t W_cap) {
    const int64_t rps = rows_per_split(g, W_cap);
    return (int)((W_cap + rps - 1) / rps);
}

}  // namespace

size_t attend_ws_bytes(const Geom &g, int64_t W_cap) {
    const size_t rows = (size_t)g.n_blk * g.Hkv * n_split_of(g, W_cap) * (size_t)(g.block_q * g.g);
    const size_t acc = rows * g.d * sizeof(float);
    const size_t ml = rows * 2 * sizeof(float);
    return ((acc + 255) & ~(size_t)255) + ((ml + 255) & ~(size_t)255);
}

hipError_t launch_attend(const Geom &g, const float *q_rot, const float *k_win,
                         const void *v_win, const int32_t *W, int64_t W_cap, float *out,
                         void *ws, hipStream_t s) {
    if (mfma_attend_path(g)) return launch_attend_mfma(g, q_rot, k_win, v_win, W, W_cap, out, s);
    AttendArgs a;
    a.q_rot = q_rot;
    a.k_win = k_win;
    a.v_win = v_win;
    a.W = W;
    a.W_cap = W_cap;
    a.rows_per_split = rows_per_split(g, W_cap);
    a.n_split = n_split_of(g, W_cap);
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
