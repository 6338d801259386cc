// attend_mfma.hip - step 4 for blocks of queries (chunked prefill) on MFMA.
//
// Ordinary causal softmax attention over each block's window (OpenReview
// discussion, "Decoding Phase"/"Prefilling Phase" pseudocode:
// flash_attention(query, key_recall, value_recall)), flash-style: key tiles of
// 32 window rows are staged in LDS and the softmax is carried online.
//
// One workgroup = 4 waves = 128 query rows of one (block, KV head); a wave
// owns 32 query rows r (query i = r / g, head h*g + r % g).  Per key tile:
//   S^T = K' Q'^T on v_mfma_f32_32x32x16_bf16 with K' and Q' each split into
//         bf16 hi + lo (three products: hi.hi + hi.lo + lo.hi, ~16-bit inputs),
//         so a lane holds one query's 16 logits of the tile and the softmax
//         statistics stay lane-local (one exchange with the partner half-wave);
//   O^T += V^T P^T with V exact in bf16 and P rounded to bf16; V is staged
//         transposed so each A fragment is one 16-byte LDS read.
// The next tile's global loads are issued before this tile's MFMAs.
#include "rea_internal.h"

#include <math.h>

namespace rea {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;
constexpr int kKT = 32;             // keys per tile
constexpr int kKPad = 136;          // K' tile row stride (bf16)
constexpr int kVPad = 40;           // V^T tile row stride (bf16)
constexpr int kRowsWG = 128;        // query rows per workgroup

struct MAttnArgs {
    const float *q_rot;     // [n_q][Hq][D]
    const float *k_win;     // [n_blk][Hkv][W_cap][D]
    const uint16_t *v_win;  // [n_blk][Hkv][W_cap][D] bf16
    const int32_t *W;       // [n_blk][Hkv]
    float *out;             // [n_q][Hq][D]
    int64_t W_cap;
    int QR, Hq, Hkv, g, n_q, block_q, n_rg;
    float scale;
};

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return b >> 16;
}

// 8 floats -> hi (bf16) and lo = bf16(x - hi), packed 2 per dword
__device__ __forceinline__ void split8(const float (&x)[8], uint4 &hi, uint4 &lo) {
    uint32_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h[e] = bf16_rne_bits(x[e]);
        l[e] = bf16_rne_bits(x[e] - __uint_as_float(h[e] << 16));
    }
    hi = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    lo = make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16));
}

__global__ __launch_bounds__(256) void k_attend_mfma(MAttnArgs a) {
    __shared__ __align__(16) uint16_t khi[2][kKT][kKPad];
    __shared__ __align__(16) uint16_t klo[2][kKT][kKPad];
    __shared__ __align__(16) uint16_t vt[2][kD][kVPad];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rg = blockIdx.x % a.n_rg;
    const int bh = blockIdx.x / a.n_rg;
    const int b = bh / a.Hkv, h = bh % a.Hkv;
    const int64_t Wbh = a.W[bh];
    const int n = lane & 31, hb = lane >> 5;

    // this lane's query column
    const int r = rg * kRowsWG + wave * 32 + n;
    const bool valid_q = r < a.QR;
    const int rq = valid_q ? r : 0;
    const int64_t qi = (int64_t)b * a.block_q + rq / a.g;
    const int hq = h * a.g + rq % a.g;
    const int64_t pos = Wbh - a.n_q + qi;

    // B fragments of Q' (hi, lo): channels ks*16 + hb*8 .. +8
    uint4 qh[8], ql[8];
    {
        const float *qrow = a.q_rot + (qi * a.Hq + hq) * kD;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const float4 u0 = *(const float4 *)(qrow + ks * 16 + hb * 8);
            const float4 u1 = *(const float4 *)(qrow + ks * 16 + hb * 8 + 4);
            const float x[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
            split8(x, qh[ks], ql[ks]);
        }
    }

    // keys this workgroup needs: up to the largest position among its rows
    int64_t rmax = (int64_t)(rg + 1) * kRowsWG - 1;
    if (rmax > a.QR - 1) rmax = a.QR - 1;
    int64_t kend = Wbh - a.n_q + (int64_t)b * a.block_q + rmax / a.g + 1;
    if (kend > Wbh) kend = Wbh;
    const int64_t n_tiles = (kend + kKT - 1) / kKT;

    const float *kb = a.k_win + (int64_t)bh * a.W_cap * kD;
    const uint16_t *vb = a.v_win + (int64_t)bh * a.W_cap * kD;
    // staging: thread -> key row tid/8, channels (tid%8)*16 .. +16
    const int skey = tid >> 3, sch = (tid & 7) * 16;
    float4 kr[4];
    uint4 vr[2];
    auto load_tile = [&](int64_t w0) {
        const int64_t w = w0 + skey;
        const bool ok = w < kend;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            kr[e] = ok ? *(const float4 *)(kb + w * kD + sch + e * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int e = 0; e < 2; ++e)
            vr[e] = ok ? *(const uint4 *)(vb + w * kD + sch + e * 8) : make_uint4(0u, 0u, 0u, 0u);
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float x[8] = {kr[2 * e].x, kr[2 * e].y, kr[2 * e].z, kr[2 * e].w,
                                kr[2 * e + 1].x, kr[2 * e + 1].y, kr[2 * e + 1].z, kr[2 * e + 1].w};
            uint4 hi, lo;
            split8(x, hi, lo);
            *(uint4 *)&khi[buf][skey][sch + e * 8] = hi;
            *(uint4 *)&klo[buf][skey][sch + e * 8] = lo;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const uint32_t w4[4] = {vr[e].x, vr[e].y, vr[e].z, vr[e].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                vt[buf][sch + e * 8 + 2 * k][skey] = (uint16_t)(w4[k] & 0xffffu);
                vt[buf][sch + e * 8 + 2 * k + 1][skey] = (uint16_t)(w4[k] >> 16);
            }
        }
    };

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) o[t][rr] = 0.f;

    int buf = 0;
    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    for (int64_t it = 0; it < n_tiles; ++it) {
        const int64_t w0 = it * kKT;
        const bool more = it + 1 < n_tiles;
        if (more) load_tile(w0 + kKT);

        // S^T tile: rows = keys (A = K'), cols = queries (B = Q'^T)
        f32x16 st = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 ah = __builtin_bit_cast(bf16x8, *(const uint4 *)&khi[buf][n][ks * 16 + hb * 8]);
            const bf16x8 al = __builtin_bit_cast(bf16x8, *(const uint4 *)&klo[buf][n][ks * 16 + hb * 8]);
            const bf16x8 bh8 = __builtin_bit_cast(bf16x8, qh[ks]);
            const bf16x8 bl8 = __builtin_bit_cast(bf16x8, ql[ks]);
            st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh8, st, 0, 0, 0);
            st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl8, st, 0, 0, 0);
            st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh8, st, 0, 0, 0);
        }
        // mask, online softmax (this lane's query; keys 8(rr/4) + 4hb + rr%4)
        float x[16];
        float mt = -INFINITY;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int64_t w = w0 + 8 * (rr >> 2) + 4 * hb + (rr & 3);
            x[rr] = (w < Wbh && w <= pos) ? st[rr] * a.scale : -INFINITY;
            mt = fmaxf(mt, x[rr]);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_run == -INFINITY) ? 0.f : expf(m_run - m_new);
        float p[16];
        float lt = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            p[rr] = (x[rr] == -INFINITY) ? 0.f : expf(x[rr] - m_new);
            lt += p[rr];
        }
        lt += __shfl_xor(lt, 32);
        l_run = l_run * alpha + lt;
        m_run = m_new;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) o[t][rr] *= alpha;

        // B fragments of P^T: k-step s covers keys 16s .. 16s+15; this lane
        // (kb = hb) needs keys 16s + 8hb + e; a lane holds keys 8a + 4hb + c.
        uint4 pb[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float send[4], recv[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) send[c] = hb == 0 ? p[4 * (2 * s + 1) + c] : p[4 * (2 * s) + c];
#pragma unroll
            for (int c = 0; c < 4; ++c) recv[c] = __shfl_xor(send[c], 32);
            float v8[8];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                v8[c] = hb == 0 ? p[4 * (2 * s) + c] : recv[c];
                v8[4 + c] = hb == 0 ? recv[c] : p[4 * (2 * s + 1) + c];
            }
            uint32_t bb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) bb[e] = bf16_rne_bits(v8[e]);
            pb[s] = make_uint4(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16), bb[4] | (bb[5] << 16),
                               bb[6] | (bb[7] << 16));
        }
        // O^T (channels x queries) += V^T (channels x keys) P^T (keys x queries)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const bf16x8 av = __builtin_bit_cast(bf16x8, *(const uint4 *)&vt[buf][t * 32 + n][s * 16 + hb * 8]);
                o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, pb[s]),
                                                               o[t], 0, 0, 0);
            }
        if (more) store_tile(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }

    if (valid_q) {
        const float inv = 1.f / l_run;
        float *orow = a.out + (qi * a.Hq + hq) * kD;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int aa = 0; aa < 4; ++aa) {
                const int c = t * 32 + 8 * aa + 4 * hb;
                *(float4 *)(orow + c) = make_float4(o[t][4 * aa] * inv, o[t][4 * aa + 1] * inv,
                                                    o[t][4 * aa + 2] * inv, o[t][4 * aa + 3] * inv);
            }
    }
}

}  // namespace

bool mfma_attend_path(const Geom &g) {
    return g.dtype == 0 && g.d == kD && g.block_q * g.g >= 32;
}

hipError_t launch_attend_mfma(const Geom &g, const float *q_rot, const float *k_win,
                              const void *v_win, const int32_t *W, int64_t W_cap, float *out,
                              hipStream_t s) {
    MAttnArgs a;
    a.q_rot = q_rot;
    a.k_win = k_win;
    a.v_win = (const uint16_t *)v_win;
    a.W = W;
    a.out = out;
    a.W_cap = W_cap;
    a.QR = g.block_q * g.g;
    a.Hq = g.Hq;
    a.Hkv = g.Hkv;
    a.g = g.g;
    a.n_q = g.n_q;
    a.block_q = g.block_q;
    a.n_rg = (a.QR + kRowsWG - 1) / kRowsWG;
    a.scale = g.scale;
    hipLaunchKernelGGL(k_attend_mfma, dim3(g.n_blk * g.Hkv * a.n_rg), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace rea
