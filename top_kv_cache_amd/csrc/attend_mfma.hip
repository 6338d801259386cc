// attend_mfma.hip - step 4 for blocks of queries (chunked prefill) on MFMA.
//
// Ordinary causal softmax attention over each block's window (OpenReview
// discussion, "Decoding Phase"/"Prefilling Phase" pseudocode:
// flash_attention(query, key_recall, value_recall)), flash-style: key tiles of
// 32 window rows are staged in LDS and the softmax is carried online.
//
// One workgroup = 8 waves = 256 query rows of one (block, KV head) (a block
// of 64 queries with g = 4 in one workgroup, so its key tiles are staged
// once); a wave owns 32 query rows r (query i = r / g, head h*g + r % g).
// Per key tile:
//   S^T = K' Q'^T on v_mfma_f32_32x32x16_bf16 with K' and Q' each split into
//         bf16 hi + lo (three products: hi.hi + hi.lo + lo.hi, ~16-bit inputs),
//         so a lane holds one query's 16 logits of the tile and the softmax
//         statistics stay lane-local (one exchange with the partner half-wave).
//         Q' carries the softmax scale times log2(e): logits are in log2
//         units and weights are single exp2s; the accumulators are rescaled
//         only in tiles where some query's maximum outgrows the reference
//         maximum the weights are taken against by more than 2^8;
//   O^T += V^T P^T with V exact in bf16 and P rounded to bf16; V is staged
//         transposed so each A fragment is one 16-byte LDS read.
// 8-wave workgroups run the tiles as a three-stage software pipeline (tile
// it+2 staged, logits of tile it+1 on the MFMA pipe while tile it's softmax
// runs on the VALU, then tile it's O update), and the two waves that share a
// SIMD take those phases in opposite order.  2-wave workgroups (at most 64
// query rows, cache source) use one tile buffer.
//
// Two sources for the tiles (template parameter):
//   window  the rotated window written by the gather step (rea_window_attend);
//   cache   inside rea_decode_step: window row w is read from the bf16 cache
//           through the selection (global ++ selected spans ++ local), and
//           rotated to position w while it is staged, with (cos, sin) from a
//           per-call table of the window positions (k_rope_table, fp64
//           angles rounded to fp32).  The queries are rotated the same way
//           from the table, so neither the window nor the rotated queries are
//           ever written.
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
constexpr int kAThreads = 512;      // 8 waves (blocks of many query rows)
constexpr int kRowsWG = kAThreads / 2;   // query rows per 8-wave workgroup (32 per wave)

constexpr float kLazy = 8.f;         // log2 of the largest unnormalised weight
constexpr int kSelCap = 4096;       // selection entries staged in LDS (cache source, 8 waves)
// 2-wave workgroups (at most 64 query rows: decode steps, small blocks) take
// at most kSmallTiles key tiles per split and stage only the selection
// entries those rows use
constexpr int kSmallTiles = 8;
constexpr int kSmallSel = kSmallTiles * 32 + 8;

struct MAttnArgs {
    // window source
    const float *q_rot;     // [n_q][Hq][D]
    const float *k_win;     // [n_blk][Hkv][W_cap][D]
    const uint16_t *v_win;  // [n_blk][Hkv][W_cap][D] bf16
    const int32_t *W;       // [n_blk][Hkv]
    // cache source
    const uint16_t *q;      // [n_q][Hq][D] bf16, un-rotated
    const uint16_t *k, *v;  // caches, element strides sh (head), st (token)
    const int32_t *sel, *n_sel;
    const float2 *rope;     // [W_cap][D/2] (cos, sin) of w * theta_c
    int64_t sh, st, T, Gp, Lp, mid_lo, n_spans;
    int S, last_len, topk;
    // both
    float *out;             // [n_q][Hq][D]
    int64_t W_cap;
    int QR, Hq, Hkv, g, n_q, block_q, n_rg, rep;
    float scale_log2;       // softmax scale * log2(e)
    // key-tile splits (cache source): split sp of a workgroup's tiles writes
    // unnormalised partials of its valid rows, merged by k_attend_merge
    int n_split, rw;        // rw: query rows per workgroup (32 per wave)
    float *part_o;          // [units][n_split][rw][D]
    float2 *part_ml;        // [units][n_split][rw]: running max, sum
    // batched decode (see Geom): per-sequence lengths and cache offsets
    const int64_t *lens;
    int hps, G, L;
    int64_t seq_stride;
};

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (round to nearest even), packed low first
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, bf16x2v));
}

// 8 floats -> hi (bf16) and lo = bf16(x - hi), packed 2 per dword
__device__ __forceinline__ void split8(const float (&x)[8], uint4 &hi, uint4 &lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = pack_bf16(x[2 * e], x[2 * e + 1]);
        l[e] = pack_bf16(x[2 * e] - __uint_as_float(h[e] << 16),
                         x[2 * e + 1] - __uint_as_float(h[e] & 0xffff0000u));
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

__device__ __forceinline__ void bf16x8_to_f32(const uint4 &u, float (&x)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}

// The occupancy hint of one wave per SIMD lets the 2-wave variant (4 staging
// groups per thread) keep everything in registers, accumulators in AGPRs,
// instead of spilling 132 bytes per lane to scratch (15-20% faster).
template <bool kCache, int NW>
__global__ __launch_bounds__(64 * NW, 1) void k_attend_mfma(MAttnArgs a) {
    static_assert(NW == 8 || (NW == 2 && kCache), "8 waves, or 2 waves on the cache source");
    constexpr int NT = 64 * NW;                 // threads
    constexpr int RW = 32 * NW;                 // query rows per workgroup
    constexpr int NB = NW == 8 ? 3 : 1;         // LDS tile buffers
    constexpr int TPR = NT / kKT;               // staging threads per key row (16 or 4)
    constexpr int PG = 16 / TPR;                // groups of 4 channel pairs (K) / 8 channels (V) per thread
    constexpr int kSel = NW == 8 ? kSelCap : kSmallSel;
    __shared__ __align__(16) uint16_t khi[NB][kKT][kKPad];
    __shared__ __align__(16) uint16_t klo[NB][kKT][kKPad];
    __shared__ __align__(16) uint16_t vt[NB][kD][kVPad];
    __shared__ int32_t ssel[kCache ? kSel : 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Later blocks of a chunk see more keys (causal): the grid runs them
    // first, so that the shorter ones fill in behind them.
    const int bid = (int)gridDim.x - 1 - (int)blockIdx.x;
    const int sp = bid % a.n_split;
    const int unit = bid / a.n_split;
    const int rg = unit % a.n_rg;
    const int bh = unit / a.n_rg;
    const int b = bh / a.Hkv, h = bh % a.Hkv;
    const int n = lane & 31, hb = lane >> 5;
    // the (block, head)'s sequence: its own regions when decoding a batch
    SeqGeom sg{};
    int64_t kv_off = 0;
    if (kCache) {
        const SeqOf so = seq_of(a.lens, h, a.hps, a.rep, a.seq_stride, a.sh, a.T);
        sg = seq_geom(so.T, a.G, a.L, a.S);
        kv_off = so.kv_off;
    }
    int64_t Wbh, sel_len = 0;
    int ns = 0;
    if (kCache) {
        // window length from the selection (only span n_spans-1 can be short,
        // and a sorted selection holds it last)
        ns = a.n_sel[bh];
        sel_len = (int64_t)ns * a.S;
        if (sg.last_len != a.S && ns > 0 && a.sel[(int64_t)bh * a.topk + ns - 1] == sg.n_spans - 1)
            sel_len -= a.S - sg.last_len;
        Wbh = sg.Gp + sel_len + sg.Lp;
    } else {
        Wbh = a.W[bh];
    }

    // this lane's query column
    const int r = rg * RW + wave * 32 + n;
    const bool valid_q = r < a.QR;
    const int rq = valid_q ? r : 0;
    const int64_t qi = (int64_t)b * a.block_q + rq / a.g;
    const int hq = h * a.g + rq % a.g;
    const int64_t pos = Wbh - a.n_q + qi;

    // keys this workgroup needs: up to the largest position among its rows,
    // and this split's share of their tiles
    int64_t rmax = (int64_t)(rg + 1) * RW - 1;
    if (rmax > a.QR - 1) rmax = a.QR - 1;
    int64_t kend = Wbh - a.n_q + (int64_t)b * a.block_q + rmax / a.g + 1;
    if (kend > Wbh) kend = Wbh;
    const int64_t n_tiles_all = (kend + kKT - 1) / kKT;
    const int64_t it0 = n_tiles_all * sp / a.n_split;
    const int64_t it1 = n_tiles_all * (sp + 1) / a.n_split;

    // the selection entries the split's rows use go to LDS (all of them with
    // 8 waves; with 2 waves a split spans at most kSmallTiles tiles)
    int64_t slot0 = 0;
    if (kCache) {
        int64_t slot1 = ns;
        if (NW != 8) {
            const int64_t wl = it0 * kKT - sg.Gp, wh = it1 * kKT - 1 - sg.Gp;
            slot0 = wl > 0 ? wl / a.S : 0;
            slot1 = wh >= 0 ? wh / a.S + 1 : 0;
            if (slot1 > ns) slot1 = ns;
            if (slot1 < slot0) slot1 = slot0;
        }
        for (int64_t t = tid; t < slot1 - slot0; t += NT)
            ssel[t] = a.sel[(int64_t)bh * a.topk + slot0 + t];
    }

    // B fragments of Q' (hi, lo): channels ks*16 + hb*8 .. +8.  The query is
    // scaled by softmax_scale * log2(e) first, so logits come out in log2
    // units and every weight is one exp2.
    uint4 qh[8], ql[8];
    const float sc = a.scale_log2;
    if (kCache) {
        // rotate the raw query to its position: channel ks*16+hb*8+e (ks < 4)
        // pairs with the same offset in ks+4, both held by this lane
        const uint16_t *qrow = a.q + (qi * a.Hq + hq) * kD;
        const float2 *rp = a.rope + pos * (kD / 2);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float x1[8], x2[8], y1[8], y2[8];
            bf16x8_to_f32(*(const uint4 *)(qrow + ks * 16 + hb * 8), x1);
            bf16x8_to_f32(*(const uint4 *)(qrow + ks * 16 + hb * 8 + kD / 2), x2);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float2 cs = rp[ks * 16 + hb * 8 + e];
                y1[e] = (x1[e] * cs.x - x2[e] * cs.y) * sc;
                y2[e] = (x2[e] * cs.x + x1[e] * cs.y) * sc;
            }
            split8(y1, qh[ks], ql[ks]);
            split8(y2, qh[ks + 4], ql[ks + 4]);
        }
    } else {
        const float *qrow = a.q_rot + (qi * a.Hq + hq) * kD;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const float4 u0 = *(const float4 *)(qrow + ks * 16 + hb * 8);
            const float4 u1 = *(const float4 *)(qrow + ks * 16 + hb * 8 + 4);
            const float x[8] = {u0.x * sc, u0.y * sc, u0.z * sc, u0.w * sc,
                                u1.x * sc, u1.y * sc, u1.z * sc, u1.w * sc};
            split8(x, qh[ks], ql[ks]);
        }
    }

    // staging (NT threads, 32 rows).  K, window (8 waves): thread -> key row
    // tid/16, channels (tid%16)*8 .. +8.  K, cache: thread -> key row tid/TPR,
    // PG groups of 4 channel pairs from (tid%TPR)*4*PG, i.e. channels c0 ..
    // c0+4 and c0+D/2 .. c0+D/2+4 per group.  V: thread -> key row tid%32, PG
    // groups of 8 channels from (tid/32)*8*PG, so lanes l and l^1 hold
    // adjacent keys and V^T is written one 32-bit word (two keys) at a time.
    const int skey = tid / TPR, sch = (tid & 15) * 8, c0 = (tid % TPR) * 4 * PG;
    const int vkey = tid & 31, vch = (tid >> 5) * 8 * PG;
    const float *kwb = a.k_win + (int64_t)bh * a.W_cap * kD;
    const uint16_t *vwb = a.v_win + (int64_t)bh * a.W_cap * kD;
    const uint16_t *kcb = a.k + kv_off;
    const uint16_t *vcb = a.v + kv_off;
    // one tile's staging registers
    struct Stage {
        float4 kr[PG][2];       // window: 8 fp32 keys; cache: 4 x (cos, sin) per group
        uint4 vr[PG];
        uint2 kc[PG][2];
    };
    // cache row of window row wl (rows past the end read window row 0: finite
    // data that is masked or multiplied by a zero weight)
    auto src_row = [&](int64_t wl) -> int64_t {
        int64_t src;
        if (wl < sg.Gp) {
            src = wl;
        } else if (wl < sg.Gp + sel_len) {
            const uint32_t o = (uint32_t)(wl - sg.Gp);
            const uint32_t qs = o / (uint32_t)a.S;
            src = sg.mid_lo + (int64_t)ssel[qs - slot0] * a.S + (o - qs * (uint32_t)a.S);
        } else {
            src = sg.T - sg.Lp + (wl - sg.Gp - sel_len);
        }
        return src * a.st;
    };
    auto load_tile = [&](Stage &stg, int64_t w0) {
        const int64_t w = w0 + skey, wv = w0 + vkey;
        const bool ok = w < kend, okv = wv < kend;
        if (kCache) {
            // lane l < 32 looks up key l of the tile (its V row); the K row
            // of key skey comes from lane skey
            const int64_t wl = ok ? w : it0 * kKT;
            const int64_t rowv = src_row(okv ? wv : it0 * kKT);
            const int64_t row = __shfl(rowv, skey);
#pragma unroll
            for (int gq = 0; gq < PG; ++gq) {
                const int c = c0 + gq * 4;
                stg.kc[gq][0] = *(const uint2 *)(kcb + row + c);
                stg.kc[gq][1] = *(const uint2 *)(kcb + row + c + kD / 2);
                stg.vr[gq] = *(const uint4 *)(vcb + rowv + vch + gq * 8);
                const float4 *rp = (const float4 *)(a.rope + wl * (kD / 2) + c);
                stg.kr[gq][0] = rp[0];
                stg.kr[gq][1] = rp[1];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 2; ++e)
                stg.kr[0][e] = ok ? *(const float4 *)(kwb + w * kD + sch + e * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
            stg.vr[0] = okv ? *(const uint4 *)(vwb + wv * kD + vch) : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    // V^T from this lane's 8-channel groups of key vkey and lane^1's (key
    // vkey^1): the even lane writes the even channels, the odd lane the odd
    // ones, each word holding (key 2m, key 2m+1)
    auto store_vt = [&](const Stage &stg, int bf) {
        const bool odd = (vkey & 1) != 0;
        uint32_t *vrow = (uint32_t *)&vt[bf][0][0];
#pragma unroll
        for (int gq = 0; gq < PG; ++gq) {
            const uint32_t w8[4] = {stg.vr[gq].x, stg.vr[gq].y, stg.vr[gq].z, stg.vr[gq].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t send = odd ? (w8[m] & 0xffffu) : (w8[m] >> 16);
                const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
                const uint32_t word = odd ? (recv | (w8[m] & 0xffff0000u)) : ((w8[m] & 0xffffu) | (recv << 16));
                const int ch = vch + gq * 8 + 2 * m + (odd ? 1 : 0);
                vrow[(ch * kVPad + (vkey & ~1)) / 2] = word;
            }
        }
    };
    auto store_tile = [&](const Stage &stg, int bf) {
        if (kCache) {
#pragma unroll
            for (int gq = 0; gq < PG; ++gq) {
                const int c = c0 + gq * 4;
                const float x1[4] = {__uint_as_float(stg.kc[gq][0].x << 16), __uint_as_float(stg.kc[gq][0].x & 0xffff0000u),
                                     __uint_as_float(stg.kc[gq][0].y << 16), __uint_as_float(stg.kc[gq][0].y & 0xffff0000u)};
                const float x2[4] = {__uint_as_float(stg.kc[gq][1].x << 16), __uint_as_float(stg.kc[gq][1].x & 0xffff0000u),
                                     __uint_as_float(stg.kc[gq][1].y << 16), __uint_as_float(stg.kc[gq][1].y & 0xffff0000u)};
                const float cs[4][2] = {{stg.kr[gq][0].x, stg.kr[gq][0].y}, {stg.kr[gq][0].z, stg.kr[gq][0].w},
                                        {stg.kr[gq][1].x, stg.kr[gq][1].y}, {stg.kr[gq][1].z, stg.kr[gq][1].w}};
                float y[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    y[e] = x1[e] * cs[e][0] - x2[e] * cs[e][1];
                    y[4 + e] = x2[e] * cs[e][0] + x1[e] * cs[e][1];
                }
                uint4 hi, lo;
                split8(y, hi, lo);
                *(uint2 *)&khi[bf][skey][c] = make_uint2(hi.x, hi.y);
                *(uint2 *)&klo[bf][skey][c] = make_uint2(lo.x, lo.y);
                *(uint2 *)&khi[bf][skey][c + kD / 2] = make_uint2(hi.z, hi.w);
                *(uint2 *)&klo[bf][skey][c + kD / 2] = make_uint2(lo.z, lo.w);
            }
        } else {
            const float x[8] = {stg.kr[0][0].x, stg.kr[0][0].y, stg.kr[0][0].z, stg.kr[0][0].w,
                                stg.kr[0][1].x, stg.kr[0][1].y, stg.kr[0][1].z, stg.kr[0][1].w};
            uint4 hi, lo;
            split8(x, hi, lo);
            *(uint4 *)&khi[bf][skey][sch] = hi;
            *(uint4 *)&klo[bf][skey][sch] = lo;
        }
        store_vt(stg, bf);
    };

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) o[t][rr] = 0.f;

    // S^T tile from buffer bf: rows = keys (A = K'), cols = queries (B = Q'^T)
    // (two accumulation chains, even and odd k-steps, so that consecutive
    // MFMAs do not wait on each other's result)
    auto logits = [&](int bf) {
        f32x16 sa = {}, sb = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 ah = __builtin_bit_cast(bf16x8, *(const uint4 *)&khi[bf][n][ks * 16 + hb * 8]);
            const bf16x8 al = __builtin_bit_cast(bf16x8, *(const uint4 *)&klo[bf][n][ks * 16 + hb * 8]);
            const bf16x8 bh8 = __builtin_bit_cast(bf16x8, qh[ks]);
            const bf16x8 bl8 = __builtin_bit_cast(bf16x8, ql[ks]);
            f32x16 &acc = (ks & 1) ? sb : sa;
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh8, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl8, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh8, acc, 0, 0, 0);
        }
        return sa + sb;
    };
    // mask (this lane's query; keys w0 + 8(rr/4) + 4hb + rr%4) and the
    // running maximum.  Tiles wholly before every query of the wave and
    // inside the window need no mask.
    auto mask_max = [&](const f32x16 &st, int64_t w0, float (&x)[16]) {
        const int w0i = (int)w0, posi = (int)pos, Wi = (int)Wbh;
        const bool whole = w0i + kKT <= Wi && w0i + kKT - 1 <= posi;
        if (__builtin_amdgcn_read_exec() == __ballot(whole)) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) x[rr] = st[rr];
        } else {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int w = w0i + 8 * (rr >> 2) + 4 * hb + (rr & 3);
                x[rr] = (w < Wi && w <= posi) ? st[rr] : -INFINITY;
            }
        }
        float mt = x[0];
#pragma unroll
        for (int rr = 1; rr < 16; ++rr) mt = fmaxf(mt, x[rr]);
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        // lazy rescale: weights are taken against m_run until some query's
        // maximum exceeds it by more than 2^kLazy (weights stay below 2^kLazy,
        // far from fp32 and bf16 overflow)
        const float m_new = fmaxf(m_run, mt);
        if (__ballot(m_new > m_run + kLazy)) {
            const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) o[t][rr] *= alpha;
            m_run = m_new;
        }
    };
    // weights, their sum, and the B fragments of P^T: k-step s covers keys 16s ..
    // 16s+15; this lane (kb = hb) needs keys 16s + 8hb + e; a lane holds keys
    // 8a + 4hb + c.  P is rounded to bf16 first (packed pairs), then
    // v_permlane32_swap of (keys 8(2s) + 4hb .., keys 8(2s+1) + 4hb ..) leaves
    // keys 16s + e in the first register and 16s + 8 + e in the second on
    // both halves.
    auto weights = [&](const float (&x)[16], uint4 (&pb)[2]) {
        // a query that has seen no key yet has m_run = -inf and every x = -inf:
        // its weights are exp2(-inf - 0) = 0
        const float mu = m_run == -INFINITY ? 0.f : m_run;
        float p[16];
        float lt = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            p[rr] = __builtin_amdgcn_exp2f(x[rr] - mu);
            lt += p[rr];
        }
        lt += __shfl_xor(lt, 32);
        l_run += lt;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint32_t e0 = pack_bf16(p[8 * s], p[8 * s + 1]);
            const uint32_t e1 = pack_bf16(p[8 * s + 2], p[8 * s + 3]);
            const uint32_t o0 = pack_bf16(p[8 * s + 4], p[8 * s + 5]);
            const uint32_t o1 = pack_bf16(p[8 * s + 6], p[8 * s + 7]);
            const auto x0 = __builtin_amdgcn_permlane32_swap(e0, o0, false, false);
            const auto x1 = __builtin_amdgcn_permlane32_swap(e1, o1, false, false);
            pb[s] = make_uint4(x0[0], x1[0], x0[1], x1[1]);
        }
    };
    // O^T (channels x queries) += V^T (channels x keys) P^T (keys x queries)
    auto accumulate = [&](int bf, const uint4 (&pb)[2]) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const bf16x8 av = __builtin_bit_cast(bf16x8, *(const uint4 *)&vt[bf][t * 32 + n][s * 16 + hb * 8]);
                o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, pb[s]),
                                                               o[t], 0, 0, 0);
            }
    };

    if (kCache) __syncthreads();        // ssel visible before the first row lookup
    if (NB == 3) {
        // Software pipeline over three tile buffers: while tile it's softmax
        // runs on the VALU, the logits of tile it+1 are on the MFMA pipe, and
        // tile it+2 is staged into the buffer tile it-1 used.  Staging and the
        // logits past the split's last tile run on clamped rows whose results
        // are never used, so the loop body has no branch around them.  One
        // barrier per tile: buffer (it+2)%3 was last read by tile it-1's
        // O update, before the previous barrier.
        //
        // Waves w and w+4 share a SIMD; they take the phases of an iteration
        // in opposite order (ping-pong) so that one wave's MFMA work overlaps
        // the other's VALU work: waves 0-3 multiply first and stage last,
        // waves 4-7 stage first (from registers loaded one iteration earlier)
        // and multiply last.
        const bool lead = wave < 4;
        Stage sa;
        if (it1 > it0) {
            load_tile(sa, it0 * kKT);
            store_tile(sa, 0);
            load_tile(sa, (it0 + 1) * kKT);
            store_tile(sa, 1);
        }
        if (!lead) load_tile(sa, (it0 + 2) * kKT);
        __syncthreads();
        f32x16 st = logits(0);
        int bcur = 0;
        for (int64_t it = it0; it < it1; ++it) {
            const int bnext = bcur == 2 ? 0 : bcur + 1;
            const int bfill = bnext == 2 ? 0 : bnext + 1;
            float x[16];
            uint4 pb[2];
            if (lead) {
                load_tile(sa, (it + 2) * kKT);
                mask_max(st, it * kKT, x);
                st = logits(bnext);
                weights(x, pb);
                accumulate(bcur, pb);
                store_tile(sa, bfill);
            } else {
                store_tile(sa, bfill);
                load_tile(sa, (it + 3) * kKT);
                mask_max(st, it * kKT, x);
                weights(x, pb);
                st = logits(bnext);
                accumulate(bcur, pb);
            }
            __syncthreads();
            bcur = bnext;
        }
    } else {
        // one buffer: every wave has read it before it is refilled
        Stage sa;
        if (it1 > it0) {
            load_tile(sa, it0 * kKT);
            store_tile(sa, 0);
        }
        __syncthreads();
        for (int64_t it = it0; it < it1; ++it) {
            const bool more = it + 1 < it1;
            if (more) load_tile(sa, (it + 1) * kKT);
            const f32x16 st = logits(0);
            float x[16];
            mask_max(st, it * kKT, x);
            uint4 pb[2];
            weights(x, pb);
            accumulate(0, pb);
            __syncthreads();
            if (more) store_tile(sa, 0);
            __syncthreads();
        }
    }

    if (a.n_split > 1) {
        // unnormalised partial of this split, valid rows only
        if (valid_q) {
            const int64_t prow = ((int64_t)unit * a.n_split + sp) * RW + wave * 32 + n;
            float *po = a.part_o + prow * kD;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int aa = 0; aa < 4; ++aa) {
                    const int c = t * 32 + 8 * aa + 4 * hb;
                    *(float4 *)(po + c) = make_float4(o[t][4 * aa], o[t][4 * aa + 1], o[t][4 * aa + 2],
                                                      o[t][4 * aa + 3]);
                }
            if (hb == 0) a.part_ml[prow] = make_float2(m_run, l_run);
        }
        return;
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

// Merge of the key-tile splits: one thread per (query row, 4 channels), 8 rows
// per workgroup; weights 2^(m_s - M) as in the online softmax.
constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void k_attend_merge(MAttnArgs a) {
    const int tid = threadIdx.x;
    const int rows = a.QR < a.rw ? a.QR : a.rw;             // rows a unit can hold
    const int per_unit = (rows + 7) / 8;
    const int unit = blockIdx.x / per_unit;
    const int r = (blockIdx.x % per_unit) * 8 + tid / 32;   // row within the workgroup's rw
    const int cq = tid % 32;
    const int rg = unit % a.n_rg, bh = unit / a.n_rg;
    const int b = bh / a.Hkv, h = bh % a.Hkv;
    const int rr = rg * a.rw + r;
    if (r >= a.rw || rr >= a.QR) return;
    float M = -INFINITY, L = 0.f;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
    constexpr int kBatch = 8;                   // partials loaded together
    for (int s0 = 0; s0 < a.n_split; s0 += kBatch) {
        float2 ml[kBatch];
        float4 x[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int s = s0 + u < a.n_split ? s0 + u : s0;
            const int64_t prow = ((int64_t)unit * a.n_split + s) * a.rw + r;
            ml[u] = a.part_ml[prow];
            x[u] = *(const float4 *)(a.part_o + prow * kD + cq * 4);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (s0 + u >= a.n_split) break;
            const float mn = fmaxf(M, ml[u].x);
            if (mn == -INFINITY) continue;
            const float f = __builtin_amdgcn_exp2f(M - mn), fo = __builtin_amdgcn_exp2f(ml[u].x - mn);
            L = L * f + ml[u].y * fo;
            A.x = A.x * f + x[u].x * fo;
            A.y = A.y * f + x[u].y * fo;
            A.z = A.z * f + x[u].z * fo;
            A.w = A.w * f + x[u].w * fo;
            M = mn;
        }
    }
    const float inv = 1.f / L;
    const int64_t qi = (int64_t)b * a.block_q + rr / a.g;
    const int hq = h * a.g + rr % a.g;
    *(float4 *)(a.out + (qi * a.Hq + hq) * kD + cq * 4) =
        make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
}

// (cos, sin) of w * theta_c for every window position w < W_cap and channel
// pair c: angles and their sine/cosine in fp64, rounded once to fp32.
struct RopeArgs {
    float2 *rope;
    int64_t n;
    int half;
    double inv_freq[kMaxHalfDim];
};

__global__ __launch_bounds__(256) void k_rope_table(RopeArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.n) return;
    const int64_t w = i / a.half;
    const int c = (int)(i % a.half);
    double sn, cs;
    sincos((double)w * a.inv_freq[c], &sn, &cs);
    a.rope[i] = make_float2((float)cs, (float)sn);
}

}  // namespace

bool mfma_attend_path(const Geom &g) {
    return g.dtype == 0 && g.d == kD && g.block_q * g.g >= 32;
}

namespace {

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Cache-source attention: 2-wave workgroups for at most 64 query rows per
// (block, head), else 8-wave workgroups of 256 rows.
int cache_waves(const Geom &g) { return g.block_q * g.g <= 64 ? 2 : 8; }

int64_t attend_units(const Geom &g) {
    const int QR = g.block_q * g.g, rw = 32 * cache_waves(g);
    return (int64_t)g.n_blk * g.Hkv * ((QR + rw - 1) / rw);
}

// Key-tile splits.  8 waves: enough workgroups for every CU (one 512-thread
// workgroup per CU), at least 8 key tiles per split.  2 waves: at most
// kSmallTiles tiles per split, and about 1024 workgroups when the window
// allows (at least 2 tiles per split).
int attend_splits(const Geom &g) {
    const int64_t units = attend_units(g);
    const int64_t tiles = (g.W_cap + kKT - 1) / kKT;
    if (cache_waves(g) == 8) {
        if (units >= 256) return 1;
        int64_t ns = (256 + units - 1) / units;
        const int64_t by_tiles = tiles / 8 > 1 ? tiles / 8 : 1;
        if (ns > by_tiles) ns = by_tiles;
        if (ns > 16) ns = 16;
        return (int)ns;
    }
    const int64_t least = (tiles + kSmallTiles - 1) / kSmallTiles;
    int64_t want = (1024 + units - 1) / units;
    const int64_t most = (tiles + 1) / 2;
    if (want > most) want = most;
    const int64_t ns = want > least ? want : least;
    return (int)(ns > 0 ? ns : 1);
}

size_t rope_bytes(const Geom &g) { return (size_t)g.W_cap * (g.d / 2) * sizeof(float2); }

}  // namespace

// Decode-sized groups (at most 8 query rows) stay on the fused VALU kernel,
// which measured faster there; 9 to 64 rows take 2-wave workgroups, more take
// 8-wave ones (which stage the whole selection: at most kSelCap entries).
bool mfma_cache_attend_path(const Geom &g) {
    if (g.dtype != 0 || g.d != kD) return false;
    const int QR = g.block_q * g.g;
    if (QR <= 8) return false;
    return QR <= 64 || g.topk <= kSelCap;
}

size_t rope_table_bytes(const Geom &g) {
    size_t b = al256(rope_bytes(g));
    const int ns = attend_splits(g);
    if (ns > 1) {
        const size_t rows = (size_t)attend_units(g) * ns * 32 * cache_waves(g);
        b += al256(rows * kD * sizeof(float)) + al256(rows * sizeof(float2));
    }
    return b;
}

hipError_t launch_attend_mfma(const Geom &g, const float *q_rot, const float *k_win,
                              const void *v_win, const int32_t *W, int64_t W_cap, float *out,
                              hipStream_t s) {
    MAttnArgs a{};
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
    a.rep = g.rep;
    a.n_q = g.n_q;
    a.block_q = g.block_q;
    a.n_rg = (a.QR + kRowsWG - 1) / kRowsWG;
    a.scale_log2 = (float)((double)g.scale * 1.4426950408889634074);
    a.n_split = 1;
    a.rw = kRowsWG;
    hipLaunchKernelGGL((k_attend_mfma<false, 8>), dim3(g.n_blk * g.Hkv * a.n_rg), dim3(kAThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attend_mfma_cache(const Geom &g, const void *q, const void *k, const void *v,
                                    const int32_t *sel, const int32_t *n_sel, float *out,
                                    void *ws, hipStream_t s, bool table_ready) {
    float2 *rope = (float2 *)ws;
    hipError_t e = hipSuccess;
    if (!table_ready) {
        RopeArgs ra;
        ra.rope = rope;
        ra.n = g.W_cap * (g.d / 2);
        ra.half = g.d / 2;
        for (int c = 0; c < kMaxHalfDim; ++c)
            ra.inv_freq[c] = c < g.d / 2 ? pow(g.theta, -2.0 * (double)c / (double)g.d) : 0.0;
        hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((ra.n + 255) / 256)), dim3(256), 0, s, ra);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    MAttnArgs a{};
    a.q = (const uint16_t *)q;
    a.k = (const uint16_t *)k;
    a.v = (const uint16_t *)v;
    a.sel = sel;
    a.n_sel = n_sel;
    a.rope = rope;
    a.sh = g.sh;
    a.st = g.st;
    a.T = g.T;
    a.Gp = g.Gp;
    a.Lp = g.Lp;
    a.mid_lo = g.mid_lo;
    a.n_spans = g.n_spans;
    a.S = g.S;
    a.last_len = g.last_len;
    a.topk = g.topk;
    a.out = out;
    a.W_cap = g.W_cap;
    a.QR = g.block_q * g.g;
    a.Hq = g.Hq;
    a.Hkv = g.Hkv;
    a.g = g.g;
    a.rep = g.rep;
    a.n_q = g.n_q;
    a.block_q = g.block_q;
    const int nw = cache_waves(g);
    a.rw = 32 * nw;
    a.n_rg = (a.QR + a.rw - 1) / a.rw;
    a.scale_log2 = (float)((double)g.scale * 1.4426950408889634074);
    a.lens = g.lens;
    a.hps = g.hps;
    a.G = g.G;
    a.L = g.L;
    a.seq_stride = g.seq_stride;
    a.n_split = attend_splits(g);
    const int64_t units = (int64_t)g.n_blk * g.Hkv * a.n_rg;
    if (a.n_split > 1) {
        char *p = (char *)ws + al256(rope_bytes(g));
        const size_t rows = (size_t)units * a.n_split * a.rw;
        a.part_o = (float *)p;
        a.part_ml = (float2 *)(p + al256(rows * kD * sizeof(float)));
    }
    if (nw == 2)
        hipLaunchKernelGGL((k_attend_mfma<true, 2>), dim3((unsigned)(units * a.n_split)), dim3(128),
                           0, s, a);
    else
        hipLaunchKernelGGL((k_attend_mfma<true, 8>), dim3((unsigned)(units * a.n_split)),
                           dim3(kAThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess || a.n_split == 1) return e;
    const int rows = a.QR < a.rw ? a.QR : a.rw;
    hipLaunchKernelGGL(k_attend_merge, dim3((unsigned)(units * ((rows + 7) / 8))),
                       dim3(kMergeThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace rea
