// score.hip - step 1a: position-agnostic token scoring with span max-reduce.
//
// For KV head h, the middle cache [G', T-L') is cut into spans of S tokens.
// The score of token t for query i is the dot product of the UN-rotated query
// with the PRE-RoPE key, summed over the query heads of h's GQA group
// (ReAttention research-map summary, "Approach": segments are chosen by the
// query/un-positioned-key dot product; OpenReview discussion, "Decoding Phase"
// pseudocode: score = query @ key[G:-L]^T).  A span's score is the maximum of
// its token scores; a block of queries sums its queries' maxima.  Token scores
// are never written out: only span scores leave the kernel, together with the
// maximum of every group of 32 consecutive spans (used by the top-k step) and,
// from the decode scorer, each group's second and third largest and the spans
// holding its top two (so the top-k need not read most groups' spans).
//
// Arithmetic: the group-summed query is formed in fp64 (exact for bf16 and,
// in practice, fp32 inputs), every product with a bf16/fp32 key element is
// exact in fp64, and sums are fp64, so span scores agree with the exact ones
// to ~1e-16 relative (for ordinary bf16 data the sums are exact).
//
// Memory (decode): the whole middle K is streamed once (2.14 GB per layer at
// 1M tokens, d=128, 8 KV heads).  A key row is read by the lanes of one DPP
// row (16 lanes x 16 B for d=128 bf16), so one load instruction reads whole
// rows, contiguous; loads are non-temporal (the cache is touched once); up to
// 32 rows per wave are loaded before any arithmetic.  Partial dot products
// are summed across a row's lanes with DPP quad-permute and mirror moves
// (symmetric pairings, so every lane of a row ends with identical bits); for
// bf16 rows of 128 elements the two halves of the 16 lanes load different
// rows in each instruction, which halves those moves (kPairRows).  Each
// workgroup owns a contiguous run of 32-span groups of one (block, KV head);
// its four waves take adjacent spans, so the workgroup reads 32 KB
// contiguous per step.  About two workgroups per compute unit run: more
// concurrent streams lowered measured bandwidth.
//
// Variants: one selection per query head (every query head of a KV head's
// group scored from one read of each key row), token-level selection (S = 1,
// one 32-token group per wave), and blocks of several queries on the VALU.
#include "rea_internal.h"

#include <math.h>

namespace rea {
namespace {

constexpr int kThreads = 256;   // 4 waves
constexpr int kWaves = kThreads / 64;
constexpr int kGroup = 32;      // spans per group maximum

struct ScoreArgs {
    const void *q;
    const unsigned char *k;
    double *out;                // [n_blk][Hkv][n_spans]
    double *gmax;               // [n_blk][Hkv][n_groups]
    // k_score_tokens: null, or the second largest score of every group (a
    // tied maximum counts twice) and the offset of a maximum in the group
    double *gsec;               // [n_blk][Hkv][n_groups]
    int32_t *garg;              // [n_blk][Hkv][n_groups]
    int64_t sh_bytes, st_bytes;
    int64_t mid_lo, mid_hi, n_spans, n_groups;   // n_spans, n_groups: also the row strides
    int S, Hq, Hkv, g, block_q, P, rep;
    // batched decode (see Geom): per-sequence lengths and cache offsets
    const int64_t *lens;
    int hps, G, L;
    int64_t T, seq_stride_bytes;
    // null, or one flag per (block, selection head): k_score_block and the
    // per-query-head decode scorers score only the flagged pairs (the exact
    // fallback of the MFMA paths)
    const uint32_t *only;
    // null, or (k_score_decode) per group the second and third largest span
    // scores [n_groups][2] and the spans holding the largest and the second
    // largest [n_groups][2] (a tied score counts again)
    double *gtop;
    int32_t *gtopi;
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt(const void *p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ double load_f64(const uint16_t *p, int64_t i) {
    return (double)__uint_as_float(((uint32_t)p[i]) << 16);
}
__device__ __forceinline__ double load_f64(const float *p, int64_t i) { return (double)p[i]; }

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

// v + (v from the lane chosen by DPP control CTRL), on the two halves of a double
template <int CTRL> __device__ __forceinline__ double dpp_add(double v) {
    const int2 x = *reinterpret_cast<const int2 *>(&v);
    int2 y;
    y.x = __builtin_amdgcn_mov_dpp(x.x, CTRL, 0xF, 0xF, false);
    y.y = __builtin_amdgcn_mov_dpp(x.y, CTRL, 0xF, 0xF, false);
    return v + *reinterpret_cast<const double *>(&y);
}

// a + (b from the lane chosen by DPP control CTRL), on the two halves of a double
template <int CTRL> __device__ __forceinline__ double dpp_add2(double a, double b) {
    const int2 x = *reinterpret_cast<const int2 *>(&b);
    int2 y;
    y.x = __builtin_amdgcn_mov_dpp(x.x, CTRL, 0xF, 0xF, false);
    y.y = __builtin_amdgcn_mov_dpp(x.y, CTRL, 0xF, 0xF, false);
    return a + *reinterpret_cast<const double *>(&y);
}

// The decode scorer's paired-row layout: bf16 rows of 128 elements (16 lanes of
// 16 bytes), 8 load instructions (32 rows) per batch.
template <typename TIn, int D, int R>
constexpr bool kPairRows = sizeof(TIn) == 2 && D == 128 && R == 8;

// Sum over the LPR consecutive lanes that share a key row.  Every step pairs
// lanes symmetrically: quad-permute xor 1, xor 2, half-row mirror, row mirror.
template <int LPR> __device__ __forceinline__ double row_sum(double v) {
    v = dpp_add<0xB1>(v);
    v = dpp_add<0x4E>(v);
    if (LPR >= 8) v = dpp_add<0x141>(v);
    if (LPR >= 16) v = dpp_add<0x140>(v);
    if (LPR >= 32) v += __shfl_xor(v, 16);
    return v;
}

// Max over the rows of a wave (lanes LPR apart).
template <int LPR> __device__ __forceinline__ double rows_max(double v) {
    for (int o = LPR; o < 64; o <<= 1) v = fmax(v, __shfl_xor(v, o));
    return v;
}

// Group bookkeeping shared by both kernels: the workgroup's group range and
// the per-group maximum across its waves (double-buffered by group parity).
struct GroupRange {
    int64_t g0, g1;
};
__device__ __forceinline__ GroupRange group_range(const ScoreArgs &a, int p, int64_t n_groups) {
    const int64_t g1 = (int64_t)(p + 1) * a.n_groups / a.P;
    return {(int64_t)p * a.n_groups / a.P, g1 < n_groups ? g1 : n_groups};
}

// The regions of the sequence that selection head hs belongs to, and the
// byte offset of its KV head in the cache.
struct Unit {
    SeqGeom sg;
    int64_t kv_off;
};
__device__ __forceinline__ Unit unit_of(const ScoreArgs &a, int hs) {
    const SeqOf so = seq_of(a.lens, hs, a.hps, a.rep, a.seq_stride_bytes, a.sh_bytes, a.T);
    return {seq_geom(so.T, a.G, a.L, a.S), so.kv_off};
}

__device__ __forceinline__ void publish_group_max(const ScoreArgs &a, double (&slot)[2][kWaves],
                                                  int64_t bh, int64_t grp, double wave_best) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) slot[grp & 1][wave] = wave_best;
    __syncthreads();
    if (threadIdx.x == 0) {
        double m = slot[grp & 1][0];
        for (int w = 1; w < kWaves; ++w) m = fmax(m, slot[grp & 1][w]);
        a.gmax[bh * a.n_groups + grp] = m;
    }
}

// The three largest span scores of a wave's spans in a group, with the spans
// of the first two; a score equal to one held counts again.
struct Top3 {
    double v1, v2, v3;
    int32_t i1, i2;
    __device__ void init() {
        v1 = v2 = v3 = -INFINITY;
        i1 = i2 = -1;
    }
    __device__ void add(double v, int32_t j) {
        if (v > v1) {
            v3 = v2;
            v2 = v1;
            i2 = i1;
            v1 = v;
            i1 = j;
        } else if (v > v2) {
            v3 = v2;
            v2 = v;
            i2 = j;
        } else if (v > v3) {
            v3 = v;
        }
    }
};

// Group maximum and the group's top three (a.gtop set).  The waves' lists go
// to LDS; after the barrier twelve lanes of one wave (a different one for
// each group, so no wave is held back every time) take the twelve entries,
// rank each against the others (value descending, then list position: a
// wave's third value, which has no span, ranks after its first two) and the
// lanes ranked 0-2 write the results.
__device__ __forceinline__ void publish_group_top(const ScoreArgs &a, double (&slot)[2][kWaves],
                                                  double (&tv)[2][kWaves][2], int32_t (&ti)[2][kWaves][2],
                                                  int64_t bh, int64_t grp, const Top3 &w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pb = (int)(grp & 1);
    if (lane == 0) {
        slot[pb][wave] = w.v1;
        tv[pb][wave][0] = w.v2;
        tv[pb][wave][1] = w.v3;
        ti[pb][wave][0] = w.i1;
        ti[pb][wave][1] = w.i2;
    }
    __syncthreads();
    if (wave == (int)(grp & (kWaves - 1)) && lane < 3 * kWaves) {
        double e[3 * kWaves];
#pragma unroll
        for (int q = 0; q < kWaves; ++q) {
            e[3 * q] = slot[pb][q];
            e[3 * q + 1] = tv[pb][q][0];
            e[3 * q + 2] = tv[pb][q][1];
        }
        const int q = lane / 3, k = lane % 3;
        const double v = k == 0 ? slot[pb][q] : tv[pb][q][k - 1];
        uint32_t rank = 0;
#pragma unroll
        for (int o = 0; o < 3 * kWaves; ++o) rank += (uint32_t)(e[o] > v) | ((uint32_t)(e[o] == v) & (uint32_t)(o < lane));
        const int64_t og = bh * a.n_groups + grp;
        if (rank == 0) {
            a.gmax[og] = v;
            a.gtopi[2 * og] = ti[pb][q][k < 2 ? k : 1];
        } else if (rank == 1) {
            a.gtop[2 * og] = v;
            a.gtopi[2 * og + 1] = ti[pb][q][k < 2 ? k : 1];
        } else if (rank == 2) {
            a.gtop[2 * og + 1] = v;
        }
    }
}

// Decode: one query per block; the group-summed query lives in registers.
// R = load instructions per batch (each instruction covers RPI rows).
template <typename TIn, int D, int R>
__global__ __launch_bounds__(kThreads) void k_score_decode(ScoreArgs a) {
    constexpr int ESZ = sizeof(TIn);
    constexpr int LPR = D * ESZ / 16;          // lanes per key row
    constexpr int RPI = 64 / LPR;              // rows per load instruction
    constexpr int EPL = 16 / ESZ;              // elements per lane
    __shared__ double slot[2][kWaves];
    __shared__ double tv[2][kWaves][2];
    __shared__ int32_t ti[2][kWaves][2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rs = lane / LPR, ch = lane % LPR;
    const int bh = blockIdx.x / a.P, p = blockIdx.x % a.P;
    const int b = bh / a.Hkv, h = bh % a.Hkv;

    double qr[EPL];
    {
        const TIn *qb = (const TIn *)a.q + (int64_t)b * a.Hq * D + (int64_t)h * a.g * D;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            double s = 0.0;
            for (int gg = 0; gg < a.g; ++gg) s += load_f64(qb, (int64_t)gg * D + ch * EPL + e);
            qr[e] = s;
        }
    }

    const Unit un = unit_of(a, h);
    const unsigned char *kh = a.k + un.kv_off + ch * 16;
    const GroupRange gr = group_range(a, p, un.sg.n_groups);
    for (int64_t grp = gr.g0; grp < gr.g1; ++grp) {
        const int64_t jend = min((grp + 1) * kGroup, un.sg.n_spans);
        double gbest = -INFINITY;
        Top3 top;
        top.init();
        for (int64_t j = grp * kGroup + wave; j < jend; j += kWaves) {
            const int64_t tb = un.sg.mid_lo + j * a.S;
            const int64_t te = min(tb + (int64_t)a.S, un.sg.mid_hi);
            double best = -INFINITY;
            if constexpr (kPairRows<TIn, D, R>) {
                // instruction r of a batch: lanes of the row's first half
                // (chunks 0-7) load row 4r + rs, lanes of the second half row
                // 4(r ^ 4) + rs (every instruction still reads whole 128-byte
                // half rows), so one mirror step turns the partial sums of
                // instructions r and r + 4 into two rows' sums over a half
                // each, and three steps within 8 lanes finish them
                const int hb = (lane >> 3) & 1;
                for (int64_t r0 = tb; r0 < te; r0 += (int64_t)R * RPI) {
                    uint4 buf[R];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const int64_t t = r0 + (r ^ (hb * 4)) * RPI + rs;
                        buf[r] = t < te ? load_nt(kh + t * a.st_bytes) : make_uint4(0u, 0u, 0u, 0u);
                    }
                    double acc[R];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        double x[EPL];
                        unpack(buf[r], x);
                        double v = 0.0;
#pragma unroll
                        for (int e = 0; e < EPL; ++e) v = fma(qr[e], x[e], v);
                        acc[r] = v;
                    }
#pragma unroll
                    for (int r = 0; r < R / 2; ++r) {
                        // this lane's row: 4r + rs (first half) or 4(r + 4) + rs
                        double v = dpp_add2<0x140>(acc[r], acc[r + R / 2]);
                        v = dpp_add<0xB1>(v);
                        v = dpp_add<0x4E>(v);
                        v = dpp_add<0x141>(v);
                        const int64_t t = r0 + (r + hb * (R / 2)) * RPI + rs;
                        if (t < te) best = fmax(best, v);
                    }
                }
                // rows of a half-row group: max over the halves and the 4 row groups
                best = fmax(best, __shfl_xor(best, 8));
                best = rows_max<LPR>(best) + 0.0;       // -0 -> +0
            } else {
            for (int64_t r0 = tb; r0 < te; r0 += (int64_t)R * RPI) {
                uint4 buf[R];
                bool ok[R];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int64_t t = r0 + r * RPI + rs;
                    ok[r] = t < te;
                    buf[r] = ok[r] ? load_nt(kh + t * a.st_bytes) : make_uint4(0u, 0u, 0u, 0u);
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    double x[EPL];
                    unpack(buf[r], x);
                    double acc = 0.0;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc = fma(qr[e], x[e], acc);
                    acc = row_sum<LPR>(acc);
                    if (ok[r]) best = fmax(best, acc);
                }
            }
            best = rows_max<LPR>(best) + 0.0;       // -0 -> +0
            }
            if (lane == 0) a.out[(int64_t)bh * a.n_spans + j] = best;
            gbest = fmax(gbest, best);
            top.add(best, (int32_t)j);
        }
        if (a.gtop)
            publish_group_top(a, slot, tv, ti, bh, grp, top);
        else
            publish_group_max(a, slot, bh, grp, gbest);
    }
}

// Decode with one selection per query head: the NH query heads of a group
// share their KV head, so each key row is loaded once and scored against all
// NH queries (NH dot products per row).  The workgroup covers KV head hp; its
// selection heads are hp*NH .. hp*NH+NH-1 (rep == NH, g == 1).
template <typename TIn, int D, int R, int NH>
__global__ __launch_bounds__(kThreads) void k_score_decode_heads(ScoreArgs a) {
    constexpr int ESZ = sizeof(TIn);
    constexpr int LPR = D * ESZ / 16;
    constexpr int RPI = 64 / LPR;
    constexpr int EPL = 16 / ESZ;
    __shared__ double slot[2][NH][kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rs = lane / LPR, ch = lane % LPR;
    const int Hp = a.Hkv / NH;                   // KV heads
    const int bp = blockIdx.x / a.P, p = blockIdx.x % a.P;
    const int b = bp / Hp, hp = bp % Hp;
    const int64_t bh0 = (int64_t)b * a.Hkv + (int64_t)hp * NH;   // first selection head
    if (a.only) {
        bool any = false;
#pragma unroll
        for (int m = 0; m < NH; ++m) any |= a.only[bh0 + m] != 0;
        if (!any) return;
    }

    double qr[NH][EPL];
    {
        const TIn *qb = (const TIn *)a.q + (int64_t)b * a.Hq * D + (int64_t)hp * NH * D;
#pragma unroll
        for (int m = 0; m < NH; ++m)
#pragma unroll
            for (int e = 0; e < EPL; ++e) qr[m][e] = load_f64(qb, (int64_t)m * D + ch * EPL + e);
    }

    const Unit un = unit_of(a, hp * NH);
    const unsigned char *kh = a.k + un.kv_off + ch * 16;
    const GroupRange gr = group_range(a, p, un.sg.n_groups);
    for (int64_t grp = gr.g0; grp < gr.g1; ++grp) {
        const int64_t jend = min((grp + 1) * kGroup, un.sg.n_spans);
        double gbest[NH];
#pragma unroll
        for (int m = 0; m < NH; ++m) gbest[m] = -INFINITY;
        for (int64_t j = grp * kGroup + wave; j < jend; j += kWaves) {
            const int64_t tb = un.sg.mid_lo + j * a.S;
            const int64_t te = min(tb + (int64_t)a.S, un.sg.mid_hi);
            double best[NH];
#pragma unroll
            for (int m = 0; m < NH; ++m) best[m] = -INFINITY;
            for (int64_t r0 = tb; r0 < te; r0 += (int64_t)R * RPI) {
                uint4 buf[R];
                bool ok[R];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int64_t t = r0 + r * RPI + rs;
                    ok[r] = t < te;
                    buf[r] = ok[r] ? load_nt(kh + t * a.st_bytes) : make_uint4(0u, 0u, 0u, 0u);
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    double x[EPL];
                    unpack(buf[r], x);
#pragma unroll
                    for (int m = 0; m < NH; ++m) {
                        double acc = 0.0;
#pragma unroll
                        for (int e = 0; e < EPL; ++e) acc = fma(qr[m][e], x[e], acc);
                        acc = row_sum<LPR>(acc);
                        if (ok[r]) best[m] = fmax(best[m], acc);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < NH; ++m) {
                const double v = rows_max<LPR>(best[m]) + 0.0;       // -0 -> +0
                if (lane == 0) a.out[(bh0 + m) * a.n_spans + j] = v;
                gbest[m] = fmax(gbest[m], v);
            }
        }
        if (lane == 0) {
#pragma unroll
            for (int m = 0; m < NH; ++m) slot[grp & 1][m][wave] = gbest[m];
        }
        __syncthreads();
        if (threadIdx.x < NH) {
            const int m = threadIdx.x;
            double v = slot[grp & 1][m][0];
            for (int w = 1; w < kWaves; ++w) v = fmax(v, slot[grp & 1][m][w]);
            a.gmax[(bh0 + m) * a.n_groups + grp] = v;
        }
    }
}

// DPP move of a double (both halves), for sums of two different registers.
template <int CTRL> __device__ __forceinline__ double dpp_mov(double v) {
    const int2 x = *reinterpret_cast<const int2 *>(&v);
    int2 y;
    y.x = __builtin_amdgcn_mov_dpp(x.x, CTRL, 0xF, 0xF, false);
    y.y = __builtin_amdgcn_mov_dpp(x.y, CTRL, 0xF, 0xF, false);
    return *reinterpret_cast<const double *>(&y);
}

// Head whose full row sum lane c (0..7 within its row) ends with after the
// reduce-scatter of k_score_heads_lds.
template <int NH> __device__ __forceinline__ int heads8_final(int c) {
    return NH == 4 ? 2 * ((c >> 2) & 1) + (c & 1) : ((c >> 2) & 1);
}

// s_waitcnt vmcnt(n) for even n <= 14 (expcnt and lgkmcnt not waited for)
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0xF70); break;
    case 2: __builtin_amdgcn_s_waitcnt(0xF72); break;
    case 4: __builtin_amdgcn_s_waitcnt(0xF74); break;
    case 6: __builtin_amdgcn_s_waitcnt(0xF76); break;
    case 8: __builtin_amdgcn_s_waitcnt(0xF78); break;
    case 10: __builtin_amdgcn_s_waitcnt(0xF7A); break;
    case 12: __builtin_amdgcn_s_waitcnt(0xF7C); break;
    default: __builtin_amdgcn_s_waitcnt(0xF7E); break;
    }
}

typedef unsigned int lds_u32x4 __attribute__((ext_vector_type(4)));

// Two 16-byte LDS reads completed (lgkmcnt(0)) inside one asm block, so that
// the compiler does not make them wait for the DMA still in flight to other
// ring slots (the slot read here is complete by an explicit vmcnt wait).
__device__ __forceinline__ void lds_read2(uint32_t a0, uint32_t a1, uint4 &o0, uint4 &o1) {
    lds_u32x4 r0, r1;
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1)
        : "v"(a0), "v"(a1)
        : "memory");
    o0 = make_uint4(r0.x, r0.y, r0.z, r0.w);
    o1 = make_uint4(r1.x, r1.y, r1.z, r1.w);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(size_t)(const void __attribute__((address_space(3))) *)p;
}

// Per-query-head decode for 256-byte key rows (bf16 d 128, fp32 d 64) and
// NH = 2 or 4 query heads per KV head.
//
// Arithmetic: 8 lanes per row, 32 bytes each, and the NH partial dot
// products of a row are reduced with a reduce-scatter instead of NH separate
// reductions.  Step 1 pairs lanes c and c^7 (half-row mirror), step 2 c and
// c^1, step 3 c and c^2.  Each lane holds its partial sums in an order fixed
// for it, so that every step adds the partner's second half to its own first
// half with no selects: for NH = 4 the order is F(c), F(c^1), F(c^7), F(c^6),
// with F(c) = 2*bit2 + bit0 the head the lane ends with (lanes c and c^2 end
// with the same head); for NH = 2 it is F(c), F(c^7) with F(c) = bit2.  Per
// row that is 6 DPP moves of doubles and 3 adds instead of NH x 3 of each.
//
// Memory: the key rows are staged through LDS by DMA (global_load_lds), so
// that many rows are in flight without holding them in registers.  Every wave
// runs its own pipeline over whole groups of 32 spans (no barriers): a stage
// is 8 rows, moved by two 1 KB copies, the first halves of the 8 rows then
// their second halves, so that lane (row r, chunk c) reads LDS at 16 * lane in
// each half (conflict-free).  kHNB stages per wave are in flight.
constexpr int kHNB = 8;
static_assert((kHNB & (kHNB - 1)) == 0, "ring slots: a power of two");

template <typename TIn, int D, int NH>
__global__ __launch_bounds__(kThreads, 2) void k_score_heads_lds(ScoreArgs a) {
    constexpr int ESZ = sizeof(TIn);
    static_assert(D * ESZ == 256, "256-byte key rows");
    static_assert(NH == 2 || NH == 4, "two or four heads");
    constexpr int EPL = 16 / ESZ;
    __shared__ __align__(16) unsigned char ring[kWaves][kHNB][2048];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int rs = lane >> 3, c = lane & 7;
    const int Hp = a.Hkv / NH;
    const int bp = blockIdx.x / a.P, p = blockIdx.x % a.P;
    const int b = bp / Hp, hp = bp % Hp;
    const int64_t bh0 = (int64_t)b * a.Hkv + (int64_t)hp * NH;
    if (a.only) {
        bool any = false;
#pragma unroll
        for (int m = 0; m < NH; ++m) any |= a.only[bh0 + m] != 0;
        if (!any) return;
    }

    int order[NH];
    if (NH == 4) {
        order[0] = heads8_final<NH>(c);
        order[1] = heads8_final<NH>(c ^ 1);
        order[2] = heads8_final<NH>(c ^ 7);
        order[3] = heads8_final<NH>(c ^ 6);
    } else {
        order[0] = heads8_final<NH>(c);
        order[1] = heads8_final<NH>(c ^ 7);
    }
    double qr[NH][2 * EPL];
    {
        const TIn *qb = (const TIn *)a.q + (int64_t)b * a.Hq * D + (int64_t)hp * NH * D;
#pragma unroll
        for (int o = 0; o < NH; ++o)
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                qr[o][e] = load_f64(qb, (int64_t)order[o] * D + c * EPL + e);
                qr[o][EPL + e] = load_f64(qb, (int64_t)order[o] * D + D / 2 + c * EPL + e);
            }
    }
    __builtin_amdgcn_s_waitcnt(0xF70);              // queries in registers before the ring starts
    const int mine = heads8_final<NH>(c);
    const bool writer = rs == 0 && ((c & 2) == 0) && (NH == 4 || (c & 1) == 0);

    // this wave's groups: g0 + wave, g0 + wave + 4, ...; stages: (span, sub)
    const Unit un = unit_of(a, hp * NH);
    const GroupRange gr = group_range(a, p, un.sg.n_groups);
    const int64_t first = gr.g0 + wave;
    const int64_t n_grp = first < gr.g1 ? (gr.g1 - first + kWaves - 1) / kWaves : 0;
    if (n_grp == 0) return;
    const int64_t last_grp = first + (n_grp - 1) * kWaves;
    const int64_t n_spans_w = (n_grp - 1) * kGroup + min((int64_t)kGroup, un.sg.n_spans - last_grp * kGroup);
    const int sps = (a.S + 7) / 8;                   // stages per span
    const int64_t n_st = n_spans_w * sps;

    const unsigned char *kh = a.k + un.kv_off;
    const uint32_t ring_w = lds_addr(&ring[wave][0][0]);
    // Stage cursors (issue side and consume side) advance incrementally: sub
    // stage within the span, span within the group, group (stride kWaves).
    struct Cursor {
        int sub, sig;
        int64_t grp, j, tb, te;
    };
    auto start = [&](Cursor &u) {
        u.sub = 0;
        u.sig = 0;
        u.grp = first;
        u.j = first * kGroup;
        u.tb = un.sg.mid_lo + u.j * a.S;
        u.te = min(u.tb + (int64_t)a.S, un.sg.mid_hi);
    };
    auto advance = [&](Cursor &u) {
        if (++u.sub < sps) return;
        u.sub = 0;
        if (++u.sig == kGroup) {
            u.sig = 0;
            u.grp += kWaves;
            u.j = u.grp * kGroup;
        } else {
            ++u.j;
        }
        u.tb = un.sg.mid_lo + u.j * a.S;
        u.te = min(u.tb + (int64_t)a.S, un.sg.mid_hi);
    };
    Cursor iss, con;
    start(iss);
    start(con);
    int64_t is = 0;                                  // stages issued
    auto issue_next = [&]() {
        if (is >= n_st) return;
        int64_t t = iss.tb + iss.sub * 8 + (lane >> 3);
        if (t >= iss.te) t = iss.tb;                 // masked when consumed
        const unsigned char *src = kh + t * a.st_bytes + (lane & 7) * 16;
        unsigned char *dst = &ring[wave][is & (kHNB - 1)][0];
        __builtin_amdgcn_global_load_lds((const void *)src,
                                         (void __attribute__((address_space(3))) *)dst, 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)(src + 128),
                                         (void __attribute__((address_space(3))) *)(dst + 1024),
                                         16, 0, 0);
        ++is;
        advance(iss);
    };
    for (int i = 0; i < kHNB - 1; ++i) issue_next();

    double best = -INFINITY, gbest = -INFINITY;
    for (int64_t it = 0; it < n_st; ++it) {
        int64_t later = n_st - 1 - it;               // stages issued after this one
        if (later > kHNB - 2) later = kHNB - 2;
        wait_vmcnt(2 * (int)later);
        issue_next();                                // refills the slot read last step
        const bool ok = con.tb + con.sub * 8 + rs < con.te;

        uint4 lo, hi;
        const uint32_t sa = ring_w + (uint32_t)((it & (kHNB - 1)) * 2048) + lane * 16;
        lds_read2(sa, sa + 1024, lo, hi);
        double acc[NH];
#pragma unroll
        for (int o = 0; o < NH; ++o) acc[o] = 0.0;
        double x[EPL];
        unpack(lo, x);
#pragma unroll
        for (int o = 0; o < NH; ++o)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[o] = fma(qr[o][e], x[e], acc[o]);
        unpack(hi, x);
#pragma unroll
        for (int o = 0; o < NH; ++o)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[o] = fma(qr[o][EPL + e], x[e], acc[o]);
        double v;
        if (NH == 4) {
            const double s0 = acc[0] + dpp_mov<0x141>(acc[2]);
            const double s1 = acc[1] + dpp_mov<0x141>(acc[3]);
            v = s0 + dpp_mov<0xB1>(s1);
        } else {
            v = acc[0] + dpp_mov<0x141>(acc[1]);
            v = v + dpp_mov<0xB1>(v);
        }
        v = v + dpp_mov<0x4E>(v);
        if (ok) best = fmax(best, v);
        if (con.sub == sps - 1) {                    // span complete
            best = rows_max<8>(best) + 0.0;          // -0 -> +0
            if (writer) a.out[(bh0 + mine) * a.n_spans + con.j] = best;
            gbest = fmax(gbest, best);
            best = -INFINITY;
            if (con.sig == kGroup - 1 || con.j == un.sg.n_spans - 1) {   // group complete
                if (writer) a.gmax[(bh0 + mine) * a.n_groups + con.grp] = gbest;
                gbest = -INFINITY;
            }
        }
        advance(con);
    }
}

// Token-level decode (S = 1: every middle token is its own span).  A wave
// takes one group of 32 consecutive tokens per step (all its rows loaded
// before any arithmetic) and writes their 32 scores with one store per
// selection head; the group maximum needs no exchange between waves.  NH > 1
// scores the NH query heads of a KV head from one read of each row (one
// selection per query head); NH == 1 scores selection head u with the summed
// queries of its group.  After the row sums every lane holds the scores of
// all the rows its lanes share (bf16 rows of 128 elements: paired rows, as in
// k_score_decode, so each half row holds half of them), so a group's two
// largest scores are formed in registers first and then merged across the
// half rows (DPP rotate by 8) and the row slots (permlane swaps, no LDS).
template <bool X16> __device__ __forceinline__ void swap_halves(double v, double &x, double &y) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t l = (uint32_t)u, hi = (uint32_t)(u >> 32);
    const auto lo2 = X16 ? __builtin_amdgcn_permlane16_swap(l, l, false, false)
                         : __builtin_amdgcn_permlane32_swap(l, l, false, false);
    const auto hi2 = X16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                         : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    x = __longlong_as_double((long long)(((uint64_t)hi2[0] << 32) | lo2[0]));
    y = __longlong_as_double((long long)(((uint64_t)hi2[1] << 32) | lo2[1]));
}

// (b1, b2) <- the two largest of the multiset {b1, b2, c1, c2} (a tie counts twice)
__device__ __forceinline__ void top2_merge(double &b1, double &b2, double c1, double c2) {
    b2 = fmax(fmin(b1, c1), fmax(b2, c2));
    b1 = fmax(b1, c1);
}

// Merge with lane l ^ 16 (X16) or l ^ 32: the swap returns this lane's pair and
// the partner's in either order, and the merge is symmetric in the two.
template <bool X16> __device__ __forceinline__ void top2_xlane(double &b1, double &b2) {
    double p1, q1, p2, q2;
    swap_halves<X16>(b1, p1, q1);
    swap_halves<X16>(b2, p2, q2);
    b1 = p1, b2 = p2;
    top2_merge(b1, b2, q1, q2);
}

template <typename TIn, int D, int NH>
__global__ __launch_bounds__(kThreads) void k_score_tokens(ScoreArgs a) {
    constexpr int ESZ = sizeof(TIn);
    constexpr int LPR = D * ESZ / 16;
    constexpr int RPI = 64 / LPR;
    constexpr int EPL = 16 / ESZ;
    constexpr int R = kGroup / RPI;              // load instructions per group
    constexpr bool PAIR = kPairRows<TIn, D, R>;
    constexpr int NV = PAIR ? R / 2 : R;         // token scores a lane holds
    static_assert(R <= LPR, "one lane per row slot writes the group's scores");
    static_assert(LPR >= 8 && LPR <= 32, "rows of 8 to 32 lanes");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rs = lane / LPR, ch = lane % LPR;
    // paired rows: the second half of a row's lanes holds rows NV.. of the group
    const int hb = PAIR ? (lane >> 3) & 1 : 0;
    const int c = PAIR ? ch & 7 : ch;            // writer lanes: c < NV
    const int Hu = a.Hkv / NH;
    const int bu = blockIdx.x / a.P, p = blockIdx.x % a.P;
    const int b = bu / Hu, u = bu % Hu;
    const int64_t bh0 = (int64_t)b * a.Hkv + (int64_t)u * NH;   // first selection head

    double qr[NH][EPL];
    {
        const TIn *qb = (const TIn *)a.q + (int64_t)b * a.Hq * D;
#pragma unroll
        for (int m = 0; m < NH; ++m)
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                double s = 0.0;
                for (int gg = 0; gg < a.g; ++gg)
                    s += load_f64(qb, ((int64_t)(u * NH + m) * a.g + gg) * D + ch * EPL + e);
                qr[m][e] = s;
            }
    }

    const Unit un = unit_of(a, u * NH);
    const unsigned char *kh = a.k + un.kv_off + ch * 16;
    const GroupRange gr = group_range(a, p, un.sg.n_groups);
    for (int64_t grp = gr.g0 + wave; grp < gr.g1; grp += kWaves) {
        const int64_t t0 = un.sg.mid_lo + grp * kGroup;
        // v[.][i] below is the score of token tl + i * RPI
        const int64_t tl = t0 + hb * NV * RPI + rs;
        uint4 buf[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t t = t0 + (PAIR ? (r ^ (hb * NV)) : r) * RPI + rs;
            buf[r] = t < un.sg.mid_hi ? load_nt(kh + t * a.st_bytes) : make_uint4(0u, 0u, 0u, 0u);
        }
        double acc[NH][R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            double x[EPL];
            unpack(buf[r], x);
#pragma unroll
            for (int m = 0; m < NH; ++m) {
                double s = 0.0;
#pragma unroll
                for (int e = 0; e < EPL; ++e) s = fma(qr[m][e], x[e], s);
                acc[m][r] = s;
            }
        }
        double v[NH][NV];
#pragma unroll
        for (int m = 0; m < NH; ++m)
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                if constexpr (PAIR) {
                    // instruction i of this half and i + NV of the mirrored half
                    // read the same row: one mirror step, then 8 lanes
                    double s = dpp_add2<0x140>(acc[m][i], acc[m][i + NV]);
                    s = dpp_add<0xB1>(s);
                    s = dpp_add<0x4E>(s);
                    s = dpp_add<0x141>(s);
                    v[m][i] = s + 0.0;                  // -0 -> +0
                } else {
                    v[m][i] = row_sum<LPR>(acc[m][i]) + 0.0;
                }
            }
        // lane (rs, c < NV) stores the score of token tl + c * RPI
        const int64_t tw = tl + c * RPI;
        const bool wr = c < NV && tw < un.sg.mid_hi;
#pragma unroll
        for (int m = 0; m < NH; ++m) {
            double mine = v[m][0], b1 = -INFINITY, b2 = -INFINITY;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                if (i > 0 && c == i) mine = v[m][i];
                const double x = tl + i * RPI < un.sg.mid_hi ? v[m][i] : -INFINITY;
                if (a.gsec) {
                    top2_merge(b1, b2, x, -INFINITY);
                } else {
                    b1 = fmax(b1, x);
                }
            }
            if (wr) a.out[(bh0 + m) * a.n_spans + (tw - un.sg.mid_lo)] = mine;
            if (a.gsec) {
                // lane l ^ 8 (the other half row, or with 8-lane rows the next
                // row slot), then l ^ 16 where it holds another row slot, then l ^ 32
                if constexpr (PAIR || LPR == 8)
                    top2_merge(b1, b2, dpp_mov<0x128>(b1), dpp_mov<0x128>(b2));
                if constexpr (LPR <= 16) top2_xlane<true>(b1, b2);
                top2_xlane<false>(b1, b2);
                // a lane holding the maximum: its token's offset in the group
                // (the only one when the second largest is smaller)
                const uint64_t hit = __ballot(wr && mine == b1);
                const int hl = hit ? __ffsll((long long)hit) - 1 : 0;
                if (lane == 0) {
                    const int hch = hl % LPR;
                    const int hc = PAIR ? hch & 7 : hch, hh = PAIR ? (hch >> 3) & 1 : 0;
                    a.gmax[(bh0 + m) * a.n_groups + grp] = b1 + 0.0;
                    a.gsec[(bh0 + m) * a.n_groups + grp] = b2 + 0.0;
                    a.garg[(bh0 + m) * a.n_groups + grp] = (hh * NV + hc) * RPI + hl / LPR;
                }
            } else {
                if constexpr (PAIR) b1 = fmax(b1, dpp_mov<0x128>(b1));
                b1 = rows_max<LPR>(b1);
                if (lane == 0) a.gmax[(bh0 + m) * a.n_groups + grp] = b1;
            }
        }
    }
}

// Blocks of several queries (chunked prefill on the VALU): the group-summed
// queries of the block sit in LDS; span score = sum over queries of the max.
template <typename TIn, int D>
__global__ __launch_bounds__(kThreads) void k_score_block(ScoreArgs a) {
    constexpr int ESZ = sizeof(TIn);
    constexpr int LPR = D * ESZ / 16;
    constexpr int RPI = 64 / LPR;
    constexpr int EPL = 16 / ESZ;
    extern __shared__ double qe[];                // [block_q][D]
    __shared__ double slot[2][kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rs = lane / LPR, ch = lane % LPR;
    const int bh = blockIdx.x / a.P, p = blockIdx.x % a.P;
    const int b = bh / a.Hkv, h = bh % a.Hkv;
    if (a.only && !a.only[bh]) return;

    const TIn *qb = (const TIn *)a.q;
    for (int idx = threadIdx.x; idx < a.block_q * D; idx += kThreads) {
        const int i = idx / D, c = idx % D;
        const int64_t row = ((int64_t)b * a.block_q + i) * a.Hq + (int64_t)h * a.g;
        double s = 0.0;
        for (int gg = 0; gg < a.g; ++gg) s += load_f64(qb, (row + gg) * D + c);
        qe[idx] = s;
    }
    __syncthreads();

    const Unit un = unit_of(a, h);
    const unsigned char *kh = a.k + un.kv_off + ch * 16;
    const GroupRange gr = group_range(a, p, un.sg.n_groups);
    for (int64_t grp = gr.g0; grp < gr.g1; ++grp) {
        const int64_t jend = min((grp + 1) * kGroup, un.sg.n_spans);
        double gbest = -INFINITY;
        for (int64_t j = grp * kGroup + wave; j < jend; j += kWaves) {
            const int64_t tb = un.sg.mid_lo + j * a.S;
            const int64_t te = min(tb + (int64_t)a.S, un.sg.mid_hi);
            double total = 0.0;
            for (int i = 0; i < a.block_q; ++i) {
                const double *qi = qe + (int64_t)i * D + ch * EPL;
                double best = -INFINITY;
                for (int64_t r0 = tb; r0 < te; r0 += RPI) {
                    const int64_t t = r0 + rs;
                    const bool ok = t < te;
                    const uint4 raw = ok ? *(const uint4 *)(kh + t * a.st_bytes)
                                         : make_uint4(0u, 0u, 0u, 0u);
                    double x[EPL];
                    unpack(raw, x);
                    double acc = 0.0;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc = fma(qi[e], x[e], acc);
                    acc = row_sum<LPR>(acc);
                    if (ok) best = fmax(best, acc);
                }
                total += rows_max<LPR>(best);
            }
            total += 0.0;
            if (lane == 0) a.out[(int64_t)bh * a.n_spans + j] = total;
            gbest = fmax(gbest, total);
        }
        publish_group_max(a, slot, bh, grp, gbest);
    }
}

// The events of a timed launch (both null when untimed).
struct Ev {
    hipEvent_t b, e;
};

template <typename TIn, int D, int R>
hipError_t launch_decode(const ScoreArgs &a, int nblocks, hipStream_t s, Ev ev) {
    return launch_struct(k_score_decode<TIn, D, R>, dim3(nblocks), dim3(kThreads), 0, s, a, ev.b,
                         ev.e);
}

template <typename TIn, int D, int NH>
hipError_t launch_heads(const Geom &g, const ScoreArgs &a, int nblocks, hipStream_t s, Ev ev) {
    const dim3 grid(nblocks), block(kThreads);
    if constexpr (D * sizeof(TIn) == 256 && (NH == 2 || NH == 4))
        return launch_struct(k_score_heads_lds<TIn, D, NH>, grid, block, 0, s, a, ev.b, ev.e);
    constexpr int RPI = 64 / (D * (int)sizeof(TIn) / 16);
    const int per_span = (g.S + RPI - 1) / RPI;
    if (per_span >= 4)
        return launch_struct(k_score_decode_heads<TIn, D, 4, NH>, grid, block, 0, s, a, ev.b, ev.e);
    if (per_span >= 2)
        return launch_struct(k_score_decode_heads<TIn, D, 2, NH>, grid, block, 0, s, a, ev.b, ev.e);
    return launch_struct(k_score_decode_heads<TIn, D, 1, NH>, grid, block, 0, s, a, ev.b, ev.e);
}

// Query heads per KV head that one multi-head decode workgroup scores
// together (0: score each selection head on its own, reading its KV head).
int multi_heads(const Geom &g) {
    if (g.block_q != 1 || g.rep < 2) return 0;
    if (g.S == 1) return g.rep <= 4 ? g.rep : 0;     // token level: at most 4 heads' scores held
    return (g.rep == 2 || g.rep == 3 || g.rep == 4 || g.rep == 8) ? g.rep : 0;
}

template <typename TIn, int D, int NH>
hipError_t launch_tokens(const ScoreArgs &a, int nblocks, hipStream_t s, Ev ev) {
    return launch_struct(k_score_tokens<TIn, D, NH>, dim3(nblocks), dim3(kThreads), 0, s, a, ev.b,
                         ev.e);
}

template <typename TIn, int D>
hipError_t launch_typed(const Geom &g, const ScoreArgs &a, int nblocks, hipStream_t s, Ev ev) {
    if (g.block_q == 1 && g.S == 1) {
        const int nh = multi_heads(g);
        if (nh == 2) return launch_tokens<TIn, D, 2>(a, nblocks, s, ev);
        if (nh == 3) return launch_tokens<TIn, D, 3>(a, nblocks, s, ev);
        if (nh == 4) return launch_tokens<TIn, D, 4>(a, nblocks, s, ev);
        return launch_tokens<TIn, D, 1>(a, nblocks, s, ev);
    }
    if (const int nh = multi_heads(g)) {
        if (nh == 2) return launch_heads<TIn, D, 2>(g, a, nblocks, s, ev);
        if (nh == 3) return launch_heads<TIn, D, 3>(g, a, nblocks, s, ev);
        if (nh == 4) return launch_heads<TIn, D, 4>(g, a, nblocks, s, ev);
        return launch_heads<TIn, D, 8>(g, a, nblocks, s, ev);
    }
    if (g.block_q == 1) {
        constexpr int RPI = 64 / (D * (int)sizeof(TIn) / 16);
        const int per_span = (g.S + RPI - 1) / RPI;       // load instructions per span
        if (per_span >= 8) return launch_decode<TIn, D, 8>(a, nblocks, s, ev);
        if (per_span >= 4) return launch_decode<TIn, D, 4>(a, nblocks, s, ev);
        if (per_span >= 2) return launch_decode<TIn, D, 2>(a, nblocks, s, ev);
        return launch_decode<TIn, D, 1>(a, nblocks, s, ev);
    }
    const size_t lds = (size_t)g.block_q * D * sizeof(double);
    return launch_struct(k_score_block<TIn, D>, dim3(nblocks), dim3(kThreads), lds, s, a, ev.b,
                         ev.e);
}

}  // namespace

int64_t score_groups(const Geom &g) { return (g.n_spans + kGroup - 1) / kGroup; }

bool score_decode_path(const Geom &g) { return g.block_q == 1 && g.S > 1 && multi_heads(g) == 0; }

hipError_t launch_score(const Geom &g, const void *q, const void *k, double *span_scores,
                        double *group_max, int num_cu, hipStream_t s, hipEvent_t ev_begin,
                        hipEvent_t ev_end, const uint32_t *only, double *group_second,
                        int32_t *group_arg, double *group_top, int32_t *group_top_idx) {
    if (g.n_spans == 0) return hipSuccess;
    ScoreArgs a;
    a.only = only;
    const bool top = score_decode_path(g) && group_top && group_top_idx;
    a.gtop = top ? group_top : nullptr;
    a.gtopi = top ? group_top_idx : nullptr;
    a.gsec = group_second;
    a.garg = group_arg;
    a.q = q;
    a.k = (const unsigned char *)k;
    a.out = span_scores;
    a.gmax = group_max;
    a.sh_bytes = g.sh * g.esize;
    a.st_bytes = g.st * g.esize;
    a.mid_lo = g.mid_lo;
    a.mid_hi = g.mid_hi;
    a.n_spans = g.n_spans;
    a.n_groups = score_groups(g);
    a.S = g.S;
    a.Hq = g.Hq;
    a.Hkv = g.Hkv;
    a.g = g.g;
    a.block_q = g.block_q;
    a.rep = g.rep;
    a.lens = g.lens;
    a.hps = g.hps;
    a.G = g.G;
    a.L = g.L;
    a.T = g.T;
    a.seq_stride_bytes = g.seq_stride * g.esize;
    // one workgroup column per (block, KV head); a multi-head decode covers the
    // rep selection heads of a KV head together
    const int nh = multi_heads(g);
    const int64_t units = (int64_t)g.n_blk * (nh ? g.Hkv / nh : g.Hkv);
    const int64_t target = (int64_t)(num_cu > 0 ? num_cu : 256) * 2;
    int64_t P = (target + units - 1) / units;
    if (P > a.n_groups) P = a.n_groups;
    if (P < 1) P = 1;
    a.P = (int)P;
    const int nblocks = (int)(units * P);
    const Ev ev{ev_begin, ev_end};
    if (g.dtype == 0)
        return g.d == 128 ? launch_typed<uint16_t, 128>(g, a, nblocks, s, ev)
                          : launch_typed<uint16_t, 64>(g, a, nblocks, s, ev);
    return g.d == 128 ? launch_typed<float, 128>(g, a, nblocks, s, ev)
                      : launch_typed<float, 64>(g, a, nblocks, s, ev);
}

}  // namespace rea
