// score_mfma.hip - step 1 for blocks of 64 queries (chunked prefill) on MFMA.
//
// A block of queries shares one selection whose span score is the sum over the
// block's queries of the span's maximum token score (ReAttention, OpenReview
// discussion, "Prefilling Phase" pseudocode: one top-k per chunk of queries;
// this library cuts a chunk into blocks).  For 64 queries against the whole
// middle cache the token scores form a real GEMM, so it runs on bf16 MFMA:
//
//   k_qprep       per (block, KV head): the fp64 group sum q_eff of each
//                 query, split as hi = bf16(q_eff), lo = bf16(q_eff - hi),
//                 stored as a 256-long bf16 row [hi | lo]; plus the error
//                 scale E_b = sum_i (gamma * ||(|hi|+|lo|)||_2 + ||q_eff-hi-lo||_2).
//   k_score_mfma  per (KV head, token range, group of 4 blocks): K tiles of 32
//                 tokens are staged once in LDS and multiplied on
//                 v_mfma_f32_32x32x16_bf16 by [hi|lo] of each wave's 64
//                 queries (K = 256: the key tile is fed twice).  The tile's
//                 token maxima, the span maximum and the sum over the block's
//                 queries are taken in the epilogue; one fp64 span score per
//                 (block, span) is written, and an upper bound of each span's
//                 largest key norm (by one wave of the grid per span: squares
//                 summed in fp32 with v_dot2, rounded up).
//   k_cert_candidates
//                 only beyond 4096 spans: per (block, KV head), the spans
//                 whose approximate score lies within twice the largest error
//                 bound of the (k+1)-th (a superset of every span the
//                 certification could keep or re-score); see there.
//   k_certify_head, k_rescore, k_certify_tail
//                 per (block, KV head): exact top-k from the approximate
//                 scores (see below): the classification per pair, the fp64
//                 re-scoring of the uncertain spans over several four-wave
//                 workgroups per pair (a chunk's few pairs then do not
//                 re-score on a handful of CUs, and many pairs share CUs three
//                 at a time), the ranking per pair.
//
// Error bound.  Every product hi*k, lo*k of two bf16 numbers is exact in fp32;
// the MFMA sums 256 of them in fp32.  With at most 255 roundings of at most
// 2^-23 relative each, |s_hat - s| <= e_i * ||k_t||_2 where
// e_i = 255*2^-23*(1+1e-6) * ||(|hi|+|lo|)||_2 + ||q_eff - hi - lo||_2.
// A span maximum moves by at most e_i * max_t ||k_t||, a block sum by
// E_b * Kbar_j.  The certification keeps every span whose interval
// [s_hat - eps, s_hat + eps] lies surely inside the top-k, drops every span
// surely outside it, re-scores the rest in fp64 (exact for bf16 inputs), and
// selects among them exactly -- so the selection equals the exact one.
#include "rea_internal.h"

#include <math.h>

namespace rea {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;             // head_dim handled here
constexpr int kQB = 64;             // queries per block
constexpr int kWavesM = 4;          // blocks (waves) per workgroup
constexpr int kTile = 32;           // tokens per MFMA tile
constexpr double kGammaMfma = 255.0 * 1.1920928955078125e-07 * (1.0 + 1e-6);   // 255 * 2^-23

__device__ __forceinline__ double bf16_to_f64(uint16_t b) {
    return (double)__uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

// ---------------------------------------------------------------------------
// k_score_mfma: grid (n_qg * Hkv * NR) with the query group slowest, so the
// workgroups sharing a key range of one head sit on one XCD; 256 threads,
// two workgroups per CU so that one hides the other's LDS and reduction
// latency.
//
// Key tiles stream through a 6-deep LDS ring filled by global_load_lds
// (16 bytes per lane straight into LDS, no staging registers), so five tiles
// are in flight while one is multiplied.  Within a tile, 16-byte chunk c of
// token row m is stored at slot c ^ (m % 16), which makes the MFMA operand
// reads bank-conflict free.  Span results are buffered in LDS and written
// after the loop, so only the ring's loads count in vmcnt.  The key norms a
// span's error bound needs are computed by one wave of the whole grid per
// span, spread evenly over the query groups.
// ---------------------------------------------------------------------------
constexpr int kNBuf = 6;
constexpr int kTileBytes = kTile * kD * 2;          // 8 KB
constexpr int kMaxSpansWG = 512;

struct MfmaArgs {
    const unsigned char *k;     // K cache (bf16)
    const uint16_t *qhl;        // [Hkv][n_q][256]
    double *out;                // [n_blk][Hkv][n_spans]
    double *kbar;               // [Hkv][n_spans]
    int64_t sh_bytes, st_bytes;
    int64_t mid_lo, mid_hi, n_spans;
    int S, Hkv, n_q, n_blk, NR, rep;
};

__device__ __forceinline__ uint4 ld16(const void *p) { return *(const uint4 *)p; }

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// Eight 16-byte LDS reads issued together and completed (lgkmcnt(0)) inside
// one asm block.  Written as asm so that the compiler does not make them wait
// for every DMA still in flight to other ring slots; the ring slot read here
// is complete by the explicit vmcnt wait and barrier that precede the call.
__device__ __forceinline__ void lds_read8(const uint32_t (&ad)[8], uint4 (&o)[8]) {
    u32x4v r0, r1, r2, r3, r4, r5, r6, r7;
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %13\n\t"
        "ds_read_b128 %6, %14\n\t"
        "ds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
          "v"(ad[7])
        : "memory");
    o[0] = make_uint4(r0.x, r0.y, r0.z, r0.w);
    o[1] = make_uint4(r1.x, r1.y, r1.z, r1.w);
    o[2] = make_uint4(r2.x, r2.y, r2.z, r2.w);
    o[3] = make_uint4(r3.x, r3.y, r3.z, r3.w);
    o[4] = make_uint4(r4.x, r4.y, r4.z, r4.w);
    o[5] = make_uint4(r5.x, r5.y, r5.z, r5.w);
    o[6] = make_uint4(r6.x, r6.y, r6.z, r6.w);
    o[7] = make_uint4(r7.x, r7.y, r7.z, r7.w);
}

// Sixteen 16-byte LDS reads: 8 channels of four fp64 rows 128 doubles apart
// (base + r * 1024 + {0, 16, 32, 48}), completed inside one asm block like
// lds_read8.
__device__ __forceinline__ void lds_read16_rows4(uint32_t base, uint4 (&o)[16]) {
    u32x4v r[16];
    asm volatile(
        "ds_read_b128 %0, %16\n\t"
        "ds_read_b128 %1, %16 offset:16\n\t"
        "ds_read_b128 %2, %16 offset:32\n\t"
        "ds_read_b128 %3, %16 offset:48\n\t"
        "ds_read_b128 %4, %16 offset:1024\n\t"
        "ds_read_b128 %5, %16 offset:1040\n\t"
        "ds_read_b128 %6, %16 offset:1056\n\t"
        "ds_read_b128 %7, %16 offset:1072\n\t"
        "ds_read_b128 %8, %16 offset:2048\n\t"
        "ds_read_b128 %9, %16 offset:2064\n\t"
        "ds_read_b128 %10, %16 offset:2080\n\t"
        "ds_read_b128 %11, %16 offset:2096\n\t"
        "ds_read_b128 %12, %16 offset:3072\n\t"
        "ds_read_b128 %13, %16 offset:3088\n\t"
        "ds_read_b128 %14, %16 offset:3104\n\t"
        "ds_read_b128 %15, %16 offset:3120\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
          "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]),
          "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
        : "v"(base)
        : "memory");
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = make_uint4(r[i].x, r[i].y, r[i].z, r[i].w);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(size_t)(const void __attribute__((address_space(3))) *)p;
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

// The value of lane l ^ 32 (v_permlane32_swap: either result half may hold
// the partner, so the caller combines both with a symmetric operation).
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ double pair_sum(double x) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    const double a = __longlong_as_double((long long)(((uint64_t)hi[0] << 32) | lo[0]));
    const double b = __longlong_as_double((long long)(((uint64_t)hi[1] << 32) | lo[1]));
    return a + b;     // own + partner in either order: the same value
}

__device__ __forceinline__ float pair_sumf(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);   // own + partner, either order
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Every lane of each 16-lane row ends with the row's sum (max): partners are
// lane^1, lane^2, then the mirror within 8 and within 16 lanes, each a
// symmetric pairing, so both partners compute the same value.
__device__ __forceinline__ double row_sum16(double v) {
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x141>(v);
    v += dpp_f64<0x140>(v);
    return v;
}
__device__ __forceinline__ double row_max16(double v) {
    v = fmax(v, dpp_f64<0xB1>(v));
    v = fmax(v, dpp_f64<0x4E>(v));
    v = fmax(v, dpp_f64<0x141>(v));
    v = fmax(v, dpp_f64<0x140>(v));
    return v;
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// ---------------------------------------------------------------------------
// k_qprep: grid (n_blk, Hkv), 1024 threads: each wave takes every 16th query
// of the block, a lane two adjacent channels (2l, 2l + 1: one 32-bit load per
// query and query head, the loads of up to four query heads issued together);
// the per-query norms are summed over the wave with DPP and read lanes, and
// the block's bound E_b is the sum of the per-query bounds, added in query
// order by one thread.
// ---------------------------------------------------------------------------
struct PrepArgs {
    const uint16_t *q;      // [n_q][Hq][D]
    uint16_t *qhl;          // [Hkv][n_q][256]
    double *qeff;           // [Hkv][n_q][D]
    double *E;              // [n_blk][Hkv]
    int Hq, Hkv, g, n_q;
};

constexpr int kPrepThreads = 1024;

// Sum over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ double wave_sum_f64(double v) {
    v = row_sum16(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

__global__ __launch_bounds__(kPrepThreads) void k_qprep(PrepArgs a) {
    __shared__ double e_q[kQB];
    const int b = blockIdx.x, h = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int kWavesP = kPrepThreads / 64;
    constexpr int QPW = kQB / kWavesP;                 // queries per wave (4)
    constexpr int GB = 4;                              // query heads loaded together
    // group sums in fp64, query heads added in order
    double s[QPW][2];
#pragma unroll
    for (int u = 0; u < QPW; ++u) s[u][0] = s[u][1] = 0.0;
    for (int g0 = 0; g0 < a.g; g0 += GB) {
        uint32_t raw[GB][QPW];
#pragma unroll
        for (int gg = 0; gg < GB; ++gg) {
            const int hq = h * a.g + (g0 + gg < a.g ? g0 + gg : a.g - 1);
#pragma unroll
            for (int u = 0; u < QPW; ++u) {
                const int64_t i = (int64_t)b * kQB + wave + u * kWavesP;
                raw[gg][u] = *(const uint32_t *)(a.q + (i * a.Hq + hq) * kD + 2 * lane);
            }
        }
#pragma unroll
        for (int gg = 0; gg < GB; ++gg)
            if (g0 + gg < a.g)
#pragma unroll
                for (int u = 0; u < QPW; ++u) {
                    s[u][0] += (double)__uint_as_float(raw[gg][u] << 16);
                    s[u][1] += (double)__uint_as_float(raw[gg][u] & 0xffff0000u);
                }
    }
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
        const int il = wave + u * kWavesP;
        const int64_t row = (int64_t)h * a.n_q + (int64_t)b * kQB + il;
        double n1 = 0.0, n2 = 0.0;
        uint32_t hi2 = 0, lo2 = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const double sv = s[u][e];
            const uint16_t hi = f32_to_bf16((float)sv);
            const double hid = bf16_to_f64(hi);
            const uint16_t lo = f32_to_bf16((float)(sv - hid));
            const double lod = bf16_to_f64(lo);
            const double r = sv - hid - lod;
            hi2 |= (uint32_t)hi << (16 * e);
            lo2 |= (uint32_t)lo << (16 * e);
            n1 += (fabs(hid) + fabs(lod)) * (fabs(hid) + fabs(lod));
            n2 += r * r;
        }
        *(uint32_t *)(a.qhl + row * 256 + 2 * lane) = hi2;
        *(uint32_t *)(a.qhl + row * 256 + kD + 2 * lane) = lo2;
        *(double2 *)(a.qeff + row * kD + 2 * lane) = make_double2(s[u][0], s[u][1]);
        n1 = wave_sum_f64(n1);
        n2 = wave_sum_f64(n2);
        if (lane == 0) e_q[il] = (kGammaMfma * sqrt(n1) + sqrt(n2)) * (1.0 + 1e-12);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double esum = 0.0;
        for (int il = 0; il < kQB; ++il) esum += e_q[il];
        a.E[(int64_t)b * a.Hkv + h] = esum * (1.0 + 1e-9);
    }
}

__global__ __launch_bounds__(256, 2) void k_score_mfma(MfmaArgs a) {
    __shared__ __align__(16) unsigned char ring[kNBuf * kTileBytes];
    __shared__ double res[kWavesM][kMaxSpansWG];
    __shared__ double kres[kMaxSpansWG];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int units = a.Hkv * a.NR;
    const int n_qg = gridDim.x / units;
    const int qg = blockIdx.x / units;
    const int rest = blockIdx.x % units;
    const int h = rest / a.NR, r = rest % a.NR;
    const int b = qg * kWavesM + wave;              // this wave's block
    const bool active = b < a.n_blk;
    const int j0 = (int)((int64_t)r * a.n_spans / a.NR), j1 = (int)((int64_t)(r + 1) * a.n_spans / a.NR);
    const int tiles_per_span = a.S / kTile;

    // B fragments: [hi|lo] of the wave's 64 queries, two 32-query tiles x 16 k-steps
    uint4 qf[2][16];
    {
        const int n = lane & 31, kb = lane >> 5;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int64_t qi = (int64_t)(active ? b : 0) * kQB + t * 32 + n;
            const uint16_t *row = a.qhl + ((int64_t)h * a.n_q + qi) * 256;
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) qf[t][ks] = ld16(row + ks * 16 + kb * 8);
        }
    }
    __builtin_amdgcn_s_waitcnt(0xF70);              // fragments in registers before the ring starts

    const unsigned char *kh = a.k + (int64_t)(h / a.rep) * a.sh_bytes;
    const int n_tiles = (j1 - j0) * tiles_per_span;
    // each wave moves 2 x 1 KB (8 token rows) of every tile; (ij, isub) is the
    // span and sub-tile of the next tile to issue
    int ij = j0, isub = 0, it_issue = 0;
    auto issue_next = [&]() {
        if (it_issue >= n_tiles) return;
        const int64_t t0 = a.mid_lo + (int64_t)ij * a.S + isub * kTile;
        unsigned char *dst = ring + (it_issue % kNBuf) * kTileBytes;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int row = (wave * 2 + jj) * 4 + (lane >> 4);
            const int chunk = (lane & 15) ^ (row & 15);
            int64_t t = t0 + row;
            if (t >= a.mid_hi) t = a.mid_hi - 1;       // rows past the middle are masked later
            __builtin_amdgcn_global_load_lds((const void *)(kh + t * a.st_bytes + chunk * 16),
                                             (void __attribute__((address_space(3))) *)(dst + (wave * 2 + jj) * 1024),
                                             16, 0, 0);
        }
        ++it_issue;
        if (++isub == tiles_per_span) {
            isub = 0;
            ++ij;
        }
    };
    for (int i = 0; i < kNBuf - 1; ++i) issue_next();

    float run[2] = {-INFINITY, -INFINITY};   // lane-local running max over the span's tiles
    double kn_run = 0.0;                     // running max of squared key norms (owner wave)
    int j = j0, sub = 0;
    for (int it = 0; it < n_tiles; ++it) {
        int later = n_tiles - 1 - it;                 // tiles issued after this one
        if (later > kNBuf - 2) later = kNBuf - 2;
        wait_vmcnt(2 * later);
        // A plain barrier, not __syncthreads(): its release fence would wait for
        // every DMA in flight.  This wave's copies into the slot are complete by
        // the vmcnt wait above, the other waves' by the barrier; every wave
        // finished reading (lgkmcnt(0)) the slot refilled below before it got here.
        __builtin_amdgcn_s_barrier();
        issue_next();
        const unsigned char *tb = ring + (it % kNBuf) * kTileBytes;
        const int64_t t0 = a.mid_lo + (int64_t)j * a.S + sub * kTile;
        const bool owner = (j & 3) == wave && ((j >> 2) % n_qg) == qg;
        // A fragments: token row m = lane%32, channel chunk ks*2 + lane/32
        uint4 af[8];
        {
            const int m = lane & 31, kb = lane >> 5;
            const uint32_t base = lds_addr(tb) + m * 256;
            uint32_t ad[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) ad[ks] = base + (((ks * 2 + kb) ^ (m & 15)) * 16);
            lds_read8(ad, af);
        }
        f32x16 acc0 = {}, acc1 = {};
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const bf16x8 A = __builtin_bit_cast(bf16x8, af[ks & 7]);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, __builtin_bit_cast(bf16x8, qf[0][ks]),
                                                           acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, __builtin_bit_cast(bf16x8, qf[1][ks]),
                                                           acc1, 0, 0, 0);
        }
        // tokens past the middle (a short last span) do not count
        const int64_t valid = a.mid_hi - t0;
        if (valid >= kTile) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                run[0] = fmaxf(run[0], acc0[rr]);
                run[1] = fmaxf(run[1], acc1[rr]);
            }
        } else {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int row = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
                if (row < valid) {
                    run[0] = fmaxf(run[0], acc0[rr]);
                    run[1] = fmaxf(run[1], acc1[rr]);
                }
            }
        }
        if (owner) {
            // squared norm of key row lane%32: this lane's half of the channels
            // (its A fragments) plus the partner lane's half, summed in fp32 by
            // v_dot2 (bf16 squares are exact in fp32; the at most 130 roundings
            // of the sums are covered by the factor applied at the span's end)
            float sq4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const uint32_t w4[4] = {af[ks].x, af[ks].y, af[ks].z, af[ks].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bf16x2 x = __builtin_bit_cast(bf16x2, w4[e]);
                    sq4[e] = __builtin_amdgcn_fdot2_f32_bf16(x, x, sq4[e], false);
                }
            }
            const float sq = pair_sumf((sq4[0] + sq4[1]) + (sq4[2] + sq4[3]));
            if ((lane & 31) < valid) kn_run = fmax(kn_run, (double)sq);
        }
        if (++sub == tiles_per_span) {
            // span done: per-query maximum (lanes l and l^32 hold the two row
            // halves), then the sum over the block's 64 queries
            const float m0 = pair_max(run[0]), m1 = pair_max(run[1]);
            const double v = row_sum16((double)m0 + (double)m1);
            const double tot = readlane_f64(v, 0) + readlane_f64(v, 16);
            if (lane == 0) res[wave][j - j0] = tot + 0.0;
            if (owner) {
                const double kn = row_max16(kn_run);
                const double km = fmax(readlane_f64(kn, 0), readlane_f64(kn, 16));
                // an upper bound of the largest norm: the fp32 sums low by
                // at most 130 * 2^-23 relative, squares below 2^-126 flushed
                if (lane == 0)
                    kres[j - j0] = sqrt(km * (1.0 + 0x1p-15) + 0x1p-119) * (1.0 + 1e-12);
            }
            run[0] = -INFINITY;
            run[1] = -INFINITY;
            kn_run = 0.0;
            sub = 0;
            ++j;
        }
    }
    __syncthreads();
    const int nsp = j1 - j0;
    for (int x = tid; x < nsp; x += 256) {
#pragma unroll
        for (int w = 0; w < kWavesM; ++w) {
            const int bw = qg * kWavesM + w;
            if (bw < a.n_blk) a.out[((int64_t)bw * a.Hkv + h) * a.n_spans + j0 + x] = res[w][x];
        }
        if ((((j0 + x) >> 2) % n_qg) == qg) a.kbar[(int64_t)h * a.n_spans + j0 + x] = kres[x];
    }
}

// ---------------------------------------------------------------------------
// k_score_heads_mfma: a decode step with one selection per query head (bf16,
// d 128, S a multiple of 32).  The NH query heads of a KV head are the
// columns, and 32 consecutive key tokens the rows, of a
// v_mfma_f32_32x32x16_bf16, so every key row is read once and scored for all
// NH heads on the matrix cores.  q_h is bf16, so each product is exact in
// fp32, and the fp32 sum of a token's 128 products is within
// gamma * ||q_h|| * ||k_t|| of the exact score (at most 128 roundings of at
// most 2^-23 relative each, whatever the order).  The span scores written are
// approximations within eps_j = E_h * Kbar_j (E_h = gamma ||q_h||, Kbar_j an
// upper bound of the span's largest key norm), and the certification below
// decides the top-k exactly (one query per pair: its fp64 re-scoring runs in
// k_certify_one).
//
// grid (Hp * P), 256 threads, two workgroups per CU: workgroup (hp, p) takes a
// contiguous run of KV head hp's groups of 32 spans.  Within a group, wave w
// scores spans w, w + 4, ..., so the four waves stream adjacent spans, each
// through its own LDS ring of kQNB tiles filled by DMA (global_load_lds;
// 16-byte chunk c of token row m at slot c ^ (m % 16), as in k_score_mfma).
// No barrier couples the waves: each writes its own spans' results and its
// own maxima of each group (gmx / gkb hold one per wave; the candidate pass
// takes their maximum), so a wave never stops issuing loads to wait for the
// others.  The DMA loads carry the non-temporal cache policy: the keys are
// read once, and keeping them out of the caches' normal replacement raises
// the read rate markedly on this pattern.
// ---------------------------------------------------------------------------
constexpr int kQNB = 2;
constexpr int kGroupH = 32;         // spans per group
constexpr double kGammaHeads = 128.0 * 1.1920928955078125e-07 * (1.0 + 1e-4);   // 128 * 2^-23

struct HeadsArgs {
    const unsigned char *k;     // K cache (bf16)
    const uint16_t *q;          // [Hq][D]: the step's one query
    double *out;                // [Hsel][n_spans] approximate span scores
    double *kbar;               // [Hp][n_spans] key-norm bounds (one per KV head)
    double *E;                  // [Hsel]
    double *gmx, *gkb;          // [Hsel][groups][4]: per 32 spans and wave, largest score / norm bound
    int64_t sh_bytes, st_bytes, mid_lo, mid_hi, n_spans;
    int S, NH, Hp, P;
};

__global__ __launch_bounds__(256, 2) void k_score_heads_mfma(HeadsArgs a) {
    __shared__ __align__(16) unsigned char ring[kWavesM][kQNB][kTileBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hp = blockIdx.x / a.P, p = blockIdx.x % a.P;
    const int64_t h0 = (int64_t)hp * a.NH;          // first selection head (query head)
    const int n = lane & 31, kb = lane >> 5;

    // B fragments: query head n (zero columns beyond NH), channels
    // ks * 16 + kb * 8 .. + 8
    uint4 qf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
        qf[ks] = n < a.NH ? ld16(a.q + (h0 + n) * kD + ks * 16 + kb * 8) : make_uint4(0u, 0u, 0u, 0u);
    if (p == 0 && wave == 0) {
        // E_h = gamma * ||q_h|| (bf16 squares and their sum exact in fp64), plus
        // a floor covering fp32 products flushed below 2^-126
        double sq = 0.0;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const uint32_t w4[4] = {qf[ks].x, qf[ks].y, qf[ks].z, qf[ks].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double x0 = (double)__uint_as_float(w4[e] << 16);
                const double x1 = (double)__uint_as_float(w4[e] & 0xffff0000u);
                sq = fma(x0, x0, fma(x1, x1, sq));
            }
        }
        sq = pair_sum(sq);
        if (lane < a.NH) a.E[h0 + lane] = kGammaHeads * sqrt(sq) * (1.0 + 1e-12) + 0x1p-50;
    }

    // the workgroup's groups [g0, g1) of 32 spans; this wave's span slots
    // are wave, wave + 4, ... of each group
    const int64_t ng = (a.n_spans + kGroupH - 1) / kGroupH;
    const int64_t g0 = (int64_t)p * ng / a.P, g1 = (int64_t)(p + 1) * ng / a.P;
    const int64_t first = g0;
    const int64_t n_grp = g1 - g0;
    const int tps = a.S / kTile;
    // every wave runs 8 span slots of every group (slots past the middle's
    // last span read a clamped row and are masked), so it writes its maxima
    // slot of every group
    const int64_t n_tiles = n_grp * (kGroupH / kWavesM) * tps;
    const unsigned char *kh = a.k + (int64_t)hp * a.sh_bytes;
    unsigned char *rw = &ring[wave][0][0];
    // tile cursors (issue side and consume side), advanced incrementally:
    // sub-tile within the span, span slot within the group (stride 4), group
    struct Cursor {
        int sub, sig;
        int64_t grp, t0;
    };
    auto advance = [&](Cursor &u) {
        if (++u.sub < tps) {
            u.t0 += kTile;
            return;
        }
        u.sub = 0;
        u.sig += kWavesM;
        if (u.sig >= kGroupH) {
            u.sig = wave;
            u.grp += 1;
        }
        u.t0 = a.mid_lo + (u.grp * kGroupH + u.sig) * a.S;
    };
    Cursor iss = {0, wave, first, a.mid_lo + (first * kGroupH + wave) * a.S};
    Cursor con = iss;
    int64_t it_issue = 0;
    int slot_i = 0, slot_c = 0;                  // ring slots of the next issue / consume
    auto issue_next = [&]() {
        if (it_issue >= n_tiles) return;
        const int64_t t0 = iss.t0;
        unsigned char *dst = rw + slot_i * kTileBytes;
        slot_i = slot_i + 1 == kQNB ? 0 : slot_i + 1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = i * 4 + (lane >> 4);
            const int chunk = (lane & 15) ^ (row & 15);
            int64_t t = t0 + row;
            if (t >= a.mid_hi) t = a.mid_hi - 1;       // rows past the middle are masked
            __builtin_amdgcn_global_load_lds((const void *)(kh + t * a.st_bytes + chunk * 16),
                                             (void __attribute__((address_space(3))) *)(dst + i * 1024),
                                             16, 0, 2);
        }
        ++it_issue;
        advance(iss);
    };
#pragma unroll
    for (int i = 0; i < kQNB - 1; ++i) issue_next();

    float run = -INFINITY;       // running maximum of this lane's rows (query n)
    float kn_run = 0.f;          // running maximum of squared key norms (row lane % 32)
    double gmax = -INFINITY, gkmax = 0.0;   // the group's maxima (lanes n < NH)
    for (int64_t it = 0; it < n_tiles; ++it) {
        int64_t later = n_tiles - 1 - it;               // tiles issued after this one
        if (later > kQNB - 2) later = kQNB - 2;
        // 8 DMA instructions per tile
        if (later == 0) __builtin_amdgcn_s_waitcnt(0xF70);   // vmcnt(0)
        else __builtin_amdgcn_s_waitcnt(0xF78);              // vmcnt(8)
        const int64_t grp = con.grp;
        const int sig = con.sig, sub = con.sub;
        const int64_t j = grp * kGroupH + sig;
        const int64_t t0 = con.t0;
        const unsigned char *tb = rw + slot_c * kTileBytes;
        slot_c = slot_c + 1 == kQNB ? 0 : slot_c + 1;
        advance(con);
        // refill the slot read in the previous step (its reads completed there)
        issue_next();
        uint4 af[8];
        {
            const int m = lane & 31;
            const uint32_t base = lds_addr(tb) + m * 256;
            uint32_t ad[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) ad[ks] = base + (((ks * 2 + kb) ^ (m & 15)) * 16);
            lds_read8(ad, af);
        }
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[ks]),
                                                          __builtin_bit_cast(bf16x8, qf[ks]),
                                                          acc, 0, 0, 0);
        // squared key norm of row lane % 32 (this lane's half of the channels,
        // then the partner's), fp32 v_dot2 sums
        float sq4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const uint32_t w4[4] = {af[ks].x, af[ks].y, af[ks].z, af[ks].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16x2 x = __builtin_bit_cast(bf16x2, w4[e]);
                sq4[e] = __builtin_amdgcn_fdot2_f32_bf16(x, x, sq4[e], false);
            }
        }
        const float sq = pair_sumf((sq4[0] + sq4[1]) + (sq4[2] + sq4[3]));
        const int64_t valid = a.mid_hi - t0;
        if ((lane & 31) < valid) kn_run = fmaxf(kn_run, sq);
        if (valid >= kTile) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) run = fmaxf(run, acc[rr]);
        } else {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int row = 8 * (rr >> 2) + 4 * kb + (rr & 3);
                if (row < valid) run = fmaxf(run, acc[rr]);
            }
        }
        if (sub == tps - 1) {
            // span done: query n's maximum (lanes n and n + 32 hold the two
            // row halves), the largest key norm over the 32 row lanes
            const double sm = (double)pair_max(run) + 0.0;
            // largest of the 32 rows' norms: DPP within each 16-lane row, then
            // the two rows of a half wave (lanes l and l ^ 32 hold the same row)
            float km = kn_run;
            km = fmaxf(km, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(km), 0xB1, 0xF, 0xF, false)));
            km = fmaxf(km, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(km), 0x4E, 0xF, 0xF, false)));
            km = fmaxf(km, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(km), 0x141, 0xF, 0xF, false)));
            km = fmaxf(km, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(km), 0x140, 0xF, 0xF, false)));
            {
                const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(km), __float_as_uint(km), false, false);
                km = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
            }
            // an upper bound: the fp32 sums low by at most 130 * 2^-23
            // relative, squares below 2^-126 flushed
            const double kbv = sqrt((double)km * (1.0 + 0x1p-15) + 0x1p-119) * (1.0 + 1e-12);
            if (j < a.n_spans) {
                if (kb == 0 && n < a.NH) a.out[(h0 + n) * a.n_spans + j] = sm;
                if (lane == 0) a.kbar[(int64_t)hp * a.n_spans + j] = kbv;
                gmax = fmax(gmax, sm);
                gkmax = fmax(gkmax, kbv);
            }
            run = -INFINITY;
            kn_run = 0.f;
            if (sig + kWavesM >= kGroupH) {      // this wave's last slot of the group
                if (kb == 0 && n < a.NH) {
                    a.gmx[((h0 + n) * ng + grp) * kWavesM + wave] = gmax;
                    a.gkb[((h0 + n) * ng + grp) * kWavesM + wave] = gkmax;
                }
                gmax = -INFINITY;
                gkmax = 0.0;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// certification: k_certify_head and k_certify_tail grid (n_blk * Hkv), 512
// threads; k_rescore grid (n_blk * Hkv * R), 256 threads
// ---------------------------------------------------------------------------
constexpr int kCThreads = 512;
constexpr int kCWaves = kCThreads / 64;
constexpr int kCCap = 4096;         // spans handled on chip
constexpr int kCBins = 2048;
constexpr int kCRank = 256;
constexpr int kCPer = kCCap / kCThreads;
constexpr int kCSplit = 256;        // uncertain spans re-scored as two items each

struct CertArgs {
    const double *shat;     // [n_blk][Hkv][n_spans]
    const double *kbar;     // [Hkv][n_spans]
    const double *E;        // [n_blk][Hkv]
    const double *qeff;     // [Hkv][n_q][D]
    const unsigned char *k;
    int32_t *sel, *nsel;
    int64_t sh_bytes, st_bytes, mid_lo, mid_hi, n_spans;
    int S, Hkv, n_q, kk, topk, rep;
    // the three certification kernels' shared state
    int R;
    int32_t *gxs;       // [pairs][kCCap] uncertain spans (positions among the ranked ones)
    uint32_t *gbits;    // [pairs][kCCap / 32] certain spans (bits by position)
    uint32_t *gcnt;     // [pairs][4]: nx, nd, decided without ranking
    double *gpart;      // [pairs][2][kCCap] per-item sums of the re-scoring
    // more than kCCap spans: the spans ranked per pair are its candidates
    // (k_cert_candidates); null when every span is ranked (position = index)
    int32_t *gcand;     // [pairs][kCCap] candidate span indices, ascending
    uint32_t *gncand;   // [pairs] candidates
    uint32_t *gover;    // [pairs] 1: too many candidates, the exact fallback selects
    // queries per pair: 64 (blocks; re-scored by k_rescore from qeff) or 1 (a
    // decode step per query head; re-scored in k_certify_tail from q1)
    int qpb;
    const uint16_t *q1;     // [Hsel][D] bf16 (qpb == 1)
    const double *gmx, *gkb;    // [pairs][groups][4] per-wave group maxima (k_certify_heads)
    // selection heads per kbar row: 1 (blocks: kbar per KV head and pair), or
    // the query heads per KV head (decode per query head: one row per KV head)
    int kbar_div;
};

// Span index of the pair's ranked span at position c.
__device__ __forceinline__ int32_t span_at(const CertArgs &a, int64_t bh, int64_t c) {
    return a.gcand ? a.gcand[bh * kCCap + c] : (int32_t)c;
}

// Spans the pair ranks: all of them, or its candidates.
__device__ __forceinline__ int64_t ranked(const CertArgs &a, int64_t bh) {
    return a.gcand ? (int64_t)a.gncand[bh] : a.n_spans;
}

struct CertShared {
    double val[kCCap];
    int32_t idx[kCCap];
    double xv[kCCap];               // exact scores of the uncertain spans
    int32_t xs[kCCap];              // their indices
    uint32_t hist[kCBins];
    uint32_t bitmap[kCCap / 32];
    double red_d[2][kCWaves];
    uint32_t red_u[kCWaves];
    uint32_t scan[kCWaves + 1];
    uint32_t count, above, nd, nx;
    int32_t bstar, cut_j;
    double cut_v, cut_u;
    double q1[kD];                  // the pair's query in fp64 (one query per pair)
    int32_t cand[kCCap];            // k_certify_heads: the pair's candidate spans, ascending
    uint32_t ncand;
};

// Span index of ranked position c, and the number of ranked spans: from the
// candidate list in LDS (L, k_certify_heads) or as span_at / ranked.
template <bool L>
__device__ __forceinline__ int32_t span_of(const CertArgs &a, const CertShared &sh, int64_t bh,
                                           int64_t c) {
    if constexpr (L) return sh.cand[c];
    return span_at(a, bh, c);
}
template <bool L>
__device__ __forceinline__ int64_t ranked_of(const CertArgs &a, const CertShared &sh, int64_t bh) {
    if constexpr (L) return (int64_t)sh.ncand;
    return ranked(a, bh);
}

__device__ __forceinline__ int c_bin(double x, double mn, double inv) {
    const double f = floor((x - mn) * inv);
    if (!(f > 0.0)) return 0;
    if (f >= (double)(kCBins - 1)) return kCBins - 1;
    return (int)f;
}

__device__ __forceinline__ void c_minmax(CertShared &sh, double &mn, double &mx) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int o = 32; o > 0; o >>= 1) {
        mn = fmin(mn, __shfl_xor(mn, o));
        mx = fmax(mx, __shfl_xor(mx, o));
    }
    if (lane == 0) {
        sh.red_d[0][wave] = mn;
        sh.red_d[1][wave] = mx;
    }
    __syncthreads();
    mn = INFINITY;
    mx = -INFINITY;
    for (int w = 0; w < kCWaves; ++w) {
        mn = fmin(mn, sh.red_d[0][w]);
        mx = fmax(mx, sh.red_d[1][w]);
    }
    __syncthreads();
}

// Slices a pairwise ranking of count entries is split into: as many as the
// workgroup's threads allow, but each covering at least 16 entries (the
// slices' counts are summed one LDS read each afterwards).
__device__ __forceinline__ uint32_t c_slices(uint32_t count) {
    uint32_t ns = count ? kCThreads / count : 1;
    if (ns > count / 16) ns = count / 16;
    return ns ? ns : 1u;
}

// Called by the 64 lanes of one wave: the bin of hist[0..kCBins) holding the
// need-th largest entry (bins counted from the top) and the count in the bins
// above it (1 <= need <= the histogram's total).  Each lane sums a run of
// kCBins / 64 bins, read in a lane-rotated order so that the lanes hit
// distinct banks; a suffix scan over the lanes picks the run, and a prefix
// scan over that run's bins, one per lane, picks the bin.
__device__ __forceinline__ void c_find_bin(const uint32_t *hist, int64_t need, int &bstar,
                                           uint32_t &above) {
    const int lane = threadIdx.x & 63;
    constexpr int bpl = kCBins / 64;
    static_assert(bpl <= 64 && (bpl & (bpl - 1)) == 0, "one run's bins fit the wave");
    uint32_t own = 0;
    for (int i = 0; i < bpl; ++i) own += hist[lane * bpl + ((i + lane) & (bpl - 1))];
    uint32_t suf = own;                          // count in bins >= lane * bpl
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_down(suf, o);
        if (lane + o < 64) suf += y;
    }
    const uint32_t after = suf - own;            // count in the runs above this lane's
    const uint64_t hit = __ballot((int64_t)after < need && need <= (int64_t)suf);
    const int L = hit ? __ffsll((long long)hit) - 1 : 0;
    const uint32_t aboveL = __shfl(after, L);
    const uint32_t c = lane < bpl ? hist[L * bpl + bpl - 1 - lane] : 0u;   // run L, top first
    uint32_t pre = c;
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(pre, o);
        if (lane >= o) pre += y;
    }
    const uint64_t at = __ballot(lane < bpl && (int64_t)(aboveL + pre) >= need);
    const int i = at ? __ffsll((long long)at) - 1 : 0;
    bstar = L * bpl + bpl - 1 - i;
    above = aboveL + __shfl(pre - c, i);
}

// need-th best of (val, idx)[0..count) under (val desc, idx asc) -> cut_v/cut_j.
// Reorders and shrinks val/idx.
__device__ __forceinline__ void c_find_kth(CertShared &sh, uint32_t count, int64_t need) {
    const int tid = threadIdx.x, lane = tid & 63;
    bool by_index = false;
    for (;;) {
        if (count <= (uint32_t)kCRank) {
            // pairwise ranks: one thread per (entry, slice of the compared
            // entries), so every thread of the workgroup takes part; 8
            // entries are read per step so the LDS latency is paid once per 8
            // comparisons, and the slices' counts are summed through LDS
            const uint32_t ns = c_slices(count);
            if ((uint32_t)tid < ns * count) {
                const uint32_t c = (uint32_t)tid % count, sl = (uint32_t)tid / count;
                const uint32_t o1 = (sl + 1) * count / ns;
                const double x = sh.val[c];
                const int32_t jc = sh.idx[c];
                uint32_t rank = 0, o = sl * count / ns;
                for (; o + 8 <= o1; o += 8) {
                    double y[8];
                    int32_t yi[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        y[u] = sh.val[o + u];
                        yi[u] = sh.idx[o + u];
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) rank += outranks(y[u], yi[u], x, jc);
                }
                for (; o < o1; ++o) {
                    const double y = sh.val[o];
                    rank += outranks(y, sh.idx[o], x, jc);
                }
                sh.hist[tid] = rank;
            }
            __syncthreads();
            for (uint32_t c = tid; c < count; c += kCThreads) {
                int64_t rank = 0;
                for (uint32_t sl = 0; sl < ns; ++sl) rank += sh.hist[sl * count + c];
                if (rank == need - 1) {
                    sh.cut_v = sh.val[c];
                    sh.cut_j = sh.idx[c];
                }
            }
            __syncthreads();
            return;
        }
        double mn = INFINITY, mx = -INFINITY;
        for (uint32_t c = tid; c < count; c += kCThreads) {
            const double key = by_index ? -(double)sh.idx[c] : sh.val[c];
            mn = fmin(mn, key);
            mx = fmax(mx, key);
        }
        c_minmax(sh, mn, mx);
        if (mn == mx) {
            by_index = true;
            continue;
        }
        const double inv = (double)kCBins / (mx - mn);
        for (int i = tid; i < kCBins; i += kCThreads) sh.hist[i] = 0u;
        __syncthreads();
        for (uint32_t c = tid; c < count; c += kCThreads) {
            const double key = by_index ? -(double)sh.idx[c] : sh.val[c];
            atomicAdd(&sh.hist[c_bin(key, mn, inv)], 1u);
        }
        __syncthreads();
        if ((tid >> 6) == 0) {
            int bb;
            uint32_t above;
            c_find_bin(sh.hist, need, bb, above);
            if (lane == 0) {
                sh.bstar = bb;
                sh.above = above;
            }
        }
        __syncthreads();
        const int bstar = sh.bstar;
        need -= sh.above;
        double rv[kCPer];
        int32_t ri[kCPer];
#pragma unroll
        for (int e = 0; e < kCPer; ++e) {
            const uint32_t c = tid + (uint32_t)e * kCThreads;
            rv[e] = c < count ? sh.val[c] : 0.0;
            ri[e] = c < count ? sh.idx[c] : -1;
        }
        if (tid == 0) sh.count = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kCPer; ++e) {
            const uint32_t c = tid + (uint32_t)e * kCThreads;
            if (c < count) {
                const double key = by_index ? -(double)ri[e] : rv[e];
                if (c_bin(key, mn, inv) == bstar) {
                    const uint32_t slot = atomicAdd(&sh.count, 1u);
                    sh.val[slot] = rv[e];
                    sh.idx[slot] = ri[e];
                }
            }
        }
        __syncthreads();
        count = sh.count;
        __syncthreads();
    }
}

// With count <= kCRank: the needL-th best of (val, idx) and the needU-th best
// of (xv, idx) under (value desc, idx asc) -> cut_v and cut_u, from one
// pairwise pass (one thread per (entry, slice of the compared entries), the
// slices' counts summed through LDS).  val, xv and idx are left unchanged.
__device__ __forceinline__ void c_find_kth_pair(CertShared &sh, uint32_t count, int64_t needL,
                                                int64_t needU) {
    const int tid = threadIdx.x;
    const uint32_t ns = c_slices(count);
    if ((uint32_t)tid < ns * count) {
        const uint32_t c = (uint32_t)tid % count, sl = (uint32_t)tid / count;
        const uint32_t o1 = (sl + 1) * count / ns;
        const double xl = sh.val[c], xu = sh.xv[c];
        const int32_t jc = sh.idx[c];
        uint32_t rl = 0, ru = 0, o = sl * count / ns;
        for (; o + 8 <= o1; o += 8) {
            double yl[8], yu[8];
            int32_t yi[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                yl[u] = sh.val[o + u];
                yu[u] = sh.xv[o + u];
                yi[u] = sh.idx[o + u];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                rl += outranks(yl[u], yi[u], xl, jc);
                ru += outranks(yu[u], yi[u], xu, jc);
            }
        }
        for (; o < o1; ++o) {
            const int32_t yi = sh.idx[o];
            rl += outranks(sh.val[o], yi, xl, jc);
            ru += outranks(sh.xv[o], yi, xu, jc);
        }
        sh.hist[tid] = rl;
        sh.hist[kCThreads + tid] = ru;
    }
    __syncthreads();
    for (uint32_t c = tid; c < count; c += kCThreads) {
        int64_t rl = 0, ru = 0;
        for (uint32_t sl = 0; sl < ns; ++sl) {
            rl += sh.hist[sl * count + c];
            ru += sh.hist[kCThreads + sl * count + c];
        }
        if (rl == needL - 1) {
            sh.cut_v = sh.val[c];
            sh.cut_j = sh.idx[c];
        }
        if (ru == needU - 1) sh.cut_u = sh.xv[c];
    }
    __syncthreads();
}

__device__ __forceinline__ double cert_eps(double Eb, double kb, double s) {
    const double e = Eb * kb;
    return e * (1.0 + 1e-9) + 1e-12 * (fabs(s) + e) + 1e-300;
}

// The steps before re-scoring: interval thresholds, then every span is
// certainly in (sh.bitmap, nd of them), certainly out, or uncertain (sh.xs,
// nx of them).  Returns false when the pair needs no ranking at all (kk == 0
// or kk >= n_spans; sel is then written).
template <bool L = false>
__device__ __forceinline__ bool cert_classify(const CertArgs &a, CertShared &sh, int64_t bh,
                                              uint32_t &nx_out, uint32_t &nd_out) {
    const int tid = threadIdx.x;
    const int h = (int)(bh % a.Hkv);
    const int64_t n = a.n_spans;
    const int kk = a.kk;
    const double *shat = a.shat + bh * n;
    const double *kbar = a.kbar + (int64_t)(h / (a.kbar_div > 1 ? a.kbar_div : 1)) * n;
    const double Eb = a.E[bh];
    int32_t *sel = a.sel ? a.sel + bh * a.topk : nullptr;
    if (tid == 0) a.nsel[bh] = kk;
    if (kk == 0 || kk >= n) {
        if (sel)
            for (int64_t i = tid; i < a.topk; i += kCThreads) sel[i] = i < kk ? (int32_t)i : -1;
        return false;
    }
    // the ranked spans (every span, or the pair's candidates: m <= kCCap),
    // their approximate scores and error bounds, every load in flight
    // together (kCPer per thread), kept in registers for the three passes
    // below; position c holds span jv
    const int64_t m = ranked_of<L>(a, sh, bh);
    double sv[kCPer], ev[kCPer];
    int32_t jv[kCPer];
    {
        double kv[kCPer];
#pragma unroll
        for (int e = 0; e < kCPer; ++e) {
            const int64_t c = tid + (int64_t)e * kCThreads;
            jv[e] = c < m ? span_of<L>(a, sh, bh, c) : 0;
        }
#pragma unroll
        for (int e = 0; e < kCPer; ++e) {
            sv[e] = shat[jv[e]];
            kv[e] = kbar[jv[e]];
        }
#pragma unroll
        for (int e = 0; e < kCPer; ++e) ev[e] = cert_eps(Eb, kv[e], sv[e]);
    }
    // tau_L = kk-th largest lower end, tau_U = (kk+1)-th largest upper end
    // (order: value desc, span index asc).  Up to kCRank ranked spans both
    // come from one pairwise pass (lower ends in val, upper ends in xv, which
    // the re-scoring fills only later); beyond that, histogram levels each.
    double tauL, tauU;
    if (m <= kCRank) {
#pragma unroll
        for (int e = 0; e < kCPer; ++e) {
            const int64_t c = tid + (int64_t)e * kCThreads;
            if (c < m) {
                sh.val[c] = sv[e] - ev[e];
                sh.xv[c] = sv[e] + ev[e];
                sh.idx[c] = jv[e];
            }
        }
        __syncthreads();
        c_find_kth_pair(sh, (uint32_t)m, kk, kk + 1);
        tauL = sh.cut_v;
        tauU = sh.cut_u;
    } else {
#pragma unroll
        for (int e = 0; e < kCPer; ++e) {
            const int64_t c = tid + (int64_t)e * kCThreads;
            if (c < m) {
                sh.val[c] = sv[e] - ev[e];
                sh.idx[c] = jv[e];
            }
        }
        __syncthreads();
        c_find_kth(sh, (uint32_t)m, kk);
        tauL = sh.cut_v;
#pragma unroll
        for (int e = 0; e < kCPer; ++e) {
            const int64_t c = tid + (int64_t)e * kCThreads;
            if (c < m) {
                sh.val[c] = sv[e] + ev[e];
                sh.idx[c] = jv[e];
            }
        }
        __syncthreads();
        c_find_kth(sh, (uint32_t)m, kk + 1);
        tauU = sh.cut_v;
    }
    // certainly in: lower end above tau_U.  Possibly in: upper end >= tau_L.
    // Bits and uncertain entries are by position.
    const int nwords = (int)((m + 31) / 32);
    for (int i = tid; i < nwords; i += kCThreads) sh.bitmap[i] = 0u;
    if (tid == 0) {
        sh.nd = 0;
        sh.nx = 0;
    }
    __syncthreads();
#pragma unroll
    for (int ei = 0; ei < kCPer; ++ei) {
        const int64_t c = tid + (int64_t)ei * kCThreads;
        if (c >= m) continue;
        const double s = sv[ei], e = ev[ei];
        if (s - e > tauU) {
            atomicOr(&sh.bitmap[c >> 5], 1u << (c & 31));
            atomicAdd(&sh.nd, 1u);
        } else if (s + e >= tauL) {
            const uint32_t slot = atomicAdd(&sh.nx, 1u);
            sh.xs[slot] = (int32_t)c;
        }
    }
    __syncthreads();
    nx_out = sh.nx;
    nd_out = sh.nd;
    return true;
}

// Exact block scores of the nx uncertain spans in sh.xs, over the query
// halves qh0 .. qh1 - 1.  This workgroup takes the work items first,
// first + step, ... of each half; each item's sum goes to
// gpart[query half * kCCap + item], and cert_gather_xv adds them up.
template <int NT, class Sh>
__device__ __forceinline__ void cert_rescore(const CertArgs &a, Sh &sh, int64_t bh, uint32_t nx,
                                             int qh0, int qh1, uint32_t first, uint32_t step,
                                             double *gpart) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int b = (int)(bh / a.Hkv), h = (int)(bh % a.Hkv);
    // exact (fp64) block scores of the uncertain spans.  The block's
    // q_eff is staged in LDS 32 queries at a time; a work item is (span,
    // part): lane = (token tl of a 32-token chunk, query half sub) and it
    // accumulates the 8 dot products of its token with queries
    // sub*16 + part*8 .. +8 in fp64 (the products of a bf16 key with q_eff
    // are exact), the per-query maxima over the 32 token lanes come from a
    // transpose-reduce, and the 16 maxima are summed.  Up to kCSplit
    // uncertain spans, the two parts of a span are separate items (the
    // 2 nx equal items then spread evenly over the waves), their sums added
    // later in a fixed order; beyond that one wave takes both parts of its
    // span in turn.
    const int tl = lane & 31, sub = lane >> 5;
    const bool split = nx <= (uint32_t)kCSplit;
    const uint32_t n_items = split ? 2 * nx : nx;
    const unsigned char *kh = a.k + (int64_t)(h / a.rep) * a.sh_bytes;
    for (int qh = qh0; qh < qh1; ++qh) {
        const double *qsrc = a.qeff + ((int64_t)h * a.n_q + (int64_t)b * kQB + qh * 32) * kD;
        {
            constexpr int QPT = 32 * kD / NT;
            double qv[QPT];
#pragma unroll
            for (int u = 0; u < QPT; ++u) qv[u] = qsrc[tid + u * NT];
#pragma unroll
            for (int u = 0; u < QPT; ++u) sh.qblk[tid + u * NT] = qv[u];
        }
        __syncthreads();
        for (uint32_t it = first; it < n_items; it += step) {
            const uint32_t x = split ? it >> 1 : it;
            const int p0 = split ? (int)(it & 1) : 0, p1 = split ? p0 + 1 : 2;
            const int64_t j = span_at(a, bh, sh.xs[x]);
            const int64_t tb = a.mid_lo + j * a.S, te = min(tb + (int64_t)a.S, a.mid_hi);
            double total = 0.0;
            for (int part = p0; part < p1; ++part) {
                double best[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) best[i] = -INFINITY;
                for (int64_t c0 = tb; c0 < te; c0 += 32) {
                    const int64_t t = c0 + tl;
                    const bool ok = t < te;
                    const unsigned char *krow = kh + (ok ? t : tb) * a.st_bytes;
                    double acc[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] = 0.0;
                    // the key row in two halves of 8 chunks, each half's
                    // loads issued together before its arithmetic
                    for (int half = 0; half < 2; ++half) {
                        uint4 kraw[8];
#pragma unroll
                        for (int cc = 0; cc < 8; ++cc) kraw[cc] = ld16(krow + (half * 8 + cc) * 16);
#pragma unroll
                        for (int cc = 0; cc < 8; ++cc) {
                            const uint32_t w4[4] = {kraw[cc].x, kraw[cc].y, kraw[cc].z, kraw[cc].w};
                            double kd[8];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                kd[2 * e] = (double)__uint_as_float(w4[e] << 16);
                                kd[2 * e + 1] = (double)__uint_as_float(w4[e] & 0xffff0000u);
                            }
                            // the 8 channels of 4 queries per LDS batch
                            // (sixteen 16-byte reads completed together;
                            // the lanes of a half-wave read the same
                            // addresses)
                            const uint32_t qc = lds_addr(sh.qblk + (sub * 16 + part * 8) * kD +
                                                         (half * 8 + cc) * 8);
                            static_assert(kD * 8 == 1024, "query rows 1024 bytes apart");
#pragma unroll
                            for (int i0 = 0; i0 < 8; i0 += 4) {
                                uint4 qv[16];
                                lds_read16_rows4(qc + (uint32_t)(i0 * kD * 8), qv);
#pragma unroll
                                for (int u = 0; u < 16; ++u) {
                                    const double q0 = __hiloint2double((int)qv[u].y, (int)qv[u].x);
                                    const double q1 = __hiloint2double((int)qv[u].w, (int)qv[u].z);
                                    const int i = i0 + (u >> 2), e = 2 * (u & 3);
                                    acc[i] = fma(q0, kd[e], acc[i]);
                                    acc[i] = fma(q1, kd[e + 1], acc[i]);
                                }
                            }
                        }
                    }
                    if (ok)
#pragma unroll
                        for (int i = 0; i < 8; ++i) best[i] = fmax(best[i], acc[i]);
                }
                // transpose-max over the 32 token lanes: after the steps
                // over lane^16, ^8, ^4 lane l keeps query slot (l/4)%8,
                // then the maxima over lane^2 and lane^1 complete it
#pragma unroll
                for (int o = 16, nv = 8; o >= 4; o >>= 1, nv >>= 1) {
                    const bool upper = (tl & o) != 0;
#pragma unroll
                    for (int i = 0; i < nv / 2; ++i) {
                        const double keep = upper ? best[i + nv / 2] : best[i];
                        const double send = upper ? best[i] : best[i + nv / 2];
                        best[i] = fmax(keep, __shfl_xor(send, o));
                    }
                }
                best[0] = fmax(best[0], __shfl_xor(best[0], 2));
                best[0] = fmax(best[0], __shfl_xor(best[0], 1));
                // sum of the 16 maxima (lanes with tl % 4 == 0 hold one each)
                double v = (tl & 3) ? 0.0 : best[0];
                for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
                total = part == p0 ? v : total + v;
            }
            if (lane == 0) gpart[qh * kCCap + it] = total;
        }
        __syncthreads();
    }
}

// One query per pair: the exact (fp64) scores of the nx uncertain spans into
// sh.xv, a wave per span; lane (token tl of a 32-token chunk, channel half kb)
// takes 64 products of its token (bf16 values are exact in fp64), the halves
// are added across lane^32 and the maximum taken over the 32 token lanes.
template <bool L = false>
__device__ __forceinline__ void cert_rescore_one(const CertArgs &a, CertShared &sh, int64_t bh,
                                                 uint32_t nx) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = (int)(bh % a.Hkv);
    const uint16_t *qh = a.q1 + (int64_t)h * kD;
    for (int c = tid; c < kD; c += kCThreads) sh.q1[c] = bf16_to_f64(qh[c]);
    __syncthreads();
    const int tl = lane & 31, kb = lane >> 5;
    const unsigned char *kh = a.k + (int64_t)(h / a.rep) * a.sh_bytes;
    for (uint32_t x = wave; x < nx; x += kCWaves) {
        const int64_t j = span_of<L>(a, sh, bh, sh.xs[x]);
        const int64_t tb = a.mid_lo + j * a.S, te = min(tb + (int64_t)a.S, a.mid_hi);
        double best = -INFINITY;
        for (int64_t c0 = tb; c0 < te; c0 += 32) {
            const int64_t t = c0 + tl;
            const bool ok = t < te;
            const unsigned char *krow = kh + (ok ? t : tb) * a.st_bytes + kb * (kD / 2) * 2;
            uint4 kr[8];
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) kr[cc] = ld16(krow + cc * 16);
            double acc = 0.0;
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                const uint32_t w4[4] = {kr[cc].x, kr[cc].y, kr[cc].z, kr[cc].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = kb * (kD / 2) + cc * 8 + 2 * e;
                    acc = fma(sh.q1[c], (double)__uint_as_float(w4[e] << 16), acc);
                    acc = fma(sh.q1[c + 1], (double)__uint_as_float(w4[e] & 0xffff0000u), acc);
                }
            }
            acc += __shfl_xor(acc, 32);
            if (ok) best = fmax(best, acc);
        }
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) best = fmax(best, __shfl_xor(best, o));
        if (lane == 0) sh.xv[x] = best + 0.0;
    }
    __syncthreads();
}

// sh.xv from the per-item sums of the re-scoring, in a fixed order: the two
// parts of a span, then the two query halves.
__device__ __forceinline__ void cert_gather_xv(CertShared &sh, const double *gpart, uint32_t nx) {
    const bool split = nx <= (uint32_t)kCSplit;
    for (uint32_t x = threadIdx.x; x < nx; x += kCThreads) {
        double xv = 0.0;
        for (int qh = 0; qh < 2; ++qh) {
            const double *p = gpart + qh * kCCap;
            const double v = split ? p[2 * x] + p[2 * x + 1] : p[x];
            xv = (qh == 0 ? v : xv + v) + 0.0;
        }
        sh.xv[x] = xv;
    }
    __syncthreads();
}

// The need best uncertain spans (sh.xv, sh.xs) join the certain ones in
// sh.bitmap, and the bitmap is compacted in span order into sel.
template <bool L = false>
__device__ __forceinline__ void cert_finish(const CertArgs &a, CertShared &sh, int64_t bh,
                                            uint32_t nx, int64_t need) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kk = a.kk;
    const int nwords = (int)((ranked_of<L>(a, sh, bh) + 31) / 32);
    int32_t *sel = a.sel ? a.sel + bh * a.topk : nullptr;
    if (need > 0) {
        // ranked by exact score, then span index
        for (uint32_t x = tid; x < nx; x += kCThreads) {
            sh.val[x] = sh.xv[x];
            sh.idx[x] = span_of<L>(a, sh, bh, sh.xs[x]);
        }
        __syncthreads();
        c_find_kth(sh, nx, need);
        const double cv = sh.cut_v;
        const int32_t cj = sh.cut_j;
        for (uint32_t x = tid; x < nx; x += kCThreads) {
            const double v = sh.xv[x];
            const int32_t c = sh.xs[x];
            const int32_t j = sh.idx[x];
            if (v > cv || (v == cv && j <= cj)) atomicOr(&sh.bitmap[c >> 5], 1u << (c & 31));
        }
        __syncthreads();
    }
    // ordered compaction of the bitmap (at most 128 words, one per thread)
    const uint32_t wv = tid < nwords ? sh.bitmap[tid] : 0u;
    {
        uint32_t x = __popc(wv);
        const uint32_t v0 = x;
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (lane == 63) sh.red_u[wave] = x;
        __syncthreads();
        if (tid == 0) {
            uint32_t acc = 0;
            for (int w = 0; w < kCWaves; ++w) {
                sh.scan[w] = acc;
                acc += sh.red_u[w];
            }
        }
        __syncthreads();
        uint32_t pos = sh.scan[wave] + x - v0;
        if (sel) {
            uint32_t w = wv;
            while (w) {
                const int bit = __ffs(w) - 1;
                w &= w - 1;
                if (pos < (uint32_t)a.topk) sel[pos] = span_of<L>(a, sh, bh, tid * 32 + bit);
                ++pos;
            }
            for (int64_t i = (int64_t)kk + tid; i < a.topk; i += kCThreads) sel[i] = -1;
        }
    }
}

// ---------------------------------------------------------------------------
// Candidates of a decode pair with one selection per query head and more than
// kCCap spans (k_certify_heads, first part), from the group maxima the
// scoring kernel wrote (largest approximate score and largest key-norm bound
// of every 32 spans, one of each per wave).  The (kk+1)-th largest group maximum tau is a lower bound of the
// (kk+1)-th largest score c' (the kk+1 best groups hold kk+1 distinct spans at
// or above it), so theta = tau - 2 eps_max <= c' - 2 eps_max and every span
// scoring below theta is certainly out (see k_cert_candidates).  Only the
// groups whose maximum reaches theta are read; their spans at or above theta,
// ascending, are the candidates.  More than kGCand such groups or kCCap such
// spans flag the pair for the exact fallback.
// ---------------------------------------------------------------------------
typedef double double4v __attribute__((ext_vector_type(4)));
constexpr int kGThreads = 512;
constexpr int kGPT = 8;                       // group maxima per thread
constexpr int kGMaxGroups = kGThreads * kGPT; // 4096 groups (131,072 spans)
constexpr int kGCand = 256;                   // candidate groups

// k_certify_heads: grid (pairs), 512 threads (kCThreads == kGThreads): the
// candidates as above, then k_certify_one's steps.  The candidate spans go to
// LDS (sh.cand) and
// the classification, re-scoring and output read them there, so neither the
// list nor its count makes a round trip through global memory.  The pair's
// gover flag is written as before; a flagged pair returns at once (the exact
// fallback selects it).
__global__ __launch_bounds__(kCThreads) void k_certify_heads(CertArgs a) {
    __shared__ CertShared sh;
    __shared__ uint32_t hist[kCBins];
    __shared__ double red[3][kGThreads / 64];
    __shared__ uint32_t wsum[kGThreads / 64];
    __shared__ uint32_t wsum8[kGPT][kGThreads / 64];
    __shared__ int32_t cgrp[kGCand];
    __shared__ uint32_t cword[kGCand];
    __shared__ int32_t s_bstar;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int NW = kGThreads / 64;
    const int64_t bh = blockIdx.x;
    const int64_t n = a.n_spans;
    const int64_t m = (n + kGroupH - 1) / kGroupH;
    const int kk = a.kk;
    auto flag_over = [&]() {
        if (tid == 0) a.gover[bh] = 1;
    };
    bool listed = false;         // candidates in sh.cand (else nothing to rank)
    if (kk == 0 || kk >= n) {
        if (tid == 0) a.gover[bh] = 0;
    } else if (m > kGMaxGroups || (int64_t)kk + 1 > m) {
        flag_over();
        return;
    } else {
        listed = true;
    }
    if (listed) {
    const double *gm = a.gmx + bh * m * kWavesM;      // [groups][4 waves]
    const double *gk = a.gkb + bh * m * kWavesM;
    double gv[kGPT];
    double mn = INFINITY, mx = -INFINITY, km = 0.0;
#pragma unroll
    for (int r = 0; r < kGPT; ++r) {
        const int64_t g = (int64_t)r * kGThreads + tid;
        if (g < m) {
            const double4v x = *(const double4v *)(gm + g * kWavesM);
            const double4v y = *(const double4v *)(gk + g * kWavesM);
            gv[r] = fmax(fmax(x[0], x[1]), fmax(x[2], x[3]));
            km = fmax(km, fmax(fmax(y[0], y[1]), fmax(y[2], y[3])));
        } else {
            gv[r] = -INFINITY;
        }
    }
#pragma unroll
    for (int r = 0; r < kGPT; ++r)
        if ((int64_t)r * kGThreads + tid < m) {
            mn = fmin(mn, gv[r]);
            mx = fmax(mx, gv[r]);
        }
    for (int o = 32; o > 0; o >>= 1) {
        mn = fmin(mn, __shfl_xor(mn, o));
        mx = fmax(mx, __shfl_xor(mx, o));
        km = fmax(km, __shfl_xor(km, o));
    }
    if (lane == 0) {
        red[0][wave] = mn;
        red[1][wave] = mx;
        red[2][wave] = km;
    }
    for (int i = tid; i < kCBins; i += kGThreads) hist[i] = 0u;
    __syncthreads();
    mn = INFINITY;
    mx = -INFINITY;
    km = 0.0;
    for (int w = 0; w < NW; ++w) {
        mn = fmin(mn, red[0][w]);
        mx = fmax(mx, red[1][w]);
        km = fmax(km, red[2][w]);
    }
    // tau: the smallest group maximum in the bins at or above the bin that
    // holds the (kk+1)-th largest (every maximum equal: tau = that value)
    double tau = mn;
    if (mn < mx) {
        const double inv = (double)kCBins / (mx - mn);
#pragma unroll
        for (int r = 0; r < kGPT; ++r)
            if ((int64_t)r * kGThreads + tid < m) atomicAdd(&hist[c_bin(gv[r], mn, inv)], 1u);
        __syncthreads();
        if (wave == 0) {
            int bb;
            uint32_t above;
            c_find_bin(hist, (int64_t)kk + 1, bb, above);
            if (lane == 0) s_bstar = bb;
        }
        __syncthreads();
        const int bstar = s_bstar;
        double lo = INFINITY;
#pragma unroll
        for (int r = 0; r < kGPT; ++r)
            if ((int64_t)r * kGThreads + tid < m && c_bin(gv[r], mn, inv) >= bstar) lo = fmin(lo, gv[r]);
        for (int o = 32; o > 0; o >>= 1) lo = fmin(lo, __shfl_xor(lo, o));
        __syncthreads();
        if (lane == 0) red[0][wave] = lo;
        __syncthreads();
        tau = INFINITY;
        for (int w = 0; w < NW; ++w) tau = fmin(tau, red[0][w]);
    }
    // eps_max bounds every span's cert_eps: E * Kbar with the largest key
    // norm, and the relative term with a magnitude that covers every span
    // at or above theta (spans below it stay below theta + eps_max)
    const double Eb = a.E[bh];
    const double eb = Eb * km * (1.0 + 1e-9) * (1.0 + 1e-9) + 1e-300;
    const double A = fabs(tau) + fmax(fabs(mn), fabs(mx)) + 4.0 * eb;
    const double eps_max = eb + 1e-12 * (A + eb) + 1e-300;
    double theta = tau - 2.0 * eps_max;
    theta -= 4e-16 * fabs(theta) + 1e-300;

    // candidate groups: maximum >= theta, ascending
    // (every batch's ballots first, then one barrier for all their counts)
    uint64_t bal[kGPT];
#pragma unroll
    for (int r = 0; r < kGPT; ++r) {
        const int64_t g = (int64_t)r * kGThreads + tid;
        bal[r] = __ballot(g < m && gv[r] >= theta);
        if (lane == 0) wsum8[r][wave] = (uint32_t)__popcll(bal[r]);
    }
    __syncthreads();
    uint32_t ncg = 0;
#pragma unroll
    for (int r = 0; r < kGPT; ++r) {
        uint32_t off = 0, tot = 0;
        for (int w = 0; w < NW; ++w) {
            off += w < wave ? wsum8[r][w] : 0u;
            tot += wsum8[r][w];
        }
        const uint32_t pos = ncg + off + (uint32_t)__popcll(bal[r] & ((1ull << lane) - 1ull));
        if (((bal[r] >> lane) & 1ull) && pos < (uint32_t)kGCand)
            cgrp[pos] = (int32_t)((int64_t)r * kGThreads + tid);
        ncg += tot;
    }
    __syncthreads();
    if (ncg > (uint32_t)kGCand) {
        flag_over();
        return;
    }
    // their spans >= theta: half a wave per group, one 32-bit word each
    const int half = tid >> 5, hl = tid & 31;
    constexpr int NH2 = kGThreads / 32;           // groups per round
    for (uint32_t c0 = 0; c0 < ncg; c0 += NH2) {
        const uint32_t c = c0 + half;
        const int64_t jj = c < ncg ? (int64_t)cgrp[c] * kGroupH + hl : 0;
        const bool keep = c < ncg && jj < n && a.shat[bh * n + jj] >= theta;
        const uint64_t bal = __ballot(keep);
        if (hl == 0 && c < ncg) cword[c] = (uint32_t)(bal >> (lane & 32));
    }
    __syncthreads();
    // ordered compaction of the words (ncg <= 256 <= threads)
    const uint32_t wv = tid < (int)ncg ? cword[tid] : 0u;
    uint32_t x = __popc(wv);
    const uint32_t v0 = x;
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    __syncthreads();
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    uint32_t base = 0, total = 0;
    for (int w = 0; w < NW; ++w) {
        base += w < wave ? wsum[w] : 0u;
        total += wsum[w];
    }
    if (total > (uint32_t)kCCap) {
        flag_over();
        return;
    }
    uint32_t pos = base + x - v0;
    uint32_t w = wv;
    while (w) {
        const int bit = __ffs(w) - 1;
        w &= w - 1;
        sh.cand[pos++] = cgrp[tid] * kGroupH + bit;
    }
    if (tid == 0) {
        sh.ncand = total;
        a.gover[bh] = 0;
    }
    }   // listed
    __syncthreads();
    uint32_t nx, nd;
    if (!cert_classify<true>(a, sh, bh, nx, nd)) return;
    const int64_t need = (int64_t)a.kk - nd;
    if (need > 0) cert_rescore_one<true>(a, sh, bh, nx);
    __syncthreads();
    cert_finish<true>(a, sh, bh, nx, need);
}

// ---------------------------------------------------------------------------
// k_cert_candidates: grid (pairs), 1024 threads; only when a pair has more
// spans than the certification ranks on chip (kCCap).  Let c' be the
// (kk+1)-th largest approximate score and eps_max the largest error bound of
// the pair.  Every span scoring below c' - 2 eps_max has an upper end below
// c' - eps_max, which is below the kk-th largest lower end and below the
// (kk+1)-th largest upper end (the kk + 1 best approximate scores keep their
// ends above c' - eps_max and c'): such spans are certainly out, and leaving
// them out of the ranking changes neither threshold.  So the certification
// ranks only the spans scoring at least theta = m* - 2 eps_max, with m* the
// smallest score in the histogram bin holding c' (m* <= c').  They are listed
// in ascending span order; more than kCCap of them (massive near-ties) flag
// the pair for the exact fallback (k_score_block on the VALU, then k_topk).
// Passes over the pair's scores: range, histogram, m*, ordered compaction.
// ---------------------------------------------------------------------------
constexpr int kPThreads = 1024;
constexpr int kPWaves = kPThreads / 64;

__global__ __launch_bounds__(kPThreads) void k_cert_candidates(CertArgs a) {
    __shared__ uint32_t hist[kCBins];
    __shared__ double red[3][kPWaves];
    __shared__ uint32_t wsum[kPWaves];
    __shared__ int32_t s_bstar;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % a.Hkv);
    const int64_t n = a.n_spans;
    const int kk = a.kk;
    if (kk == 0 || kk >= n) {
        // nothing to rank (k_certify_head writes the selection)
        if (tid == 0) {
            a.gncand[bh] = 0;
            a.gover[bh] = 0;
        }
        return;
    }
    const double *shat = a.shat + bh * n;
    const double *kbar = a.kbar + (int64_t)(h / (a.kbar_div > 1 ? a.kbar_div : 1)) * n;

    // range of the scores, largest key norm
    double mn = INFINITY, mx = -INFINITY, km = 0.0;
    for (int64_t j = tid; j < n; j += kPThreads) {
        const double x = shat[j];
        mn = fmin(mn, x);
        mx = fmax(mx, x);
        km = fmax(km, kbar[j]);
    }
    for (int o = 32; o > 0; o >>= 1) {
        mn = fmin(mn, __shfl_xor(mn, o));
        mx = fmax(mx, __shfl_xor(mx, o));
        km = fmax(km, __shfl_xor(km, o));
    }
    if (lane == 0) {
        red[0][wave] = mn;
        red[1][wave] = mx;
        red[2][wave] = km;
    }
    __syncthreads();
    mn = INFINITY;
    mx = -INFINITY;
    km = 0.0;
    for (int w = 0; w < kPWaves; ++w) {
        mn = fmin(mn, red[0][w]);
        mx = fmax(mx, red[1][w]);
        km = fmax(km, red[2][w]);
    }
    if (mn == mx) {
        // every span scores the same: all of them would be ranked
        if (tid == 0) {
            a.gncand[bh] = 0;
            a.gover[bh] = 1;
        }
        return;
    }
    // cert_eps grows with the key norm and with |score|
    const double eps_max = cert_eps(a.E[bh], km, fmax(fabs(mn), fabs(mx)));
    const double inv = (double)kCBins / (mx - mn);

    // histogram, and the bin b* holding the (kk+1)-th largest score
    for (int i = tid; i < kCBins; i += kPThreads) hist[i] = 0u;
    __syncthreads();
    for (int64_t j = tid; j < n; j += kPThreads) atomicAdd(&hist[c_bin(shat[j], mn, inv)], 1u);
    __syncthreads();
    if (wave == 0) {
        int bb;
        uint32_t above;
        c_find_bin(hist, (int64_t)kk + 1, bb, above);
        if (lane == 0) s_bstar = bb;
    }
    __syncthreads();
    const int bstar = s_bstar;

    // m*: the smallest score in bin b*
    double mb = INFINITY;
    for (int64_t j = tid; j < n; j += kPThreads) {
        const double x = shat[j];
        if (c_bin(x, mn, inv) == bstar) mb = fmin(mb, x);
    }
    for (int o = 32; o > 0; o >>= 1) mb = fmin(mb, __shfl_xor(mb, o));
    __syncthreads();
    if (lane == 0) red[0][wave] = mb;
    __syncthreads();
    mb = INFINITY;
    for (int w = 0; w < kPWaves; ++w) mb = fmin(mb, red[0][w]);
    // theta = m* - 2 eps_max, lowered past the subtraction's rounding
    double theta = mb - 2.0 * eps_max;
    theta -= 4e-16 * fabs(theta) + 1e-300;

    // the spans scoring >= theta, in ascending order
    int32_t *cand = a.gcand + bh * kCCap;
    uint32_t total = 0;
    for (int64_t base = 0; base < n; base += kPThreads) {
        const int64_t j = base + tid;
        const bool keep = j < n && shat[j] >= theta;
        const uint64_t bal = __ballot(keep);
        const uint32_t before = (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wsum[wave] = (uint32_t)__popcll(bal);
        __syncthreads();
        uint32_t off = 0, tot = 0;
        for (int w = 0; w < kPWaves; ++w) {
            const uint32_t c = wsum[w];
            off += w < wave ? c : 0u;
            tot += c;
        }
        const uint32_t pos = total + off + before;
        if (keep && pos < (uint32_t)kCCap) cand[pos] = (int32_t)j;
        total += tot;
        __syncthreads();
    }
    if (tid == 0) {
        const bool over = total > (uint32_t)kCCap;
        a.gncand[bh] = over ? 0u : total;
        a.gover[bh] = over ? 1u : 0u;
    }
}

// Certification in three kernels: the classification per pair, the
// re-scoring spread over a.R workgroups per pair (grid pairs x R, a pair's
// workgroups adjacent so that they land on different XCDs), then the final
// ranking per pair.  State passes through gxs / gbits / gcnt / gpart.
__global__ __launch_bounds__(kCThreads) void k_certify_head(CertArgs a) {
    __shared__ CertShared sh;
    const int64_t bh = blockIdx.x;
    uint32_t *cnt = a.gcnt + bh * 4;
    uint32_t nx, nd;
    if (a.gover && a.gover[bh]) {
        // too many candidates: the exact fallback selects this pair
        if (threadIdx.x == 0) cnt[2] = 1u;
        return;
    }
    if (!cert_classify(a, sh, bh, nx, nd)) {
        if (threadIdx.x == 0) cnt[2] = 1u;
        return;
    }
    for (uint32_t i = threadIdx.x; i < nx; i += kCThreads) a.gxs[bh * kCCap + i] = sh.xs[i];
    const int nwords = (int)((ranked(a, bh) + 31) / 32);
    for (int i = threadIdx.x; i < nwords; i += kCThreads) a.gbits[bh * (kCCap / 32) + i] = sh.bitmap[i];
    if (threadIdx.x == 0) {
        cnt[0] = nx;
        cnt[1] = nd;
        cnt[2] = 0u;
    }
}

// What the split re-scoring keeps on chip (a third of CertShared, so that
// several of its workgroups share a CU).
struct RescoreShared {
    int32_t xs[kCCap];
    double qblk[32 * kD];
};

constexpr int kRThreads = 256;      // k_rescore: 4 waves, three workgroups per CU
constexpr int kRWaves = kRThreads / 64;

__global__ __launch_bounds__(kRThreads, 3) void k_rescore(CertArgs a) {
    __shared__ RescoreShared sh;
    const int64_t bh = blockIdx.x / a.R;
    const uint32_t r = blockIdx.x % a.R;
    const uint32_t *cnt = a.gcnt + bh * 4;
    if (cnt[2]) return;
    const uint32_t nx = cnt[0], nd = cnt[1];
    if ((int64_t)a.kk - nd <= 0) return;
    // workgroup r takes query half r % 2 and its share of that half's items
    const int qh = (int)(r & 1);
    const uint32_t first = (r >> 1) * kRWaves, step = (uint32_t)(a.R / 2) * kRWaves;
    const uint32_t n_items = nx <= (uint32_t)kCSplit ? 2 * nx : nx;
    if (first >= n_items) return;
    for (uint32_t i = threadIdx.x; i < nx; i += kRThreads) sh.xs[i] = a.gxs[bh * kCCap + i];
    __syncthreads();
    cert_rescore<kRThreads>(a, sh, bh, nx, qh, qh + 1, first + (threadIdx.x >> 6), step,
                            a.gpart + bh * 2 * kCCap);
}

// One query per pair (a decode step per query head): classification, fp64
// re-scoring of the uncertain spans and ranking in one workgroup per pair.
__global__ __launch_bounds__(kCThreads) void k_certify_one(CertArgs a) {
    __shared__ CertShared sh;
    const int64_t bh = blockIdx.x;
    if (a.gover && a.gover[bh]) return;      // too many candidates: the exact fallback selects
    uint32_t nx, nd;
    if (!cert_classify(a, sh, bh, nx, nd)) return;
    const int64_t need = (int64_t)a.kk - nd;
    if (need > 0) cert_rescore_one(a, sh, bh, nx);
    __syncthreads();
    cert_finish(a, sh, bh, nx, need);
}

__global__ __launch_bounds__(kCThreads) void k_certify_tail(CertArgs a) {
    __shared__ CertShared sh;
    const int64_t bh = blockIdx.x;
    const uint32_t *cnt = a.gcnt + bh * 4;
    if (cnt[2]) return;
    const uint32_t nx = cnt[0], nd = cnt[1];
    const int64_t need = (int64_t)a.kk - nd;
    const int nwords = (int)((ranked(a, bh) + 31) / 32);
    for (int i = threadIdx.x; i < nwords; i += kCThreads) sh.bitmap[i] = a.gbits[bh * (kCCap / 32) + i];
    if (need > 0) {
        for (uint32_t i = threadIdx.x; i < nx; i += kCThreads) sh.xs[i] = a.gxs[bh * kCCap + i];
        __syncthreads();
        if (a.qpb == 1)
            cert_rescore_one(a, sh, bh, nx);
        else
            cert_gather_xv(sh, a.gpart + bh * 2 * kCCap, nx);
    }
    __syncthreads();
    cert_finish(a, sh, bh, nx, need);
}

}  // namespace

bool mfma_block_path(const Geom &g) {
    return g.dtype == 0 && g.d == kD && g.block_q == kQB && g.S % kTile == 0 && g.n_spans > 0;
}

// Workgroups that re-score one (block, KV head) pair's uncertain spans: an
// even number (half per query half) that gives the grid about 1024 four-wave
// workgroups, at least 2 and at most 16 (32 waves per query half: up to 16
// uncertain spans re-scored in one round).
int cert_ways(const Geom &g) {
    const int64_t pairs = (int64_t)g.n_blk * g.Hkv;
    const int64_t r = 1024 / pairs;
    return (int)((r < 2 ? 2 : r > 16 ? 16 : r) & ~(int64_t)1);
}

size_t cert_split_bytes(const Geom &g) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t pairs = (size_t)g.n_blk * g.Hkv;
    return al(pairs * kCCap * sizeof(int32_t)) + al(pairs * (kCCap / 32) * sizeof(uint32_t)) +
           al(pairs * 4 * sizeof(uint32_t)) + al(pairs * 2 * kCCap * sizeof(double));
}

// More spans than the certification ranks on chip: candidate lists, their
// counts, the overflow flags and the exact fallback's group maxima.
size_t cert_many_bytes(const Geom &g) {
    if (g.n_spans <= kCCap) return 0;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t pairs = (size_t)g.n_blk * g.Hkv;
    return al(pairs * kCCap * sizeof(int32_t)) + 2 * al(pairs * sizeof(uint32_t)) +
           al(pairs * (size_t)score_groups(g) * sizeof(double));
}

size_t mfma_ws_bytes(const Geom &g) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return al((size_t)g.Hkv * g.n_q * 256 * sizeof(uint16_t)) +       // [hi|lo]
           al((size_t)g.Hkv * g.n_q * kD * sizeof(double)) +           // q_eff
           al((size_t)g.n_blk * g.Hkv * sizeof(double)) +              // E
           al((size_t)g.Hkv * g.n_spans * sizeof(double)) +            // key-norm maxima
           cert_split_bytes(g) +                                       // certification state
           cert_many_bytes(g);                                         // candidates, fallback
}

hipError_t launch_score_select_mfma(const Geom &g, const void *q, const void *k,
                                    double *span_scores, int32_t *sel, int32_t *n_sel,
                                    void *ws, int num_cu, hipStream_t s,
                                    hipEvent_t ev_begin, hipEvent_t ev_end) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    char *p = (char *)ws;
    uint16_t *qhl = (uint16_t *)p;
    p += al((size_t)g.Hkv * g.n_q * 256 * sizeof(uint16_t));
    double *qeff = (double *)p;
    p += al((size_t)g.Hkv * g.n_q * kD * sizeof(double));
    double *E = (double *)p;
    p += al((size_t)g.n_blk * g.Hkv * sizeof(double));
    double *kbar = (double *)p;
    p += al((size_t)g.Hkv * g.n_spans * sizeof(double));

    PrepArgs pa{(const uint16_t *)q, qhl, qeff, E, g.Hq, g.Hkv, g.g, g.n_q};
    hipLaunchKernelGGL(k_qprep, dim3(g.n_blk, g.Hkv), dim3(kPrepThreads), 0, s, pa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    MfmaArgs ma;
    ma.k = (const unsigned char *)k;
    ma.qhl = qhl;
    ma.out = span_scores;
    ma.kbar = kbar;
    ma.sh_bytes = g.sh * g.esize;
    ma.st_bytes = g.st * g.esize;
    ma.mid_lo = g.mid_lo;
    ma.mid_hi = g.mid_hi;
    ma.n_spans = g.n_spans;
    ma.S = g.S;
    ma.Hkv = g.Hkv;
    ma.rep = g.rep;
    ma.n_q = g.n_q;
    ma.n_blk = g.n_blk;
    const int n_qg = (g.n_blk + kWavesM - 1) / kWavesM;
    const int64_t units = (int64_t)n_qg * g.Hkv;
    int64_t NR = ((int64_t)(num_cu > 0 ? num_cu : 256) * 2 + units - 1) / units;
    const int64_t NRmin = (g.n_spans + kMaxSpansWG - 1) / kMaxSpansWG;
    if (NR < NRmin) NR = NRmin;
    if (NR > g.n_spans) NR = g.n_spans;
    if (NR < 1) NR = 1;
    ma.NR = (int)NR;
    e = launch_struct(k_score_mfma, dim3((unsigned)(units * NR)), dim3(256), 0, s, ma, ev_begin,
                      ev_end);
    if (e != hipSuccess) return e;

    CertArgs ca;
    ca.shat = span_scores;
    ca.kbar = kbar;
    ca.E = E;
    ca.qeff = qeff;
    ca.k = (const unsigned char *)k;
    ca.sel = sel;
    ca.nsel = n_sel;
    ca.sh_bytes = ma.sh_bytes;
    ca.st_bytes = ma.st_bytes;
    ca.mid_lo = g.mid_lo;
    ca.mid_hi = g.mid_hi;
    ca.n_spans = g.n_spans;
    ca.S = g.S;
    ca.Hkv = g.Hkv;
    ca.rep = g.rep;
    ca.n_q = g.n_q;
    ca.kk = g.k_sel;
    ca.topk = g.topk;
    ca.R = cert_ways(g);
    ca.qpb = kQB;
    ca.q1 = nullptr;
    ca.kbar_div = 1;
    ca.gmx = nullptr;
    ca.gkb = nullptr;
    const unsigned pairs = (unsigned)(g.n_blk * g.Hkv);
    ca.gxs = (int32_t *)p;
    p += al((size_t)pairs * kCCap * sizeof(int32_t));
    ca.gbits = (uint32_t *)p;
    p += al((size_t)pairs * (kCCap / 32) * sizeof(uint32_t));
    ca.gcnt = (uint32_t *)p;
    p += al((size_t)pairs * 4 * sizeof(uint32_t));
    ca.gpart = (double *)p;
    p += al((size_t)pairs * 2 * kCCap * sizeof(double));
    const bool many = g.n_spans > kCCap;
    double *fb_gmax = nullptr;
    ca.gcand = nullptr;
    ca.gncand = nullptr;
    ca.gover = nullptr;
    if (many) {
        ca.gcand = (int32_t *)p;
        p += al((size_t)pairs * kCCap * sizeof(int32_t));
        ca.gncand = (uint32_t *)p;
        p += al((size_t)pairs * sizeof(uint32_t));
        ca.gover = (uint32_t *)p;
        p += al((size_t)pairs * sizeof(uint32_t));
        fb_gmax = (double *)p;
        if ((e = launch_struct(k_cert_candidates, dim3(pairs), dim3(kPThreads), 0, s, ca)) !=
            hipSuccess)
            return e;
    }
    if ((e = launch_struct(k_certify_head, dim3(pairs), dim3(kCThreads), 0, s, ca)) != hipSuccess)
        return e;
    if ((e = launch_struct(k_rescore, dim3(pairs * ca.R), dim3(kRThreads), 0, s, ca)) != hipSuccess)
        return e;
    if ((e = launch_struct(k_certify_tail, dim3(pairs), dim3(kCThreads), 0, s, ca)) != hipSuccess)
        return e;
    if (!many) return hipSuccess;
    // pairs flagged in gover: exact fp64 span scores on the VALU (overwriting
    // their approximations) and the ordinary top-k; the other pairs' workgroups
    // return at once
    if ((e = launch_score(g, q, k, span_scores, fb_gmax, num_cu, s, nullptr, nullptr, ca.gover)) !=
        hipSuccess)
        return e;
    return launch_topk(g, span_scores, fb_gmax, sel, n_sel, s, ca.gover);
}

bool heads_mfma_path(const Geom &g) {
    return g.dtype == 0 && g.d == kD && g.block_q == 1 && g.n_q == 1 && g.g == 1 &&
           g.rep >= 2 && g.rep <= 32 && g.S % kTile == 0 && g.n_spans > 0 && !g.lens && !g.seg;
}

size_t heads_ws_bytes(const Geom &g) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t ng = (size_t)((g.n_spans + kGroupH - 1) / kGroupH);
    return al((size_t)(g.Hkv / g.rep) * g.n_spans * sizeof(double)) + // key-norm bounds, per KV head
           al((size_t)g.Hkv * sizeof(double)) +                        // E
           2 * al((size_t)g.Hkv * ng * kWavesM * sizeof(double)) +     // group maxima per wave
           cert_many_bytes(g);                                         // candidates, fallback
}

hipError_t launch_score_select_heads(const Geom &g, const void *q, const void *k,
                                     double *span_scores, int32_t *sel, int32_t *n_sel,
                                     void *ws, int num_cu, hipStream_t s,
                                     hipEvent_t ev_begin, hipEvent_t ev_end) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t ng = (size_t)((g.n_spans + kGroupH - 1) / kGroupH);
    char *p = (char *)ws;
    double *kbar = (double *)p;
    p += al((size_t)(g.Hkv / g.rep) * g.n_spans * sizeof(double));
    double *E = (double *)p;
    p += al((size_t)g.Hkv * sizeof(double));
    double *gmx = (double *)p;
    p += al((size_t)g.Hkv * ng * kWavesM * sizeof(double));
    double *gkb = (double *)p;
    p += al((size_t)g.Hkv * ng * kWavesM * sizeof(double));

    HeadsArgs ha;
    ha.k = (const unsigned char *)k;
    ha.q = (const uint16_t *)q;
    ha.out = span_scores;
    ha.kbar = kbar;
    ha.E = E;
    ha.gmx = gmx;
    ha.gkb = gkb;
    ha.sh_bytes = g.sh * g.esize;
    ha.st_bytes = g.st * g.esize;
    ha.mid_lo = g.mid_lo;
    ha.mid_hi = g.mid_hi;
    ha.n_spans = g.n_spans;
    ha.S = g.S;
    ha.NH = g.rep;
    ha.Hp = g.Hkv / g.rep;
    // two workgroups per CU, split evenly over the KV heads (runs of whole groups)
    int64_t P = ((int64_t)(num_cu > 0 ? num_cu : 256) * 2 + ha.Hp - 1) / ha.Hp;
    if (P > (int64_t)ng) P = (int64_t)ng;
    if (P < 1) P = 1;
    ha.P = (int)P;
    hipError_t e = launch_struct(k_score_heads_mfma, dim3((unsigned)(ha.Hp * P)), dim3(256), 0, s,
                                 ha, ev_begin, ev_end);
    if (e != hipSuccess) return e;

    CertArgs ca = {};
    ca.shat = span_scores;
    ca.kbar = kbar;
    ca.E = E;
    ca.qeff = nullptr;
    ca.k = (const unsigned char *)k;
    ca.sel = sel;
    ca.nsel = n_sel;
    ca.sh_bytes = ha.sh_bytes;
    ca.st_bytes = ha.st_bytes;
    ca.mid_lo = g.mid_lo;
    ca.mid_hi = g.mid_hi;
    ca.n_spans = g.n_spans;
    ca.S = g.S;
    ca.Hkv = g.Hkv;
    ca.rep = g.rep;
    ca.n_q = 1;
    ca.kk = g.k_sel;
    ca.topk = g.topk;
    ca.qpb = 1;
    ca.q1 = (const uint16_t *)q;
    ca.gmx = gmx;
    ca.gkb = gkb;
    ca.kbar_div = g.rep;
    const unsigned pairs = (unsigned)(g.n_blk * g.Hkv);
    const bool many = g.n_spans > kCCap;
    double *fb_gmax = nullptr;
    if (many) {
        ca.gcand = (int32_t *)p;
        p += al((size_t)pairs * kCCap * sizeof(int32_t));
        ca.gncand = (uint32_t *)p;
        p += al((size_t)pairs * sizeof(uint32_t));
        ca.gover = (uint32_t *)p;
        p += al((size_t)pairs * sizeof(uint32_t));
        fb_gmax = (double *)p;
        if ((e = launch_struct(k_certify_heads, dim3(pairs), dim3(kCThreads), 0, s, ca)) !=
            hipSuccess)
            return e;
    } else if ((e = launch_struct(k_certify_one, dim3(pairs), dim3(kCThreads), 0, s, ca)) !=
               hipSuccess) {
        return e;
    }
    if (!many) return hipSuccess;
    // flagged pairs: exact fp64 scores on the VALU, then the ordinary top-k
    if ((e = launch_score(g, q, k, span_scores, fb_gmax, num_cu, s, nullptr, nullptr, ca.gover)) !=
        hipSuccess)
        return e;
    return launch_topk(g, span_scores, fb_gmax, sel, n_sel, s, ca.gover);
}

}  // namespace rea
