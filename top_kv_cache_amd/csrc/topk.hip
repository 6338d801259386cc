// topk.hip - step 1b: keep the k highest-scoring spans per (block, KV head).
//
// ReAttention keeps the top-k middle segments by score (OpenReview
// discussion, "Decoding Phase" pseudocode: idx_recall = score.topk; the NIAH
// reply's settings use 127 spans of 32 tokens).  Order used here: higher score
// first, equal scores -> lower span index first.  The selection is emitted in
// ascending span order, which is the order the spans take in the window.
//
// One 512-thread workgroup per (block, KV head).  The scoring kernel also
// wrote the maximum of every group of 32 consecutive spans.  Fast path (at
// most 2048 groups):
//   1. tau, a lower bound of the k-th largest group maximum, from one
//      histogram level over the group maxima: the lower edge of the bin
//      holding the k-th largest (lowered by far more than the binning's
//      rounding), below every maximum in that bin and the ones above.  It also bounds the
//      k-th largest score from below (the k best groups hold k distinct
//      scores), so every selected span scores >= tau and lies in a group
//      whose maximum is >= tau; at most 256 such groups are accepted (more
//      only with massive ties).  With at most 4096 spans every span score is
//      held in registers instead: the same level is taken over the span
//      scores themselves (when k is close to the group count the group bound
//      keeps most spans, the span bound about k of them), and the spans
//      scoring >= tau are the candidates of step 3 without step 2;
//   2. the spans of those groups with score >= tau (all spans scoring >= tau)
//      are loaded into LDS; when the decode scorer also wrote each group's
//      second and third largest scores and the spans of its top two, a
//      candidate group whose third largest is below tau holds at most those
//      two, taken from registers, and only the other groups' span scores
//      are read (usually none: no second round trip to memory);
//   3. with at most 192 of them, each one's rank among them (score desc,
//      index asc) is its global rank: ranks < k are kept and each kept span is
//      written at the count of kept indices below its own.  Otherwise the
//      cutoff e* (the k-th best) is found in LDS by histogram levels; span j
//      is selected iff score_j > score* or (score_j == score* and j <= j*);
//      each candidate group becomes one 32-bit word of a bitmap over the
//      spans, and one block scan over the words writes the indices in
//      ascending order.
// More groups (token level), or more candidate groups than the fast path
// holds: the large path takes the same steps with the group maxima held in
// registers (up to 32,768 groups, fp32 rounded up) or streamed, up to 8192
// candidate groups and 8192 candidate spans, the cutoff always by histogram
// levels and the output from one selection word per candidate group.
// Histogram level: 2048 equal-width bins between the candidates' min and max
// (on the large path's first level: between tau and the largest group
// maximum, which hold every candidate), bin = floor((x - min) * (2048 /
// (max - min))) in fp64 -- monotone in x, so bins are ordered; only the bin
// holding the k-th best survives.  Once all survivors share one score the
// order is by index, so the level key becomes the negated index.  At most 64
// survivors are ranked pairwise.  Otherwise a generic path makes the same
// decisions with passes over all scores in global memory.
#include "rea_internal.h"

#include <math.h>

namespace rea {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kGroup = 32;
constexpr int kMaxGroups = 2048;
constexpr int kCandCap = 8192;
constexpr int kPerThread = kCandCap / kThreads;             // 16
constexpr int kBins = 2048;
constexpr int kRankMax = 64;
constexpr int kMaxCandGroups = kCandCap / kGroup;        // 256
constexpr int kPairCap = 192;       // candidates ranked pairwise (else histogram levels)
constexpr int kSmallPer = 8;        // spans per thread below which tau comes from the spans

struct FastShared {
    double val[kCandCap];
    int32_t idx[kCandCap];
    double gval[kMaxGroups];
    int32_t gidx[kMaxGroups];
    uint32_t hist[kBins];
    uint32_t bitmap[kMaxGroups];
    int32_t cgrp[kMaxCandGroups];
    int32_t cxgrp[kMaxCandGroups];      // candidate groups whose span scores are read
};

// generic path state
constexpr int kGBins = 4096;
constexpr int kGCap = 2048;
constexpr int kGMaxLevels = 12;
struct GenericShared {
    uint32_t hist[kGBins];
    double cand_v[kGCap];
    int32_t cand_j[kGCap];
    double lev_mn[kGMaxLevels];
    double lev_inv[kGMaxLevels];
    int32_t lev_bin[kGMaxLevels];
};

// large path state (many groups, or many candidate groups)
constexpr int kLGroups = 8192;      // candidate groups held, ascending
static_assert(8 * kWaves == 64, "one wave scans the slice counts of a batch");
struct LargeShared {
    double val[kCandCap];
    int32_t idx[kCandCap];
    uint32_t hist[kBins];
    int32_t cgrp[kLGroups];
    uint32_t wcnt[8 * kWaves];          // per (batch slot, wave), or per wave
    uint32_t wpre[8 * kWaves + 1];
};

struct Common {
    double red_d[2][kWaves];
    uint32_t red_u[kWaves];
    uint32_t scan[kWaves + 1];
    uint32_t count;
    // candidate counters of the fast paths, cleared before a barrier that
    // comes anyway, so that no barrier is spent on clearing them
    uint32_t cgroups, cspans, cxgroups;
    uint32_t nkept, ndrop;              // pairwise ranking: kept / dropped candidates
    uint32_t above;
    int32_t bstar;
    int32_t found;
    int32_t cut_j;
    double cut_v;
};

__device__ __forceinline__ int bin_of(double x, double mn, double inv, int nbins) {
    const double f = floor((x - mn) * inv);
    if (!(f > 0.0)) return 0;                       // also x == mn with inv == inf
    if (f >= (double)(nbins - 1)) return nbins - 1;
    return (int)f;
}

// Workgroup min / max / sum; every thread gets the results.
// LDS slots for the flagged items of U per-lane flags, appended at *counter:
// one atomic per wave (the wave's flags are counted with ballots), not one per
// item, so thousands of appends do not serialise on one LDS address.  Every
// lane of the wave must take part.
template <int U>
__device__ __forceinline__ void wave_append(uint32_t *counter, const bool (&flag)[U],
                                            uint32_t (&slot)[U]) {
    const int lane = threadIdx.x & 63;
    unsigned long long bal[U];
    uint32_t pre[U], tot = 0;
#pragma unroll
    for (int e = 0; e < U; ++e) {
        bal[e] = __ballot(flag[e]);
        pre[e] = tot;
        tot += (uint32_t)__popcll(bal[e]);
    }
    uint32_t base = 0;
    if (lane == 0 && tot) base = atomicAdd(counter, tot);
    base = (uint32_t)__shfl((int)base, 0);
#pragma unroll
    for (int e = 0; e < U; ++e)
        slot[e] = base + pre[e] +
                  __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal[e], 0u));
}

__device__ __forceinline__ void block_minmax_count(Common &cm, double &mn, double &mx, uint32_t &cnt) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int o = 32; o > 0; o >>= 1) {
        mn = fmin(mn, __shfl_xor(mn, o));
        mx = fmax(mx, __shfl_xor(mx, o));
        cnt += __shfl_xor(cnt, o);
    }
    if (lane == 0) {
        cm.red_d[0][wave] = mn;
        cm.red_d[1][wave] = mx;
        cm.red_u[wave] = cnt;
    }
    __syncthreads();
    mn = INFINITY;
    mx = -INFINITY;
    cnt = 0;
    for (int w = 0; w < kWaves; ++w) {
        mn = fmin(mn, cm.red_d[0][w]);
        mx = fmax(mx, cm.red_d[1][w]);
        cnt += cm.red_u[w];
    }
    __syncthreads();
}

// Workgroup min / max with one barrier (the LDS slots must not be written
// again before a later barrier).
__device__ __forceinline__ void block_minmax1(Common &cm, double &mn, double &mx) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int o = 32; o > 0; o >>= 1) {
        mn = fmin(mn, __shfl_xor(mn, o));
        mx = fmax(mx, __shfl_xor(mx, o));
    }
    if (lane == 0) {
        cm.red_d[0][wave] = mn;
        cm.red_d[1][wave] = mx;
    }
    __syncthreads();
    mn = INFINITY;
    mx = -INFINITY;
    for (int w = 0; w < kWaves; ++w) {
        mn = fmin(mn, cm.red_d[0][w]);
        mx = fmax(mx, cm.red_d[1][w]);
    }
}

// A value at or below every x with bin_of(x, mn, inv, kBins) >= b: the bin's
// lower edge, lowered by far more than the rounding of the binning.
__device__ __forceinline__ double bin_floor(double mn, double mx, int b) {
    const double e = mn + (mx - mn) * ((double)b / (double)kBins);
    return e - 1e-12 * (fabs(mn) + fabs(mx) + fabs(e)) - 1e-300;
}

// Exclusive prefix sum of v over the workgroup in thread order.
__device__ __forceinline__ uint32_t block_excl_sum(Common &cm, uint32_t v, uint32_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) cm.red_u[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t acc = 0;
        for (int w = 0; w < kWaves; ++w) {
            cm.scan[w] = acc;
            acc += cm.red_u[w];
        }
        cm.scan[kWaves] = acc;
    }
    __syncthreads();
    const uint32_t r = cm.scan[wave] + x - v;
    *total = cm.scan[kWaves];
    __syncthreads();
    return r;
}

// Wave 0 finds the bin holding the need-th best (bins counted from the top);
// sets cm.bstar and cm.above (candidates in higher bins).  Each lane sums a run
// of nbins/64 bins (read in a lane-rotated order, so the 64 lanes hit distinct
// banks), a suffix scan over the lanes picks the run, and the wave then scans
// that run's bins in parallel.
__device__ __forceinline__ void find_bin(Common &cm, const uint32_t *hist, int nbins, int64_t need) {
    const int lane = threadIdx.x & 63;
    if ((threadIdx.x >> 6) == 0) {
        const int bpl = nbins / 64;           // 32 or 64
        uint32_t own = 0;
        for (int i = 0; i < bpl; ++i) own += hist[lane * bpl + ((i + lane) & (bpl - 1))];
        uint32_t suf = own;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_down(suf, o);
            if (lane + o < 64) suf += y;
        }
        const uint32_t after = suf - own;       // candidates in runs above this lane's
        const unsigned long long hit =
            __ballot((int64_t)after < need && need <= (int64_t)suf);
        const int L = __ffsll((long long)hit) - 1;
        const uint32_t aboveL = __shfl(after, L);
        // bins of run L, top first: lane i < bpl holds bin L*bpl + bpl-1-i
        const uint32_t c = lane < bpl ? hist[L * bpl + bpl - 1 - lane] : 0u;
        uint32_t pre = c;                       // inclusive prefix from the top
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(pre, o);
            if (lane >= o) pre += y;
        }
        const unsigned long long at =
            __ballot(lane < bpl && (int64_t)(aboveL + pre) >= need);
        const int i = __ffsll((long long)at) - 1;
        if (lane == i) {
            cm.bstar = L * bpl + bpl - 1 - i;
            cm.above = aboveL + pre - c;
        }
    }
    __syncthreads();
}

// The need-th best of `count` (<= kCandCap) LDS entries (val, idx) under
// (val desc, idx asc); result in cm.cut_v / cm.cut_j.  Reorders and shrinks
// the arrays.  With lo0 < hi0 (every value known to lie in [lo0, hi0]) the
// first histogram level spans that range instead of a min / max pass.
__device__ __forceinline__ void find_kth(Common &cm, uint32_t *hist, double *val, int32_t *idx,
                         uint32_t count, int64_t need, double lo0 = 0.0, double hi0 = -1.0) {
    const int tid = threadIdx.x;
    bool by_index = false;
    bool given = lo0 < hi0;
    for (;;) {
        if (count <= (uint32_t)kRankMax) {
            // pairwise ranks; 8 entries are read per step so the LDS latency
            // is paid once per 8 comparisons
            for (uint32_t c = tid; c < count; c += kThreads) {
                const double x = val[c];
                const int32_t jc = idx[c];
                int rank = 0;
                uint32_t o = 0;
                for (; o + 8 <= count; o += 8) {
                    double y[8];
                    int32_t yi[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        y[u] = val[o + u];
                        yi[u] = idx[o + u];
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) rank += outranks(y[u], yi[u], x, jc);
                }
                for (; o < count; ++o) rank += outranks(val[o], idx[o], x, jc);
                if (rank == need - 1) {
                    cm.cut_v = x;
                    cm.cut_j = jc;
                }
            }
            __syncthreads();
            return;
        }
        double mn = lo0, mx = hi0;
        if (!given) {
            mn = INFINITY;
            mx = -INFINITY;
            uint32_t dummy = 0;
            for (uint32_t c = tid; c < count; c += kThreads) {
                const double k = by_index ? -(double)idx[c] : val[c];
                mn = fmin(mn, k);
                mx = fmax(mx, k);
            }
            block_minmax_count(cm, mn, mx, dummy);
            if (mn == mx) {      // every survivor has this score: order by index
                by_index = true;
                continue;
            }
        }
        given = false;
        const double inv = (double)kBins / (mx - mn);
        for (int i = tid; i < kBins; i += kThreads) hist[i] = 0u;
        __syncthreads();
        for (uint32_t c0 = 0; c0 < count; c0 += 4 * kThreads) {
            double k[4];             // (4 reads issued before the atomics)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t c = c0 + e * kThreads + tid;
                const uint32_t cc = c < count ? c : 0u;
                k[e] = by_index ? -(double)idx[cc] : val[cc];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (c0 + e * kThreads + tid < count) atomicAdd(&hist[bin_of(k[e], mn, inv, kBins)], 1u);
        }
        __syncthreads();
        find_bin(cm, hist, kBins, need);
        const int bstar = cm.bstar;
        need -= cm.above;
        // keep the survivors (bin == bstar)
        double rv[kPerThread];
        int32_t ri[kPerThread];
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) {
            const uint32_t c = tid + (uint32_t)e * kThreads;
            rv[e] = c < count ? val[c] : 0.0;
            ri[e] = c < count ? idx[c] : -1;
        }
        if (tid == 0) cm.count = 0;
        __syncthreads();
        bool keep[kPerThread];
        uint32_t slot[kPerThread];
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) {
            const uint32_t c = tid + (uint32_t)e * kThreads;
            const double k = by_index ? -(double)ri[e] : rv[e];
            keep[e] = c < count && bin_of(k, mn, inv, kBins) == bstar;
        }
        wave_append(&cm.count, keep, slot);
#pragma unroll
        for (int e = 0; e < kPerThread; ++e)
            if (keep[e]) {
                val[slot[e]] = rv[e];
                idx[slot[e]] = ri[e];
            }
        __syncthreads();
        count = cm.count;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// large path: the fast path's decisions with the group maxima streamed from
// global memory (any number of groups), for at most kLGroups candidate groups
// and kCandCap candidate spans.  Returns false (uniformly, before writing any
// output) when either bound is exceeded.
// ---------------------------------------------------------------------------
// Streams the group maxima in batches of 8 per thread (one batch covers
// 8 * kThreads consecutive groups, e-major), calling f(i, x) for each.
template <typename F>
__device__ __forceinline__ void for_each_gmax(const double *gm, int64_t m, F f) {
    constexpr int B = 16;                       // loads in flight per thread
    const int tid = threadIdx.x;
    for (int64_t b0 = 0; b0 < m; b0 += B * kThreads) {
        double x[B];
#pragma unroll
        for (int e = 0; e < B; ++e) {
            const int64_t i = b0 + e * kThreads + tid;
            x[e] = gm[i < m ? i : m - 1];
        }
#pragma unroll
        for (int e = 0; e < B; ++e) {
            const int64_t i = b0 + e * kThreads + tid;
            if (i < m) f(i, x[e]);
        }
    }
}

// The group maxima as steps 1-2 of the large path read them: streamed from
// global memory (16 loads in flight per thread) each time, or, when there are
// at most kGReg * kThreads of them, loaded once into registers as fp32 values
// rounded up.  In registers wave w holds the contiguous chunk of kGReg * 64
// groups from w * kGReg * 64 on, lane l of it the groups chunk + k * 64 + l
// (k < kGReg): every load is coalesced, and ascending group order is (wave,
// k, lane) order.  Rounding up is monotone, so with the rounded values step 1
// finds a tau_r <= the rounded kk-th largest maximum, and the fp32 value just
// below tau_r is <= the exact kk-th largest maximum: a valid bound.  Step 2
// then keeps every group whose rounded maximum reaches it, a superset of the
// groups whose exact maximum does.
constexpr int kGReg = 64;
template <bool kRegs> struct GmaxSource {
    const double *gm;
    int64_t m;
    float reg[kRegs ? kGReg : 1];
    __device__ static int64_t chunk() { return (int64_t)(threadIdx.x >> 6) * (kGReg * 64); }
    __device__ void load() {
        if constexpr (kRegs) {
            constexpr int C = 16;                   // loads in flight per thread
            const int64_t c0 = chunk() + (threadIdx.x & 63);
#pragma unroll
            for (int k0 = 0; k0 < kGReg; k0 += C) {
                if (chunk() + (int64_t)k0 * 64 >= m) break;   // (wave-uniform) past the end
                double x[C];
#pragma unroll
                for (int k = 0; k < C; ++k) {
                    const int64_t i = c0 + (int64_t)(k0 + k) * 64;
                    x[k] = gm[i < m ? i : m - 1];
                }
#pragma unroll
                for (int k = 0; k < C; ++k) reg[k0 + k] = __double2float_ru(x[k]);
            }
        }
    }
    template <typename F> __device__ void each(F f) const {
        if constexpr (kRegs) {
            const int64_t c0 = chunk() + (threadIdx.x & 63);
#pragma unroll
            for (int k = 0; k < kGReg; ++k) {
                const int64_t i = c0 + (int64_t)k * 64;
                // (an empty asm pins the widening to this pass; hoisted out of
                // the passes, 64 doubles would not fit in registers)
                float v = reg[k];
                __asm__ volatile("" : "+v"(v));
                if (i < m) f(i, (double)v);
            }
        } else {
            for_each_gmax(gm, m, f);
        }
    }
    // (streamed only) batch of 8 * kThreads groups from b0:
    // x[e] = gm[b0 + e * kThreads + tid]
    __device__ void batch(int64_t b0, double (&x)[8]) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t i = b0 + e * kThreads + threadIdx.x;
            x[e] = gm[i < m ? i : m - 1];
        }
    }
};

template <bool kRegs>
__device__ __forceinline__ uint32_t large_tau_groups(Common &cm, LargeShared &L, const double *gm,
                                                     int64_t m, int kk, double &tau_out,
                                                     double &max_out) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    GmaxSource<kRegs> src{gm, m, {}};
    src.load();
    // 1. tau: the lower edge of the histogram bin holding the kk-th largest
    //    maximum (a lower bound of the kk-th largest span score)
    double mn = INFINITY, mx = -INFINITY;
    src.each([&](int64_t, double x) {
        mn = fmin(mn, x);
        mx = fmax(mx, x);
    });
    block_minmax1(cm, mn, mx);
    max_out = mx;
    double tau = mn;
    if (mn != mx) {
        const double inv = (double)kBins / (mx - mn);
        for (int i = tid; i < kBins; i += kThreads) L.hist[i] = 0u;
        __syncthreads();
        src.each([&](int64_t, double x) { atomicAdd(&L.hist[bin_of(x, mn, inv, kBins)], 1u); });
        __syncthreads();
        find_bin(cm, L.hist, kBins, kk);
        tau = bin_floor(mn, mx, cm.bstar);
    }
    if constexpr (kRegs) tau = (double)nextafterf((float)tau, -INFINITY);
    tau_out = tau;
    // 2. candidate groups (maximum >= tau) in ascending order
    if constexpr (kRegs) {
        // each wave counts its chunk's candidates (per lane, then summed over
        // the wave), one prefix over the kWaves counts places the
        // chunks, then each wave writes its candidates in (k, lane) order
        const float tf = (float)tau;          // exact: tau is an fp32 value here
        const int64_t c0 = GmaxSource<true>::chunk() + lane;
        uint32_t cnt = 0;
#pragma unroll
        for (int k = 0; k < kGReg; ++k) cnt += (c0 + (int64_t)k * 64 < m && src.reg[k] >= tf) ? 1u : 0u;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
        if (lane == 0) L.wcnt[wave] = cnt;
        __syncthreads();
        uint32_t off = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t v = L.wcnt[w];
            off += w < wave ? v : 0u;
            total += v;
        }
#pragma unroll
        for (int k = 0; k < kGReg; ++k) {
            const int64_t i = c0 + (int64_t)k * 64;
            const bool keep = i < m && src.reg[k] >= tf;
            const unsigned long long bk = __ballot(keep);
            if (keep) {
                const uint32_t slot = off + __builtin_amdgcn_mbcnt_hi(
                    (uint32_t)(bk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bk, 0u));
                if (slot < (uint32_t)kLGroups) L.cgrp[slot] = (int32_t)i;
            }
            off += (uint32_t)__popcll(bk);
        }
        __syncthreads();
        return total;
    }
    // per batch of 8 * kThreads groups, the count of every (e, wave) slice
    // orders the writes
    uint32_t ncg = 0;
    for (int64_t b0 = 0; b0 < m; b0 += 8 * kThreads) {
        double x[8];
        src.batch(b0, x);
        unsigned long long bal[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t i = b0 + e * kThreads + tid;
            bal[e] = __ballot(i < m && x[e] >= tau);
            if (lane == 0) L.wcnt[e * kWaves + wave] = (uint32_t)__popcll(bal[e]);
        }
        __syncthreads();
        if (wave == 0) {                 // exclusive prefix over the 64 slices
            const uint32_t v = L.wcnt[lane];
            uint32_t incl = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            L.wpre[lane] = incl - v;
            if (lane == 63) L.wpre[64] = incl;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t off = ncg + L.wpre[e * kWaves + wave];
            const unsigned long long bb2 = bal[e];
            if ((bb2 >> lane) & 1ull) {
                const uint32_t below = __builtin_amdgcn_mbcnt_hi(
                    (uint32_t)(bb2 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bb2, 0u));
                const uint32_t slot = off + below;
                if (slot < (uint32_t)kLGroups) L.cgrp[slot] = (int32_t)(b0 + e * kThreads + tid);
            }
        }
        ncg += L.wpre[64];
        __syncthreads();                 // wcnt / wpre are rewritten by the next batch
    }
    return ncg;
}

__device__ __forceinline__ bool large_path(Common &cm, LargeShared &L, const double *sc,
                                           const double *gm, const double *gs, const int32_t *ga,
                                           int64_t n, int64_t m, int kk, int topk, int32_t *sel) {
    const int tid = threadIdx.x, lane = tid & 63;
    double tau, gmx;
    const uint32_t ncg = m <= (int64_t)kGReg * kThreads
                             ? large_tau_groups<true>(cm, L, gm, m, kk, tau, gmx)
                             : large_tau_groups<false>(cm, L, gm, m, kk, tau, gmx);
    if (ncg > (uint32_t)kLGroups) return false;
    if (tid == 0) {
        cm.count = 0;
        cm.above = 0;
    }
    __syncthreads();
    // 3. their spans scoring >= tau.  A candidate is recorded by its position
    //    p = c * 32 + o (o: its offset in candidate group c, the groups
    //    ascending), which orders like its span index.
    //    With the scorer's second largest scores: a group whose second
    //    largest is below tau holds exactly one candidate, its maximum (at
    //    the offset the scorer recorded), appended here without reading the
    //    group; the others are listed (mlist, over the histogram's LDS) and
    //    read span by span below.  More of them than the list holds: every
    //    group is read.
    int32_t *mlist = reinterpret_cast<int32_t *>(L.hist);
    constexpr uint32_t kMList = kBins;
    constexpr int U = 32;                  // groups in flight per half wave below
    constexpr int GPI = kThreads / 32;     // groups per pass (16)
    uint32_t nread = ncg;                  // groups read span by span
    bool listed = false;
    // (a single pass of reads, at most GPI * U groups, is no slower than the
    // pass over the second maxima that would replace it)
    if (gs && ncg > (uint32_t)(GPI * U)) {
        constexpr int V = 8;               // candidate groups per thread and pass
        for (uint32_t c0 = 0; c0 < ncg; c0 += kThreads * V) {
            int32_t gi[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const uint32_t c = c0 + e * kThreads + tid;
                gi[e] = L.cgrp[c < ncg ? c : ncg - 1];
            }
            double v1[V], v2[V];
            int32_t off[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                v1[e] = gm[gi[e]];
                v2[e] = gs[gi[e]];
                off[e] = ga[gi[e]];
            }
            bool single[V];
            uint32_t slot[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const uint32_t c = c0 + e * kThreads + tid;
                // (the maxima tau was taken from are rounded up: check)
                single[e] = c < ncg && v2[e] < tau && v1[e] >= tau;
                if (c < ncg && !(v2[e] < tau)) {
                    const uint32_t k2 = atomicAdd(&cm.above, 1u);
                    if (k2 < kMList) mlist[k2] = (int32_t)c;
                }
            }
            wave_append(&cm.count, single, slot);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                if (single[e] && slot[e] < (uint32_t)kCandCap) {
                    L.val[slot[e]] = v1[e];
                    L.idx[slot[e]] = (int32_t)((c0 + e * kThreads + tid) * kGroup + off[e]);
                }
            }
        }
        __syncthreads();
        nread = cm.above;
        listed = nread <= kMList;
        if (!listed) {
            // too many groups to list: read them all, from no candidates
            nread = ncg;
            __syncthreads();
            if (tid == 0) cm.count = 0;
        }
        __syncthreads();
    }
    // half a wave per group read, U groups in flight
    const int half = tid >> 5, hl = tid & 31;
    for (uint32_t c0 = 0; c0 < nread; c0 += GPI * U) {
        double x[U];
        bool ok[U];
        // (the group index is read unconditionally, clamped, so the LDS reads
        // are issued together and the loads follow without a wait per read)
        uint32_t cv[U];
        int32_t gi[U];
#pragma unroll
        for (int e = 0; e < U; ++e) {
            const uint32_t r = c0 + e * GPI + half;
            const uint32_t rc = r < nread ? r : nread - 1;
            cv[e] = listed ? (uint32_t)mlist[rc] : rc;
        }
#pragma unroll
        for (int e = 0; e < U; ++e) gi[e] = L.cgrp[cv[e]];
#pragma unroll
        for (int e = 0; e < U; ++e) {
            // (span indices are below 2^31: 32-bit offsets from one base)
            const uint32_t r = c0 + e * GPI + half;
            const uint32_t j = (uint32_t)gi[e] * kGroup + hl;
            ok[e] = r < nread && j < (uint64_t)n;
            x[e] = sc[j < (uint64_t)n ? j : (uint32_t)(n - 1)];
        }
        bool keep[U];
        uint32_t slot[U];
#pragma unroll
        for (int e = 0; e < U; ++e) keep[e] = ok[e] && x[e] >= tau;
        wave_append(&cm.count, keep, slot);
#pragma unroll
        for (int e = 0; e < U; ++e) {
            if (keep[e] && slot[e] < (uint32_t)kCandCap) {
                L.val[slot[e]] = x[e];
                L.idx[slot[e]] = (int32_t)(cv[e] * kGroup + hl);
            }
        }
    }
    __syncthreads();
    const uint32_t count = cm.count;
    __syncthreads();
    if (count > (uint32_t)kCandCap) return false;
    // the candidates stay in registers for step 5 (the cutoff search below
    // reorders the LDS copy)
    double rv[kPerThread];
    int32_t rp[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        const uint32_t c = tid + (uint32_t)e * kThreads;
        rv[e] = c < count ? L.val[c] : 0.0;
        rp[e] = c < count ? L.idx[c] : -1;
    }
    __syncthreads();
    // 4. the kk-th best candidate = the cutoff (every candidate lies in
    //    [tau, the largest group maximum]: its score is >= tau and <= its
    //    group's maximum, rounded up or exact)
    find_kth(cm, L.hist, L.val, L.idx, count, kk, tau, gmx);
    const double cv = cm.cut_v;
    const int64_t cj = cm.cut_j;
    // 5. one selection word per candidate group (over the candidate values,
    //    which are no longer needed), set from the candidates in registers
    //    (every selected span is a candidate), then one ordered scan writes
    //    the indices
    uint32_t *words = reinterpret_cast<uint32_t *>(L.val);
    for (uint32_t c = tid; c < ncg; c += kThreads) words[c] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        const int32_t pp = rp[e];
        if (pp >= 0 && (rv[e] > cv || (rv[e] == cv && pp <= cj)))
            atomicOr(&words[pp >> 5], 1u << (pp & 31));
    }
    __syncthreads();
    constexpr int WPT = kLGroups / kThreads;           // 16 words per thread
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
        const uint32_t c = (uint32_t)(tid * WPT + i);
        mine += c < ncg ? (uint32_t)__popc(words[c]) : 0u;
    }
    uint32_t tot;
    uint32_t pos = block_excl_sum(cm, mine, &tot);
    if (sel) {
        for (int i = 0; i < WPT; ++i) {
            const uint32_t c = (uint32_t)(tid * WPT + i);
            if (c >= ncg) break;
            uint32_t w = words[c];
            while (w) {
                const int bit = __ffs(w) - 1;
                w &= w - 1;
                if (pos < (uint32_t)topk) sel[pos] = L.cgrp[c] * kGroup + bit;
                ++pos;
            }
        }
        for (int64_t i = (int64_t)kk + tid; i < topk; i += kThreads) sel[i] = -1;
    }
    return true;
}

// ---------------------------------------------------------------------------
// generic path: the same decisions with global-memory passes (any n)
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool g_candidate(const GenericShared &gs, int nlev, double x) {
    for (int l = 0; l < nlev; ++l) {
        if (x < gs.lev_mn[l]) return false;
        if (bin_of(x, gs.lev_mn[l], gs.lev_inv[l], kGBins) != gs.lev_bin[l]) return false;
    }
    return true;
}

__device__ __forceinline__ void generic_cutoff(Common &cm, GenericShared &gs, const double *sc, int64_t n,
                               int64_t need) {
    const int tid = threadIdx.x;
    int nlev = 0;
    for (;;) {
        double mn = INFINITY, mx = -INFINITY;
        uint32_t cnt = 0;
        for (int64_t j = tid; j < n; j += kThreads) {
            const double x = sc[j];
            if (g_candidate(gs, nlev, x)) {
                mn = fmin(mn, x);
                mx = fmax(mx, x);
                ++cnt;
            }
        }
        block_minmax_count(cm, mn, mx, cnt);
        if (cnt <= (uint32_t)kGCap) {
            if (tid == 0) cm.count = 0;
            __syncthreads();
            for (int64_t j = tid; j < n; j += kThreads) {
                const double x = sc[j];
                if (g_candidate(gs, nlev, x)) {
                    const uint32_t slot = atomicAdd(&cm.count, 1u);
                    gs.cand_v[slot] = x;
                    gs.cand_j[slot] = (int32_t)j;
                }
            }
            __syncthreads();
            const uint32_t m = cm.count;
            for (uint32_t c = tid; c < m; c += kThreads) {
                const double x = gs.cand_v[c];
                const int32_t jc = gs.cand_j[c];
                int64_t rank = 0;
                for (uint32_t o = 0; o < m; ++o) {
                    const double y = gs.cand_v[o];
                    rank += outranks(y, gs.cand_j[o], x, jc);
                }
                if (rank == need - 1) {
                    cm.cut_v = x;
                    cm.cut_j = jc;
                }
            }
            __syncthreads();
            return;
        }
        if (mn == mx || nlev == kGMaxLevels) {
            // equal scores (or an extreme dynamic range): walk the candidates in
            // index order; equal scores are ordered by index, others are ranked
            // against all candidates
            if (tid == 0) cm.found = 0;
            __syncthreads();
            uint32_t before = 0;
            for (int64_t base = 0; base < n; base += kThreads) {
                const int64_t j = base + tid;
                bool f = false;
                double x = 0.0;
                if (j < n) {
                    x = sc[j];
                    f = g_candidate(gs, nlev, x);
                }
                if (mn != mx && f) {
                    int64_t rank = 0;
                    for (int64_t o = 0; o < n; ++o) {
                        const double y = sc[o];
                        rank += g_candidate(gs, nlev, y) && (y > x || (y == x && o < j));
                    }
                    if (rank == need - 1) {
                        cm.cut_v = x;
                        cm.cut_j = (int32_t)j;
                        cm.found = 1;
                    }
                }
                uint32_t tot;
                const uint32_t pre = block_excl_sum(cm, f ? 1u : 0u, &tot);
                if (mn == mx && f && before + pre == (uint32_t)(need - 1)) {
                    cm.cut_v = x;
                    cm.cut_j = (int32_t)j;
                    cm.found = 1;
                }
                before += tot;
                __syncthreads();
                if (cm.found) break;
            }
            __syncthreads();
            return;
        }
        const double inv = (double)kGBins / (mx - mn);
        for (int i = tid; i < kGBins; i += kThreads) gs.hist[i] = 0u;
        __syncthreads();
        for (int64_t j = tid; j < n; j += kThreads) {
            const double x = sc[j];
            if (g_candidate(gs, nlev, x)) atomicAdd(&gs.hist[bin_of(x, mn, inv, kGBins)], 1u);
        }
        __syncthreads();
        find_bin(cm, gs.hist, kGBins, need);
        if (tid == 0) {
            gs.lev_mn[nlev] = mn;
            gs.lev_inv[nlev] = inv;
            gs.lev_bin[nlev] = cm.bstar;
        }
        need -= cm.above;
        ++nlev;
        __syncthreads();
    }
}

__device__ __forceinline__ void generic_emit(Common &cm, const double *sc, int64_t n, int32_t *sel, int topk) {
    const double cv = cm.cut_v;
    const int64_t cj = cm.cut_j;
    uint32_t written = 0;
    for (int64_t base = 0; base < n; base += kThreads) {
        const int64_t j = base + threadIdx.x;
        bool f = false;
        if (j < n) {
            const double x = sc[j];
            f = x > cv || (x == cv && j <= cj);
        }
        uint32_t tot;
        const uint32_t pre = block_excl_sum(cm, f ? 1u : 0u, &tot);
        if (f && written + pre < (uint32_t)topk) sel[written + pre] = (int32_t)j;
        written += tot;
    }
}

// With every span scoring >= tau in (f.val, f.idx)[0..count), count <=
// kPairCap: a candidate's rank among them (score desc, index asc) is its
// global rank, so ranks < kk are kept and each kept span is written at the
// count of kept indices below its own.  Both counts are split into slices of
// the compared range, one thread per (entry, slice), summed through LDS.
__device__ __forceinline__ void rank_pairwise_emit(Common &cm, FastShared &f, uint32_t count, int kk,
                                                   int topk, int32_t *sel) {
    const int tid = threadIdx.x;
    // 3'. every span scoring >= tau is a candidate, so a candidate's rank
    //     among them (score desc, index asc) is its rank among all spans:
    //     rank every candidate pairwise and keep ranks < kk.  The same pass
    //     counts the candidates of lower index, so a kept span's output
    //     position is that count less the dropped candidates below it (or
    //     the kept ones below it, whichever list is shorter).  The counts
    //     are split into slices of the compared range, one thread per
    //     (entry, slice), summed through LDS.
    if (tid == 0) {
        cm.nkept = 0;
        cm.ndrop = 0;
    }
    const uint32_t ns = count ? kThreads / count : 1;         // >= 2 (count <= kPairCap)
    if (tid < ns * count) {
        const uint32_t c = tid % count, sl = tid / count;
        const uint32_t o0 = sl * count / ns, o1 = (sl + 1) * count / ns;
        const double x = f.val[c];
        const int32_t jc = f.idx[c];
        uint32_t rank = 0, lt = 0, o = o0;
        for (; o + 8 <= o1; o += 8) {
            double y[8];
            int32_t yi[8];
#pragma unroll
            for (int u2 = 0; u2 < 8; ++u2) {
                y[u2] = f.val[o + u2];
                yi[u2] = f.idx[o + u2];
            }
#pragma unroll
            for (int u2 = 0; u2 < 8; ++u2) {
                rank += outranks(y[u2], yi[u2], x, jc);
                lt += (uint32_t)(yi[u2] < jc);
            }
        }
        for (; o < o1; ++o) {
            const int32_t yi = f.idx[o];
            rank += outranks(f.val[o], yi, x, jc);
            lt += (uint32_t)(yi < jc);
        }
        f.hist[tid] = rank;
        f.hist[kThreads + tid] = lt;
    }
    __syncthreads();
    uint32_t rank = 0, lt = 0;
    int32_t jt = 0;
    if ((uint32_t)tid < count) {
        for (uint32_t sl = 0; sl < ns; ++sl) {
            rank += f.hist[sl * count + tid];
            lt += f.hist[kThreads + sl * count + tid];
        }
        jt = f.idx[tid];
        // kept indices from the front of gidx, dropped ones from the back
        if (rank < (uint32_t)kk)
            f.gidx[atomicAdd(&cm.nkept, 1u)] = jt;
        else
            f.gidx[kMaxGroups - 1 - atomicAdd(&cm.ndrop, 1u)] = jt;
    }
    __syncthreads();
    if (sel) {
        if ((uint32_t)tid < count && rank < (uint32_t)kk) {
            const uint32_t nk = cm.nkept, nd = cm.ndrop;
            const bool by_drop = nd <= nk;
            const int32_t *lst = by_drop ? &f.gidx[kMaxGroups - nd] : &f.gidx[0];
            const uint32_t nl = by_drop ? nd : nk;
            uint32_t below = 0, o = 0;
            for (; o + 8 <= nl; o += 8) {
                int32_t yi[8];
#pragma unroll
                for (int u2 = 0; u2 < 8; ++u2) yi[u2] = lst[o + u2];
#pragma unroll
                for (int u2 = 0; u2 < 8; ++u2) below += (uint32_t)(yi[u2] < jt);
            }
            for (; o < nl; ++o) below += (uint32_t)(lst[o] < jt);
            sel[by_drop ? lt - below : below] = jt;
        }
        for (int64_t i = (int64_t)kk + tid; i < topk; i += kThreads) sel[i] = -1;
    }
}

// The selection bitmap f.bitmap[0..m) (one word per 32 spans) compacted in
// ascending span order into sel, padded with -1 after kk entries.
__device__ __forceinline__ void emit_bitmap(Common &cm, FastShared &f, int64_t m, int kk, int topk,
                                            int32_t *sel) {
    const int tid = threadIdx.x;
    constexpr int WPT = kMaxGroups / kThreads;      // 4 words per thread
    uint32_t words[WPT];
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
        const int wi = tid * WPT + i;
        words[i] = wi < m ? f.bitmap[wi] : 0u;
        mine += __popc(words[i]);
    }
    uint32_t tot;
    uint32_t pos = block_excl_sum(cm, mine, &tot);
    if (sel) {
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            uint32_t w = words[i];
            while (w) {
                const int bit = __ffs(w) - 1;
                w &= w - 1;
                if (pos < (uint32_t)topk) sel[pos] = (tid * WPT + i) * kGroup + bit;
                ++pos;
            }
        }
        for (int64_t i = (int64_t)kk + tid; i < topk; i += kThreads) sel[i] = -1;
    }
}

struct TopkArgs {
    const double *scores;       // [n_blk * Hkv][n_stride]
    const double *gmax;         // [n_blk * Hkv][m_stride]
    int32_t *sel, *nsel;
    int64_t n_stride, m_stride;
    int topk, Hkv, S;
    // the (block, selection head)'s sequence: length lens[h / hps] (batched
    // decode) or T; its span count and group count follow from G, L and S
    const int64_t *lens;
    int hps;
    int64_t T, G, L;
    // null, or one flag per (block, head): only the flagged pairs are selected
    const uint32_t *only;
    // null, or per group the second largest score and the offset of a maximum
    // (token-level scorer): the large path then reads only the candidate
    // groups with two or more spans at or above its bound
    const double *gsec;
    const int32_t *garg;
    // null, or per group its second and third largest span scores and the
    // spans holding its largest and second largest (decode scorer): a
    // candidate group whose third largest is below the bound then gives its
    // one or two candidates without its span scores being read
    const double *gtop;
    const int32_t *gtopi;
};

__global__ __launch_bounds__(kThreads) void k_topk(TopkArgs ta) {
    __shared__ Common cm;
    __shared__ union {
        FastShared f;
        LargeShared l;
        GenericShared g;
    } u;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bh = blockIdx.x;
    if (ta.only && !ta.only[bh]) return;
    const int h = (int)(bh % ta.Hkv);
    int64_t T = ta.T;
    if (ta.lens) {
        T = ta.lens[h / ta.hps];
        T = T < 1 ? 1 : (T > ta.T ? ta.T : T);
    }
    const SeqGeom sg = seq_geom(T, ta.G, ta.L, ta.S);
    const int64_t n = sg.n_spans, m = sg.n_groups;
    const int topk = ta.topk;
    const int kk = (int)(topk < n ? topk : n);
    const double *sc = ta.scores + bh * ta.n_stride;
    const double *gm = ta.gmax + bh * ta.m_stride;
    int32_t *sel = ta.sel ? ta.sel + bh * topk : nullptr;
    if (tid == 0) ta.nsel[bh] = kk;

    if (kk == 0 || kk >= n) {       // nothing or everything
        if (sel)
            for (int64_t i = tid; i < topk; i += kThreads) sel[i] = i < kk ? (int32_t)i : -1;
        return;
    }

    if (n <= (int64_t)kThreads * kSmallPer) {
        // few spans (at most 128 groups): every span score is held in
        // registers.  tau = the lower edge of the histogram bin holding the
        // kk-th largest score; the candidates are the spans scoring >= tau,
        // taken straight from the registers (the group maxima bound little
        // when k is close to the group count).
        FastShared &f = u.f;
        double sr[kSmallPer];
#pragma unroll
        for (int e = 0; e < kSmallPer; ++e) {
            const int64_t i = tid + (int64_t)e * kThreads;
            sr[e] = sc[i < n ? i : n - 1];
        }
        for (int i = tid; i < kBins; i += kThreads) f.hist[i] = 0u;
        if (tid == 0) cm.cspans = 0;       // ordered by block_minmax1's barrier
        double mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < kSmallPer; ++e)
            if (tid + (int64_t)e * kThreads < n) {
                mn = fmin(mn, sr[e]);
                mx = fmax(mx, sr[e]);
            }
        block_minmax1(cm, mn, mx);
        double tau = mn;
        if (mn < mx) {
            const double inv = (double)kBins / (mx - mn);
#pragma unroll
            for (int e = 0; e < kSmallPer; ++e)
                if (tid + (int64_t)e * kThreads < n) atomicAdd(&f.hist[bin_of(sr[e], mn, inv, kBins)], 1u);
            __syncthreads();
            find_bin(cm, f.hist, kBins, kk);
            tau = bin_floor(mn, mx, cm.bstar);
        }
        bool keep[kSmallPer];
        uint32_t slot[kSmallPer];
#pragma unroll
        for (int e = 0; e < kSmallPer; ++e) keep[e] = tid + (int64_t)e * kThreads < n && sr[e] >= tau;
        wave_append(&cm.cspans, keep, slot);
#pragma unroll
        for (int e = 0; e < kSmallPer; ++e)
            if (keep[e]) {
                f.val[slot[e]] = sr[e];
                f.idx[slot[e]] = tid + e * kThreads;
            }
        __syncthreads();
        const uint32_t count = cm.cspans;   // not cleared again in this call
        if (count <= (uint32_t)kPairCap) {
            rank_pairwise_emit(cm, f, count, kk, topk, sel);
            return;
        }
        // the cutoff among the candidates, then a bitmap over the spans
        find_kth(cm, f.hist, f.val, f.idx, count, kk);
        const double cv = cm.cut_v;
        const int64_t cj = cm.cut_j;
        for (int i = tid; i < m; i += kThreads) f.bitmap[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kSmallPer; ++e) {
            const int32_t j = tid + e * kThreads;
            if (keep[e] && (sr[e] > cv || (sr[e] == cv && j <= cj))) atomicOr(&f.bitmap[j >> 5], 1u << (j & 31));
        }
        __syncthreads();
        emit_bitmap(cm, f, m, kk, topk, sel);
        return;
    }

    if (m <= kMaxGroups) {
        FastShared &f = u.f;
        constexpr int GPT = kMaxGroups / kThreads;         // group maxima per thread (4)
        double gr[GPT];
        double2 g23[GPT];              // second and third largest of the group
        int2 gij[GPT];                 // spans of the largest and second largest
        // (with k above half the candidate-group capacity the first bound
        // usually keeps too many groups and the second bound lists them
        // again, so the top three are not worth loading)
        const bool tops = ta.gtop != nullptr && kk <= kMaxCandGroups / 2;
#pragma unroll
        for (int e = 0; e < GPT; ++e) {
            const int i = tid + e * kThreads;
            const int64_t ic = i < m ? i : m - 1;
            gr[e] = gm[ic];
            if (tops) {
                g23[e] = *(const double2 *)(ta.gtop + 2 * (bh * ta.m_stride + ic));
                gij[e] = *(const int2 *)(ta.gtopi + 2 * (bh * ta.m_stride + ic));
            }
        }
        // 1. tau <= the kk-th largest group maximum (every span competes if
        //    kk > m): one histogram level over the group maxima finds the bin
        //    b* holding the kk-th largest, and tau is b*'s lower edge (bins
        //    are monotone in the value, so every maximum in bins >= b* is at
        //    or above it).
        double tau = -INFINITY;
        if (tid == 0) {
            cm.cgroups = 0;
            cm.cspans = 0;
            cm.cxgroups = 0;
        }
        if (kk > m) __syncthreads();         // else ordered by block_minmax1's barrier
        if (kk <= m) {
            for (int i = tid; i < kBins; i += kThreads) f.hist[i] = 0u;
            double mn = INFINITY, mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < GPT; ++e)
                if (tid + e * kThreads < m) {
                    mn = fmin(mn, gr[e]);
                    mx = fmax(mx, gr[e]);
                }
            block_minmax1(cm, mn, mx);
            if (mn == mx) {
                tau = mn;
            } else {
                const double inv = (double)kBins / (mx - mn);
#pragma unroll
                for (int e = 0; e < GPT; ++e)
                    if (tid + e * kThreads < m) atomicAdd(&f.hist[bin_of(gr[e], mn, inv, kBins)], 1u);
                __syncthreads();
                find_bin(cm, f.hist, kBins, kk);
                tau = bin_floor(mn, mx, cm.bstar);
            }
        }
        // candidate groups: maximum >= tau (about k appends: one LDS atomic
        // each is cheaper than the ballots).  With the groups' top three, a
        // group whose third largest score is below tau holds at most two
        // spans at or above it, its largest and maybe its second, appended
        // here; the others are listed in cxgrp and their span scores read
        // below.
#pragma unroll
        for (int e = 0; e < GPT; ++e) {
            const int i = tid + e * kThreads;
            if (i < m && gr[e] >= tau) {
                const uint32_t slot = atomicAdd(&cm.cgroups, 1u);
                if (slot < (uint32_t)kMaxCandGroups) f.cgrp[slot] = i;
                if (tops) {
                    if (g23[e].y < tau) {
                        const bool two = g23[e].x >= tau;
                        const uint32_t s = atomicAdd(&cm.cspans, two ? 2u : 1u);
                        f.val[s] = gr[e];
                        f.idx[s] = gij[e].x;
                        if (two) {
                            f.val[s + 1] = g23[e].x;
                            f.idx[s + 1] = gij[e].y;
                        }
                    } else {
                        const uint32_t s = atomicAdd(&cm.cxgroups, 1u);
                        if (s < (uint32_t)kMaxCandGroups) f.cxgrp[s] = i;
                    }
                }
            }
        }
        __syncthreads();
        uint32_t ncg = cm.cgroups;
        bool split = tops;              // candidates in place but for the cxgrp groups'
        if (ncg > (uint32_t)kMaxCandGroups && kk <= m) {
            // One histogram level left every group of the kk-th largest
            // maximum's bin above tau, more than the candidate capacity (a
            // wide bin: a few far larger maxima stretch the range).  tau
            // becomes the kk-th largest group maximum itself, ranked among
            // the groups at or above the first bound; it still bounds the
            // kk-th largest span score from below (the kk best groups each
            // hold a span at their maximum).  (Every thread has read ncg
            // before the counters are cleared again: barriers come first.)
            split = false;
            if (tid == 0) cm.count = 0;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < GPT; ++e) {
                const int i = tid + e * kThreads;
                if (i < m && gr[e] >= tau) {
                    const uint32_t slot = atomicAdd(&cm.count, 1u);
                    f.val[slot] = gr[e];
                    f.idx[slot] = i;
                }
            }
            __syncthreads();
            const uint32_t cnt = cm.count;
            __syncthreads();
            find_kth(cm, f.hist, f.val, f.idx, cnt, kk);
            tau = cm.cut_v;
            if (tid == 0) {
                cm.cgroups = 0;
                cm.cspans = 0;
            }
            __syncthreads();
#pragma unroll
            for (int e = 0; e < GPT; ++e) {
                const int i = tid + e * kThreads;
                if (i < m && gr[e] >= tau) {
                    const uint32_t slot = atomicAdd(&cm.cgroups, 1u);
                    if (slot < (uint32_t)kMaxCandGroups) f.cgrp[slot] = i;
                }
            }
            __syncthreads();
            ncg = cm.cgroups;
        }
        constexpr int CPT = kMaxCandGroups / (kThreads / 32);   // 16
        const int half = tid >> 5, hl = tid & 31;
        if (split && ncg <= (uint32_t)kMaxCandGroups) {
            // 2'. the spans scoring >= tau of the groups listed in cxgrp
            //     (usually none or a few); the others are in place already
            const uint32_t ncx = cm.cxgroups;
            if (ncx > 0) {
                double cx[CPT];
                int32_t cjx[CPT];
#pragma unroll
                for (int it = 0; it < CPT; ++it) {
                    const uint32_t c = half + it * (kThreads / 32);
                    cjx[it] = -1;
                    cx[it] = -INFINITY;
                    if (c < ncx) {
                        const int64_t j = (int64_t)f.cxgrp[c] * kGroup + hl;
                        if (j < n) {
                            cjx[it] = (int32_t)j;
                            cx[it] = sc[j];
                        }
                    }
                }
#pragma unroll
                for (int it = 0; it < CPT; ++it) {
                    if (cjx[it] >= 0 && cx[it] >= tau) {
                        const uint32_t slot = atomicAdd(&cm.cspans, 1u);
                        f.val[slot] = cx[it];
                        f.idx[slot] = cjx[it];
                    }
                }
                __syncthreads();
            }
            const uint32_t count = cm.cspans;
            if (count <= (uint32_t)kPairCap) {
                rank_pairwise_emit(cm, f, count, kk, topk, sel);
                return;
            }
            if (count <= (uint32_t)kMaxGroups) {
                // 3''. the cutoff among the candidates (find_kth reorders
                //      val / idx, so they are copied first), then a bitmap over
                //      the spans and the ordered output
                for (uint32_t c = tid; c < count; c += kThreads) {
                    f.gval[c] = f.val[c];
                    f.gidx[c] = f.idx[c];
                }
                for (int i = tid; i < m; i += kThreads) f.bitmap[i] = 0u;
                __syncthreads();
                find_kth(cm, f.hist, f.val, f.idx, count, kk);
                const double cv = cm.cut_v;
                const int64_t cj = cm.cut_j;
                for (uint32_t c = tid; c < count; c += kThreads) {
                    const double x = f.gval[c];
                    const int32_t j = f.gidx[c];
                    if (x > cv || (x == cv && j <= cj)) atomicOr(&f.bitmap[j >> 5], 1u << (j & 31));
                }
                __syncthreads();
                emit_bitmap(cm, f, m, kk, topk, sel);
                return;
            }
            // more candidates than that: the full pass below
            __syncthreads();
            if (tid == 0) cm.cspans = 0;
            __syncthreads();
        }
        if (ncg <= (uint32_t)kMaxCandGroups) {
            // 2. their spans with score >= tau; half a wave per group, every
            //    load issued before any is used (addresses clamped in range)
            double cx[CPT];
            int32_t cjx[CPT];            // span index, -1 where (group, lane) is not a span
#pragma unroll
            for (int it = 0; it < CPT; ++it) {
                const uint32_t c = half + it * (kThreads / 32);
                const int64_t j = (int64_t)f.cgrp[c < ncg ? c : 0] * kGroup + hl;
                cjx[it] = (c < ncg && j < n) ? (int32_t)j : -1;
                cx[it] = sc[j < n ? j : n - 1];
            }
#pragma unroll
            for (int it = 0; it < CPT; ++it) {
                if (cjx[it] >= 0 && cx[it] >= tau) {
                    const uint32_t slot = atomicAdd(&cm.cspans, 1u);
                    f.val[slot] = cx[it];
                    f.idx[slot] = cjx[it];
                }
            }
            __syncthreads();
            const uint32_t count = cm.cspans;   // not cleared again in this call
            if (count <= (uint32_t)kPairCap) {
                // 3'. every span scoring >= tau is a candidate: rank them pairwise
                rank_pairwise_emit(cm, f, count, kk, topk, sel);
                return;
            }
            // 3. cutoff, bitmap words of the candidate groups, ordered output
            find_kth(cm, f.hist, f.val, f.idx, count, kk);
            const double cv = cm.cut_v;
            const int64_t cj = cm.cut_j;
            for (int i = tid; i < m; i += kThreads) f.bitmap[i] = 0u;
            __syncthreads();
#pragma unroll
            for (int it = 0; it < CPT; ++it) {
                const uint32_t c = half + it * (kThreads / 32);
                const bool pick = cjx[it] >= 0 && (cx[it] > cv || (cx[it] == cv && cjx[it] <= cj));
                const unsigned long long bal = __ballot(pick);
                if (hl == 0 && c < ncg) f.bitmap[f.cgrp[c]] = (uint32_t)(bal >> (lane & 32));
            }
            __syncthreads();
            emit_bitmap(cm, f, m, kk, topk, sel);
            (void)wave;
            return;
        }
        // too many groups at or above the bound: the large path below
        __syncthreads();
    }

    if (kk <= m && large_path(cm, u.l, sc, gm, ta.gsec ? ta.gsec + bh * ta.m_stride : nullptr,
                              ta.garg ? ta.garg + bh * ta.m_stride : nullptr, n, m, kk, topk, sel))
        return;

    generic_cutoff(cm, u.g, sc, n, kk);
    if (sel) {
        generic_emit(cm, sc, n, sel, topk);
        for (int64_t i = (int64_t)kk + tid; i < topk; i += kThreads) sel[i] = -1;
    }
}

// Token segments: one workgroup per (block, selection head).  Selected token
// u_i (ascending, middle-relative) covers [a_i, b_i) = [u_i - (seg-1)/2,
// u_i - (seg-1)/2 + seg) clipped to the middle; both ends are non-decreasing
// in i, so token i adds [max(a_i, b_{i-1}), b_i) to the union, and an
// exclusive scan of those lengths places every token of the union in order.
constexpr int kWThreads = 256;

struct WidenArgs {
    const int32_t *sel_tok, *nsel_tok;
    int32_t *sel, *n_sel;
    int k_tok, cap, seg, Hkv;
    const int64_t *lens;
    int hps;
    int64_t T, G, L;
};

__global__ __launch_bounds__(kWThreads) void k_widen(WidenArgs a) {
    __shared__ uint32_t red[kWThreads / 64 + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % a.Hkv);
    int64_t T = a.T;
    if (a.lens) {
        T = a.lens[h / a.hps];
        T = T < 1 ? 1 : (T > a.T ? a.T : T);
    }
    const SeqGeom sg = seq_geom(T, a.G, a.L, 1);
    const int64_t n_mid = sg.n_spans;
    const int kk = a.nsel_tok[bh];
    const int32_t *tok = a.sel_tok + bh * a.k_tok;
    int32_t *out = a.sel ? a.sel + bh * a.cap : nullptr;
    const int left = (a.seg - 1) / 2;
    uint32_t written = 0;
    for (int base = 0; base < kk; base += kWThreads) {
        const int i = base + tid;
        int64_t lo = 0, hi = 0;
        if (i < kk) {
            const int64_t u = tok[i];
            int64_t a0 = u - left, b0 = u - left + a.seg;
            a0 = a0 < 0 ? 0 : a0;
            b0 = b0 > n_mid ? n_mid : b0;
            int64_t prev_b = -1;
            if (i > 0) {
                prev_b = (int64_t)tok[i - 1] - left + a.seg;
                prev_b = prev_b > n_mid ? n_mid : prev_b;
            }
            lo = a0 > prev_b ? a0 : prev_b;
            hi = b0;
        }
        const uint32_t len = hi > lo ? (uint32_t)(hi - lo) : 0u;
        // exclusive scan of len in thread order
        uint32_t x = len;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (lane == 63) red[wave] = x;
        __syncthreads();
        uint32_t off = 0, tot = 0;
        for (int w = 0; w < kWThreads / 64; ++w) {
            off += w < wave ? red[w] : 0u;
            tot += red[w];
        }
        const uint32_t pos = written + off + x - len;
        if (out)
            for (uint32_t e = 0; e < len; ++e)
                if (pos + e < (uint32_t)a.cap) out[pos + e] = (int32_t)(lo + e);
        written += tot;
        __syncthreads();
    }
    if (out)
        for (int64_t i = (int64_t)written + tid; i < a.cap; i += kWThreads) out[i] = -1;
    if (tid == 0) a.n_sel[bh] = (int32_t)(written < (uint32_t)a.cap ? written : (uint32_t)a.cap);
}

}  // namespace

hipError_t launch_widen(const Geom &g, const int32_t *sel_tok, const int32_t *nsel_tok,
                        int32_t *sel, int32_t *n_sel, hipStream_t s) {
    WidenArgs a;
    a.sel_tok = sel_tok;
    a.nsel_tok = nsel_tok;
    a.sel = sel;
    a.n_sel = n_sel;
    a.k_tok = g.k_tok;
    a.cap = g.topk;
    a.seg = g.seg;
    a.Hkv = g.Hkv;
    a.lens = g.lens;
    a.hps = g.hps;
    a.T = g.T;
    a.G = g.G;
    a.L = g.L;
    hipLaunchKernelGGL(k_widen, dim3(g.n_blk * g.Hkv), dim3(kWThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_topk(const Geom &g, const double *span_scores, const double *group_max,
                       int32_t *sel, int32_t *n_sel, hipStream_t s, const uint32_t *only,
                       const double *group_second, const int32_t *group_arg,
                       const double *group_top, const int32_t *group_top_idx) {
    const int nbh = g.n_blk * g.Hkv;
    TopkArgs ta;
    ta.only = only;
    ta.gsec = group_second;
    ta.garg = group_arg;
    ta.gtop = group_top_idx ? group_top : nullptr;
    ta.gtopi = group_top ? group_top_idx : nullptr;
    ta.scores = span_scores;
    ta.gmax = group_max;
    ta.sel = sel;
    ta.nsel = n_sel;
    ta.n_stride = g.n_spans;
    ta.m_stride = score_groups(g);
    ta.topk = g.topk;
    ta.Hkv = g.Hkv;
    ta.S = g.S;
    ta.lens = g.lens;
    ta.hps = g.hps;
    ta.T = g.T;
    ta.G = g.G;
    ta.L = g.L;
    hipLaunchKernelGGL(k_topk, dim3(nbh), dim3(kThreads), 0, s, ta);
    return hipGetLastError();
}

}  // namespace rea
