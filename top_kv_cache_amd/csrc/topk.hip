// topk.hip - step 1b: keep the k highest-scoring spans per (block, KV head).
//
// ReAttention keeps the top-k middle segments by score (OpenReview
// discussion, "Decoding Phase" pseudocode: idx_recall = score.topk; the NIAH
// reply's settings use 127 spans of 32 tokens).  Order used here: higher score
// first, equal scores -> lower span index first.  The selection is emitted in
// ascending span order, which is the order the spans take in the window.
//
// Algorithm (one 1024-thread workgroup per (block, KV head); scores are read
// from L2, never sorted):
//   1. find the cutoff element e* = the k-th best under (score desc, index
//      asc).  Candidates start as all spans; each level takes min/max of the
//      candidates, histograms them into 4096 equal-width bins, keeps the bin
//      that holds the k-th best and counts the candidates above it.  Once at
//      most 2048 candidates remain they are ranked exactly in LDS; if they are
//      all equal, e* is the right one of them by index order.
//   2. span j is selected iff score_j > score* or (score_j == score* and
//      j <= j*); a block-wide ordered compaction writes the indices ascending.
// Binning uses floor((x - min) * (4096 / (max - min))) in fp64, which is
// monotone in x, so no element can land in a bin out of order.
#include "rea_internal.h"

#include <math.h>

namespace rea {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 4096;
constexpr int kCap = 2048;
constexpr int kMaxLevels = 12;

struct TopkShared {
    uint32_t hist[kBins];
    double cand_v[kCap];
    int32_t cand_j[kCap];
    double lev_mn[kMaxLevels];
    double lev_inv[kMaxLevels];
    int32_t lev_bin[kMaxLevels];
    double red_d[2][kWaves];
    uint32_t red_u[kWaves];
    uint32_t scan[kWaves + 1];
    uint32_t n_cand;
    int32_t cut_j;
    double cut_v;
    int32_t found;
};

__device__ __forceinline__ int bin_of(double x, double mn, double inv) {
    const double f = floor((x - mn) * inv);
    if (!(f > 0.0)) return 0;                      // also x == mn with inv == inf
    if (f >= (double)(kBins - 1)) return kBins - 1;
    return (int)f;
}

__device__ __forceinline__ bool is_candidate(const TopkShared &sh, int nlev, double x) {
    for (int l = 0; l < nlev; ++l) {
        if (x < sh.lev_mn[l]) return false;
        if (bin_of(x, sh.lev_mn[l], sh.lev_inv[l]) != sh.lev_bin[l]) return false;
    }
    return true;
}

// Exclusive prefix of `flag` over the workgroup in thread order; returns the
// prefix and writes the total to *total.  All threads must call it.
__device__ uint32_t block_excl_scan(TopkShared &sh, bool flag, uint32_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned long long m = __ballot(flag);
    const uint32_t in_wave = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) sh.red_u[wave] = (uint32_t)__popcll(m);
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t acc = 0;
        for (int w = 0; w < kWaves; ++w) {
            sh.scan[w] = acc;
            acc += sh.red_u[w];
        }
        sh.scan[kWaves] = acc;
    }
    __syncthreads();
    const uint32_t r = sh.scan[wave] + in_wave;
    *total = sh.scan[kWaves];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kThreads) void k_topk(const double *__restrict__ scores_all,
                                                   int64_t n, int kk, int topk,
                                                   int32_t *__restrict__ sel_all,
                                                   int32_t *__restrict__ nsel_all) {
    __shared__ TopkShared sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bh = blockIdx.x;
    const double *sc = scores_all + bh * n;
    int32_t *sel = sel_all ? sel_all + bh * topk : nullptr;
    if (tid == 0) nsel_all[bh] = kk;

    if (kk == 0 || kk >= n) {       // nothing or everything
        if (sel)
            for (int64_t i = tid; i < topk; i += kThreads) sel[i] = i < kk ? (int32_t)i : -1;
        return;
    }

    int nlev = 0;
    int64_t need = kk;              // rank (1-based) of e* among current candidates
    for (;;) {
        // min / max / count over the candidates
        double mn = INFINITY, mx = -INFINITY;
        uint32_t cnt = 0;
        for (int64_t j = tid; j < n; j += kThreads) {
            const double x = sc[j];
            if (is_candidate(sh, nlev, x)) {
                mn = fmin(mn, x);
                mx = fmax(mx, x);
                ++cnt;
            }
        }
        for (int o = 32; o > 0; o >>= 1) {
            mn = fmin(mn, __shfl_xor(mn, o));
            mx = fmax(mx, __shfl_xor(mx, o));
            cnt += __shfl_xor(cnt, o);
        }
        if (lane == 0) {
            sh.red_d[0][wave] = mn;
            sh.red_d[1][wave] = mx;
            sh.red_u[wave] = cnt;
        }
        __syncthreads();
        mn = INFINITY;
        mx = -INFINITY;
        cnt = 0;
        for (int w = 0; w < kWaves; ++w) {
            mn = fmin(mn, sh.red_d[0][w]);
            mx = fmax(mx, sh.red_d[1][w]);
            cnt += sh.red_u[w];
        }
        __syncthreads();

        if (cnt <= (uint32_t)kCap) {
            // gather the candidates and rank them exactly in LDS
            if (tid == 0) sh.n_cand = 0;
            __syncthreads();
            for (int64_t j = tid; j < n; j += kThreads) {
                const double x = sc[j];
                if (is_candidate(sh, nlev, x)) {
                    const uint32_t slot = atomicAdd(&sh.n_cand, 1u);
                    sh.cand_v[slot] = x;
                    sh.cand_j[slot] = (int32_t)j;
                }
            }
            __syncthreads();
            const int m = (int)sh.n_cand;
            for (int c = tid; c < m; c += kThreads) {
                const double v = sh.cand_v[c];
                const int32_t jc = sh.cand_j[c];
                int rank = 0;
                for (int o = 0; o < m; ++o) {
                    const double vo = sh.cand_v[o];
                    rank += (vo > v) || (vo == v && sh.cand_j[o] < jc);
                }
                if (rank == need - 1) {
                    sh.cut_v = v;
                    sh.cut_j = jc;
                }
            }
            __syncthreads();
            break;
        }
        if (mn == mx) {
            // all candidates are equal: e* is the need-th of them in index order
            if (tid == 0) sh.found = 0;
            __syncthreads();
            uint32_t before = 0;
            for (int64_t base = 0; base < n; base += kThreads) {
                const int64_t j = base + tid;
                const bool f = j < n && is_candidate(sh, nlev, sc[j]);
                uint32_t tot;
                const uint32_t pre = block_excl_scan(sh, f, &tot);
                if (f && before + pre == (uint32_t)(need - 1)) {
                    sh.cut_j = (int32_t)j;
                    sh.cut_v = sc[j];
                    sh.found = 1;
                }
                before += tot;
                __syncthreads();
                if (sh.found) break;
            }
            break;
        }
        if (nlev == kMaxLevels) {
            // levels exhausted (only for scores spread over an extreme dynamic
            // range): rank every candidate against all others, O(n^2)
            for (int64_t j = tid; j < n; j += kThreads) {
                const double x = sc[j];
                if (!is_candidate(sh, nlev, x)) continue;
                int64_t rank = 0;
                for (int64_t o = 0; o < n; ++o) {
                    const double y = sc[o];
                    if (is_candidate(sh, nlev, y) && (y > x || (y == x && o < j))) ++rank;
                }
                if (rank == need - 1) {
                    sh.cut_v = x;
                    sh.cut_j = (int32_t)j;
                }
            }
            __syncthreads();
            break;
        }

        // one histogram level
        const double inv = (double)kBins / (mx - mn);
        for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0u;
        __syncthreads();
        for (int64_t j = tid; j < n; j += kThreads) {
            const double x = sc[j];
            if (is_candidate(sh, nlev, x)) atomicAdd(&sh.hist[bin_of(x, mn, inv)], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            int64_t above = 0;
            int b = kBins - 1;
            for (; b > 0; --b) {
                if (above + sh.hist[b] >= need) break;
                above += sh.hist[b];
            }
            sh.lev_mn[nlev] = mn;
            sh.lev_inv[nlev] = inv;
            sh.lev_bin[nlev] = b;
            sh.red_u[0] = (uint32_t)above;
        }
        __syncthreads();
        need -= sh.red_u[0];
        ++nlev;
        __syncthreads();
    }

    // ordered compaction of the selected spans
    const double cv = sh.cut_v;
    const int64_t cj = sh.cut_j;
    uint32_t written = 0;
    for (int64_t base = 0; base < n; base += kThreads) {
        const int64_t j = base + tid;
        bool f = false;
        if (j < n) {
            const double x = sc[j];
            f = x > cv || (x == cv && j <= cj);
        }
        uint32_t tot;
        const uint32_t pre = block_excl_scan(sh, f, &tot);
        if (f && sel && written + pre < (uint32_t)topk) sel[written + pre] = (int32_t)j;
        written += tot;
    }
    if (sel)
        for (int64_t i = (int64_t)kk + tid; i < topk; i += kThreads) sel[i] = -1;
}

}  // namespace

hipError_t launch_topk(const Geom &g, const double *span_scores, int32_t *sel, int32_t *n_sel,
                       hipStream_t s) {
    const int nbh = g.n_blk * g.Hkv;
    hipLaunchKernelGGL(k_topk, dim3(nbh), dim3(kThreads), 0, s, span_scores, g.n_spans,
                       g.k_sel, g.topk, sel, n_sel);
    return hipGetLastError();
}

}  // namespace rea
