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
//                 (block, span) is written.  The first query group also writes
//                 each span's largest key norm.
//   k_certify     per (block, KV head): exact top-k from the approximate
//                 scores (see below).
//
// Error bound.  Every product hi*k, lo*k of two bf16 numbers is exact in fp32;
// the MFMA sums 256 of them in fp32.  With at most 255 roundings of at most
// 2^-23 relative each, |s_hat - s| <= e_i * ||k_t||_2 where
// e_i = 255*2^-23*(1+1e-6) * ||(|hi|+|lo|)||_2 + ||q_eff - hi - lo||_2.
// A span maximum moves by at most e_i * max_t ||k_t||, a block sum by
// E_b * Kbar_j.  k_certify keeps every span whose interval
// [s_hat - eps, s_hat + eps] lies surely inside the top-k, drops every span
// surely outside it, re-scores the rest in fp64 (exact for bf16 inputs), and
// selects among them exactly -- so the selection equals the exact one.
#include "rea_internal.h"

#include <math.h>

namespace rea {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;             // head_dim handled here
constexpr int kQB = 64;             // queries per block
constexpr int kWavesM = 4;          // blocks (waves) per workgroup
constexpr int kTile = 32;           // tokens per MFMA tile
constexpr int kRowPad = 136;        // LDS row stride (bf16) of a staged key tile
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
// k_qprep: grid (n_blk, Hkv), 128 threads (one per channel)
// ---------------------------------------------------------------------------
struct PrepArgs {
    const uint16_t *q;      // [n_q][Hq][D]
    uint16_t *qhl;          // [Hkv][n_q][256]
    double *qeff;           // [Hkv][n_q][D]
    double *E;              // [n_blk][Hkv]
    int Hq, Hkv, g, n_q;
};

__global__ __launch_bounds__(kD) void k_qprep(PrepArgs a) {
    __shared__ double red[kD / 64][2];
    __shared__ double esum;
    const int b = blockIdx.x, h = blockIdx.y, c = threadIdx.x;
    const int lane = c & 63, wave = c >> 6;
    if (c == 0) esum = 0.0;
    __syncthreads();
    for (int il = 0; il < kQB; ++il) {
        const int64_t i = (int64_t)b * kQB + il;
        double s = 0.0;
        for (int gg = 0; gg < a.g; ++gg) s += bf16_to_f64(a.q[(i * a.Hq + h * a.g + gg) * kD + c]);
        const uint16_t hi = f32_to_bf16((float)s);
        const double hid = bf16_to_f64(hi);
        const uint16_t lo = f32_to_bf16((float)(s - hid));
        const double lod = bf16_to_f64(lo);
        const double r = s - hid - lod;
        const int64_t row = (int64_t)h * a.n_q + i;
        a.qhl[row * 256 + c] = hi;
        a.qhl[row * 256 + kD + c] = lo;
        a.qeff[row * kD + c] = s;
        double n1 = (fabs(hid) + fabs(lod)) * (fabs(hid) + fabs(lod));
        double n2 = r * r;
        for (int o = 32; o > 0; o >>= 1) {
            n1 += __shfl_xor(n1, o);
            n2 += __shfl_xor(n2, o);
        }
        if (lane == 0) {
            red[wave][0] = n1;
            red[wave][1] = n2;
        }
        __syncthreads();
        if (c == 0) {
            const double s1 = red[0][0] + red[1][0], s2 = red[0][1] + red[1][1];
            esum += (kGammaMfma * sqrt(s1) + sqrt(s2)) * (1.0 + 1e-12);
        }
        __syncthreads();
    }
    if (c == 0) a.E[(int64_t)b * a.Hkv + h] = esum * (1.0 + 1e-9);
}

// ---------------------------------------------------------------------------
// k_score_mfma: grid (n_qg * Hkv * NR) with the query group slowest, so the
// workgroups sharing a key range of one head sit on one XCD; 256 threads.
// ---------------------------------------------------------------------------
struct MfmaArgs {
    const unsigned char *k;     // K cache (bf16)
    const uint16_t *qhl;        // [Hkv][n_q][256]
    double *out;                // [n_blk][Hkv][n_spans]
    double *kbar;               // [Hkv][n_spans]
    int64_t sh_bytes, st_bytes;
    int64_t mid_lo, mid_hi, n_spans;
    int S, Hkv, n_q, n_blk, NR;
};

__device__ __forceinline__ uint4 ld16(const void *p) { return *(const uint4 *)p; }

__global__ __launch_bounds__(256) void k_score_mfma(MfmaArgs a) {
    __shared__ __align__(16) uint16_t kt[2][kTile][kRowPad];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int units = a.Hkv * a.NR;
    const int qg = blockIdx.x / units;
    const int rest = blockIdx.x % units;
    const int h = rest / a.NR, r = rest % a.NR;
    const int b = qg * kWavesM + wave;              // this wave's block
    const bool active = b < a.n_blk;
    const int64_t j0 = (int64_t)r * a.n_spans / a.NR, j1 = (int64_t)(r + 1) * a.n_spans / a.NR;
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

    const unsigned char *kh = a.k + (int64_t)h * a.sh_bytes;
    // staging: thread -> (token rows tid/16 and tid/16 + 16, 16-byte chunk tid%16);
    // the next tile's rows are loaded into registers before this tile's MFMAs
    // and written to the other LDS buffer after them
    const int srow = tid >> 4, schk = tid & 15;
    uint4 nxt[2];
    auto load_rows = [&](int64_t t0) {
#pragma unroll
        for (int hr = 0; hr < 2; ++hr) {
            const int64_t t = t0 + srow + hr * 16;
            nxt[hr] = t < a.mid_hi ? ld16(kh + t * a.st_bytes + schk * 16) : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_rows = [&](int bufi) {
#pragma unroll
        for (int hr = 0; hr < 2; ++hr) *(uint4 *)&kt[bufi][srow + hr * 16][schk * 8] = nxt[hr];
    };
    auto tile_t0 = [&](int64_t it) {
        return a.mid_lo + (j0 + it / tiles_per_span) * a.S + (int64_t)(it % tiles_per_span) * kTile;
    };

    const int64_t n_tiles = (j1 - j0) * tiles_per_span;
    int buf = 0;
    if (n_tiles > 0) {
        load_rows(tile_t0(0));
        store_rows(0);
    }
    __syncthreads();
    float run[2] = {-INFINITY, -INFINITY};   // running max over the span's tiles
    double kn_run = 0.0;                     // running max of squared key norms
    for (int64_t it = 0; it < n_tiles; ++it) {
        const int64_t j = j0 + it / tiles_per_span;
        const int sub = (int)(it % tiles_per_span);
        const int64_t t0 = tile_t0(it);
        const bool more = it + 1 < n_tiles;
        if (more) load_rows(tile_t0(it + 1));
        if (sub == 0) {
            run[0] = -INFINITY;
            run[1] = -INFINITY;
            kn_run = 0.0;
        }
        // A fragments: token row m = lane%32, channels ks*16 + (lane/32)*8 .. +8
        uint4 af[8];
        {
            const int m = lane & 31, kb = lane >> 5;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) af[ks] = *(const uint4 *)&kt[buf][m][ks * 16 + kb * 8];
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
        const int64_t valid = a.mid_hi - t0;           // tokens of this tile inside the middle
        float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int row = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
            if (row < valid) {
                m0 = fmaxf(m0, acc0[rr]);
                m1 = fmaxf(m1, acc1[rr]);
            }
        }
        m0 = fmaxf(m0, __shfl_xor(m0, 32));
        m1 = fmaxf(m1, __shfl_xor(m1, 32));
        run[0] = fmaxf(run[0], m0);
        run[1] = fmaxf(run[1], m1);
        if (qg == 0 && wave == 0 && lane < kTile) {
            // squared norm of key row `lane` of this tile, fp64
            if (lane < valid) {
                double s = 0.0;
                for (int c = 0; c < kD; ++c) {
                    const double x = bf16_to_f64(kt[buf][lane][c]);
                    s = fma(x, x, s);
                }
                kn_run = fmax(kn_run, s);
            }
        }
        if (sub == tiles_per_span - 1) {
            // span done: sum over the block's 64 queries (lanes 0..31 hold queries
            // n and 32+n after the cross-half max)
            double v = (double)run[0] + (double)run[1];
            for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o);
            if (active && lane == 0) a.out[((int64_t)b * a.Hkv + h) * a.n_spans + j] = v + 0.0;
            if (qg == 0 && wave == 0) {
                double kn = kn_run;
                for (int o = 16; o > 0; o >>= 1) kn = fmax(kn, __shfl_xor(kn, o));
                if (lane == 0) a.kbar[(int64_t)h * a.n_spans + j] = sqrt(kn) * (1.0 + 1e-12);
            }
        }
        if (more) store_rows(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
}

// ---------------------------------------------------------------------------
// k_certify: grid (n_blk * Hkv), 512 threads
// ---------------------------------------------------------------------------
constexpr int kCThreads = 512;
constexpr int kCWaves = kCThreads / 64;
constexpr int kCCap = 4096;         // spans handled on chip
constexpr int kCBins = 2048;
constexpr int kCRank = 256;
constexpr int kCPer = kCCap / kCThreads;

struct CertArgs {
    const double *shat;     // [n_blk][Hkv][n_spans]
    const double *kbar;     // [Hkv][n_spans]
    const double *E;        // [n_blk][Hkv]
    const double *qeff;     // [Hkv][n_q][D]
    const unsigned char *k;
    int32_t *sel, *nsel;
    int64_t sh_bytes, st_bytes, mid_lo, mid_hi, n_spans;
    int S, Hkv, n_q, kk, topk;
};

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
    double cut_v;
};

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

// need-th best of (val, idx)[0..count) under (val desc, idx asc) -> cut_v/cut_j.
// Reorders and shrinks val/idx.
__device__ __forceinline__ void c_find_kth(CertShared &sh, uint32_t count, int64_t need) {
    const int tid = threadIdx.x, lane = tid & 63;
    bool by_index = false;
    for (;;) {
        if (count <= (uint32_t)kCRank) {
            for (uint32_t c = tid; c < count; c += kCThreads) {
                const double x = sh.val[c];
                const int32_t jc = sh.idx[c];
                int64_t rank = 0;
                for (uint32_t o = 0; o < count; ++o) {
                    const double y = sh.val[o];
                    rank += (y > x) || (y == x && sh.idx[o] < jc);
                }
                if (rank == need - 1) {
                    sh.cut_v = x;
                    sh.cut_j = jc;
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
            constexpr int bpl = kCBins / 64;
            uint32_t own = 0;
            for (int i = 0; i < bpl; ++i) own += sh.hist[lane * bpl + i];
            uint32_t suf = own;
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_down(suf, o);
                if (lane + o < 64) suf += y;
            }
            const uint32_t after = suf - own;
            if ((int64_t)after < need && need <= (int64_t)suf) {
                uint32_t above = after;
                int bb = lane * bpl + bpl - 1;
                for (; bb > lane * bpl; --bb) {
                    if ((int64_t)(above + sh.hist[bb]) >= need) break;
                    above += sh.hist[bb];
                }
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

__device__ __forceinline__ double cert_eps(double Eb, double kb, double s) {
    const double e = Eb * kb;
    return e * (1.0 + 1e-9) + 1e-12 * (fabs(s) + e) + 1e-300;
}

__global__ __launch_bounds__(kCThreads) void k_certify(CertArgs a) {
    __shared__ CertShared sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bh = blockIdx.x;
    const int b = (int)(bh / a.Hkv), h = (int)(bh % a.Hkv);
    const int64_t n = a.n_spans;
    const int kk = a.kk;
    const double *shat = a.shat + bh * n;
    const double *kbar = a.kbar + (int64_t)h * n;
    const double Eb = a.E[bh];
    int32_t *sel = a.sel ? a.sel + bh * a.topk : nullptr;
    if (tid == 0) a.nsel[bh] = kk;
    if (kk == 0 || kk >= n) {
        if (sel)
            for (int64_t i = tid; i < a.topk; i += kCThreads) sel[i] = i < kk ? (int32_t)i : -1;
        return;
    }
    // tau_L = kk-th largest lower end, tau_U = (kk+1)-th largest upper end
    for (int64_t j = tid; j < n; j += kCThreads) {
        const double s = shat[j];
        sh.val[j] = s - cert_eps(Eb, kbar[j], s);
        sh.idx[j] = (int32_t)j;
    }
    __syncthreads();
    c_find_kth(sh, (uint32_t)n, kk);
    const double tauL = sh.cut_v;
    for (int64_t j = tid; j < n; j += kCThreads) {
        const double s = shat[j];
        sh.val[j] = s + cert_eps(Eb, kbar[j], s);
        sh.idx[j] = (int32_t)j;
    }
    __syncthreads();
    c_find_kth(sh, (uint32_t)n, kk + 1);
    const double tauU = sh.cut_v;
    // certainly in: lower end above tau_U.  Possibly in: upper end >= tau_L.
    const int nwords = (int)((n + 31) / 32);
    for (int i = tid; i < nwords; i += kCThreads) sh.bitmap[i] = 0u;
    if (tid == 0) {
        sh.nd = 0;
        sh.nx = 0;
    }
    __syncthreads();
    for (int64_t j = tid; j < n; j += kCThreads) {
        const double s = shat[j], e = cert_eps(Eb, kbar[j], s);
        if (s - e > tauU) {
            atomicOr(&sh.bitmap[j >> 5], 1u << (j & 31));
            atomicAdd(&sh.nd, 1u);
        } else if (s + e >= tauL) {
            const uint32_t slot = atomicAdd(&sh.nx, 1u);
            sh.xs[slot] = (int32_t)j;
        }
    }
    __syncthreads();
    const uint32_t nd = sh.nd, nx = sh.nx;
    const int64_t need = (int64_t)kk - nd;
    if (need > 0) {
        // exact (fp64) block scores of the uncertain spans: a wave per span,
        // 16 lanes per key row, the group-summed queries read from L2
        const int rs = lane >> 4, ch = lane & 15;
        const unsigned char *kh = a.k + (int64_t)h * a.sh_bytes + ch * 16;
        const double *qb = a.qeff + ((int64_t)h * a.n_q + (int64_t)b * kQB) * kD + ch * 8;
        for (uint32_t x = wave; x < nx; x += kCWaves) {
            const int64_t j = sh.xs[x];
            const int64_t tb = a.mid_lo + j * a.S, te = min(tb + (int64_t)a.S, a.mid_hi);
            double total = 0.0;
            for (int il = 0; il < kQB; ++il) {
                double qv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) qv[e] = qb[(int64_t)il * kD + e];
                double best = -INFINITY;
                for (int64_t t0 = tb; t0 < te; t0 += 4) {
                    const int64_t t = t0 + rs;
                    const bool ok = t < te;
                    const uint4 raw = ok ? ld16(kh + t * a.st_bytes) : make_uint4(0u, 0u, 0u, 0u);
                    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
                    double acc = 0.0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc = fma(qv[2 * e], (double)__uint_as_float(w4[e] << 16), acc);
                        acc = fma(qv[2 * e + 1], (double)__uint_as_float(w4[e] & 0xffff0000u), acc);
                    }
                    for (int o = 1; o < 16; o <<= 1) acc += __shfl_xor(acc, o);
                    if (ok) best = fmax(best, acc);
                }
                best = fmax(best, __shfl_xor(best, 16));
                best = fmax(best, __shfl_xor(best, 32));
                total += best;
            }
            if (lane == 0) sh.xv[x] = total + 0.0;
        }
        __syncthreads();
        for (uint32_t x = tid; x < nx; x += kCThreads) {
            sh.val[x] = sh.xv[x];
            sh.idx[x] = sh.xs[x];
        }
        __syncthreads();
        c_find_kth(sh, nx, need);
        const double cv = sh.cut_v;
        const int32_t cj = sh.cut_j;
        for (uint32_t x = tid; x < nx; x += kCThreads) {
            const double v = sh.xv[x];
            const int32_t j = sh.xs[x];
            if (v > cv || (v == cv && j <= cj)) atomicOr(&sh.bitmap[j >> 5], 1u << (j & 31));
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
                if (pos < (uint32_t)a.topk) sel[pos] = tid * 32 + bit;
                ++pos;
            }
            for (int64_t i = (int64_t)kk + tid; i < a.topk; i += kCThreads) sel[i] = -1;
        }
    }
}

}  // namespace

bool mfma_block_path(const Geom &g) {
    return g.dtype == 0 && g.d == kD && g.block_q == kQB && g.S % kTile == 0 && g.n_spans > 0 &&
           g.n_spans <= kCCap;
}

size_t mfma_ws_bytes(const Geom &g) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return al((size_t)g.Hkv * g.n_q * 256 * sizeof(uint16_t)) +       // [hi|lo]
           al((size_t)g.Hkv * g.n_q * kD * sizeof(double)) +           // q_eff
           al((size_t)g.n_blk * g.Hkv * sizeof(double)) +              // E
           al((size_t)g.Hkv * g.n_spans * sizeof(double));             // key-norm maxima
}

hipError_t launch_score_select_mfma(const Geom &g, const void *q, const void *k,
                                    double *span_scores, int32_t *sel, int32_t *n_sel,
                                    void *ws, int num_cu, hipStream_t s) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    char *p = (char *)ws;
    uint16_t *qhl = (uint16_t *)p;
    p += al((size_t)g.Hkv * g.n_q * 256 * sizeof(uint16_t));
    double *qeff = (double *)p;
    p += al((size_t)g.Hkv * g.n_q * kD * sizeof(double));
    double *E = (double *)p;
    p += al((size_t)g.n_blk * g.Hkv * sizeof(double));
    double *kbar = (double *)p;

    PrepArgs pa{(const uint16_t *)q, qhl, qeff, E, g.Hq, g.Hkv, g.g, g.n_q};
    hipLaunchKernelGGL(k_qprep, dim3(g.n_blk, g.Hkv), dim3(kD), 0, s, pa);
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
    ma.n_q = g.n_q;
    ma.n_blk = g.n_blk;
    const int n_qg = (g.n_blk + kWavesM - 1) / kWavesM;
    const int64_t units = (int64_t)n_qg * g.Hkv;
    int64_t NR = ((int64_t)(num_cu > 0 ? num_cu : 256) * 2 + units - 1) / units;
    if (NR > g.n_spans) NR = g.n_spans;
    if (NR < 1) NR = 1;
    ma.NR = (int)NR;
    hipLaunchKernelGGL(k_score_mfma, dim3((unsigned)(units * NR)), dim3(256), 0, s, ma);
    e = hipGetLastError();
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
    ca.n_q = g.n_q;
    ca.kk = g.k_sel;
    ca.topk = g.topk;
    hipLaunchKernelGGL(k_certify, dim3(g.n_blk * g.Hkv), dim3(kCThreads), 0, s, ca);
    return hipGetLastError();
}

}  // namespace rea
