// decode_attend.hip - steps 2-4 fused for small query groups (decode).
//
// Same result as gather + RoPE (window.hip) followed by window attention
// (attend.hip), without writing the window: every window row is read straight
// from the cache, rotated to its window position in registers and attended.
// The window is global [0, G') ++ selected spans in ascending order ++ local
// [T-L', T) (OpenReview discussion, "Decoding Phase" pseudocode); row w turns
// by angle w * theta^(-2c/d) (rotate-half RoPE, research-map summary,
// "Approach": positions are assigned after the concatenation); query i of a
// block is rotated to W - n_q + i and sees rows w <= that position.
//
//   k_fused_split    one workgroup per (run of rows_wg window rows, KV head,
//                    block), 4 waves.  One round trip fetches the selection
//                    slots the run can touch and the raw queries; the queries
//                    are rotated while the first rows load.  The run is taken
//                    in sub-splits of 64 rows: a 16-lane DPP row of a wave is
//                    a stream of 4 consecutive rows of each sub-split, and the
//                    loads of the next sub-split are issued before the current
//                    one is attended, so a workgroup keeps K/V loads in
//                    flight for its whole run.  A lane holds D/32 channel
//                    pairs (c, c + D/2) of its stream's rows.  The rotation of
//                    a stream's first row comes from rope_cs, the next rows'
//                    by one complex multiplication with (cos, sin) of the
//                    channel's frequency (fp32 for bf16 inputs, fp64 for fp32
//                    inputs); the rotated key is fp32.  Logits are kept in
//                    log2 units (the softmax scale carries log2 e) so weights
//                    are single exp2s.  Each stream keeps an online (m, l,
//                    acc) over its rows; the workgroup's 16 streams are merged
//                    through LDS and one partial per workgroup is written.
//                    rows_wg is a multiple of 64 chosen on the host: 128 when
//                    one row run per workgroup already fills the GPU (a
//                    single decode: 63 workgroups per KV head at 7968 rows),
//                    longer for batches, so that the workgroups the registers
//                    allow per CU (two or three) stream their runs.
//   k_fused_combine  workgroups per (KV head, block) merge the splits:
//                    out = sum_s 2^(m_s-M) acc_s / sum_s 2^(m_s-M) l_s
//                    (maxima m_s in log2 units).
#include "rea_internal.h"

#include <math.h>

#include <type_traits>

namespace rea {
namespace {

constexpr int kThreads = 256;
constexpr int kSL = 4;                          // rows per stream and sub-split
constexpr int kSub = 4 * 4 * kSL;               // rows per sub-split: waves x streams x rows
constexpr int kPartRows = 128;                  // the shortest row run (workspace sizing)
constexpr int kSelCap = 1024;                   // selection slots a workgroup stages
constexpr int kCombBatch = 8;                   // partials loaded together by the merge

struct FusedArgs {
    const unsigned char *k, *v;
    const void *q;
    const int32_t *sel, *n_sel;
    float *part_acc;        // [n_blk][Hkv][n_split][QR][D]
    float *part_ml;         // [n_blk][Hkv][n_split][QR][2]: m, l
    float *out;             // [n_q][Hq][D]
    int64_t sh, st;         // elements
    int64_t T, Gp, Lp, mid_lo, n_spans;
    int S, last_len, topk, Hkv, Hq, g, n_q, block_q, QR, n_split, rep;
    int rows_wg;            // window rows per workgroup (multiple of kSub); n_split runs
    int comb_tpi;           // merge phases per item (power of two)
    // batched decode (see Geom): per-sequence lengths and cache offsets
    const int64_t *lens;
    int hps, G, L;
    int64_t seq_stride;
    float scale_log2;       // softmax scale * log2(e): logits in log2 units
    double frev_hi[kMaxHalfDim], frev_lo[kMaxHalfDim];   // theta_c / 2pi as hi + lo
    double step_c[kMaxHalfDim], step_s[kMaxHalfDim];     // cos, sin of theta_c
};

// (cos, sin) of the angle w * theta_c, from the fractional number of turns
// t = frac(w * theta_c / 2pi): the product is split exactly (fma) so t is
// good to ~1e-16 for any w < 2^31; then the quadrant is taken out and Taylor
// polynomials in fp32 on |x| <= pi/4 give cos and sin to fp32 rounding
// (truncation below 3e-9).
__device__ __forceinline__ void rope_cs(int64_t w, double fhi, double flo, float &c, float &s) {
    const double wd = (double)w;
    const double p = wd * fhi;
    const double e = fma(wd, fhi, -p);
    const double t = (p - rint(p)) + (e + wd * flo);
    const double qd = rint(t * 4.0);
    const int q = (int)qd & 3;
    const float x = (float)(t - qd * 0.25) * 6.28318530717958647692f;
    const float x2 = x * x;
    float sp = fmaf(x2, 2.75573192e-6f, -1.98412698e-4f);      // 1/9!, -1/7!
    sp = fmaf(x2, sp, 8.33333333e-3f);                          // 1/5!
    sp = fmaf(x2, sp, -1.66666667e-1f);                         // -1/3!
    const float sx = fmaf(x * x2, sp, x);
    float cp = fmaf(x2, -2.75573192e-7f, 2.48015873e-5f);       // -1/10!, 1/8!
    cp = fmaf(x2, cp, -1.38888889e-3f);                         // -1/6!
    cp = fmaf(x2, cp, 4.16666667e-2f);                          // 1/4!
    cp = fmaf(x2, cp, -0.5f);
    const float cx = fmaf(x2, cp, 1.f);
    c = q == 0 ? cx : q == 1 ? -sx : q == 2 ? -cx : sx;
    s = q == 0 ? sx : q == 1 ? cx : q == 2 ? -sx : -cx;
}

// PPL consecutive stored elements (the lane's share of one half of a row).
template <typename TIn, int PPL> struct Part;
template <> struct Part<uint16_t, 4> {
    uint2 a;
    __device__ void load(const uint16_t *p) { a = *(const uint2 *)p; }
    __device__ void get(float (&x)[4]) const {
        x[0] = __uint_as_float(a.x << 16);
        x[1] = __uint_as_float(a.x & 0xffff0000u);
        x[2] = __uint_as_float(a.y << 16);
        x[3] = __uint_as_float(a.y & 0xffff0000u);
    }
};
template <> struct Part<uint16_t, 2> {
    uint32_t a;
    __device__ void load(const uint16_t *p) { a = *(const uint32_t *)p; }
    __device__ void get(float (&x)[2]) const {
        x[0] = __uint_as_float(a << 16);
        x[1] = __uint_as_float(a & 0xffff0000u);
    }
};
template <> struct Part<float, 4> {
    float4 a;
    __device__ void load(const float *p) { a = *(const float4 *)p; }
    __device__ void get(float (&x)[4]) const {
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    }
};
template <> struct Part<float, 2> {
    float2 a;
    __device__ void load(const float *p) { a = *(const float2 *)p; }
    __device__ void get(float (&x)[2]) const {
        x[0] = a.x; x[1] = a.y;
    }
};

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum
// (partners lane^1, lane^2, mirror within 8, mirror within 16).
__device__ __forceinline__ float row_sum16f(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

// Barrier that orders LDS only: global loads issued before it stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The K and V rows of one stream in one sub-split.
template <typename TIn, int PPL> struct RowsKV {
    Part<TIn, PPL> k1[kSL], k2[kSL], v1[kSL], v2[kSL];
};

template <typename TIn, int D, int QRM>
__global__ __launch_bounds__(kThreads) void k_fused_split(FusedArgs a) {
    constexpr int HALF = D / 2;
    constexpr int PPL = HALF / 16;              // channel pairs per lane
    constexpr int NA = 2 * PPL;                 // accumulated channels per lane and query row
    constexpr int QPT = (QRM * HALF + kThreads - 1) / kThreads;   // query pairs per thread
    constexpr int SPT = kSelCap / kThreads;     // selection slots per thread
    __shared__ float qs[QRM][D];
    __shared__ int32_t ssel[kSelCap];
    __shared__ double tab[HALF][4];             // theta_c/2pi (hi, lo), cos and sin of theta_c
    __shared__ float sm[16][QRM], sl[16][QRM], sf[16][QRM], smax[QRM];
    __shared__ float sacc[16][QRM][D];
    using RT = typename std::conditional<sizeof(TIn) == 2, float, double>::type;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sp = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int64_t bh = (int64_t)b * a.Hkv + h;
    const int64_t w0 = (int64_t)sp * a.rows_wg;
    const SeqOf so = seq_of(a.lens, h, a.hps, a.rep, a.seq_stride, a.sh, a.T);
    const SeqGeom sg = seq_geom(so.T, a.G, a.L, a.S);

    // One round trip: the selection count, the selection slots this run's
    // rows can touch (row w >= G' lies in slot (w - G') / S; the host keeps
    // rows_wg / S + 2 <= kSelCap), and the raw query elements.
    const int ns = a.n_sel[bh];
    const int64_t slot0 = w0 > sg.Gp ? (w0 - sg.Gp) / a.S : 0;
    int64_t nslot = (int64_t)a.rows_wg / a.S + 2;
    if (nslot > (int64_t)a.topk - slot0) nslot = (int64_t)a.topk - slot0;
    int32_t sv[SPT];
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        const int idx = tid + u * kThreads;
        sv[u] = idx < nslot ? a.sel[bh * a.topk + slot0 + idx] : 0;
    }
    float qx1[QPT], qx2[QPT];
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
        const int idx = tid + j * kThreads, r = idx / HALF, c = idx % HALF;
        qx1[j] = qx2[j] = 0.f;
        if (r < a.QR) {
            const int64_t i = (int64_t)b * a.block_q + r / a.g;
            const TIn *qp = (const TIn *)a.q + (i * a.Hq + h * a.g + r % a.g) * D;
            if (sizeof(TIn) == 2) {
                qx1[j] = __uint_as_float((uint32_t)((const uint16_t *)qp)[c] << 16);
                qx2[j] = __uint_as_float((uint32_t)((const uint16_t *)qp)[c + HALF] << 16);
            } else {
                qx1[j] = ((const float *)qp)[c];
                qx2[j] = ((const float *)qp)[c + HALF];
            }
        }
    }
    double fh = 0.0, fl = 0.0, scs = 0.0, ssn = 0.0;
    if (tid < HALF) {
        fh = a.frev_hi[tid];
        fl = a.frev_lo[tid];
        scs = a.step_c[tid];
        ssn = a.step_s[tid];
    }
#pragma unroll
    for (int u = 0; u < SPT; ++u) ssel[tid + u * kThreads] = sv[u];
    if (tid < HALF) {
        tab[tid][0] = fh;
        tab[tid][1] = fl;
        tab[tid][2] = scs;
        tab[tid][3] = ssn;
    }
    // window length: only span n_spans-1 can be short, and a sorted selection
    // holds it last
    int64_t sel_len = (int64_t)ns * a.S;
    if (sg.last_len != a.S && ns > 0 && a.sel[bh * a.topk + ns - 1] == sg.n_spans - 1)
        sel_len -= a.S - sg.last_len;
    const int64_t Wbh = sg.Gp + sel_len + sg.Lp;
    __syncthreads();

    // this run's rows [w0, wend) in sub-splits of kSub; rows past the window
    // are skipped, and within the last sub-split they load token 0 (finite
    // data whose logits are masked and weights are 0)
    const int64_t wend = w0 + a.rows_wg < Wbh ? w0 + a.rows_wg : Wbh;
    const int nsub = wend > w0 ? (int)((wend - w0 + kSub - 1) / kSub) : 0;
    const int rho = lane >> 4, c0 = (lane & 15) * PPL;
    const int soff = wave * (4 * kSL) + rho * kSL;      // the stream's first row in a sub-split
    const TIn *kb = (const TIn *)a.k + so.kv_off;
    const TIn *vb = (const TIn *)a.v + so.kv_off;

    auto issue = [&](int sub, RowsKV<TIn, PPL> &rk) {
        const int64_t wf = w0 + (int64_t)sub * kSub + soff;
        const int64_t o0 = wf - sg.Gp;
        const uint32_t oc = (uint32_t)(o0 > 0 ? o0 : 0);
        int oq = (int)(oc / (uint32_t)a.S), orr = (int)(oc - (uint32_t)oq * (uint32_t)a.S);
        // the usual case: the stream's kSL rows are consecutive cache rows
        // (inside the window, in one region, within one selected span), so
        // the first row's source and the row stride address them all
        const bool run = wf + kSL <= Wbh &&
                         (o0 + kSL <= 0 || o0 >= sel_len || (o0 >= 0 && o0 + kSL <= sel_len && orr + kSL <= a.S));
        if (run) {
            const int64_t src = o0 < 0 ? wf
                              : o0 < sel_len ? sg.mid_lo + (int64_t)ssel[oq - slot0] * a.S + orr
                                             : sg.T - sg.Lp + (o0 - sel_len);
            const TIn *kp = kb + src * a.st + c0, *vp = vb + src * a.st + c0;
#pragma unroll
            for (int i = 0; i < kSL; ++i) {
                rk.k1[i].load(kp + i * a.st);
                rk.k2[i].load(kp + i * a.st + HALF);
                rk.v1[i].load(vp + i * a.st);
                rk.v2[i].load(vp + i * a.st + HALF);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < kSL; ++i) {
            const int64_t w = wf + i, o = o0 + i;
            int64_t src = 0;
            if (w < Wbh) {
                if (o < 0)
                    src = w;
                else if (o < sel_len)
                    src = sg.mid_lo + (int64_t)ssel[oq - slot0] * a.S + orr;
                else
                    src = sg.T - sg.Lp + (o - sel_len);
            }
            const int64_t row = src * a.st;
            rk.k1[i].load(kb + row + c0);
            rk.k2[i].load(kb + row + c0 + HALF);
            rk.v1[i].load(vb + row + c0);
            rk.v2[i].load(vb + row + c0 + HALF);
            if (o >= 0 && ++orr == a.S) {
                orr = 0;
                ++oq;
            }
        }
    };

    RowsKV<TIn, PPL> ra, rb;
    if (nsub > 0) issue(0, ra);

    // while they load: the query rows r = (query r / g, head h*g + r % g)
    // rotated to their positions and rounded to fp32
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
        const int idx = tid + j * kThreads, r = idx / HALF, c = idx % HALF;
        if (r < QRM) {
            float y1 = 0.f, y2 = 0.f;
            if (r < a.QR) {
                const int64_t i = (int64_t)b * a.block_q + r / a.g;
                float co, sn;
                rope_cs(Wbh - a.n_q + i, tab[c][0], tab[c][1], co, sn);
                // (the softmax scale, in log2 units, is folded in here)
                y1 = (qx1[j] * co - qx2[j] * sn) * a.scale_log2;
                y2 = (qx2[j] * co + qx1[j] * sn) * a.scale_log2;
            }
            qs[r][c] = y1;
            qs[r][c + HALF] = y2;
        }
    }
    lds_barrier();

    float q1[QRM][PPL], q2[QRM][PPL];
#pragma unroll
    for (int r = 0; r < QRM; ++r)
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
            q1[r][p] = qs[r][c0 + p];
            q2[r][p] = qs[r][c0 + p + HALF];
        }
    RT cst[PPL], snt[PPL];
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
        cst[p] = (RT)tab[c0 + p][2];
        snt[p] = (RT)tab[c0 + p][3];
    }

    // (cos, sin) of (kSub - kSL) theta_c: a stream's next sub-split starts that
    // many rows after the row its per-row steps reach, so one complex step
    // carries the rotation over instead of evaluating it again (fp64 powers of
    // the per-row step, rounded to RT)
    RT cj[PPL], sj[PPL];
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
        double rc = 1.0, rs = 0.0, bc = tab[c0 + p][2], bs = tab[c0 + p][3];
        for (int e = kSub - kSL; e > 0; e >>= 1) {
            if (e & 1) {
                const double t = rc * bc - rs * bs;
                rs = rs * bc + rc * bs;
                rc = t;
            }
            const double t = bc * bc - bs * bs;
            bs = 2.0 * bc * bs;
            bc = t;
        }
        cj[p] = (RT)rc;
        sj[p] = (RT)rs;
    }
    RT cs_run[PPL], sn_run[PPL];        // rotation of the row after the last consumed one
    bool started = false;

    // the stream's running softmax state over its rows.  The running maximum
    // starts at the lowest finite float, not -inf: every finite logit reaches
    // it, and a masked row (logit -inf) then gets weight exp2(-inf) = 0 with
    // no test (while every row so far is masked the state stays 0 and rescales
    // by exp2(0)).
    float m[QRM], l[QRM], acc[QRM][NA];
#pragma unroll
    for (int r = 0; r < QRM; ++r) {
        m[r] = -__FLT_MAX__;
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < NA; ++e) acc[r][e] = 0.f;
    }
    const int Wi = (int)Wbh;

    const int64_t pos_min = Wbh - a.n_q + (int64_t)b * a.block_q;   // the first query row's position
    auto consume = [&](int sub, const RowsKV<TIn, PPL> &rk) {
        const int64_t wf = w0 + (int64_t)sub * kSub + soff;
        const int wfi = (int)wf;
        // rotation of the stream's first row (evaluated for the first
        // sub-split, carried over from the previous one by one complex step
        // after that), then one step per row (bf16 inputs step in fp32, a few
        // fp32 ulps per sub-split; fp32 inputs in fp64)
        RT cs[PPL], sn[PPL];
        if (!started) {
#pragma unroll
            for (int p = 0; p < PPL; ++p) {
                float c1, s1;
                rope_cs(wf, tab[c0 + p][0], tab[c0 + p][1], c1, s1);
                cs[p] = c1;
                sn[p] = s1;
            }
            started = true;
        } else {
#pragma unroll
            for (int p = 0; p < PPL; ++p) {
                cs[p] = cs_run[p] * cj[p] - sn_run[p] * sj[p];
                sn[p] = sn_run[p] * cj[p] + cs_run[p] * sj[p];
            }
        }
        // logits of the rows, in log2 units (the scale carries log2 e).  A row
        // past the window adds -inf; a row after a query row's own position
        // is masked per query row, tested only where the sub-split reaches
        // the first query row's position (the same test for the workgroup).
        // Query rows r >= QR need no mask: their staged query is 0 and their
        // results are never written.
        const bool causal = w0 + (int64_t)(sub + 1) * kSub - 1 > pos_min;
        float lg[kSL][QRM];
#pragma unroll
        for (int i = 0; i < kSL; ++i) {
            float x1[PPL], x2[PPL];
            rk.k1[i].get(x1);
            rk.k2[i].get(x2);
            const float madd = wfi + i < Wi ? 0.f : -INFINITY;
            float y1[PPL], y2[PPL];
#pragma unroll
            for (int p = 0; p < PPL; ++p) {
                const float c = (float)cs[p], s = (float)sn[p];
                y1[p] = x1[p] * c - x2[p] * s;
                y2[p] = x2[p] * c + x1[p] * s;
                const RT cn = cs[p] * cst[p] - sn[p] * snt[p];
                sn[p] = sn[p] * cst[p] + cs[p] * snt[p];
                cs[p] = cn;
            }
#pragma unroll
            for (int r = 0; r < QRM; ++r) {
                // each of the row's 16 lanes starts from the row's mask term
                // (0, or -inf past the window), so their sum carries it
                float d = madd;
#pragma unroll
                for (int p = 0; p < PPL; ++p) {
                    d = fmaf(q1[r][p], y1[p], d);
                    d = fmaf(q2[r][p], y2[p], d);
                }
                d = row_sum16f(d);
                if (causal) {
                    const int pos = Wi - a.n_q + b * a.block_q + r / a.g;
                    if (wfi + i > pos) d = -INFINITY;
                }
                lg[i][r] = d;
            }
        }
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
            cs_run[p] = cs[p];
            sn_run[p] = sn[p];
        }
        // online softmax: the state is rescaled to a new maximum only when a
        // row exceeds the current one by more than 2^8 (weights up to 2^8
        // stay far inside fp32), and only when some stream of the wave needs
        // it; the first real row always does (from the floor)
#pragma unroll
        for (int r = 0; r < QRM; ++r) {
            float mx = m[r];
#pragma unroll
            for (int i = 0; i < kSL; ++i) mx = fmaxf(mx, lg[i][r]);
            const bool grow = mx > m[r] + 8.f;
            if (__builtin_amdgcn_ballot_w64(grow)) {
                const float f = grow ? __builtin_amdgcn_exp2f(m[r] - mx) : 1.f;   // 0 from the floor
                l[r] *= f;
#pragma unroll
                for (int e = 0; e < NA; ++e) acc[r][e] *= f;
                if (grow) m[r] = mx;
            }
        }
#pragma unroll
        for (int i = 0; i < kSL; ++i) {
            float x1[PPL], x2[PPL];
            rk.v1[i].get(x1);
            rk.v2[i].get(x2);
#pragma unroll
            for (int r = 0; r < QRM; ++r) {
                // exp2(-inf) = 0 covers masked rows
                const float p = __builtin_amdgcn_exp2f(lg[i][r] - m[r]);
                l[r] += p;
#pragma unroll
                for (int e = 0; e < PPL; ++e) {
                    acc[r][e] = fmaf(p, x1[e], acc[r][e]);
                    acc[r][PPL + e] = fmaf(p, x2[e], acc[r][PPL + e]);
                }
            }
        }
    };

    // two sub-splits in flight: the next one's loads are issued before the
    // current one is attended
    for (int sub = 0; sub < nsub; sub += 2) {
        if (sub + 1 < nsub) issue(sub + 1, rb);
        consume(sub, ra);
        if (sub + 1 < nsub) {
            if (sub + 2 < nsub) issue(sub + 2, ra);
            consume(sub + 1, rb);
        }
    }

    // the workgroup's 16 streams -> LDS, then one merge per (query row, channel)
    const int st_id = wave * 4 + rho;
#pragma unroll
    for (int r = 0; r < QRM; ++r) {
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
            sacc[st_id][r][c0 + p] = acc[r][p];
            sacc[st_id][r][c0 + p + HALF] = acc[r][PPL + p];
        }
        if ((lane & 15) == 0) {
            sm[st_id][r] = m[r];
            sl[st_id][r] = l[r];
        }
    }
    __syncthreads();
    if (tid < 16 * QRM) {
        // weight of stream s for query row r: 2^(m_s - M_r)
        const int s2 = tid / QRM, r = tid % QRM;
        float M = -INFINITY;
#pragma unroll
        for (int t = 0; t < 16; ++t) M = fmaxf(M, sm[t][r]);
        sf[s2][r] = sm[s2][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm[s2][r] - M);
        if (s2 == 0) smax[r] = M;
    }
    __syncthreads();
    const int64_t pbase = bh * a.n_split * a.QR;
    for (int idx = tid; idx < a.QR * D; idx += kThreads) {
        const int r = idx / D, c = idx % D;
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const float f = sf[t][r];
            L = fmaf(sl[t][r], f, L);
            A = fmaf(sacc[t][r][c], f, A);
        }
        const int64_t slot = pbase + (int64_t)sp * a.QR + r;
        a.part_acc[slot * D + c] = A;
        if (c == 0) *(float2 *)(a.part_ml + slot * 2) = make_float2(smax[r], L);
    }
}

// grid (Hkv, n_blk, item slices): merges the splits of one (block, KV head).
// Thread = (query row r, channel quad, split phase j); comb_tpi phases, so
// each thread folds at most kCombBatch splits (one round of loads) into a
// running (m, l, acc), and the phases are folded in LDS.  A workgroup takes
// kThreads / comb_tpi of the QR x D/4 items.
template <int D>
__global__ __launch_bounds__(kThreads) void k_fused_combine(FusedArgs a) {
    constexpr int NQ = D / 4;
    __shared__ float cm[kThreads], cl[kThreads];
    __shared__ float4 ca[kThreads];
    const int tid = threadIdx.x;
    const int h = blockIdx.x, b = blockIdx.y;
    const int64_t bh = (int64_t)b * a.Hkv + h;
    const int64_t pbase = bh * a.n_split * a.QR;
    const int items = a.QR * NQ;
    const int tpi = a.comb_tpi, ipw = kThreads / tpi;
    const int il = tid % ipw, j = tid / ipw;
    const int item = blockIdx.z * ipw + il;
    const bool live = item < items;
    const int r = live ? item / NQ : 0, cq = item % NQ;
    float M = -INFINITY, L = 0.f;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) {
        for (int s0 = j; s0 < a.n_split; s0 += kCombBatch * tpi) {
            float2 ml[kCombBatch];
            float4 x[kCombBatch];
#pragma unroll
            for (int u = 0; u < kCombBatch; ++u) {
                const int s = s0 + u * tpi;
                const int64_t slot = pbase + (int64_t)(s < a.n_split ? s : 0) * a.QR + r;
                ml[u] = *(const float2 *)(a.part_ml + slot * 2);
                x[u] = *(const float4 *)(a.part_acc + slot * D + cq * 4);
                if (s >= a.n_split) ml[u].x = -INFINITY;
            }
#pragma unroll
            for (int u = 0; u < kCombBatch; ++u) {
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
    }
    cm[tid] = M;
    cl[tid] = L;
    ca[tid] = A;
    __syncthreads();
    if (j == 0 && live) {
        for (int jj = 1; jj < tpi; ++jj) {
            const int o = jj * ipw + il;
            const float mn = fmaxf(M, cm[o]);
            if (mn == -INFINITY) continue;
            const float f = __builtin_amdgcn_exp2f(M - mn), fo = __builtin_amdgcn_exp2f(cm[o] - mn);
            L = L * f + cl[o] * fo;
            A.x = A.x * f + ca[o].x * fo;
            A.y = A.y * f + ca[o].y * fo;
            A.z = A.z * f + ca[o].z * fo;
            A.w = A.w * f + ca[o].w * fo;
            M = mn;
        }
        const float inv = 1.f / L;
        const int64_t i = (int64_t)b * a.block_q + r / a.g;
        const int hq = h * a.g + r % a.g;
        *(float4 *)(a.out + (i * a.Hq + hq) * D + cq * 4) =
            make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
    }
}

template <typename TIn, int D, int QRM>
hipError_t launch_typed(const Geom &g, const FusedArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((k_fused_split<TIn, D, QRM>), dim3(a.n_split, g.Hkv, g.n_blk),
                       dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ipw = kThreads / a.comb_tpi;
    const int slices = (a.QR * (D / 4) + ipw - 1) / ipw;
    hipLaunchKernelGGL((k_fused_combine<D>), dim3(g.Hkv, g.n_blk, slices), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename TIn, int D>
hipError_t launch_qr(const Geom &g, const FusedArgs &a, hipStream_t s) {
    if (a.QR == 1) return launch_typed<TIn, D, 1>(g, a, s);
    if (a.QR == 2) return launch_typed<TIn, D, 2>(g, a, s);
    // 3 query rows (e.g. 24 query heads over 8 KV heads): a fourth row would be
    // a quarter more logit and P.V work for nothing
    if (a.QR == 3) return launch_typed<TIn, D, 3>(g, a, s);
    return a.QR <= 4 ? launch_typed<TIn, D, 4>(g, a, s) : launch_typed<TIn, D, 8>(g, a, s);
}

// Partials the workspace holds per (block, KV head): runs of the shortest
// length.
int fused_max_parts(int64_t W_cap) { return (int)((W_cap + kPartRows - 1) / kPartRows); }

// Window rows per workgroup: 128, or longer when (block, head) units are many,
// so that about `per_cu` workgroups per CU stream their runs; at most the
// rows whose selection slots fit kSelCap.
int fused_rows_wg(const Geom &g, int num_cu, int per_cu) {
    const int64_t units = (int64_t)g.n_blk * g.Hkv;
    const int64_t target = (int64_t)(num_cu > 0 ? num_cu : 256) * per_cu;
    int64_t rows = (g.W_cap * units + target - 1) / target;
    rows = (rows + kSub - 1) / kSub * kSub;
    if (rows < kPartRows) rows = kPartRows;
    const int64_t cap = (int64_t)(kSelCap - 2) * g.S / kSub * kSub;
    if (rows > cap) rows = cap;
    if (rows < kSub) rows = kSub;
    return (int)rows;
}

}  // namespace

bool fused_decode_path(const Geom &g) { return g.block_q * g.g <= 8 && !mfma_block_path(g); }

size_t fused_ws_bytes(const Geom &g) {
    const size_t rows = (size_t)g.n_blk * g.Hkv * fused_max_parts(g.W_cap) * (size_t)(g.block_q * g.g);
    return ((rows * g.d * sizeof(float) + 255) & ~(size_t)255) +
           ((rows * 2 * sizeof(float) + 255) & ~(size_t)255);
}

hipError_t launch_fused_decode(const Geom &g, const void *k, const void *v, const void *q,
                               const int32_t *sel, const int32_t *n_sel, float *out, void *ws,
                               int num_cu, hipStream_t s) {
    FusedArgs a;
    a.k = (const unsigned char *)k;
    a.v = (const unsigned char *)v;
    a.q = q;
    a.sel = sel;
    a.n_sel = n_sel;
    a.out = out;
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
    a.Hkv = g.Hkv;
    a.Hq = g.Hq;
    a.g = g.g;
    a.rep = g.rep;
    a.lens = g.lens;
    a.hps = g.hps;
    a.G = g.G;
    a.L = g.L;
    a.seq_stride = g.seq_stride;
    a.n_q = g.n_q;
    a.block_q = g.block_q;
    a.QR = g.block_q * g.g;
    // workgroups per CU that the registers allow: three for one query row
    // (bf16 d 128: 146 VGPRs), two up to eight rows
    a.rows_wg = fused_rows_wg(g, num_cu, a.QR == 1 ? 3 : 2);
    a.n_split = (int)((g.W_cap + a.rows_wg - 1) / a.rows_wg);
    // merge phases: the fewest (a power of two) that leave each thread at
    // most kCombBatch splits, and at least enough to fill the workgroup
    int tpi = 1;
    while (tpi < 64 && tpi * kCombBatch < a.n_split) tpi *= 2;
    while (kThreads / tpi > a.QR * (g.d / 4) && tpi < kThreads) tpi *= 2;
    a.comb_tpi = tpi;
    a.scale_log2 = (float)((double)g.scale * 1.4426950408889634074);
    for (int c = 0; c < kMaxHalfDim; ++c) {
        const double f = c < g.d / 2 ? pow(g.theta, -2.0 * (double)c / (double)g.d) : 0.0;
        const long double turns = (long double)f / (2.0L * 3.14159265358979323846264338327950288L);
        a.frev_hi[c] = (double)turns;
        a.frev_lo[c] = (double)(turns - (long double)a.frev_hi[c]);
        a.step_c[c] = cos(f);
        a.step_s[c] = sin(f);
    }
    const size_t rows = (size_t)g.n_blk * g.Hkv * fused_max_parts(g.W_cap) * (size_t)a.QR;
    a.part_acc = (float *)ws;
    a.part_ml = (float *)((char *)ws + ((rows * g.d * sizeof(float) + 255) & ~(size_t)255));
    if (g.dtype == 0)
        return g.d == 128 ? launch_qr<uint16_t, 128>(g, a, s) : launch_qr<uint16_t, 64>(g, a, s);
    return g.d == 128 ? launch_qr<float, 128>(g, a, s) : launch_qr<float, 64>(g, a, s);
}

}  // namespace rea
