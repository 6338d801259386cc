// rea_api.cpp - the C ABI declared in include/rea.h: argument validation,
// size queries, workspace carving and the launch sequences.
//
// Validation is pure host code and runs before any HIP call, so every error
// status is observable on a machine without a GPU.  Nothing here allocates
// device memory or synchronises: all buffers come from the caller and all
// kernels are enqueued on the caller's stream.
#include "rea.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "rea_internal.h"

namespace {

thread_local char g_err[512] = "";

rea_status fail(rea_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Validate problem + params and derive the geometry.  No HIP call.
rea_status make_geom(const rea_problem *p, const rea_params *a, rea::Geom *g) {
    if (!p || !a) return fail(REA_EINVAL, "problem or params is NULL");
    if (p->struct_size != sizeof(rea_problem))
        return fail(REA_EINVAL, "rea_problem.struct_size %u != %zu", p->struct_size,
                    sizeof(rea_problem));
    if (a->struct_size != sizeof(rea_params))
        return fail(REA_EINVAL, "rea_params.struct_size %u != %zu", a->struct_size,
                    sizeof(rea_params));
    if (p->dtype != REA_BF16 && p->dtype != REA_F32)
        return fail(REA_EDTYPE, "dtype %d is neither REA_BF16 nor REA_F32", p->dtype);
    if (!p->q || !p->k || !p->v) return fail(REA_EINVAL, "q, k or v is NULL");
    if (p->n_q < 1) return fail(REA_ESHAPE, "n_q %d < 1", p->n_q);
    if (p->n_kv_heads < 1) return fail(REA_ESHAPE, "n_kv_heads %d < 1", p->n_kv_heads);
    if (p->n_q_heads < 1 || p->n_q_heads % p->n_kv_heads != 0)
        return fail(REA_ESHAPE, "n_q_heads %d is not a positive multiple of n_kv_heads %d",
                    p->n_q_heads, p->n_kv_heads);
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(REA_EUNSUPPORTED, "head_dim %d: the library implements 64 and 128",
                    p->head_dim);
    if (p->T < p->n_q || p->T >= ((int64_t)1 << 31))
        return fail(REA_ESHAPE, "T %lld must satisfy n_q <= T < 2^31", (long long)p->T);
    if (a->G < 0 || a->L < 0) return fail(REA_EINVAL, "G %d and L %d must be >= 0", a->G, a->L);
    if (a->S < 1) return fail(REA_EINVAL, "span size S %d < 1", a->S);
    if (a->topk < 0) return fail(REA_EINVAL, "topk %d < 0", a->topk);
    if (a->block_q < 1) return fail(REA_EINVAL, "block_q %d < 1", a->block_q);
    if (a->select_flags & ~(REA_SELECT_PER_Q_HEAD | REA_SELECT_TOKEN_SEGMENTS))
        return fail(REA_EINVAL, "select_flags 0x%x has unknown bits", a->select_flags);
    const bool segs = (a->select_flags & REA_SELECT_TOKEN_SEGMENTS) != 0;
    if (segs && (int64_t)a->topk * a->S >= ((int64_t)1 << 30))
        return fail(REA_EUNSUPPORTED, "topk * S too large for token segments");
    if (!(a->rope_theta > 0.0) || !isfinite(a->rope_theta))
        return fail(REA_EINVAL, "rope_theta must be finite and > 0");
    if (!isfinite(a->softmax_scale)) return fail(REA_EINVAL, "softmax_scale is not finite");
    if (p->n_q % a->block_q != 0)
        return fail(REA_ESHAPE, "n_q %d is not a multiple of block_q %d", p->n_q, a->block_q);
    if (p->kv_stride_tok < p->head_dim)
        return fail(REA_ESHAPE, "kv_stride_tok %lld < head_dim %d", (long long)p->kv_stride_tok,
                    p->head_dim);
    if (p->kv_stride_head < p->T * p->kv_stride_tok)
        return fail(REA_ESHAPE, "kv_stride_head %lld < T * kv_stride_tok",
                    (long long)p->kv_stride_head);

    const int esize = p->dtype == REA_BF16 ? 2 : 4;
    if (!aligned(p->q, 16) || !aligned(p->k, 16) || !aligned(p->v, 16))
        return fail(REA_EALIGN, "q, k and v must be 16-byte aligned");
    if ((p->kv_stride_tok * esize) % 16 != 0 || (p->kv_stride_head * esize) % 16 != 0)
        return fail(REA_EALIGN, "kv strides must be multiples of 16 bytes");

    g->dtype = p->dtype;
    g->esize = esize;
    g->n_q = p->n_q;
    g->Hq = p->n_q_heads;
    if (a->select_flags & REA_SELECT_PER_Q_HEAD) {   // every query head selects
        g->Hkv = p->n_q_heads;
        g->g = 1;
        g->rep = p->n_q_heads / p->n_kv_heads;
    } else {
        g->Hkv = p->n_kv_heads;
        g->g = p->n_q_heads / p->n_kv_heads;
        g->rep = 1;
    }
    g->d = p->head_dim;
    g->T = p->T;
    g->Gp = a->G < p->T ? a->G : p->T;
    g->Lp = a->L < p->T - g->Gp ? a->L : p->T - g->Gp;
    g->mid_lo = g->Gp;
    g->mid_hi = p->T - g->Lp;
    const int64_t n_mid = g->mid_hi - g->mid_lo;
    // token segments: kernels see one-token spans, a selection holds up to
    // topk * S tokens
    g->seg = segs ? a->S : 0;
    g->k_tok = a->topk;
    g->S = segs ? 1 : a->S;
    g->topk = segs ? a->topk * a->S : a->topk;
    g->n_spans = (n_mid + g->S - 1) / g->S;
    g->block_q = a->block_q;
    g->n_blk = p->n_q / a->block_q;
    g->k_sel = (int)(g->topk < g->n_spans ? g->topk : g->n_spans);
    g->last_len = g->n_spans > 0 ? (int)(n_mid - (g->n_spans - 1) * g->S) : 0;
    int64_t wc = g->Gp + (int64_t)g->k_sel * g->S + g->Lp;
    g->W_cap = wc < p->T ? wc : p->T;
    g->sh = p->kv_stride_head;
    g->st = p->kv_stride_tok;
    g->scale = a->softmax_scale > 0.f ? a->softmax_scale : (float)(1.0 / sqrt((double)g->d));
    g->theta = a->rope_theta;
    g->lens = nullptr;
    g->hps = g->Hkv;
    g->seq_stride = 0;
    g->G = a->G;
    g->L = a->L;

    if (n_mid > 0 && p->n_q > g->Lp)
        return fail(REA_ESHAPE,
                    "the %d queries must lie in the local region (L' = %lld) unless T <= G + L",
                    p->n_q, (long long)g->Lp);
    if ((int64_t)g->n_blk * g->Hkv * (g->n_spans > 0 ? g->n_spans : 1) >= ((int64_t)1 << 40))
        return fail(REA_EUNSUPPORTED, "too many spans");
    if (g->block_q > 1 && (size_t)g->block_q * g->d * sizeof(double) > 65536)
        return fail(REA_EUNSUPPORTED, "block_q %d too large for head_dim %d (needs <= %d)",
                    g->block_q, g->d, (int)(65536 / (g->d * sizeof(double))));
    return REA_OK;
}

struct Carve {
    char *base;
    size_t off;
    template <typename T> T *take(size_t bytes) {
        T *p = base ? (T *)(base + off) : nullptr;
        off += align256(bytes);
        return p;
    }
};

size_t score_scores_bytes(const rea::Geom &g) {
    return (size_t)g.n_blk * g.Hkv * (size_t)g.n_spans * sizeof(double);
}

size_t group_max_bytes(const rea::Geom &g) {
    return (size_t)g.n_blk * g.Hkv * (size_t)rea::score_groups(g) * sizeof(double);
}

// The token scorer (spans of one token, one query per block) also records
// each group's second largest score and where its maximum lies.
bool token_groups(const rea::Geom &g) { return g.S == 1 && g.block_q == 1; }

// score_select workspace: [span scores unless the caller keeps them][group
// maxima (+ second maxima and offsets of the maxima for the token scorer, or
// second and third maxima and the spans of the first two for the decode
// scorer), or the MFMA path's query rows / bounds]
size_t select_aux_bytes(const rea::Geom &g) {
    if (rea::mfma_block_path(g)) return align256(rea::mfma_ws_bytes(g));
    if (rea::heads_mfma_path(g)) return align256(rea::heads_ws_bytes(g));
    const size_t gm = align256(group_max_bytes(g));
    if (token_groups(g)) return 2 * gm + align256(group_max_bytes(g) / 2);
    if (rea::score_decode_path(g)) return gm + align256(2 * group_max_bytes(g)) + align256(group_max_bytes(g));
    return gm;
}

// token segments: the best tokens before widening, [n_blk][Hkv][k_tok] + counts
size_t seg_tok_bytes(const rea::Geom &g) {
    if (!g.seg) return 0;
    return align256((size_t)g.n_blk * g.Hkv * g.k_tok * sizeof(int32_t)) +
           align256((size_t)g.n_blk * g.Hkv * sizeof(int32_t));
}

size_t score_ws_bytes(const rea::Geom &g, bool caller_scores) {
    return (caller_scores ? 0 : align256(score_scores_bytes(g))) + select_aux_bytes(g) +
           seg_tok_bytes(g);
}

// Steps 1a+1b on whichever path fits the problem.
hipError_t launch_select(const rea::Geom &g, const void *q, const void *k, double *scores,
                         void *aux, void *seg_ws, int32_t *sel, int32_t *n_sel, int num_cu,
                         hipStream_t s, const rea_timing *timing) {
    if (rea::mfma_block_path(g))
        return rea::launch_score_select_mfma(g, q, k, scores, sel, n_sel, aux, num_cu, s,
                                             timing ? (hipEvent_t)timing->score_begin : nullptr,
                                             timing ? (hipEvent_t)timing->score_end : nullptr);
    if (rea::heads_mfma_path(g))
        return rea::launch_score_select_heads(g, q, k, scores, sel, n_sel, aux, num_cu, s,
                                              timing ? (hipEvent_t)timing->score_begin : nullptr,
                                              timing ? (hipEvent_t)timing->score_end : nullptr);
    double *gsec = nullptr, *gtop = nullptr;
    int32_t *garg = nullptr, *gtopi = nullptr;
    if (token_groups(g)) {
        gsec = (double *)((char *)aux + align256(group_max_bytes(g)));
        garg = (int32_t *)((char *)gsec + align256(group_max_bytes(g)));
    } else if (rea::score_decode_path(g)) {
        gtop = (double *)((char *)aux + align256(group_max_bytes(g)));
        gtopi = (int32_t *)((char *)gtop + align256(2 * group_max_bytes(g)));
    }
    hipError_t e = rea::launch_score(g, q, k, scores, (double *)aux, num_cu, s,
                                     timing ? (hipEvent_t)timing->score_begin : nullptr,
                                     timing ? (hipEvent_t)timing->score_end : nullptr, nullptr,
                                     gsec, garg, gtop, gtopi);
    if (e != hipSuccess) return e;
    if (!g.seg)
        return rea::launch_topk(g, scores, (const double *)aux, sel, n_sel, s, nullptr, gsec, garg,
                                gtop, gtopi);
    // token segments: the k_tok best tokens, then their widened union
    rea::Geom gt = g;
    gt.topk = g.k_tok;
    gt.k_sel = g.k_tok < g.n_spans ? g.k_tok : (int)g.n_spans;
    Carve c{(char *)seg_ws, 0};
    int32_t *sel_tok = c.take<int32_t>((size_t)g.n_blk * g.Hkv * g.k_tok * sizeof(int32_t));
    int32_t *nsel_tok = c.take<int32_t>((size_t)g.n_blk * g.Hkv * sizeof(int32_t));
    e = rea::launch_topk(gt, scores, (const double *)aux, sel_tok, nsel_tok, s, nullptr, gsec, garg);
    if (e != hipSuccess) return e;
    return rea::launch_widen(g, sel_tok, nsel_tok, sel, n_sel, s);
}

size_t decode_ws_bytes(const rea::Geom &g) {
    Carve c{nullptr, 0};
    c.take<double>(score_scores_bytes(g));
    c.take<char>(select_aux_bytes(g));
    c.take<char>(seg_tok_bytes(g));
    c.take<int32_t>((size_t)g.n_blk * g.Hkv * g.topk * sizeof(int32_t));
    c.take<int32_t>((size_t)g.n_blk * g.Hkv * sizeof(int32_t));
    if (rea::mfma_cache_attend_path(g)) {
        c.take<char>(rea::rope_table_bytes(g));
        return c.off;
    }
    if (rea::fused_decode_path(g)) {
        c.take<char>(rea::fused_ws_bytes(g));
        return c.off;
    }
    c.take<int32_t>((size_t)g.n_blk * g.Hkv * sizeof(int32_t));
    c.take<float>((size_t)g.n_blk * g.Hkv * g.W_cap * g.d * sizeof(float));
    c.take<char>((size_t)g.n_blk * g.Hkv * g.W_cap * g.d * g.esize);
    c.take<float>((size_t)g.n_q * g.Hq * g.d * sizeof(float));
    c.take<char>(rea::attend_ws_bytes(g, g.W_cap));
    return c.off;
}

rea_status device_ready(int *num_cu) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(REA_ENODEVICE, "no HIP device available");
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(REA_ENODEVICE, "cannot query device %d", dev);
    }
    *num_cu = n;
    return REA_OK;
}

rea_status launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(REA_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
    return REA_OK;
}

rea_status check_ws(void *ws, size_t have, size_t need) {
    if (need > 0 && !ws) return fail(REA_EWORKSPACE, "workspace is NULL, %zu bytes needed", need);
    if (have < need) return fail(REA_EWORKSPACE, "workspace %zu bytes < %zu needed", have, need);
    if (ws && !aligned(ws, 256)) return fail(REA_EALIGN, "workspace must be 256-byte aligned");
    return REA_OK;
}

rea_status check_sel(const rea::Geom &g, const int32_t *sel, const int32_t *n_sel) {
    if (!n_sel) return fail(REA_EINVAL, "n_sel is NULL");
    if (g.topk > 0 && !sel) return fail(REA_EINVAL, "sel is NULL while topk > 0");
    if (!aligned(n_sel, 4) || (sel && !aligned(sel, 4)))
        return fail(REA_EALIGN, "sel / n_sel must be 4-byte aligned");
    return REA_OK;
}

rea_status check_window(const rea::Geom &g, const void *k_win, const void *v_win,
                        int32_t W_cap) {
    if (!k_win || !v_win) return fail(REA_EINVAL, "k_win or v_win is NULL");
    if (!aligned(k_win, 16) || !aligned(v_win, 16))
        return fail(REA_EALIGN, "k_win and v_win must be 16-byte aligned");
    if (W_cap < g.W_cap)
        return fail(REA_ESHAPE, "W_cap %d < %lld (the largest possible window)", W_cap,
                    (long long)g.W_cap);
    return REA_OK;
}

}  // namespace

extern "C" {

int rea_abi_version(void) { return REA_ABI_VERSION; }

const char *rea_status_string(int status) {
    switch (status) {
    case REA_OK: return "REA_OK";
    case REA_EINVAL: return "REA_EINVAL";
    case REA_ESHAPE: return "REA_ESHAPE";
    case REA_EDTYPE: return "REA_EDTYPE";
    case REA_EALIGN: return "REA_EALIGN";
    case REA_EWORKSPACE: return "REA_EWORKSPACE";
    case REA_ENODEVICE: return "REA_ENODEVICE";
    case REA_ELAUNCH: return "REA_ELAUNCH";
    case REA_EUNSUPPORTED: return "REA_EUNSUPPORTED";
    default: return "REA_UNKNOWN";
    }
}

const char *rea_last_error(void) { return g_err; }

rea_status rea_query_sizes(const rea_problem *p, const rea_params *a, rea_sizes *out) {
    g_err[0] = 0;
    if (!out) return fail(REA_EINVAL, "out is NULL");
    rea::Geom g;
    rea_status st = make_geom(p, a, &g);
    if (st != REA_OK) return st;
    out->n_blocks = g.n_blk;
    out->n_spans = g.n_spans;
    out->k_sel = g.k_sel;
    out->W_cap = g.W_cap;
    out->ws_score_select = score_ws_bytes(g, false);
    out->ws_window_attend = rea::attend_ws_bytes(g, g.W_cap);
    out->ws_decode_step = decode_ws_bytes(g);
    out->n_sel_heads = g.Hkv;
    return REA_OK;
}

size_t rea_workspace_bytes(const rea_problem *p, const rea_params *a) {
    rea_sizes s;
    if (rea_query_sizes(p, a, &s) != REA_OK) return (size_t)-1;
    size_t need = s.ws_score_select;
    if (s.ws_window_attend > need) need = s.ws_window_attend;
    if (s.ws_decode_step > need) need = s.ws_decode_step;
    return need;
}

rea_status rea_score_select(const rea_problem *p, const rea_params *a, int32_t *sel,
                            int32_t *n_sel, double *span_scores, void *ws, size_t ws_bytes,
                            void *stream) {
    g_err[0] = 0;
    rea::Geom g;
    rea_status st = make_geom(p, a, &g);
    if (st != REA_OK) return st;
    if ((st = check_sel(g, sel, n_sel)) != REA_OK) return st;
    if (span_scores && !aligned(span_scores, 8))
        return fail(REA_EALIGN, "span_scores must be 8-byte aligned");
    if ((st = check_ws(ws, ws_bytes, score_ws_bytes(g, span_scores != nullptr))) != REA_OK)
        return st;
    int num_cu = 0;
    if ((st = device_ready(&num_cu)) != REA_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    Carve c{(char *)ws, 0};
    double *scores = span_scores ? span_scores : c.take<double>(score_scores_bytes(g));
    void *aux = c.take<char>(select_aux_bytes(g));
    void *seg_ws = c.take<char>(seg_tok_bytes(g));
    return launched(launch_select(g, p->q, p->k, scores, aux, seg_ws, sel, n_sel, num_cu, s,
                                  nullptr),
                    "score_select");
}

rea_status rea_gather_rope(const rea_problem *p, const rea_params *a, const int32_t *sel,
                           const int32_t *n_sel, float *k_win, void *v_win, float *q_rot,
                           int32_t *W, int32_t W_cap, void *stream) {
    g_err[0] = 0;
    rea::Geom g;
    rea_status st = make_geom(p, a, &g);
    if (st != REA_OK) return st;
    if ((st = check_sel(g, sel, n_sel)) != REA_OK) return st;
    if ((st = check_window(g, k_win, v_win, W_cap)) != REA_OK) return st;
    if (!q_rot || !W) return fail(REA_EINVAL, "q_rot or W is NULL");
    if (!aligned(q_rot, 16) || !aligned(W, 4)) return fail(REA_EALIGN, "q_rot / W misaligned");
    int num_cu = 0;
    if ((st = device_ready(&num_cu)) != REA_OK) return st;
    return launched(rea::launch_gather_rope(g, p->k, p->v, p->q, sel, n_sel, k_win, v_win,
                                            q_rot, W, W_cap, (hipStream_t)stream),
                    "gather_rope");
}

rea_status rea_window_attend(const rea_problem *p, const rea_params *a, const float *q_rot,
                             const float *k_win, const void *v_win, const int32_t *W,
                             int32_t W_cap, float *out, void *ws, size_t ws_bytes,
                             void *stream) {
    g_err[0] = 0;
    rea::Geom g;
    rea_status st = make_geom(p, a, &g);
    if (st != REA_OK) return st;
    if ((st = check_window(g, k_win, v_win, W_cap)) != REA_OK) return st;
    if (!q_rot || !W || !out) return fail(REA_EINVAL, "q_rot, W or out is NULL");
    if (!aligned(q_rot, 16) || !aligned(W, 4) || !aligned(out, 16))
        return fail(REA_EALIGN, "q_rot / W / out misaligned");
    if ((st = check_ws(ws, ws_bytes, rea::attend_ws_bytes(g, W_cap))) != REA_OK) return st;
    int num_cu = 0;
    if ((st = device_ready(&num_cu)) != REA_OK) return st;
    return launched(rea::launch_attend(g, q_rot, k_win, v_win, W, W_cap, out, ws,
                                       (hipStream_t)stream),
                    "window_attend");
}

}  // extern "C"

namespace {

// rea_decode_step's body.  rope_rows (may be NULL): in, the number of RoPE
// table rows already valid at the start of ws (from an earlier step on the
// same workspace, theta and head_dim); out, the rows valid after this step
// (0 when the step's path does not keep the table there).
// Host-side checks of rea_decode_step's arguments other than the workspace;
// *g gets the geometry.
rea_status decode_args(const rea_problem *p, const rea_params *a, const float *out,
                       const int32_t *sel, const int32_t *n_sel, rea::Geom *g) {
    rea_status st = make_geom(p, a, g);
    if (st != REA_OK) return st;
    if (!out) return fail(REA_EINVAL, "out is NULL");
    if (!aligned(out, 16)) return fail(REA_EALIGN, "out must be 16-byte aligned");
    if ((sel && !aligned(sel, 4)) || (n_sel && !aligned(n_sel, 4)))
        return fail(REA_EALIGN, "sel / n_sel must be 4-byte aligned");
    return REA_OK;
}

rea_status decode_step(const rea_problem *p, const rea_params *a, float *out, int32_t *sel,
                       int32_t *n_sel, void *ws, size_t ws_bytes, void *stream,
                       const rea_timing *timing, int64_t *rope_rows) {
    rea::Geom g;
    rea_status st = decode_args(p, a, out, sel, n_sel, &g);
    if (st != REA_OK) return st;
    if ((st = check_ws(ws, ws_bytes, decode_ws_bytes(g))) != REA_OK) return st;
    int num_cu = 0;
    if ((st = device_ready(&num_cu)) != REA_OK) return st;

    Carve c{(char *)ws, 0};
    // the MFMA attention's RoPE table goes first: the same place in every step
    const bool mfma_cache = rea::mfma_cache_attend_path(g);
    void *rws = mfma_cache ? c.take<char>(rea::rope_table_bytes(g)) : nullptr;
    const bool table_ready = mfma_cache && rope_rows && *rope_rows >= g.W_cap;
    if (rope_rows) *rope_rows = mfma_cache ? (table_ready ? *rope_rows : g.W_cap) : 0;
    double *scores = c.take<double>(score_scores_bytes(g));
    void *aux = c.take<char>(select_aux_bytes(g));
    void *seg_ws = c.take<char>(seg_tok_bytes(g));
    int32_t *ws_sel = c.take<int32_t>((size_t)g.n_blk * g.Hkv * g.topk * sizeof(int32_t));
    int32_t *ws_nsel = c.take<int32_t>((size_t)g.n_blk * g.Hkv * sizeof(int32_t));
    int32_t *use_sel = sel ? sel : ws_sel;
    int32_t *use_nsel = n_sel ? n_sel : ws_nsel;
    if (g.topk == 0) use_sel = sel;   // may be NULL: nothing is selected
    hipStream_t s = (hipStream_t)stream;
    if ((st = launched(launch_select(g, p->q, p->k, scores, aux, seg_ws, use_sel, use_nsel, num_cu, s,
                                     timing),
                       "score_select")) != REA_OK)
        return st;
    if (mfma_cache)
        return launched(rea::launch_attend_mfma_cache(g, p->q, p->k, p->v, use_sel, use_nsel, out,
                                                      rws, s, table_ready),
                        "window attention from the cache (MFMA)");
    if (rea::fused_decode_path(g)) {
        void *fws = c.take<char>(rea::fused_ws_bytes(g));
        return launched(rea::launch_fused_decode(g, p->k, p->v, p->q, use_sel, use_nsel, out,
                                                 fws, num_cu, s),
                        "fused gather + window attention");
    }
    int32_t *Wlen = c.take<int32_t>((size_t)g.n_blk * g.Hkv * sizeof(int32_t));
    float *k_win = c.take<float>((size_t)g.n_blk * g.Hkv * g.W_cap * g.d * sizeof(float));
    void *v_win = c.take<char>((size_t)g.n_blk * g.Hkv * g.W_cap * g.d * g.esize);
    float *q_rot = c.take<float>((size_t)g.n_q * g.Hq * g.d * sizeof(float));
    void *att_ws = c.take<char>(rea::attend_ws_bytes(g, g.W_cap));
    if ((st = launched(rea::launch_gather_rope(g, p->k, p->v, p->q, use_sel, use_nsel, k_win,
                                               v_win, q_rot, Wlen, g.W_cap, s),
                       "gather_rope")) != REA_OK)
        return st;
    return launched(rea::launch_attend(g, q_rot, k_win, v_win, Wlen, g.W_cap, out, att_ws, s),
                    "window_attend");
}

}  // namespace

extern "C" {

rea_status rea_decode_step(const rea_problem *p, const rea_params *a, float *out,
                           int32_t *sel, int32_t *n_sel, void *ws, size_t ws_bytes,
                           void *stream) {
    g_err[0] = 0;
    return decode_step(p, a, out, sel, n_sel, ws, ws_bytes, stream, nullptr, nullptr);
}

rea_status rea_decode_step_timed(const rea_problem *p, const rea_params *a, float *out,
                                 int32_t *sel, int32_t *n_sel, void *ws, size_t ws_bytes,
                                 void *stream, const rea_timing *timing) {
    g_err[0] = 0;
    return decode_step(p, a, out, sel, n_sel, ws, ws_bytes, stream, timing, nullptr);
}

}  // extern "C"

// ---- hooks for entry points defined in other translation units --------------

namespace rea {

void api_clear_error() { g_err[0] = 0; }

rea_status api_error(rea_status st, const char *msg) { return fail(st, "%s", msg); }

rea_status decode_check(const rea_problem *p, const rea_params *a, const float *out,
                        const int32_t *sel, const int32_t *n_sel, size_t *ws_bytes) {
    Geom g;
    rea_status st = decode_args(p, a, out, sel, n_sel, &g);
    if (st != REA_OK) return st;
    *ws_bytes = decode_ws_bytes(g);
    return REA_OK;
}

rea_status decode_step_ws(const rea_problem *p, const rea_params *a, float *out, int32_t *sel,
                          int32_t *n_sel, void *ws, size_t ws_bytes, void *stream) {
    return decode_step(p, a, out, sel, n_sel, ws, ws_bytes, stream, nullptr, nullptr);
}

}  // namespace rea

// ---- chunked prefill ------------------------------------------------------

namespace {

int32_t block_for(int32_t n, int32_t bq) {
    if (n % bq == 0) return bq;
    for (int32_t b = bq < n ? bq : n; b > 1; --b)
        if (n % b == 0) return b;
    return 1;
}

// The chunk plan; calls emit(start, n_q, block_q) for each chunk in order.
// Chunk c's blocks follow chunk c-1's in the numbering of rea_prefill's
// selection outputs.
template <typename F>
rea_status prefill_plan(const rea_problem *p, const rea_params *a, int32_t chunk, F emit) {
    if (!p || !a) return fail(REA_EINVAL, "problem or params is NULL");
    if (p->n_q != p->T)
        return fail(REA_EINVAL, "prefill needs every prompt token as a query (n_q %d != T %lld)",
                    p->n_q, (long long)p->T);
    if (a->block_q < 1) return fail(REA_EINVAL, "block_q %d < 1", a->block_q);
    if (chunk < 1 || chunk > a->L || chunk % a->block_q != 0)
        return fail(REA_EINVAL, "chunk %d must lie in [1, L = %d] and be a multiple of block_q %d",
                    chunk, a->L, a->block_q);
    const int64_t T = p->T;
    int64_t first = (int64_t)a->G + a->L < T ? (int64_t)a->G + a->L : T;
    first -= first % a->block_q;
    int64_t pos = 0;
    if (first > 0) {
        rea_status st = emit(0, (int32_t)first, a->block_q);
        if (st != REA_OK) return st;
        pos = first;
    }
    while (pos < T) {
        const int32_t n = (int32_t)(T - pos < chunk ? T - pos : chunk);
        rea_status st = emit(pos, n, block_for(n, a->block_q));
        if (st != REA_OK) return st;
        pos += n;
    }
    return REA_OK;
}

// The problem and params of one chunk: the cache cut after the chunk.
void chunk_view(const rea_problem *p, const rea_params *a, int64_t start, int32_t n, int32_t bq,
                rea_problem *pc, rea_params *ac) {
    *pc = *p;
    pc->T = start + n;
    pc->n_q = n;
    pc->q = (const char *)p->q + (size_t)start * p->n_q_heads * p->head_dim *
                                     (p->dtype == REA_BF16 ? 2 : 4);
    *ac = *a;
    ac->block_q = bq;
}

}  // namespace

extern "C" {

rea_status rea_prefill_plan(const rea_problem *p, const rea_params *a, int32_t chunk,
                            rea_chunk *chunks, int32_t cap, int32_t *n_chunks,
                            int64_t *n_blocks, size_t *ws_bytes) {
    g_err[0] = 0;
    if (!n_chunks || !ws_bytes) return fail(REA_EINVAL, "n_chunks or ws_bytes is NULL");
    if (cap > 0 && !chunks) return fail(REA_EINVAL, "chunks is NULL while cap > 0");
    int32_t count = 0;
    int64_t blocks = 0;
    size_t need = 0;
    rea_status st = prefill_plan(p, a, chunk, [&](int64_t start, int32_t n, int32_t bq) {
        rea_problem pc;
        rea_params ac;
        chunk_view(p, a, start, n, bq, &pc, &ac);
        rea::Geom g;
        rea_status s2 = make_geom(&pc, &ac, &g);
        if (s2 != REA_OK) return s2;
        const size_t w = decode_ws_bytes(g);
        if (w > need) need = w;
        if (count < cap) chunks[count] = rea_chunk{start, n, bq, blocks};
        ++count;
        blocks += n / bq;
        return REA_OK;
    });
    if (st != REA_OK) return st;
    *n_chunks = count;
    if (n_blocks) *n_blocks = blocks;
    *ws_bytes = need;
    return REA_OK;
}

rea_status rea_prefill(const rea_problem *p, const rea_params *a, int32_t chunk, float *out,
                       int32_t *sel, int32_t *n_sel, void *ws, size_t ws_bytes, void *stream) {
    g_err[0] = 0;
    if (!out) return fail(REA_EINVAL, "out is NULL");
    if (!sel != !n_sel) return fail(REA_EINVAL, "give both sel and n_sel, or neither");
    if ((sel && !aligned(sel, 4)) || (n_sel && !aligned(n_sel, 4)))
        return fail(REA_EALIGN, "sel / n_sel must be 4-byte aligned");
    int32_t count = 0;
    size_t need = 0;
    rea_status st = rea_prefill_plan(p, a, chunk, nullptr, 0, &count, nullptr, &need);
    if (st != REA_OK) return st;
    if ((st = check_ws(ws, ws_bytes, need)) != REA_OK) return st;
    // rows per block of the selection outputs: the selection heads and the
    // capacity of one selection, as rea_score_select lays them out (the plan
    // has validated p and a)
    const int64_t heads = (a->select_flags & REA_SELECT_PER_Q_HEAD) ? p->n_q_heads : p->n_kv_heads;
    const int64_t cap_sel =
        (a->select_flags & REA_SELECT_TOKEN_SEGMENTS) ? (int64_t)a->topk * a->S : a->topk;
    // the chunks share the workspace, so the RoPE table of the window
    // positions is built once (again only when the window capacity grows)
    int64_t rope_rows = 0, block = 0;
    return prefill_plan(p, a, chunk, [&](int64_t start, int32_t n, int32_t bq) {
        rea_problem pc;
        rea_params ac;
        chunk_view(p, a, start, n, bq, &pc, &ac);
        float *oc = out + (size_t)start * p->n_q_heads * p->head_dim;
        int32_t *sc = sel ? sel + block * heads * cap_sel : nullptr;
        int32_t *nc = n_sel ? n_sel + block * heads : nullptr;
        block += n / bq;
        return decode_step(&pc, &ac, oc, sc, nc, ws, ws_bytes, stream, nullptr, &rope_rows);
    });
}

}  // extern "C"

// ---- batched decode ---------------------------------------------------------

namespace {

// Validates one sequence's problem and the batch, then folds the batch into
// the selection heads: sequence b owns selection heads [b * H_sel, (b+1) * H_sel)
// and query heads [b * Hq, (b+1) * Hq); its cache starts b * kv_stride_seq
// elements after p->k / p->v.  Kernels re-derive every sequence's regions from
// its own length.
rea_status make_batch_geom(const rea_problem *p, const rea_params *a, int32_t batch,
                           rea::Geom *g) {
    rea_status st = make_geom(p, a, g);
    if (st != REA_OK) return st;
    if (batch < 1) return fail(REA_EINVAL, "batch %d < 1", batch);
    if (p->n_q != 1 || a->block_q != 1)
        return fail(REA_EUNSUPPORTED, "batched decode takes one query per sequence (n_q %d, "
                    "block_q %d)", p->n_q, a->block_q);
    if (a->L < 1)
        return fail(REA_EINVAL, "batched decode needs L >= 1 (the query token is local)");
    const bool mfma = rea::mfma_cache_attend_path(*g) && g->g <= 64;
    if (!mfma && !rea::fused_decode_path(*g))
        return fail(REA_EUNSUPPORTED, "batched decode needs at most %d query heads per selection "
                    "head (have %d)", g->dtype == 0 && g->d == 128 ? 64 : 8, g->g);
    if ((int64_t)batch * g->Hkv >= ((int64_t)1 << 24) || (int64_t)batch * g->Hq >= ((int64_t)1 << 24))
        return fail(REA_EUNSUPPORTED, "batch %d too large", batch);
    g->hps = g->Hkv;
    g->Hkv *= batch;
    g->Hq *= batch;
    return REA_OK;
}

}  // namespace

extern "C" {

rea_status rea_decode_batch_workspace(const rea_problem *p, const rea_params *a, int32_t batch,
                                      size_t *ws_bytes) {
    g_err[0] = 0;
    if (!ws_bytes) return fail(REA_EINVAL, "ws_bytes is NULL");
    rea::Geom g;
    rea_status st = make_batch_geom(p, a, batch, &g);
    if (st != REA_OK) return st;
    *ws_bytes = decode_ws_bytes(g);
    return REA_OK;
}

rea_status rea_decode_batch(const rea_problem *p, const rea_params *a, int32_t batch,
                            const int64_t *lengths, int64_t kv_stride_seq, float *out,
                            int32_t *sel, int32_t *n_sel, void *ws, size_t ws_bytes,
                            void *stream) {
    g_err[0] = 0;
    rea::Geom g;
    rea_status st = make_batch_geom(p, a, batch, &g);
    if (st != REA_OK) return st;
    if (!lengths) return fail(REA_EINVAL, "lengths is NULL");
    if (!aligned(lengths, 8)) return fail(REA_EALIGN, "lengths must be 8-byte aligned");
    if (kv_stride_seq < (int64_t)p->n_kv_heads * p->kv_stride_head)
        return fail(REA_ESHAPE, "kv_stride_seq %lld < n_kv_heads * kv_stride_head",
                    (long long)kv_stride_seq);
    if ((kv_stride_seq * g.esize) % 16 != 0)
        return fail(REA_EALIGN, "kv_stride_seq must be a multiple of 16 bytes");
    g.lens = lengths;
    g.seq_stride = kv_stride_seq;
    if (!out) return fail(REA_EINVAL, "out is NULL");
    if (!aligned(out, 16)) return fail(REA_EALIGN, "out must be 16-byte aligned");
    if ((sel && !aligned(sel, 4)) || (n_sel && !aligned(n_sel, 4)))
        return fail(REA_EALIGN, "sel / n_sel must be 4-byte aligned");
    if ((st = check_ws(ws, ws_bytes, decode_ws_bytes(g))) != REA_OK) return st;
    int num_cu = 0;
    if ((st = device_ready(&num_cu)) != REA_OK) return st;

    Carve c{(char *)ws, 0};
    double *scores = c.take<double>(score_scores_bytes(g));
    void *aux = c.take<char>(select_aux_bytes(g));
    void *seg_ws = c.take<char>(seg_tok_bytes(g));
    int32_t *ws_sel = c.take<int32_t>((size_t)g.n_blk * g.Hkv * g.topk * sizeof(int32_t));
    int32_t *ws_nsel = c.take<int32_t>((size_t)g.n_blk * g.Hkv * sizeof(int32_t));
    int32_t *use_sel = sel ? sel : ws_sel;
    int32_t *use_nsel = n_sel ? n_sel : ws_nsel;
    if (g.topk == 0) use_sel = sel;
    hipStream_t s = (hipStream_t)stream;
    if ((st = launched(launch_select(g, p->q, p->k, scores, aux, seg_ws, use_sel, use_nsel, num_cu, s,
                                     nullptr),
                       "batched score_select")) != REA_OK)
        return st;
    if (rea::mfma_cache_attend_path(g)) {
        void *rws = c.take<char>(rea::rope_table_bytes(g));
        return launched(rea::launch_attend_mfma_cache(g, p->q, p->k, p->v, use_sel, use_nsel, out,
                                                      rws, s),
                        "batched window attention from the cache (MFMA)");
    }
    void *fws = c.take<char>(rea::fused_ws_bytes(g));
    return launched(rea::launch_fused_decode(g, p->k, p->v, p->q, use_sel, use_nsel, out, fws,
                                             num_cu, s),
                    "batched gather + window attention");
}

}  // extern "C"
