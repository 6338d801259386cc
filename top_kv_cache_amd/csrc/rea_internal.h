// rea_internal.h - declarations shared by the host API (rea_api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "rea.h"

namespace rea {

// Validated geometry of one call (all values derived on the host).
struct Geom {
    int dtype;          // 0 bf16, 1 f32
    int esize;          // bytes per stored element
    int n_q, Hq, d;
    int Hkv;            // selection heads: the KV heads, or the query heads when each selects
    int g;              // query heads per selection head (1 when each query head selects)
    int rep;            // selection heads per cache head: selection head h reads KV head h / rep
    int64_t T;
    int64_t Gp, Lp;     // G' = min(G,T), L' = min(L, T-G')
    int64_t mid_lo, mid_hi;
    int64_t n_spans;    // ceil((mid_hi - mid_lo) / S)
    int S, topk, block_q, n_blk;
    int k_sel;          // min(topk, n_spans)
    // token segments: the kernels see spans of one token (S = 1); k_tok best
    // tokens are picked and each is widened to seg tokens; topk (= k_tok *
    // seg) is then the capacity of a selection.  seg = 0: span selection.
    int seg, k_tok;
    int last_len;       // length of span n_spans-1 (S unless the middle is ragged)
    int64_t W_cap;      // min(T, G' + k_sel*S + L')
    int64_t sh, st;     // K/V strides (elements) per head / per token
    float scale;        // softmax scale
    double theta;       // RoPE base
    // batched decode: selection heads [b * hps, (b + 1) * hps) belong to
    // sequence b, whose cache starts seq_stride elements after sequence b-1's
    // and whose length is lens[b] (device memory; nullptr: one sequence of T)
    const int64_t *lens;
    int hps;            // selection heads per sequence (Hkv when not batched)
    int64_t seq_stride;
    int G, L;           // the hyperparameters (regions are re-derived per sequence)
};

// Regions of one sequence of T tokens (the host derives the same for a
// single sequence): G' = min(G, T), L' = min(L, T - G'), middle [G', T - L')
// cut into spans of S from its start, in groups of 32 spans.
struct SeqGeom {
    int64_t T, Gp, Lp, mid_lo, mid_hi, n_spans, n_groups;
    int last_len;
};
__host__ __device__ inline SeqGeom seq_geom(int64_t T, int64_t G, int64_t L, int64_t S) {
    SeqGeom r;
    r.T = T;
    r.Gp = G < T ? G : T;
    r.Lp = L < T - r.Gp ? L : T - r.Gp;
    r.mid_lo = r.Gp;
    r.mid_hi = T - r.Lp;
    const int64_t n_mid = r.mid_hi - r.mid_lo;
    r.n_spans = (n_mid + S - 1) / S;
    r.n_groups = (r.n_spans + 31) / 32;
    r.last_len = r.n_spans > 0 ? (int)(n_mid - (r.n_spans - 1) * S) : 0;
    return r;
}

// The sequence of selection head h: its length (lens[b] clamped to [1, Tcap],
// or Tcap) and the element offset of its KV head in the cache.
struct SeqOf {
    int64_t T;
    int64_t kv_off;
};
__device__ __forceinline__ SeqOf seq_of(const int64_t *lens, int h, int hps, int rep,
                                        int64_t seq_stride, int64_t sh, int64_t Tcap) {
    const int b = h / hps;
    SeqOf r;
    int64_t T = Tcap;
    if (lens) {
        T = lens[b];
        T = T < 1 ? 1 : (T > Tcap ? Tcap : T);
    }
    r.T = T;
    r.kv_off = (int64_t)b * seq_stride + (int64_t)((h - b * hps) / rep) * sh;
    return r;
}

constexpr int kMaxHalfDim = 64;   // head_dim <= 128

// 1 when (y, yi) ranks before (x, xi) in the selection order (higher score
// first, the lower index first among equal scores), else 0.  Bitwise, not
// short-circuit, so that ranking loops compile without branches.
__device__ __forceinline__ uint32_t outranks(double y, int32_t yi, double x, int32_t xi) {
    return (uint32_t)(y > x) | ((uint32_t)(y == x) & (uint32_t)(yi < xi));
}

// ---- launchers (each returns hipGetLastError() of its launches) ----------

// Launches a kernel whose one parameter is an argument struct.  Non-null
// events take the start and end times of the dispatch itself (hipExtLaunchKernel
// stamps them from the kernel's own completion signal), so timing a kernel adds
// no marker packets, and no idle gaps, around it on the stream.
template <typename A>
hipError_t launch_struct(void (*kern)(A), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                         const A &a, hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr) {
    void *args[] = {const_cast<A *>(&a)};
    return hipExtLaunchKernel((const void *)kern, grid, block, args, lds, s, ev_begin, ev_end, 0);
}

// Step 1a: span scores [n_blk][Hkv][n_spans] (double) and the maximum of every
// group of 32 consecutive spans [n_blk][Hkv][score_groups(g)].  Non-null
// events time the scoring kernel's dispatch.  only (blocks of several queries):
// null, or one flag per (block, KV head) in device memory; then only the
// flagged pairs are scored.
int64_t score_groups(const Geom &g);
// group_second / group_arg (token level, S = 1, only): null, or arrays like
// group_max receiving each group's second largest score (a tied maximum
// counts twice) and the offset of a maximum within the group.
hipError_t launch_score(const Geom &g, const void *q, const void *k, double *span_scores,
                        double *group_max, int num_cu, hipStream_t s,
                        hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr,
                        const uint32_t *only = nullptr, double *group_second = nullptr,
                        int32_t *group_arg = nullptr, double *group_top = nullptr,
                        int32_t *group_top_idx = nullptr);
// Whether launch_score takes the plain decode scorer (one query, spans of
// S > 1, each selection head scored on its own): only that scorer fills
// group_top ([..][groups][2] doubles: each group's second and third largest
// span scores) and group_top_idx ([..][groups][2]: the spans holding its
// largest and second largest), when both are given.
bool score_decode_path(const Geom &g);

// Token segments: widen each selected token (sel_tok [n_blk*Hkv][k_tok],
// middle-relative, ascending) to g.seg tokens and write the union, ascending,
// to sel [n_blk*Hkv][g.topk] and its size to n_sel.
hipError_t launch_widen(const Geom &g, const int32_t *sel_tok, const int32_t *nsel_tok,
                        int32_t *sel, int32_t *n_sel, hipStream_t s);

// Step 1b: top-k per (block, KV head) from the span scores and group maxima;
// only: null, or device flags per (block, KV head) selecting the pairs to run.
// group_second / group_arg: null, or the scorer's arrays above (the large
// path then reads only the groups with two or more candidates).
// group_top / group_top_idx: null, or the decode scorer's arrays above (a
// candidate group whose third largest score is below the bound then gives its
// candidates from them, without its span scores being read).
hipError_t launch_topk(const Geom &g, const double *span_scores, const double *group_max,
                       int32_t *sel, int32_t *n_sel, hipStream_t s,
                       const uint32_t *only = nullptr, const double *group_second = nullptr,
                       const int32_t *group_arg = nullptr, const double *group_top = nullptr,
                       const int32_t *group_top_idx = nullptr);

// Step 1 for blocks of 64 queries on MFMA (bf16, d 128, S a multiple of 32):
// approximate span scores with a proven error bound, then an exact top-k that
// re-scores the uncertain spans in fp64.
bool mfma_block_path(const Geom &g);
size_t mfma_ws_bytes(const Geom &g);
hipError_t launch_score_select_mfma(const Geom &g, const void *q, const void *k,
                                    double *span_scores, int32_t *sel, int32_t *n_sel,
                                    void *ws, int num_cu, hipStream_t s,
                                    hipEvent_t ev_begin, hipEvent_t ev_end);

// Step 1 of a decode step with one selection per query head (bf16, d 128, S a
// multiple of 32, one sequence): the query heads of a KV head scored together
// on MFMA (approximate span scores with a proven bound), then the exact top-k
// by the certification.
bool heads_mfma_path(const Geom &g);
size_t heads_ws_bytes(const Geom &g);
hipError_t launch_score_select_heads(const Geom &g, const void *q, const void *k,
                                     double *span_scores, int32_t *sel, int32_t *n_sel,
                                     void *ws, int num_cu, hipStream_t s,
                                     hipEvent_t ev_begin, hipEvent_t ev_end);

// Steps 2-3: window rows (K rotated fp32, V copied) + lengths, then the queries.
hipError_t launch_gather_rope(const Geom &g, const void *k, const void *v, const void *q,
                              const int32_t *sel, const int32_t *n_sel, float *k_win,
                              void *v_win, float *q_rot, int32_t *W, int64_t W_cap,
                              hipStream_t s);

// Steps 2-4 fused for at most 8 query rows per (block, KV head): the window
// is read from the cache and attended without being written.
bool fused_decode_path(const Geom &g);
size_t fused_ws_bytes(const Geom &g);
hipError_t launch_fused_decode(const Geom &g, const void *k, const void *v, const void *q,
                               const int32_t *sel, const int32_t *n_sel, float *out, void *ws,
                               int num_cu, hipStream_t s);

// Steps 2-4 for more than 8 bf16 query rows per block and KV head inside
// rea_decode_step: the MFMA attention reads the window rows from the cache
// through the selection.  ws holds rope_table_bytes(g): the RoPE table of the
// window positions (first, so that consecutive calls on one workspace find it
// at the same place) and, for grids too small to fill the GPU, the partials
// of the key-tile splits.  table_ready: the table already holds rows
// [0, W_cap) (row w depends on w, d and theta only), so it is not rebuilt.
bool mfma_cache_attend_path(const Geom &g);
size_t rope_table_bytes(const Geom &g);
hipError_t launch_attend_mfma_cache(const Geom &g, const void *q, const void *k, const void *v,
                                    const int32_t *sel, const int32_t *n_sel, float *out,
                                    void *ws, hipStream_t s, bool table_ready = false);

// Step 4 for query blocks of at least 32 rows (bf16, d 128) on MFMA.
bool mfma_attend_path(const Geom &g);
hipError_t launch_attend_mfma(const Geom &g, const float *q_rot, const float *k_win,
                              const void *v_win, const int32_t *W, int64_t W_cap, float *out,
                              hipStream_t s);

// Step 4: split-window attention + combine (MFMA for large query blocks).
size_t attend_ws_bytes(const Geom &g, int64_t W_cap);
hipError_t launch_attend(const Geom &g, const float *q_rot, const float *k_win,
                         const void *v_win, const int32_t *W, int64_t W_cap, float *out,
                         void *ws, hipStream_t s);

// ---- host entry-point hooks (rea_api.cpp) --------------------------------

// Clear / set the calling thread's error detail (rea_last_error).
void api_clear_error();
rea_status api_error(rea_status st, const char *msg);
// rea_decode_step's host checks of everything but the workspace, and the
// workspace bytes the step needs.  No HIP call.
rea_status decode_check(const rea_problem *p, const rea_params *a, const float *out,
                        const int32_t *sel, const int32_t *n_sel, size_t *ws_bytes);
// rea_decode_step on a given workspace (does not clear the error detail).
rea_status decode_step_ws(const rea_problem *p, const rea_params *a, float *out, int32_t *sel,
                          int32_t *n_sel, void *ws, size_t ws_bytes, void *stream);

}  // namespace rea
