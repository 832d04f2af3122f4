// bkv_api.hip -- the C ABI of include/bkv.h: validation and launches.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "bkv.h"
#include "bkv_internal.hpp"
#include "bkv_step.hpp"

namespace {

constexpr int32_t kMaxLen = 8192;    // scores of one unit live in LDS
constexpr int32_t kMaxBq = 32;       // B_Q^max: one FPS wave holds 32 candidates
constexpr int32_t kMaxGroup = 8;     // query heads per KV head

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int check_shape(const bkv_shape* s) {
    if (!s) return BKV_EINVAL;
    if (s->n_layers <= 0 || s->batch <= 0 || s->n_q_heads <= 0 || s->n_kv_heads <= 0) return BKV_EINVAL;
    if (s->n_q_heads % s->n_kv_heads) return BKV_EINVAL;
    if (s->n_q_heads / s->n_kv_heads > kMaxGroup) return BKV_EUNSUPPORTED;
    if (s->head_dim != 64 && s->head_dim != 128) return BKV_EUNSUPPORTED;
    if (s->n_beacon < 0 || s->n_recent_q < 0 || s->n_beacon + s->n_recent_q < 1) return BKV_EINVAL;
    if (s->n_beacon + s->n_recent_q > kMaxBq) return BKV_EUNSUPPORTED;
    if (s->qcap < s->n_beacon + s->n_recent_q) return BKV_EINVAL;
    if (s->cap <= 0 || s->budget < 0 || s->n_prefix < 0 || s->n_recent_kv < 0) return BKV_EINVAL;
    if (s->flags & ~(BKV_CAUSAL_RECENT | BKV_POOL_MEAN | BKV_BEACON_INITIAL | BKV_BEACON_RANDOM | BKV_BEACON_NAIVE))
        return BKV_EINVAL;
    const uint32_t src = s->flags & (BKV_BEACON_INITIAL | BKV_BEACON_RANDOM | BKV_BEACON_NAIVE);
    if (src & (src - 1)) return BKV_EINVAL;   // at most one source
    const int64_t units = (int64_t)s->n_layers * s->batch * s->n_kv_heads;
    const int64_t qbufs = (int64_t)s->n_layers * s->batch * s->n_q_heads;
    if (units > INT32_MAX || qbufs > INT32_MAX) return BKV_ERANGE;
    return BKV_OK;
}

int check_len(const bkv_shape* s, int32_t n_len) {
    if (n_len <= 0) return BKV_ERANGE;
    if (n_len > s->cap) return BKV_ERANGE;
    if (n_len > kMaxLen) return BKV_EUNSUPPORTED;
    return BKV_OK;
}

int check_keep(const bkv_shape* s, int32_t n_len) {
    if (n_len > s->budget && s->budget < s->n_prefix + s->n_recent_kv) return BKV_ERANGE;
    return BKV_OK;
}

int units_of(const bkv_shape* s) { return s->n_layers * s->batch * s->n_kv_heads; }
int qbufs_of(const bkv_shape* s) { return s->n_layers * s->batch * s->n_q_heads; }

int hip_status(hipError_t e) { return e == hipSuccess ? BKV_OK : BKV_EHIP; }

int src_of(const bkv_shape* s) {
    if (s->flags & BKV_BEACON_INITIAL) return bkv::kSrcInitial;
    if (s->flags & BKV_BEACON_RANDOM) return bkv::kSrcRandom;
    if (s->flags & BKV_BEACON_NAIVE) return bkv::kSrcNaive;
    return bkv::kSrcFps;
}

bkv::FpsArgs fps_args(const bkv_shape* s, bkv_bf16* qbuf, int32_t* qcount, const bkv_bf16* q_new,
                      const bkv_bf16* q_recent, int32_t* fps_sel) {
    bkv::FpsArgs a;
    a.qbuf = qbuf;
    a.qcount = qcount;
    a.q_new = q_new;
    a.q_recent = q_recent;
    a.fps_sel = fps_sel;
    a.nbuf = qbufs_of(s);
    a.qcap = s->qcap;
    a.n_beacon = s->n_beacon;
    a.n_recent_q = s->n_recent_q;
    a.src = src_of(s);
    a.seed = s->seed;
    a.compress = 0;
    return a;
}

// FPS over rows [0, n_rows) of every buffer of q (buffer b's rows start at b * stride rows), into the query
// buffers: the prefill kernel, or the initial / random rules.
int launch_sample(const bkv_shape* s, const bkv_bf16* q, int64_t stride_rows, int32_t n_rows, bkv_bf16* qbuf,
                  int32_t* qcount, int32_t* fps_sel, hipStream_t st) {
    bkv::PrefillArgs a;
    a.q = q;
    a.q_stride = stride_rows * s->head_dim;
    a.qbuf = qbuf;
    a.qcount = qcount;
    a.fps_sel = fps_sel;
    a.nbuf = qbufs_of(s);
    a.P = n_rows;
    a.qcap = s->qcap;
    a.n_beacon = s->n_beacon;
    a.src = src_of(s) == bkv::kSrcNaive ? bkv::kSrcFps : src_of(s);
    a.seed = s->seed;
    a.lds_bytes = 0;
    if (a.src != bkv::kSrcFps) return hip_status(bkv::launch_prefill_src(a, s->head_dim, st));
    return hip_status(bkv::launch_prefill(a, s->head_dim, st));
}

bkv::ScoreArgs score_args(const bkv_shape* s, const bkv_bf16* K, int32_t n_len, const bkv_bf16* qbuf,
                          const int32_t* qcount, const bkv_bf16* q_recent, const int32_t* pos_recent,
                          const int32_t* t, const float* rope_cs, int32_t rope_rows, float* scores) {
    bkv::ScoreArgs a;
    a.K = K;
    a.qbuf = qbuf;
    a.qcount = qcount;
    a.q_recent = q_recent;
    a.pos_recent = pos_recent;
    a.t = t;
    a.rope_cs = rope_cs;
    a.scores = scores;
    a.units = units_of(s);
    a.n_len = n_len;
    a.cap = s->cap;
    a.batch = s->batch;
    a.hkv = s->n_kv_heads;
    a.G = s->n_q_heads / s->n_kv_heads;
    a.qcap = s->qcap;
    a.n_beacon = s->n_beacon;
    a.n_recent_q = s->n_recent_q;
    a.causal = (s->flags & BKV_CAUSAL_RECENT) ? 1 : 0;
    a.pool_mean = (s->flags & BKV_POOL_MEAN) ? 1 : 0;
    a.rope_rows = rope_rows;
    return a;
}

int check_score_ptrs(const bkv_bf16* K, const bkv_bf16* qbuf, const int32_t* qcount,
                     const bkv_bf16* q_recent, const int32_t* pos_recent, const int32_t* t,
                     const float* rope_cs, int32_t rope_rows, const bkv_shape* s) {
    if (!K || !qbuf || !qcount || !t || !rope_cs) return BKV_EINVAL;
    if (s->n_recent_q > 0 && (!q_recent || !pos_recent)) return BKV_EINVAL;
    if (!aligned16(K) || !aligned16(qbuf) || !aligned16(rope_cs)) return BKV_EINVAL;
    if (q_recent && !aligned16(q_recent)) return BKV_EINVAL;
    if (!aligned4(qcount) || !aligned4(t) || (pos_recent && !aligned4(pos_recent))) return BKV_EINVAL;
    if (rope_rows <= 0) return BKV_ERANGE;
    return BKV_OK;
}

}  // namespace

extern "C" {

int bkv_version(void) { return BKV_ABI_VERSION; }

const char* bkv_strerror(int code) {
    switch (code) {
        case BKV_OK: return "ok";
        case BKV_EINVAL: return "invalid argument (null or misaligned pointer, inconsistent shape)";
        case BKV_EUNSUPPORTED: return "unsupported shape (head_dim, group size, buffer or length limits)";
        case BKV_ERANGE: return "size out of range (n_len vs cap, budget vs forced keeps, table rows)";
        case BKV_EHIP: return "HIP kernel launch failed";
        default: return "unknown error";
    }
}

int bkv_rope_table(double theta, int32_t head_dim, int32_t p0, int32_t p1, float* host_out) {
    if (!host_out || head_dim <= 0 || (head_dim & 1) || p0 < 0 || p1 <= p0) return BKV_EINVAL;
    const int32_t h = head_dim / 2;
    for (int32_t i = 0; i < h; ++i) {
        const double f = pow(theta, -(double)(2 * i) / (double)head_dim);
        for (int32_t p = p0; p < p1; ++p) {
            const double ang = (double)p * f;
            float* o = host_out + ((size_t)(p - p0) * h + i) * 2;
            o[0] = (float)cos(ang);
            o[1] = (float)sin(ang);
        }
    }
    return BKV_OK;
}

int bkv_fps_update(const bkv_shape* s, bkv_bf16* qbuf, int32_t* qcount, const bkv_bf16* q_new,
                   int32_t* fps_sel, void* stream) {
    int e = check_shape(s);
    if (e) return e;
    if (!qbuf || !qcount || !q_new) return BKV_EINVAL;
    if (!aligned16(qbuf) || !aligned16(q_new) || !aligned4(qcount)) return BKV_EINVAL;
    if (fps_sel && !aligned4(fps_sel)) return BKV_EINVAL;
    bkv::FpsArgs a = fps_args(s, qbuf, qcount, q_new, nullptr, fps_sel);
    return hip_status(bkv::launch_fps(a, s->head_dim, false, (hipStream_t)stream));
}

int bkv_fps_merge(const bkv_shape* s, bkv_bf16* qbuf, int32_t* qcount, const bkv_bf16* q_recent,
                  int32_t* fps_sel, void* stream) {
    int e = check_shape(s);
    if (e) return e;
    if (!qbuf || !qcount || (s->n_recent_q > 0 && !q_recent)) return BKV_EINVAL;
    if (!aligned16(qbuf) || (q_recent && !aligned16(q_recent)) || !aligned4(qcount)) return BKV_EINVAL;
    if (fps_sel && !aligned4(fps_sel)) return BKV_EINVAL;
    bkv::FpsArgs a = fps_args(s, qbuf, qcount, nullptr, q_recent, fps_sel);
    return hip_status(bkv::launch_fps(a, s->head_dim, true, (hipStream_t)stream));
}

int bkv_fps_prefill(const bkv_shape* s, const bkv_bf16* q_prompt, int32_t n_prompt, bkv_bf16* qbuf,
                    int32_t* qcount, int32_t* fps_sel, void* stream) {
    int e = check_shape(s);
    if (e) return e;
    if (n_prompt < 0 || !qbuf || !qcount || (n_prompt > 0 && !q_prompt)) return BKV_EINVAL;
    if (n_prompt > BKV_PREFILL_MAX) return BKV_EUNSUPPORTED;
    if (!aligned16(qbuf) || (q_prompt && !aligned16(q_prompt)) || !aligned4(qcount)) return BKV_EINVAL;
    if (fps_sel && !aligned4(fps_sel)) return BKV_EINVAL;
    return launch_sample(s, q_prompt, n_prompt, n_prompt, qbuf, qcount, fps_sel, (hipStream_t)stream);
}

int bkv_fps_history(const bkv_shape* s, const bkv_bf16* hist, int32_t hcap, int32_t n_rows, bkv_bf16* qbuf,
                    int32_t* qcount, int32_t* fps_sel, void* stream) {
    int e = check_shape(s);
    if (e) return e;
    if (hcap < 0 || n_rows < 0 || n_rows > hcap || !qbuf || !qcount || (n_rows > 0 && !hist)) return BKV_EINVAL;
    if (n_rows > BKV_PREFILL_MAX) return BKV_EUNSUPPORTED;
    if (!aligned16(qbuf) || (hist && !aligned16(hist)) || !aligned4(qcount)) return BKV_EINVAL;
    if (fps_sel && !aligned4(fps_sel)) return BKV_EINVAL;
    return launch_sample(s, hist, hcap, n_rows, qbuf, qcount, fps_sel, (hipStream_t)stream);
}

int bkv_history_append(const bkv_shape* s, bkv_bf16* hist, int32_t hcap, int32_t* hcount, const bkv_bf16* q_new,
                       void* stream) {
    int e = check_shape(s);
    if (e) return e;
    if (hcap < 0 || !hist || !hcount || !q_new) return BKV_EINVAL;
    if (!aligned16(hist) || !aligned16(q_new) || !aligned4(hcount)) return BKV_EINVAL;
    bkv::HistArgs a;
    a.hist = hist;
    a.hcount = hcount;
    a.q_new = q_new;
    a.qbufs = qbufs_of(s);
    a.hcap = hcap;
    return hip_status(bkv::launch_history_append(a, s->head_dim, (hipStream_t)stream));
}

int bkv_fps_compress(const bkv_shape* s, bkv_bf16* qbuf, int32_t* qcount, int32_t* fps_sel, void* stream) {
    int e = check_shape(s);
    if (e) return e;
    if (!qbuf || !qcount || !aligned16(qbuf) || !aligned4(qcount)) return BKV_EINVAL;
    if (fps_sel && !aligned4(fps_sel)) return BKV_EINVAL;
    if (src_of(s) != bkv::kSrcFps) return BKV_OK;   // only continual FPS buffers hold uncompressed rows
    bkv::FpsArgs a = fps_args(s, qbuf, qcount, nullptr, nullptr, fps_sel);
    a.compress = 1;
    return hip_status(bkv::launch_fps(a, s->head_dim, false, (hipStream_t)stream));
}

size_t bkv_workspace_bytes(const bkv_shape* s, int32_t n_len) {
    (void)s;
    (void)n_len;
    return 0;
}

int bkv_score(const bkv_shape* s, const bkv_bf16* K, int32_t n_len, const bkv_bf16* qbuf,
              const int32_t* qcount, const bkv_bf16* q_recent, const int32_t* pos_recent, const int32_t* t,
              const float* rope_cs, int32_t rope_rows, float* scores, void* stream) {
    int e = check_shape(s);
    if (e) return e;
    if ((e = check_len(s, n_len))) return e;
    if ((e = check_score_ptrs(K, qbuf, qcount, q_recent, pos_recent, t, rope_cs, rope_rows, s))) return e;
    if (!scores || !aligned4(scores)) return BKV_EINVAL;
    bkv::ScoreArgs a = score_args(s, K, n_len, qbuf, qcount, q_recent, pos_recent, t, rope_cs, rope_rows, scores);
    return hip_status(bkv::launch_score(a, s->head_dim, (hipStream_t)stream));
}

int bkv_select(const bkv_shape* s, const float* scores, int32_t n_len, int32_t* idx, void* stream) {
    int e = check_shape(s);
    if (e) return e;
    if ((e = check_len(s, n_len))) return e;
    if ((e = check_keep(s, n_len))) return e;
    if (!scores || !idx || !aligned4(scores) || !aligned4(idx)) return BKV_EINVAL;
    bkv::SelectArgs a;
    a.scores = scores;
    a.idx = idx;
    a.units = units_of(s);
    a.n_len = n_len;
    a.budget = s->budget;
    a.n_prefix = s->n_prefix;
    a.n_recent_kv = s->n_recent_kv;
    return hip_status(bkv::launch_select(a, (hipStream_t)stream));
}

int bkv_compact(const bkv_shape* s, bkv_bf16* K, bkv_bf16* V, int32_t n_len, const int32_t* idx, void* stream) {
    int e = check_shape(s);
    if (e) return e;
    if ((e = check_len(s, n_len))) return e;
    if (!K || !V || !idx || !aligned16(K) || !aligned16(V) || !aligned4(idx)) return BKV_EINVAL;
    bkv::CompactArgs a;
    a.K = K;
    a.V = V;
    a.idx = idx;
    a.units = units_of(s);
    a.n_len = n_len;
    a.cap = s->cap;
    a.budget = s->budget;
    return hip_status(bkv::launch_compact(a, s->head_dim, (hipStream_t)stream));
}

int bkv_evict(const bkv_shape* s, bkv_bf16* K, bkv_bf16* V, int32_t n_len, bkv_bf16* qbuf, int32_t* qcount,
              const bkv_bf16* q_recent, const int32_t* pos_recent, const int32_t* t, const float* rope_cs,
              int32_t rope_rows, int32_t* idx_out, float* scores_out, int32_t* fps_sel_out, void* stream) {
    int e = check_shape(s);
    if (e) return e;
    if ((e = check_len(s, n_len))) return e;
    if ((e = check_keep(s, n_len))) return e;
    if ((e = check_score_ptrs(K, qbuf, qcount, q_recent, pos_recent, t, rope_cs, rope_rows, s))) return e;
    if (!V || !aligned16(V)) return BKV_EINVAL;
    if ((idx_out && !aligned4(idx_out)) || (scores_out && !aligned4(scores_out)) ||
        (fps_sel_out && !aligned4(fps_sel_out)))
        return BKV_EINVAL;
    hipStream_t st = (hipStream_t)stream;

    bkv::EvictArgs ea;
    ea.sc = score_args(s, K, n_len, qbuf, qcount, q_recent, pos_recent, t, rope_cs, rope_rows, scores_out);
    ea.K = K;
    ea.V = V;
    ea.idx = idx_out;
    ea.budget = s->budget;
    ea.n_prefix = s->n_prefix;
    ea.n_recent_kv = s->n_recent_kv;
    if ((e = hip_status(bkv::launch_evict(ea, s->head_dim, st)))) return e;

    bkv::FpsArgs fa = fps_args(s, qbuf, qcount, nullptr, q_recent, fps_sel_out);
    return hip_status(bkv::launch_fps(fa, s->head_dim, true, st));
}

int bkv_append_kv(const bkv_shape* s, bkv_bf16* K, bkv_bf16* V, int32_t L, const bkv_bf16* k_new,
                  const bkv_bf16* v_new, const int32_t* pos, const float* rope_cs, int32_t rope_rows, void* stream) {
    int e = check_shape(s);
    if (e) return e;
    if (L < 0 || L >= s->cap || rope_rows <= 0) return BKV_ERANGE;
    if (!K || !V || !k_new || !v_new || !pos || !rope_cs) return BKV_EINVAL;
    if (!aligned16(K) || !aligned16(V) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(rope_cs) ||
        !aligned4(pos))
        return BKV_EINVAL;
    bkv::AppendArgs aa;
    aa.K = K;
    aa.V = V;
    aa.k_new = k_new;
    aa.v_new = v_new;
    aa.pos = pos;
    aa.rope_cs = rope_cs;
    aa.units = units_of(s);
    aa.cap = s->cap;
    aa.L = L;
    aa.batch = s->batch;
    aa.hkv = s->n_kv_heads;
    aa.rope_rows = rope_rows;
    return hip_status(bkv::launch_append(aa, s->head_dim, (hipStream_t)stream));
}

int bkv_decode_attention(const bkv_shape* s, const bkv_bf16* K, const bkv_bf16* V, int32_t n_len,
                         const bkv_bf16* q, const int32_t* pos, const float* rope_cs, int32_t rope_rows, float* out,
                         void* stream) {
    int e = check_shape(s);
    if (e) return e;
    if (n_len <= 0 || n_len > s->cap || rope_rows <= 0) return BKV_ERANGE;
    if (!K || !V || !q || !pos || !rope_cs || !out) return BKV_EINVAL;
    if (!aligned16(K) || !aligned16(V) || !aligned16(q) || !aligned16(rope_cs) || !aligned4(pos) || !aligned4(out))
        return BKV_EINVAL;
    bkv::AttnArgs a;
    a.K = K;
    a.V = V;
    a.q = q;
    a.pos = pos;
    a.rope_cs = rope_cs;
    a.out = out;
    a.units = units_of(s);
    a.n_len = n_len;
    a.cap = s->cap;
    a.batch = s->batch;
    a.hkv = s->n_kv_heads;
    a.G = s->n_q_heads / s->n_kv_heads;
    a.rope_rows = rope_rows;
    return hip_status(bkv::launch_attention(a, s->head_dim, (hipStream_t)stream));
}

int bkv_decode_step(const bkv_shape* s, bkv_bf16* K, bkv_bf16* V, int32_t L, const bkv_bf16* k_new,
                    const bkv_bf16* v_new, const int32_t* pos, bkv_bf16* qbuf, int32_t* qcount,
                    const bkv_bf16* q_new, bkv_bf16* q_recent, int32_t* pos_recent, const float* rope_cs,
                    int32_t rope_rows, int32_t* fps_sel, void* stream) {
    int e = check_shape(s);
    if (e) return e;
    if (L < 0 || L >= s->cap || rope_rows <= 0) return BKV_ERANGE;
    if (!K || !V || !k_new || !v_new || !pos || !qbuf || !qcount || !q_new || !rope_cs) return BKV_EINVAL;
    if (!aligned16(K) || !aligned16(V) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(qbuf) ||
        !aligned16(q_new) || !aligned16(rope_cs) || !aligned4(pos) || !aligned4(qcount))
        return BKV_EINVAL;
    const int32_t ring0 = s->cap - s->n_recent_q;   // first step of the recent phase
    const bool ring = L >= ring0;
    if (ring && (!q_recent || !pos_recent || !aligned16(q_recent) || !aligned4(pos_recent))) return BKV_EINVAL;
    if (fps_sel && !aligned4(fps_sel)) return BKV_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    // the buffers' FPS kernels (the update, or the compression at the first ring step) size their grid from
    // an occupancy query: made here, before anything is enqueued, so that its failure enqueues nothing
    const bool fps_src = src_of(s) == bkv::kSrcFps;
    if (fps_src && (!ring || L == ring0)) {
        int64_t fit = 0;
        if ((e = hip_status(bkv::fps_grid_limit(s->head_dim, &fit)))) return e;
    }

    bkv::AppendArgs aa;
    aa.K = K;
    aa.V = V;
    aa.k_new = k_new;
    aa.v_new = v_new;
    aa.pos = pos;
    aa.rope_cs = rope_cs;
    aa.units = units_of(s);
    aa.cap = s->cap;
    aa.L = L;
    aa.batch = s->batch;
    aa.hkv = s->n_kv_heads;
    aa.rope_rows = rope_rows;
    if (!ring && fps_src) {   // collection phase: the buffer update appends the key and value in the same launch
        const bkv::FpsArgs fa = fps_args(s, qbuf, qcount, q_new, nullptr, fps_sel);
        return hip_status(bkv::launch_fps_step(fa, aa, s->head_dim, st));
    }
    if ((e = hip_status(bkv::launch_append(aa, s->head_dim, st)))) return e;

    if (ring && L == ring0 && fps_src) {   // freeze: buffers still holding more than n_beacon rows are sampled
        bkv::FpsArgs ca = fps_args(s, qbuf, qcount, nullptr, nullptr, nullptr);
        ca.compress = 1;
        if ((e = hip_status(bkv::launch_fps(ca, s->head_dim, false, st)))) return e;
    }
    if (ring) {
        bkv::RingArgs ra;
        ra.q_recent = q_recent;
        ra.pos_recent = pos_recent;
        ra.q_new = q_new;
        ra.pos = pos;
        ra.qbufs = qbufs_of(s);
        ra.batch = s->batch;
        ra.n_recent_q = s->n_recent_q;
        ra.slot = L - ring0;
        return hip_status(bkv::launch_ring(ra, s->head_dim, st));
    }
    bkv::FpsArgs fa = fps_args(s, qbuf, qcount, q_new, nullptr, fps_sel);
    return hip_status(bkv::launch_fps(fa, s->head_dim, false, st));
}

}  // extern "C"
