// bkv_internal.hpp -- kernel argument blocks and launchers (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bkv.h"

namespace bkv {

struct FpsArgs {
    bkv_bf16* qbuf;            // [nbuf][qcap][d]
    int32_t* qcount;           // [nbuf]
    const bkv_bf16* q_new;     // [nbuf][d]          (update)
    const bkv_bf16* q_recent;  // [nbuf][n_recent_q][d] (merge)
    int32_t* fps_sel;          // [nbuf][n_beacon] or null
    int nbuf, qcap, n_beacon, n_recent_q;
    int src;                   // beacon source: kSrcFps, kSrcInitial, kSrcRandom, kSrcNaive
    uint32_t seed;             // key of the random-history draws
    int compress;              // update without an append: sample the buffers holding more than n_beacon rows
};

constexpr int kSrcFps = 0, kSrcInitial = 1, kSrcRandom = 2, kSrcNaive = 3;

struct PrefillArgs {
    const bkv_bf16* q;         // prompt queries: buffer b's rows are q[b * q_stride + i * d], i < P
    int64_t q_stride;          // elements from one buffer's first row to the next buffer's
    bkv_bf16* qbuf;            // [nbuf][qcap][d]
    int32_t* qcount;           // [nbuf]
    int32_t* fps_sel;          // [nbuf][n_beacon] or null
    int nbuf, P, qcap, n_beacon;
    int src;                   // beacon source
    uint32_t seed;
    int lds_bytes;             // LDS a workgroup may take (set at launch)
};

struct ScoreArgs {
    const bkv_bf16* K;         // [units][cap][d]
    const bkv_bf16* qbuf;      // [qbufs][qcap][d]
    const int32_t* qcount;     // [qbufs]
    const bkv_bf16* q_recent;  // [qbufs][n_recent_q][d]
    const int32_t* pos_recent; // [batch][n_recent_q]
    const int32_t* t;          // [batch]
    const float* rope_cs;      // [rope_rows][d/2][2]
    float* scores;             // [units][n_len]
    int units, n_len, cap, batch, hkv, G, qcap, n_beacon, n_recent_q, causal, pool_mean, rope_rows;
};

struct SelectArgs {
    const float* scores;       // [units][n_len]
    int32_t* idx;              // [units][budget]
    int units, n_len, budget, n_prefix, n_recent_kv;
};

struct CompactArgs {
    bkv_bf16* K;               // [units][cap][d]
    bkv_bf16* V;
    const int32_t* idx;        // [units][budget]
    int units, n_len, cap, budget;
};

struct EvictArgs {
    ScoreArgs sc;              // scoring inputs (sc.scores: optional copy of the scores, may be null)
    bkv_bf16* K;               // [units][cap][d], in place
    bkv_bf16* V;
    int32_t* idx;              // [units][budget], optional copy of the keep set (may be null)
    int budget, n_prefix, n_recent_kv;
};

struct AppendArgs {
    bkv_bf16* K;               // [units][cap][d]
    bkv_bf16* V;
    const bkv_bf16* k_new;     // [units][d] pre-RoPE
    const bkv_bf16* v_new;     // [units][d]
    const int32_t* pos;        // [batch]
    const float* rope_cs;      // [rope_rows][d/2][2]
    int units, cap, L, batch, hkv, rope_rows;
};

struct AttnArgs {
    const bkv_bf16* K;         // [units][cap][d] post-RoPE
    const bkv_bf16* V;
    const bkv_bf16* q;         // [qbufs][d] pre-RoPE
    const int32_t* pos;        // [batch]
    const float* rope_cs;      // [rope_rows][d/2][2]
    float* out;                // [qbufs][d]
    int units, n_len, cap, batch, hkv, G, rope_rows;
};

struct RingArgs {
    bkv_bf16* q_recent;        // [qbufs][n_recent_q][d]
    int32_t* pos_recent;       // [batch][n_recent_q]
    const bkv_bf16* q_new;     // [qbufs][d]
    const int32_t* pos;        // [batch]
    int qbufs, batch, n_recent_q, slot;
};

struct HistArgs {
    bkv_bf16* hist;            // [qbufs][hcap][d]
    int32_t* hcount;           // [qbufs]
    const bkv_bf16* q_new;     // [qbufs][d]
    int qbufs, hcap;
};

hipError_t launch_fps(const FpsArgs& a, int d, bool merge, hipStream_t st);
hipError_t launch_prefill(const PrefillArgs& a, int d, hipStream_t st);
// initial / random beacon sources: one offer per buffer, the merge of the recents, the prefill
hipError_t launch_offer(const FpsArgs& a, int d, hipStream_t st);
hipError_t launch_offer_merge(const FpsArgs& a, int d, hipStream_t st);
hipError_t launch_prefill_src(const PrefillArgs& a, int d, hipStream_t st);
hipError_t launch_score(const ScoreArgs& a, int d, hipStream_t st);
hipError_t launch_select(const SelectArgs& a, hipStream_t st);
hipError_t launch_compact(const CompactArgs& a, int d, hipStream_t st);
hipError_t launch_append(const AppendArgs& a, int d, hipStream_t st);
hipError_t launch_evict(const EvictArgs& a, int d, hipStream_t st);
hipError_t launch_ring(const RingArgs& a, int d, hipStream_t st);
hipError_t launch_history_append(const HistArgs& a, int d, hipStream_t st);
// the update kernel's grid (workgroups resident at once); queried before a call's first launch
hipError_t fps_grid_limit(int d, int64_t* out);
hipError_t launch_attention(const AttnArgs& a, int d, hipStream_t st);

}  // namespace bkv
