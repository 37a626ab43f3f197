// Shared device-side definitions for the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator dies, workgroups dealt round-robin

enum MaskKind { kMaskNone = 0, kMaskCausal = 1, kMaskWindow = 2, kMaskDocument = 3 };

// Compute units of the current device (read once per process; host code).
int device_cus();

// Arguments of one prefill launch (already validated on the host).
struct PrefillParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv, Nq, Nk;
    int group;          // Hq / Hkv
    float scale_log2;   // scale * log2(e): scores go straight to the base-2 domain
    float scale;        // scale itself (the fp32 kernel's score modifications)
    int mask_kind;
    int window;         // clamped to [1, Nk] on the host
    const int32_t* doc_offsets;
    int num_docs;
    int num_q_tiles;
    int q_tile_pairs;          // > 0: workgroup u takes query tiles num_q_tiles-1-u and u (set by the launcher)
    int sink_end;              // window mask: keys [0, sink_end) stay visible too (0: none)
    const float* sink_logits;  // [Hq] learned sink logit per query head, or null
    float softcap;             // > 0: score -> softcap * tanh(score / softcap); 0: off
    const float* alibi_slopes; // [Hq] or null: score += slope * (key - query position)
    int soft_exp2 = 0;         // 0, 2 or 4: weights per lane and 16-key block from the software 2^x
    int num_cus = 256;         // compute units of the device (the wave-priority phase)
};

// Arguments of one chunked-prefill launch over the paged cache (validated on
// the host).  Queries, outputs and LSEs are token-major: row t of q is token
// t of the concatenated chunks, [total_q, Hq, d].
struct PagedPrefillParams {
    const uint16_t* q;
    const uint16_t* k_pages;    // [num_pages, Hkv, 16, d]
    const uint16_t* v_pages;
    const int32_t* block_table; // [num_seqs, max_pages]
    const int32_t* seq_lens;    // [num_seqs]: cached tokens, the chunk included
    const int32_t* q_offsets;   // [num_seqs + 1]: chunk s is rows q_offsets[s] .. q_offsets[s+1]
    uint16_t* o;
    float* lse;                 // [total_q, Hq] or null
    int num_seqs, Hq, Hkv, group, max_pages;
    int max_len;                // max_seq_len: seq_lens entries are clamped to [0, max_len] before use
    int num_q_tiles;            // query tiles of the longest chunk
    float scale_log2;
    int mask_kind;              // none, causal or window
    int window;
    int sink_end;               // window mask: keys [0, sink_end) stay visible too
    const float* sink_logits;   // [Hq] or null
    float softcap;              // as in PrefillParams
    const float* alibi_slopes;
};

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Score modifications of one query head, in the base-2 domain of the
// kernels (FlexAttention's score_mod, "Attention and matrix kernels" page,
// How it works).  With x = scale * q.k, a soft cap c gives
//   c tanh(x / c) = c - 2c / (e^(2x/c) + 1),   e^(2x/c) = 2^(q.k * cap_k),
// and the ALiBi-style bias adds slope * (key - query position) after it.
// The logit times log2(e) is then cap_l2 - 2 cap_l2 / (2^(q.k cap_k) + 1) +
// slope_l2 * (key - query position); without a cap the first terms are
// q.k * scale_l2.
struct ScoreMod {
    float cap_k;      // 2 scale log2(e) / c; 0: no cap
    float cap_l2;     // c log2(e)
    float scale_l2;   // scale log2(e)
    float slope_l2;   // this head's slope times log2(e); 0 without slopes
};

__device__ __forceinline__ ScoreMod make_score_mod(float scale_log2, float softcap, const float* slopes, int hq) {
    ScoreMod m;
    m.cap_k = softcap > 0.f ? 2.f * scale_log2 / softcap : 0.f;
    m.cap_l2 = softcap * kLog2e;
    m.scale_l2 = scale_log2;
    m.slope_l2 = slopes != nullptr ? slopes[hq] * kLog2e : 0.f;
    return m;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// First key position of the document that holds key position `pos` (pos >= 0).
__host__ __device__ __forceinline__ int doc_start(const int32_t* off, int num_docs, int pos) {
    int lo = 0, hi = num_docs - 1;  // answer t in [0, num_docs-1] with off[t] <= pos
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= pos) lo = mid; else hi = mid - 1;
    }
    return off[lo];
}

// Visible keys of query row i form one interval [lo, hi] (inclusive) for every
// mask kind; an empty row has lo > hi.  Query i sits at key position
// pos = i + Nk - Nq.  Both ends are non-decreasing in i, which is what lets a
// tile of rows bound its key range by its first and last row.
__host__ __device__ __forceinline__ void row_interval(const PrefillParams& p, int i, int& lo, int& hi) {
    if (i < 0 || i >= p.Nq) { lo = p.Nk; hi = -1; return; }
    const int pos = i + p.Nk - p.Nq;
    if (p.mask_kind == kMaskNone) { lo = 0; hi = p.Nk - 1; return; }
    hi = pos < p.Nk - 1 ? pos : p.Nk - 1;
    if (pos < 0) { lo = 0; hi = -1; return; }
    if (p.mask_kind == kMaskCausal) {
        lo = 0;
    } else if (p.mask_kind == kMaskWindow) {
        lo = pos - p.window + 1;
        lo = lo > 0 ? lo : 0;
    } else {
        lo = doc_start(p.doc_offsets, p.num_docs, pos);
    }
}

// Query rows that see some key of [k0, k_last] (0 <= k0 <= k_last < Nk), as
// the range [first, last] (empty when first > last): from the first row whose
// interval reaches k0 (hi >= k0) to the last row whose interval starts at or
// before k_last (lo <= k_last), or every later row when sink keys lie in the
// range.  Both ends are monotone in the row.  With row = pos + Nq - Nk, a
// masked row's end min(pos, Nk - 1) reaches k0 exactly when pos >= k0, and a
// window row's start max(pos - W + 1, 0) is at most k_last exactly when
// pos <= k_last + W - 1; so only document masks, whose starts come from the
// offsets, search the rows.
__host__ __device__ __forceinline__ void query_rows_seeing(const PrefillParams& p, int k0, int k_last, int& first,
                                                           int& last) {
    const int shift = p.Nq - p.Nk;
    if (p.mask_kind == kMaskNone) {
        first = 0;
        last = p.Nq - 1;
        return;
    }
    first = k0 + shift;
    first = first < 0 ? 0 : (first > p.Nq ? p.Nq : first);
    if (k0 < p.sink_end || p.mask_kind == kMaskCausal) {
        last = p.Nq - 1;
    } else if (p.mask_kind == kMaskWindow) {
        last = k_last + p.window - 1 + shift;
        last = last < -1 ? -1 : (last > p.Nq - 1 ? p.Nq - 1 : last);
    } else {
        int a = -1, z = p.Nq - 1;
        while (a < z) {
            const int mid = (a + z + 1) >> 1;
            int l, h;
            row_interval(p, mid, l, h);
            if (l <= k_last) a = mid; else z = mid - 1;
        }
        last = a;
    }
}

// Sink tokens (StreamingLLM's, "Attention Is the Bottleneck", Sliding windows
// and local:global layers) add a second visible interval [0, sink_end) to a
// window row's [lo, hi] (causality still applies: only keys <= hi).  A
// workgroup then visits the sink tiles [0, s0) first and its window tiles
// after them; iteration it runs tile tile_of(it).  When the sink tiles reach
// the window tiles the union is one range starting at tile 0.
struct TileRange {
    int s0;        // sink tiles visited before the window range
    int t_begin;   // first tile of the window range
    int n;         // iterations
};

__device__ __forceinline__ TileRange tile_range(int lo_wg, int hi_wg, int sink_end, int bn) {
    TileRange r;
    int t_begin = lo_wg / bn;
    const int t_end = hi_wg >= lo_wg ? hi_wg / bn : t_begin - 1;
    int s0 = 0;
    if (t_end >= t_begin && sink_end > 0) {
        const int sk = min((sink_end + bn - 1) / bn, t_end + 1);
        if (sk >= t_begin) t_begin = 0;
        else s0 = sk;
    }
    r.s0 = s0;
    r.t_begin = t_begin;
    r.n = t_end >= t_begin ? s0 + t_end - t_begin + 1 : 0;
    return r;
}

__device__ __forceinline__ int tile_of(const TileRange& r, int it) { return it < r.s0 ? it : r.t_begin + it - r.s0; }

// Row statistics to output scale and LSE, folding in an optional learned
// sink (base-2 logit s2, -inf for none) as one more denominator term with a
// zero value (gpt-oss's per-head sink, same page and section):
//   O = acc * a / (l_o * a + b),  LSE = ln 2 * (M + log2(l_lse * a + b))
// with M = max(m_run, s2), a = 2^(m_run - M), b = 2^(s2 - M), so nothing
// overflows whichever term dominates.  Without a sink this is acc / l_o and
// m_run + log2(l_lse); a row that saw no key and has no sink gets 0 / -inf.
__device__ __forceinline__ void finish_row(float m_run, float l_o, float l_lse, float s2, float& inv, float& lse) {
    const float M = fmaxf(m_run, s2);
    if (M == -__builtin_inff()) {
        inv = 0.f;
        lse = -__builtin_inff();
        return;
    }
    const float a = __builtin_amdgcn_exp2f(m_run - M);
    const float b = __builtin_amdgcn_exp2f(s2 - M);
    const float den = l_o * a + b;
    inv = den > 0.f ? a / den : 0.f;
    lse = (M + __builtin_amdgcn_logf(l_lse * a + b)) * kLn2;
}

// Workgroup id -> (b*Hkv + kv head, q tile, head within the group).
// Tiles are issued heaviest first (descending q tile: under causal-type masks
// later tiles see more keys).  When the (batch, kv head) pairs divide evenly
// over the dies, every die gets whole pairs, so the K/V of a pair stays in
// that die's own L2.
__device__ __forceinline__ void decode_work(int id, int nbk, int nqt, int group,
                                            int& bk, int& qt, int& g) {
    int qrev, r;
    if (nbk % kNumXcd == 0) {
        const int x = id % kNumXcd, u = id / kNumXcd;
        const int bpx = nbk / kNumXcd;
        qrev = u / (bpx * group);
        r = u % (bpx * group);
        bk = x * bpx + r / group;
    } else {
        qrev = id / (nbk * group);
        r = id % (nbk * group);
        bk = r / group;
    }
    g = r % group;
    qt = nqt - 1 - qrev;
}

// Workgroup id -> (sequence * Hkv + kv head, q tile, head within the group)
// for chunked prefill over the paged cache.  All workgroups of one (sequence,
// KV head) pair are issued together, on one die, so that pair's cached K/V
// (which every query tile and every head of the group re-reads) is fetched
// from HBM about once and then served from that die's L2.  With the query-
// tile-major order of decode_work a die would cycle through all its pairs'
// caches at once, far more than its L2 holds.  Pairs are dealt to the dies
// round-robin (pair x, x + 8, ... on die x) when they divide evenly.
__device__ __forceinline__ void decode_work_pair_major(int id, int nbk, int nqt, int group,
                                                       int& bk, int& qt, int& g) {
    const int per_pair = nqt * group;
    int r;
    if (nbk % kNumXcd == 0) {
        const int x = id % kNumXcd, u = id / kNumXcd;
        bk = (u / per_pair) * kNumXcd + x;
        r = u % per_pair;
    } else {
        bk = id / per_pair;
        r = id % per_pair;
    }
    qt = nqt - 1 - r / group;   // within a pair, the later (heavier) query tiles first
    g = r % group;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 f = {a, b};
    bf16x2 h = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

// acc + lo + hi of a packed bf16 pair (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16x2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3f803f80u), acc,
                                           false);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

}  // namespace xattn
