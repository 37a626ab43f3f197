// C ABI of the attention library: argument checks, launch geometry, status codes.
#include <stdio.h>
#include <string.h>

#include "../../include/exact_attn.h"
#include "common.hpp"

namespace xattn {
int launch_prefill_bf16(const PrefillParams& p, int d, hipStream_t stream);
int prefill_bf16_rows_per_block();
int launch_prefill_f32(const PrefillParams& p, int d, hipStream_t stream);
int launch_paged_prefill_bf16(const PagedPrefillParams& p, int d, hipStream_t stream);
}  // namespace xattn

#include "decode_params.hpp"
#include "backward_params.hpp"

namespace {

thread_local char g_hip_msg[256] = "HIP error";

constexpr long long kMaxSeq = 1LL << 28;     // keeps every row / position index in int32
constexpr long long kMaxGrid = 1LL << 24;    // workgroups per launch (x 256 threads < 2^32)

int hip_status(hipError_t e) {
    if (e == hipSuccess) return ATTN_OK;
    snprintf(g_hip_msg, sizeof g_hip_msg, "HIP error: %s", hipGetErrorString(e));
    return ATTN_ERR_HIP;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// sink tokens: window mask only, >= 0; sink logits: any kind, 4-byte aligned
bool sinks_ok(const attn_mask& m) {
    if (m.sink_tokens < 0) return false;
    if (m.sink_tokens > 0 && m.kind != ATTN_MASK_SLIDING_WINDOW) return false;
    return ((uintptr_t)m.sink_logits & 3u) == 0;
}

// score modifications: soft cap finite and >= 0 (NaN fails), slopes 4-byte aligned
bool mods_ok(const attn_mask& m) {
    if (!(m.softcap >= 0.f) || m.softcap == __builtin_inff()) return false;
    return ((uintptr_t)m.alibi_slopes & 3u) == 0;
}

}  // namespace

extern "C" const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
        case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
        case ATTN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case ATTN_ERR_HIP: return g_hip_msg;
        default: return "unknown status";
    }
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                        attn_mask mask, int dtype, hipStream_t stream) {
    if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0 || d < 0) return ATTN_ERR_INVALID_ARGUMENT;
    if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_INVALID_ARGUMENT;
    if (mask.kind < ATTN_MASK_NONE || mask.kind > ATTN_MASK_DOCUMENT) return ATTN_ERR_INVALID_ARGUMENT;
    if (mask.kind == ATTN_MASK_SLIDING_WINDOW && mask.window < 1) return ATTN_ERR_INVALID_ARGUMENT;
    if (mask.kind == ATTN_MASK_DOCUMENT && (mask.num_docs < 1 || mask.doc_offsets == nullptr))
        return ATTN_ERR_INVALID_ARGUMENT;
    if (!sinks_ok(mask) || !mods_ok(mask)) return ATTN_ERR_INVALID_ARGUMENT;
    if (!(scale == scale) || scale <= 0.f || scale == __builtin_inff()) return ATTN_ERR_INVALID_ARGUMENT;
    if (Hkv == 0 ? Hq != 0 : (Hq % Hkv) != 0) return ATTN_ERR_INVALID_ARGUMENT;
    if (mask.soft_exp2 != 0 && mask.soft_exp2 != 2 && mask.soft_exp2 != 4) return ATTN_ERR_INVALID_ARGUMENT;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (mask.soft_exp2 != 0 &&
        (d != 128 || dtype != ATTN_DTYPE_BF16 || mask.softcap > 0.f || mask.alibi_slopes != nullptr))
        return ATTN_ERR_UNSUPPORTED;
    if (Nq > kMaxSeq || Nk > kMaxSeq) return ATTN_ERR_UNSUPPORTED;
    if ((long long)B * Hq * Nq == 0) return ATTN_OK;  // nothing to write
    if (q == nullptr || o == nullptr) return ATTN_ERR_INVALID_ARGUMENT;
    if (Nk > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_INVALID_ARGUMENT;
    const long long rows_per_block = dtype == ATTN_DTYPE_BF16 ? xattn::prefill_bf16_rows_per_block() : 128;
    const long long tiles = (Nq + rows_per_block - 1) / rows_per_block;
    if ((long long)B * Hq * tiles > kMaxGrid) return ATTN_ERR_UNSUPPORTED;

    xattn::PrefillParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk;
    p.group = Hq / Hkv;
    p.scale_log2 = scale * xattn::kLog2e;
    p.scale = scale;
    p.mask_kind = mask.kind;
    p.window = mask.kind == ATTN_MASK_SLIDING_WINDOW ? (mask.window < Nk ? mask.window : (Nk > 0 ? Nk : 1)) : 0;
    p.doc_offsets = mask.kind == ATTN_MASK_DOCUMENT ? mask.doc_offsets : nullptr;
    p.num_docs = mask.kind == ATTN_MASK_DOCUMENT ? mask.num_docs : 0;
    p.num_q_tiles = (int)tiles;
    p.q_tile_pairs = 0;
    p.sink_end = mask.kind == ATTN_MASK_SLIDING_WINDOW ? mask.sink_tokens : 0;
    p.sink_logits = mask.sink_logits;
    p.softcap = mask.softcap;
    p.alibi_slopes = mask.alibi_slopes;
    p.soft_exp2 = mask.soft_exp2;

    if (dtype == ATTN_DTYPE_BF16)
        xattn::launch_prefill_bf16(p, d, stream);
    else
        xattn::launch_prefill_f32(p, d, stream);
    return hip_status(hipGetLastError());
}

extern "C" size_t attn_paged_decode_workspace_size(int num_seqs, int Hq, int d, int max_seq_len) {
    if (num_seqs < 0 || Hq < 0 || max_seq_len < 0 || (d != 64 && d != 128)) return 0;
    return xattn::decode_workspace_bytes(num_seqs, Hq, d, max_seq_len);
}

namespace {

// Argument checks of a paged decode call, everything but the workspace.
int decode_args_ok(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                   const int32_t* seq_lens, void* o, int num_seqs, int Hq, int Hkv, int d, int page_size,
                   int max_pages_per_seq, int max_seq_len, float scale, const float* sink_logits, float softcap,
                   const float* alibi_slopes) {
    if (num_seqs < 0 || Hq < 0 || Hkv < 0 || d < 0 || max_pages_per_seq < 0 || max_seq_len < 0)
        return ATTN_ERR_INVALID_ARGUMENT;
    if (Hkv == 0 ? Hq != 0 : (Hq % Hkv) != 0) return ATTN_ERR_INVALID_ARGUMENT;
    if (!(scale == scale) || scale <= 0.f || scale == __builtin_inff()) return ATTN_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)sink_logits & 3u) != 0) return ATTN_ERR_INVALID_ARGUMENT;
    if (!(softcap >= 0.f) || softcap == __builtin_inff() || ((uintptr_t)alibi_slopes & 3u) != 0)
        return ATTN_ERR_INVALID_ARGUMENT;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (page_size != 16) return ATTN_ERR_UNSUPPORTED;
    if ((long long)max_pages_per_seq * page_size < max_seq_len) return ATTN_ERR_INVALID_ARGUMENT;
    if (max_seq_len > kMaxSeq) return ATTN_ERR_UNSUPPORTED;
    if ((long long)num_seqs * Hq == 0) return ATTN_OK;
    if (q == nullptr || o == nullptr || seq_lens == nullptr) return ATTN_ERR_INVALID_ARGUMENT;
    if (max_seq_len > 0 && (k_pages == nullptr || v_pages == nullptr || block_table == nullptr))
        return ATTN_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o))
        return ATTN_ERR_INVALID_ARGUMENT;
    const long long splits = (max_seq_len + xattn::kSplitTokens - 1) / xattn::kSplitTokens;
    if ((long long)num_seqs * Hkv * (splits > 0 ? splits : 1) > kMaxGrid) return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

void decode_launch(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                   const int32_t* seq_lens, void* o, float* lse, int num_seqs, int Hq, int Hkv, int d,
                   int max_pages_per_seq, int max_seq_len, float scale, const float* sink_logits, float softcap,
                   const float* alibi_slopes, void* workspace, hipStream_t stream) {
    xattn::DecodeParams p;
    p.q = (const uint16_t*)q; p.kp = (const uint16_t*)k_pages; p.vp = (const uint16_t*)v_pages;
    p.block_table = block_table; p.seq_lens = seq_lens;
    p.o = (uint16_t*)o; p.lse = lse;
    p.num_seqs = num_seqs; p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
    p.max_pages = max_pages_per_seq; p.max_splits = 0; p.max_len = max_seq_len;
    p.scale_log2 = scale * xattn::kLog2e;
    p.sink_logits = sink_logits;
    p.softcap = softcap;
    p.alibi_slopes = alibi_slopes;
    p.ws_o = nullptr; p.ws_lse = nullptr;
    xattn::launch_decode(p, d, max_seq_len, workspace, stream);
}

}  // namespace

extern "C" int attn_paged_decode(const void* q, const void* k_pages, const void* v_pages,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 void* o, float* lse,
                                 int num_seqs, int Hq, int Hkv, int d, int page_size,
                                 int max_pages_per_seq, int max_seq_len, float scale, const float* sink_logits,
                                 float softcap, const float* alibi_slopes,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const int st = decode_args_ok(q, k_pages, v_pages, block_table, seq_lens, o, num_seqs, Hq, Hkv, d, page_size,
                                  max_pages_per_seq, max_seq_len, scale, sink_logits, softcap, alibi_slopes);
    if (st != ATTN_OK || (long long)num_seqs * Hq == 0) return st;
    const size_t need = xattn::decode_workspace_bytes(num_seqs, Hq, d, max_seq_len);
    if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned16(workspace)) return ATTN_ERR_INVALID_ARGUMENT;
    decode_launch(q, k_pages, v_pages, block_table, seq_lens, o, lse, num_seqs, Hq, Hkv, d, max_pages_per_seq,
                  max_seq_len, scale, sink_logits, softcap, alibi_slopes, workspace, stream);
    return hip_status(hipGetLastError());
}

extern "C" int attn_paged_decode_noalloc(const void* q, const void* k_pages, const void* v_pages,
                                         const int32_t* block_table, const int32_t* seq_lens,
                                         void* o, float* lse,
                                         int num_seqs, int Hq, int Hkv, int d, int page_size,
                                         int max_pages_per_seq, int max_seq_len, float scale,
                                         const float* sink_logits, float softcap, const float* alibi_slopes,
                                         hipStream_t stream) {
    const int st = decode_args_ok(q, k_pages, v_pages, block_table, seq_lens, o, num_seqs, Hq, Hkv, d, page_size,
                                  max_pages_per_seq, max_seq_len, scale, sink_logits, softcap, alibi_slopes);
    if (st != ATTN_OK || (long long)num_seqs * Hq == 0) return st;
    if (xattn::decode_workspace_bytes(num_seqs, Hq, d, max_seq_len) > xattn::kNoAllocScratchBytes)
        return ATTN_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    const hipError_t e = xattn::decode_scratch(&ws);
    if (e != hipSuccess) return hip_status(e);
    decode_launch(q, k_pages, v_pages, block_table, seq_lens, o, lse, num_seqs, Hq, Hkv, d, max_pages_per_seq,
                  max_seq_len, scale, sink_logits, softcap, alibi_slopes, ws, stream);
    return hip_status(hipGetLastError());
}

extern "C" int attn_paged_prefill(const void* q, const void* k_pages, const void* v_pages,
                                  const int32_t* block_table, const int32_t* seq_lens, const int32_t* q_offsets,
                                  void* o, float* lse,
                                  int num_seqs, int Hq, int Hkv, int d, int page_size,
                                  int max_pages_per_seq, int max_seq_len, int max_q_len, float scale,
                                  attn_mask mask, hipStream_t stream) {
    if (num_seqs < 0 || Hq < 0 || Hkv < 0 || d < 0 || max_pages_per_seq < 0 || max_seq_len < 0 || max_q_len < 0)
        return ATTN_ERR_INVALID_ARGUMENT;
    if (Hkv == 0 ? Hq != 0 : (Hq % Hkv) != 0) return ATTN_ERR_INVALID_ARGUMENT;
    if (!(scale == scale) || scale <= 0.f || scale == __builtin_inff()) return ATTN_ERR_INVALID_ARGUMENT;
    if (mask.kind < ATTN_MASK_NONE || mask.kind > ATTN_MASK_DOCUMENT) return ATTN_ERR_INVALID_ARGUMENT;
    if (mask.kind == ATTN_MASK_SLIDING_WINDOW && mask.window < 1) return ATTN_ERR_INVALID_ARGUMENT;
    if (!sinks_ok(mask) || !mods_ok(mask)) return ATTN_ERR_INVALID_ARGUMENT;
    if (mask.kind == ATTN_MASK_DOCUMENT) return ATTN_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (page_size != 16) return ATTN_ERR_UNSUPPORTED;
    if ((long long)max_pages_per_seq * page_size < max_seq_len) return ATTN_ERR_INVALID_ARGUMENT;
    if (max_seq_len > kMaxSeq || max_q_len > kMaxSeq) return ATTN_ERR_UNSUPPORTED;
    if ((long long)num_seqs * Hq * max_q_len == 0) return ATTN_OK;   // no query row
    if (q == nullptr || o == nullptr || seq_lens == nullptr || q_offsets == nullptr)
        return ATTN_ERR_INVALID_ARGUMENT;
    if (max_seq_len > 0 && (k_pages == nullptr || v_pages == nullptr || block_table == nullptr))
        return ATTN_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o))
        return ATTN_ERR_INVALID_ARGUMENT;
    const long long rows_per_block = xattn::prefill_bf16_rows_per_block();
    const long long tiles = (max_q_len + rows_per_block - 1) / rows_per_block;
    if ((long long)num_seqs * Hq * tiles > kMaxGrid) return ATTN_ERR_UNSUPPORTED;

    xattn::PagedPrefillParams p;
    p.q = (const uint16_t*)q; p.k_pages = (const uint16_t*)k_pages; p.v_pages = (const uint16_t*)v_pages;
    p.block_table = block_table; p.seq_lens = seq_lens; p.q_offsets = q_offsets;
    p.o = (uint16_t*)o; p.lse = lse;
    p.num_seqs = num_seqs; p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
    p.max_pages = max_pages_per_seq;
    p.max_len = max_seq_len;
    p.num_q_tiles = (int)tiles;
    p.scale_log2 = scale * xattn::kLog2e;
    p.mask_kind = mask.kind;
    p.window = mask.kind == ATTN_MASK_SLIDING_WINDOW ? mask.window : 0;
    p.sink_end = mask.kind == ATTN_MASK_SLIDING_WINDOW ? mask.sink_tokens : 0;
    p.sink_logits = mask.sink_logits;
    p.softcap = mask.softcap;
    p.alibi_slopes = mask.alibi_slopes;
    xattn::launch_paged_prefill_bf16(p, d, stream);
    return hip_status(hipGetLastError());
}

extern "C" size_t attn_bwd_workspace_size(int B, int Hq, int Nq) {
    if (B < 0 || Hq < 0 || Nq < 0) return 0;
    return xattn::backward_workspace_bytes(B, Hq, Nq);
}

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, float* dsink,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, attn_mask mask, int dtype,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0 || d < 0) return ATTN_ERR_INVALID_ARGUMENT;
    if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_INVALID_ARGUMENT;
    if (mask.kind < ATTN_MASK_NONE || mask.kind > ATTN_MASK_DOCUMENT) return ATTN_ERR_INVALID_ARGUMENT;
    if (mask.kind == ATTN_MASK_SLIDING_WINDOW && mask.window < 1) return ATTN_ERR_INVALID_ARGUMENT;
    if (mask.kind == ATTN_MASK_DOCUMENT && (mask.num_docs < 1 || mask.doc_offsets == nullptr))
        return ATTN_ERR_INVALID_ARGUMENT;
    if (!sinks_ok(mask) || !mods_ok(mask)) return ATTN_ERR_INVALID_ARGUMENT;
    if (!(scale == scale) || scale <= 0.f || scale == __builtin_inff()) return ATTN_ERR_INVALID_ARGUMENT;
    if (Hkv == 0 ? Hq != 0 : (Hq % Hkv) != 0) return ATTN_ERR_INVALID_ARGUMENT;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (Nq > kMaxSeq || Nk > kMaxSeq) return ATTN_ERR_UNSUPPORTED;
    if ((long long)B * Hkv * Nk == 0 && (long long)B * Hq * Nq == 0) return ATTN_OK;
    if (q == nullptr || o == nullptr || dout == nullptr || lse == nullptr || dq == nullptr) {
        if ((long long)B * Hq * Nq > 0) return ATTN_ERR_INVALID_ARGUMENT;
    }
    if ((long long)B * Hkv * Nk > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
        return ATTN_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv) || ((uintptr_t)lse & 3u) != 0 || ((uintptr_t)dsink & 3u) != 0)
        return ATTN_ERR_INVALID_ARGUMENT;
    const size_t need = xattn::backward_workspace_bytes(B, Hq, Nq);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ATTN_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned16(workspace)) return ATTN_ERR_INVALID_ARGUMENT;
    const long long q_tiles = (Nq + 127) / 128, k_tiles = (Nk + 127) / 128;
    if ((long long)B * Hq * q_tiles > kMaxGrid || (long long)B * Hkv * k_tiles > kMaxGrid ||
        (long long)B * Hq * Nq / 16 > kMaxGrid)
        return ATTN_ERR_UNSUPPORTED;
    // the fp32 passes take one wave per row and per key
    if (dtype == ATTN_DTYPE_F32 && ((long long)B * Hq * Nq / 4 > kMaxGrid || (long long)B * Hkv * Nk / 4 > kMaxGrid))
        return ATTN_ERR_UNSUPPORTED;

    xattn::BackwardParams p;
    p.q = (const uint16_t*)q; p.k = (const uint16_t*)k; p.v = (const uint16_t*)v;
    p.o = (const uint16_t*)o; p.dO = (const uint16_t*)dout; p.lse = lse;
    p.dq = (uint16_t*)dq; p.dk = (uint16_t*)dk; p.dv = (uint16_t*)dv;
    p.dsink = mask.sink_logits != nullptr ? dsink : nullptr;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk; p.group = Hq / Hkv;
    p.scale = scale;
    p.scale_log2 = scale * xattn::kLog2e;
    p.mask_kind = mask.kind;
    p.window = mask.kind == ATTN_MASK_SLIDING_WINDOW ? (mask.window < Nk ? mask.window : (Nk > 0 ? Nk : 1)) : 0;
    p.doc_offsets = mask.kind == ATTN_MASK_DOCUMENT ? mask.doc_offsets : nullptr;
    p.num_docs = mask.kind == ATTN_MASK_DOCUMENT ? mask.num_docs : 0;
    p.sink_end = mask.kind == ATTN_MASK_SLIDING_WINDOW ? mask.sink_tokens : 0;
    p.sink_logits = mask.sink_logits;
    p.softcap = mask.softcap;
    p.alibi_slopes = mask.alibi_slopes;
    p.num_q_tiles = (int)q_tiles;
    p.num_k_tiles = (int)k_tiles;
    // with no query rows the dK/dV pass still runs and writes zeros
    if (dtype == ATTN_DTYPE_BF16) xattn::launch_backward(p, d, workspace, stream);
    else xattn::launch_backward_f32(p, d, workspace, stream);
    return hip_status(hipGetLastError());
}
