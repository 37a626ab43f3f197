// Launch arguments of the paged split-K decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace xattn {

constexpr int kSplitTokens = 1024;  // keys per split of one (sequence, KV head)
constexpr int kPage = 16;          // tokens per KV page

struct DecodeParams {
    const uint16_t* q;
    const uint16_t* kp;
    const uint16_t* vp;
    const int32_t* block_table;
    const int32_t* seq_lens;
    uint16_t* o;
    float* lse;
    float* ws_o;     // [num_seqs, Hq, max_splits, d]
    float* ws_lse;   // [num_seqs, Hq, max_splits], base-2 log-sum-exp
    int num_seqs, Hq, Hkv, group, max_pages, max_splits;
    float scale_log2;
    const float* sink_logits;   // [Hq] learned sink logit per query head, or null
    float softcap;              // > 0: score -> softcap * tanh(score / softcap)
    const float* alibi_slopes;  // [Hq] or null: score += slope * (key - (seq_len - 1))
};

size_t decode_workspace_bytes(int num_seqs, int Hq, int d, int max_seq_len);
int launch_decode(DecodeParams p, int d, int max_seq_len, void* ws, hipStream_t stream);

}  // namespace xattn
