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
    int max_len;     // max_seq_len: every seq_lens entry is clamped to [0, max_len] before use, so the
                     // splits and the combine stay inside the table row and the workspace
    float scale_log2;
    const float* sink_logits;   // [Hq] learned sink logit per query head, or null
    float softcap;              // > 0: score -> softcap * tanh(score / softcap)
    const float* alibi_slopes;  // [Hq] or null: score += slope * (key - (seq_len - 1))
};

// A sequence length as the kernels use it: the caller promises
// 0 <= seq_lens[s] <= max_seq_len; the clamp keeps a broken promise inside
// the block-table row and the workspace (the result is then defined by the
// clamped length, not an out-of-bounds read).
__device__ __forceinline__ int clamped_len(const DecodeParams& p, int s) {
    const int len = p.seq_lens[s];
    return len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
}

// Size of the device scratch array behind the allocation-free decode entry
// point (the decode workspace of one call must fit in it).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;

size_t decode_workspace_bytes(int num_seqs, int Hq, int d, int max_seq_len);
// This device's address of the scratch array (looked up once per device,
// with that device current).
hipError_t decode_scratch(void** ptr);
int launch_decode(DecodeParams p, int d, int max_seq_len, void* ws, hipStream_t stream);

}  // namespace xattn
