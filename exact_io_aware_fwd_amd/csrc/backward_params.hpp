// Launch arguments of the attention backward kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace xattn {

struct BackwardParams {
    const uint16_t* q;     // [B, Hq, Nq, d] bf16
    const uint16_t* k;     // [B, Hkv, Nk, d]
    const uint16_t* v;
    const uint16_t* o;     // forward output [B, Hq, Nq, d]
    const uint16_t* dO;    // gradient of the loss w.r.t. o
    const float* lse;      // forward LSE [B, Hq, Nq], natural log
    uint16_t* dq;
    uint16_t* dk;          // [B, Hkv, Nk, d]: summed over each group's query heads
    uint16_t* dv;
    float* dsink;          // [Hq] or null
    // per-row statistics (written by the dQ pass, or by the fp32 path's prep pass), each [B, Hq, Nq]
    float* ws_nl;          // -LSE * log2(e) (0 for a row that sees nothing)
    float* ws_d;           // D = rowsum(dO o O)
    int32_t* ws_lo;        // visible key interval [lo, hi] of the row
    int32_t* ws_hi;
    int B, Hq, Hkv, Nq, Nk, group;
    float scale;
    float scale_log2;      // scale * log2(e)
    int mask_kind, window;
    const int32_t* doc_offsets;
    int num_docs;
    int sink_end;          // window mask: keys [0, sink_end) visible too
    const float* sink_logits;
    float softcap;             // > 0: scores went through softcap * tanh(score / softcap)
    const float* alibi_slopes; // [Hq] or null: score += slope * (key - query position)
    int num_q_tiles;       // 128-row query tiles (dQ pass)
    int num_k_tiles;       // 128-key tiles (dK/dV pass)
    int num_cus;           // compute units of the device (the dQ pass's priority phase)
};

size_t backward_workspace_bytes(int B, int Hq, int Nq);
int launch_backward(BackwardParams p, int d, void* ws, hipStream_t stream);   // d: 64 or 128
int launch_backward_f32(BackwardParams p, int d, void* ws, hipStream_t stream);   // fp32 tensors, same workspace
// dsink[h] from the saved LSE and the workspace's D (no-op without a sink gradient)
void launch_dsink(const BackwardParams& p, hipStream_t stream);

}  // namespace xattn
