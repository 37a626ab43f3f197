// Paged split-K decode for gfx950 (bf16 KV cache, one query token per sequence).
//
// Decode reads the whole KV cache for a single query row, so it is bound by
// HBM bandwidth ("Attention Is the Bottleneck", Prefill and decode are
// different problems).  To give every CU work even with few sequences, each
// (sequence, KV head) is cut into splits of kSplitTokens keys that are
// attended independently and merged afterwards with a log-sum-exp combine
// (Flash-Decoding section).  K/V are read through the block table, one
// 16-token page at a time (paged-attention kernels, "Attention and matrix
// kernels" page; Paging and prefix sharing).
//
// decode_split: one workgroup per (sequence, KV head, split).  The query
// heads that share the KV head (GQA) are handled four at a time, so each K/V
// byte loaded serves four query rows.
//   1. scores: Q'K^T on the matrix cores (v_mfma_f32_16x16x32_bf16), with the
//      four query heads replicated over the 16 MFMA rows so every lane ends up
//      holding all four heads' scores for its token; scaled to base 2 and
//      parked in LDS (masked slots past the sequence end are -inf);
//   2. exact max and sum of the split's scores per head (no online rescaling:
//      the whole split's scores fit in LDS);
//   3. P·V on the vector ALUs, 8 head-dim columns x 4 heads per lane, then a
//      reduction over lanes and waves; the normalised partial output and its
//      base-2 log-sum-exp go to the workspace.
// decode_combine: per (sequence, query head), merge the splits' partials.
#include "common.hpp"
#include "decode_params.hpp"

namespace xattn {

template <int D>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
    constexpr int T = kSplitTokens;
    constexpr int NM = D / 32;              // MFMA steps over the head dim
    constexpr int CL = D / 8;               // lanes covering one token row with 16-byte loads
    constexpr int TPI = 64 / CL;            // tokens per wave-wide load
    __shared__ __attribute__((aligned(16))) float sc[T][4];  // scores, then probabilities
    __shared__ float stat_m[4], stat_l[4];
    __shared__ __attribute__((aligned(16))) float red[4][4][D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = blockIdx.x % p.max_splits;
    const int rest = blockIdx.x / p.max_splits;
    const int hkv = rest % p.Hkv;
    const int s = rest / p.Hkv;
    const int len = p.seq_lens[s];
    const int tok0 = split * T;
    if (tok0 >= len) return;
    const int ntok = min(T, len - tok0);
    const int npages = (ntok + kPage - 1) / kPage;
    const int page0 = tok0 / kPage;
    const int32_t* bt = p.block_table + (size_t)s * p.max_pages + page0;

    for (int hc = 0; hc < p.group; hc += 4) {
        // ---- 1. scores
        bf16x8 qa[NM];
        {
            const int hl = hc + (lane & 3);            // MFMA row (lane & 15) -> head hc + row % 4
            const bool hv = hl < p.group;
            const uint16_t* qrow = p.q + ((size_t)s * p.Hq + hkv * p.group + (hv ? hl : 0)) * D;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                u32x4 w = hv ? *(const u32x4*)(qrow + m * 32 + (lane >> 4) * 8) : u32x4{0, 0, 0, 0};
                qa[m] = __builtin_bit_cast(bf16x8, w);
            }
        }
        for (int pg = wave; pg < npages; pg += 4) {
            const int phys = bt[pg];
            const uint16_t* kpage = p.kp + ((size_t)phys * p.Hkv + hkv) * (size_t)(kPage * D);
            const int t_in = pg * kPage + (lane & 15);
            const bool tv = t_in < ntok;
            f32x4 acc = f32x4{};
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                u32x4 w = tv ? *(const u32x4*)(kpage + (lane & 15) * D + m * 32 + (lane >> 4) * 8) : u32x4{0, 0, 0, 0};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[m], __builtin_bit_cast(bf16x8, w), acc, 0, 0, 0);
            }
            if (lane < 16) {
                f32x4 v;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = tv ? acc[r] * p.scale_log2 : neg_inf();
                *(f32x4*)(&sc[t_in][0]) = v;
            }
        }
        __syncthreads();
        // ---- 2. per-head max and sum over the split (wave w takes head w)
        {
            const int r = wave;
            float mx = neg_inf();
            for (int t = lane; t < ntok; t += 64) mx = fmaxf(mx, sc[t][r]);
            mx = wave_max(mx);
            float sum = 0.f;
            for (int t = lane; t < ntok; t += 64) {
                const float e = fast_exp2(sc[t][r] - mx);
                sc[t][r] = e;
                sum += e;
            }
            sum = wave_sum(sum);
            if (lane == 0) { stat_m[r] = mx; stat_l[r] = sum; }
        }
        __syncthreads();
        // ---- 3. P V: lane covers columns 8*(lane % CL) .. +8 of token (lane / CL) of each load
        float oacc[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) oacc[r][e] = 0.f;
        for (int pg = wave; pg < npages; pg += 4) {
            const int phys = bt[pg];
            const uint16_t* vpage = p.vp + ((size_t)phys * p.Hkv + hkv) * (size_t)(kPage * D);
#pragma unroll
            for (int it = 0; it < kPage / TPI; ++it) {
                const int tp = it * TPI + lane / CL;
                const int t_in = pg * kPage + tp;
                if (t_in < ntok) {
                    const u32x4 w = *(const u32x4*)(vpage + tp * D + (lane % CL) * 8);
                    const f32x4 pr = *(const f32x4*)(&sc[t_in][0]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float v0 = bf16_lo(w[j]), v1 = bf16_hi(w[j]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            oacc[r][2 * j] = __builtin_fmaf(pr[r], v0, oacc[r][2 * j]);
                            oacc[r][2 * j + 1] = __builtin_fmaf(pr[r], v1, oacc[r][2 * j + 1]);
                        }
                    }
                }
            }
        }
        // reduce over the lanes that hold other tokens of the same columns
#pragma unroll
        for (int off = CL; off < 64; off <<= 1)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) oacc[r][e] += __shfl_xor(oacc[r][e], off);
        if (lane < CL) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                *(f32x4*)(&red[wave][r][lane * 8]) = f32x4{oacc[r][0], oacc[r][1], oacc[r][2], oacc[r][3]};
                *(f32x4*)(&red[wave][r][lane * 8 + 4]) = f32x4{oacc[r][4], oacc[r][5], oacc[r][6], oacc[r][7]};
            }
        }
        __syncthreads();
        for (int idx = tid; idx < 4 * D; idx += 256) {
            const int r = idx / D, c = idx % D;
            const int hl = hc + r;
            if (hl < p.group) {
                const float l = stat_l[r];
                const float v = (red[0][r][c] + red[1][r][c] + red[2][r][c] + red[3][r][c]) / l;
                const size_t row = ((size_t)s * p.Hq + hkv * p.group + hl) * p.max_splits + split;
                p.ws_o[row * D + c] = v;
                if (c == 0) p.ws_lse[row] = stat_m[r] + fast_log2(l);
            }
        }
        __syncthreads();  // sc / red reused by the next head chunk
    }
}

// One wave per (sequence, query head): O = sum_s w_s o_s / sum_s w_s with
// w_s = 2^(lse_s - max lse); LSE = ln2 * (max + log2 sum w).
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
    constexpr int CPL = D / 64;  // columns per lane
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pair = blockIdx.x * 4 + wave;
    if (pair >= p.num_seqs * p.Hq) return;
    const int s = pair / p.Hq;
    const int len = p.seq_lens[s];
    const int ns = (len + kSplitTokens - 1) / kSplitTokens;
    uint16_t* orow = p.o + (size_t)pair * D;
    if (ns <= 0) {
        for (int c = lane; c < D; c += 64) orow[c] = 0;
        if (p.lse != nullptr && lane == 0) p.lse[pair] = neg_inf();
        return;
    }
    const float* wl = p.ws_lse + (size_t)pair * p.max_splits;
    const float* wo = p.ws_o + (size_t)pair * p.max_splits * D;
    float mx = neg_inf();
    for (int i = lane; i < ns; i += 64) mx = fmaxf(mx, wl[i]);
    mx = wave_max(mx);
    float acc[CPL] = {};
    float den = 0.f;
    for (int i = 0; i < ns; ++i) {
        const float w = fast_exp2(wl[i] - mx);
        den += w;
#pragma unroll
        for (int e = 0; e < CPL; ++e) acc[e] = __builtin_fmaf(w, wo[(size_t)i * D + lane * CPL + e], acc[e]);
    }
    const float inv = 1.f / den;
    if (CPL == 2) {
        *(uint32_t*)(orow + lane * 2) = pack_bf16x2(acc[0] * inv, acc[CPL - 1] * inv);
    } else {
        const uint32_t w = pack_bf16x2(acc[0] * inv, 0.f);
        orow[lane] = (uint16_t)(w & 0xffffu);
    }
    if (p.lse != nullptr && lane == 0) p.lse[pair] = (mx + fast_log2(den)) * kLn2;
}

size_t decode_workspace_bytes(int num_seqs, int Hq, int d, int max_seq_len) {
    const size_t max_splits = (size_t)((max_seq_len + kSplitTokens - 1) / kSplitTokens);
    const size_t rows = (size_t)num_seqs * Hq * (max_splits > 0 ? max_splits : 1);
    const size_t o_bytes = rows * d * sizeof(float);
    const size_t l_bytes = rows * sizeof(float);
    return ((o_bytes + 255) / 256) * 256 + l_bytes;
}

int launch_decode(DecodeParams p, int d, int max_seq_len, void* ws, hipStream_t stream) {
    const int max_splits = (max_seq_len + kSplitTokens - 1) / kSplitTokens;
    p.max_splits = max_splits > 0 ? max_splits : 1;
    const size_t rows = (size_t)p.num_seqs * p.Hq * p.max_splits;
    p.ws_o = (float*)ws;
    p.ws_lse = (float*)((char*)ws + ((rows * d * sizeof(float) + 255) / 256) * 256);
    if (max_splits > 0) {
        const int blocks = p.num_seqs * p.Hkv * p.max_splits;
        if (d == 128)
            hipLaunchKernelGGL(decode_split_kernel<128>, dim3(blocks), dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL(decode_split_kernel<64>, dim3(blocks), dim3(256), 0, stream, p);
    }
    const int cblocks = (p.num_seqs * p.Hq + 3) / 4;
    if (d == 128)
        hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(cblocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(cblocks), dim3(256), 0, stream, p);
    return 0;
}

}  // namespace xattn
