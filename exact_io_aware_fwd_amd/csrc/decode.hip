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
// decode_split: one workgroup (4 waves) per (sequence, KV head, split of
// kSplitTokens keys).  Workgroup ids run over the KV heads fastest, so the 8
// heads' 4 KiB chunks of a page, which sit side by side in memory, are fetched
// at about the same time.  Wave w takes pages w, w+4, ... of the split and
// streams them HBM -> LDS through its own ring of kRing page slots
// (buffer_load ... lds, no registers held per page), so each wave keeps 16 KiB
// in flight with only wave-local waits.  The query heads that share the KV
// head (GQA) are handled four at a time, so each K/V byte serves four rows.
//   1. scores: Q'K^T on the matrix cores (v_mfma_f32_16x16x32_bf16), with the
//      four query heads replicated over the 16 MFMA rows so every lane ends up
//      holding all four heads' scores for its token; scaled to base 2 and
//      parked in the wave's LDS rows (slots past the sequence end are -inf);
//   2. the wave's exact max and sum over its own tokens (no online rescaling);
//      the V copies are already in flight;
//   3. P.V on the vector ALUs, 8 head-dim columns x 4 heads per lane;
//   4. the four waves' partials are merged by log-sum-exp and the split's
//      normalised output and base-2 log-sum-exp go to the workspace.
// decode_combine: per (sequence, query head), merge the splits' partials.
#include "common.hpp"
#include "decode_params.hpp"

#include <type_traits>

namespace xattn {

typedef __attribute__((address_space(3))) void lds_void;

// Calls f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N-1>{}).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

constexpr int kRing = 4;   // pages each wave keeps in flight (its own LDS ring)

// One page (16 tokens x d of one KV head) copied HBM -> LDS into a ring slot
// with buffer_load_dwordx4 ... lds, 1 KiB per instruction.  The buffer covers
// only the page's valid tokens, so slots past the sequence end read as zero
// (whatever they hold in memory, NaN included).  voff[j] is this lane's source
// offset for instruction j; it decides where each 16-byte chunk lands.
template <int D>
__device__ __forceinline__ void load_page(const uint16_t* page, int valid_tokens, uint8_t* slot,
                                          const uint32_t (&voff)[D / 32]) {
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)page, (short)0, valid_tokens * D * 2,
                                                                  0x00020000);
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(slot + j * 1024), 16, voff[j], 0, 0, 0);
}

// Wait until at most N of this wave's direct copies are still in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

template <int D>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeParams p) {
    constexpr int T = kSplitTokens;
    constexpr int NM = D / 32;              // MFMA steps over the head dim = 1 KiB copies per page
    constexpr int CL = D / 8;               // lanes covering one token row with 16-byte reads
    constexpr int TPI = 64 / CL;            // tokens per wave-wide read
    constexpr int IT = kPage / TPI;         // reads per lane per V page
    constexpr int PAGE_BYTES = kPage * D * 2;
    constexpr int WP = T / kPage / 4;       // pages per wave in a full split
    // ring slot k of wave w is slot<k>[w]: one array per slot index, so each
    // read names the slot whose copy it waits for
    __shared__ __attribute__((aligned(1024))) uint8_t slot0[4][PAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t slot1[4][PAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t slot2[4][PAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t slot3[4][PAGE_BYTES];
    static_assert(kRing == 4, "one array per ring slot");
    __shared__ __attribute__((aligned(16))) float sc[4][T / 4][4];      // per wave: its tokens x 4 heads
    __shared__ float red_m[4][4], red_l[4][4];
    // each wave's partial output [4 heads][D] reuses its own slot 0 once its
    // last page has been read
    auto red_o = [&](int w) { return (float(*)[D])slot0[w]; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hkv = blockIdx.x % p.Hkv;
    const int rest = blockIdx.x / p.Hkv;
    const int split = rest % p.max_splits;
    const int s = rest / p.max_splits;
    const int len = p.seq_lens[s];
    const int tok0 = split * T;
    if (tok0 >= len) return;
    const int ntok = min(T, len - tok0);
    const int npages = (ntok + kPage - 1) / kPage;
    const int page0 = tok0 / kPage;
    // physical page of logical page page0 + i sits in lane i (i < npages <= 32)
    const int bt_lane = lane < npages ? p.block_table[(size_t)s * p.max_pages + page0 + lane] : 0;
    const size_t head_stride = (size_t)kPage * D;             // elements per (page, kv head)
    // this wave takes pages wave, wave + 4, ...
    const int my_pages = npages > wave ? (npages - wave + 3) / 4 : 0;
    float (*scw)[4] = sc[wave];
    // slot k of this wave's ring, resolved at compile time for constant k
#define XATTN_SLOT(k) ((k) % kRing == 0 ? slot0[wave] : (k) % kRing == 1 ? slot1[wave] : (k) % kRing == 2 ? slot2[wave] : slot3[wave])

    // Copy offsets.  K pages are XOR-swizzled by token row (16-byte chunk c of
    // row r sits at chunk c ^ r), so the MFMA operand reads of 16 rows at one
    // chunk hit 16 different banks; V pages stay row-major (their reads take
    // whole rows).
    uint32_t koff[NM], voff[NM];
#pragma unroll
    for (int j = 0; j < NM; ++j) {
        const int r = j * (1024 / (D * 2)) + lane / CL;
        const int pc = lane % CL;
        koff[j] = (uint32_t)(r * D * 2 + ((pc ^ (r % CL)) << 4));
        voff[j] = (uint32_t)(r * D * 2 + (pc << 4));
    }
    // MFMA operand reads of a K page: row (lane & 15), logical chunk m * 4 + (lane >> 4)
    int kread[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int r = lane & 15, c = m * 4 + (lane >> 4);
        kread[m] = r * D * 2 + ((c ^ (r % CL)) << 4);
    }

    auto page_ptr = [&](const uint16_t* base, int i) {
        const int phys = __builtin_amdgcn_readlane(bt_lane, wave + 4 * i);
        return base + ((size_t)phys * p.Hkv + hkv) * head_stride;
    };
    auto page_valid = [&](int i) { return min(kPage, ntok - (wave + 4 * i) * kPage); };

    for (int hc = 0; hc < p.group; hc += 4) {
        // ---- 1. scores: Q' K^T, four heads replicated over the 16 MFMA rows
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
        __builtin_amdgcn_s_waitcnt(0x0F70);   // q landed before the ring copies start counting
#pragma unroll
        for (int i = 0; i < kRing; ++i)
            if (i < my_pages) load_page<D>(page_ptr(p.kp, i), page_valid(i), XATTN_SLOT(i), koff);
        float mloc[4] = {neg_inf(), neg_inf(), neg_inf(), neg_inf()};
        // One K page: wait for its copy, scores on the matrix cores, refill
        // the slot with the page kRing ahead, park the scores.  FULL (all WP
        // pages present) lets every wait count be a constant.
        auto k_page = [&](auto full_tag, auto i_tag) {
            constexpr bool FULL = decltype(full_tag)::value;
            constexpr int i = decltype(i_tag)::value;
            if (FULL) wait_vm<(WP - 1 - i < kRing - 1 ? WP - 1 - i : kRing - 1) * NM>();
            else wait_vm<0>();
            f32x4 acc = f32x4{};
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const u32x4 w = *(const u32x4*)(XATTN_SLOT(i) + kread[m]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[m], __builtin_bit_cast(bf16x8, w), acc, 0, 0, 0);
            }
            if (i + kRing < my_pages) {
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this slot's reads retired
                load_page<D>(page_ptr(p.kp, i + kRing), page_valid(i + kRing), XATTN_SLOT(i), koff);
            }
            const int t_in = (wave + 4 * i) * kPage + (lane & 15);
            if (lane < 16) {
                f32x4 v;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = t_in < ntok ? acc[r] * p.scale_log2 : neg_inf();
                *(f32x4*)(&scw[i * kPage + lane][0]) = v;
#pragma unroll
                for (int r = 0; r < 4; ++r) mloc[r] = fmaxf(mloc[r], v[r]);
            }
        };
        if (my_pages == WP) {
            static_for<WP>([&](auto i_tag) { k_page(std::true_type{}, i_tag); });
        } else {
            static_for<WP>([&](auto i_tag) {
                if (decltype(i_tag)::value < my_pages) k_page(std::false_type{}, i_tag);
            });
        }
        // V copies start now and land during the softmax
#pragma unroll
        for (int i = 0; i < kRing; ++i)
            if (i < my_pages) load_page<D>(page_ptr(p.vp, i), page_valid(i), XATTN_SLOT(i), voff);
        // ---- 2. this wave's own max and sum over its tokens
        float sm[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) mloc[r] = wave_max(mloc[r]);
        {
            f32x4 part = f32x4{};
            for (int t = lane; t < my_pages * kPage; t += 64) {
                f32x4 v = *(const f32x4*)(&scw[t][0]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v[r] = fast_exp2(v[r] - (mloc[r] == neg_inf() ? 0.f : mloc[r]));
                    part[r] += v[r];
                }
                *(f32x4*)(&scw[t][0]) = v;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sm[r] = wave_sum(part[r]);
        }
        // ---- 3. P V: lane covers columns 8*(lane % CL) .. +8 of token (lane / CL) of each read
        float oacc[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) oacc[r][e] = 0.f;
        auto v_page = [&](auto full_tag, auto i_tag) {
            constexpr bool FULL = decltype(full_tag)::value;
            constexpr int i = decltype(i_tag)::value;
            if (FULL) wait_vm<(WP - 1 - i < kRing - 1 ? WP - 1 - i : kRing - 1) * NM>();
            else wait_vm<0>();
            u32x4 vv[IT];
#pragma unroll
            for (int it = 0; it < IT; ++it)
                vv[it] = *(const u32x4*)(XATTN_SLOT(i) + (it * TPI + lane / CL) * D * 2 + (lane % CL) * 16);
            if (i + kRing < my_pages) {
                __builtin_amdgcn_s_waitcnt(0xC07F);
                load_page<D>(page_ptr(p.vp, i + kRing), page_valid(i + kRing), XATTN_SLOT(i), voff);
            }
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                // weights of slots past the end are 0 (their scores were -inf) and their values 0
                const f32x4 pr = *(const f32x4*)(&scw[i * kPage + it * TPI + lane / CL][0]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float v0 = bf16_lo(vv[it][j]), v1 = bf16_hi(vv[it][j]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        oacc[r][2 * j] = __builtin_fmaf(pr[r], v0, oacc[r][2 * j]);
                        oacc[r][2 * j + 1] = __builtin_fmaf(pr[r], v1, oacc[r][2 * j + 1]);
                    }
                }
            }
        };
        if (my_pages == WP) {
            static_for<WP>([&](auto i_tag) { v_page(std::true_type{}, i_tag); });
        } else {
            static_for<WP>([&](auto i_tag) {
                if (decltype(i_tag)::value < my_pages) v_page(std::false_type{}, i_tag);
            });
        }
        // reduce over the lanes that hold other tokens of the same columns
#pragma unroll
        for (int off = CL; off < 64; off <<= 1)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) oacc[r][e] += __shfl_xor(oacc[r][e], off);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's ring reads retired
        if (lane < CL) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                *(f32x4*)(&red_o(wave)[r][lane * 8]) = f32x4{oacc[r][0], oacc[r][1], oacc[r][2], oacc[r][3]};
                *(f32x4*)(&red_o(wave)[r][lane * 8 + 4]) = f32x4{oacc[r][4], oacc[r][5], oacc[r][6], oacc[r][7]};
            }
        }
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                red_m[wave][r] = mloc[r];
                red_l[wave][r] = sm[r];
            }
        }
        __syncthreads();
        // ---- 4. merge the four waves' partials (log-sum-exp) and store the split's result
        for (int idx = tid; idx < 4 * D; idx += 256) {
            const int r = idx / D, c = idx % D;
            const int hl = hc + r;
            if (hl < p.group) {
                float M = neg_inf();
#pragma unroll
                for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w][r]);
                float num = 0.f, den = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float sc_w = red_m[w][r] == neg_inf() ? 0.f : fast_exp2(red_m[w][r] - M);
                    num = __builtin_fmaf(sc_w, red_o(w)[r][c], num);
                    den = __builtin_fmaf(sc_w, red_l[w][r], den);
                }
                const size_t row = ((size_t)s * p.Hq + hkv * p.group + hl) * p.max_splits + split;
                p.ws_o[row * D + c] = num / den;
                if (c == 0) p.ws_lse[row] = M + fast_log2(den);
            }
        }
        __syncthreads();  // sc / red / ring reused by the next head chunk
    }
#undef XATTN_SLOT
}

// One wave per (sequence, query head): O = sum_s w_s o_s / sum_s w_s with
// w_s = 2^(lse_s - max lse); LSE = ln2 * (max + log2 sum w).  Lane i reads
// split i's LSE (up to 64 splits per pass), and the per-split partial rows are
// read 8 at a time so their loads overlap.
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
    // a learned per-head sink joins the merge as one more split with a zero
    // partial output (base-2 logit s2; -inf when there is none)
    const float s2 = p.sink_logits != nullptr ? p.sink_logits[pair % p.Hq] * kLog2e : neg_inf();
    if (ns <= 0) {
        for (int c = lane; c < D; c += 64) orow[c] = 0;
        if (p.lse != nullptr && lane == 0) p.lse[pair] = p.sink_logits != nullptr ? p.sink_logits[pair % p.Hq] : neg_inf();
        return;
    }
    const float* wl = p.ws_lse + (size_t)pair * p.max_splits;
    const float* wo = p.ws_o + (size_t)pair * p.max_splits * D;
    float mx = neg_inf();
    for (int i = lane; i < ns; i += 64) mx = fmaxf(mx, wl[i]);
    mx = fmaxf(wave_max(mx), s2);
    float acc[CPL] = {};
    float den = 0.f;
    for (int i0 = 0; i0 < ns; i0 += 64) {
        const int cnt = min(64, ns - i0);
        const float w_lane = lane < cnt ? fast_exp2(wl[i0 + lane] - mx) : 0.f;
        den += wave_sum(w_lane);
        int i = 0;
        for (; i + 8 <= cnt; i += 8) {
            float v[8][CPL];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int e = 0; e < CPL; ++e) v[u][e] = wo[(size_t)(i0 + i + u) * D + lane * CPL + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_lane), i + u));
#pragma unroll
                for (int e = 0; e < CPL; ++e) acc[e] = __builtin_fmaf(w, v[u][e], acc[e]);
            }
        }
        for (; i < cnt; ++i) {
            const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_lane), i));
#pragma unroll
            for (int e = 0; e < CPL; ++e) acc[e] = __builtin_fmaf(w, wo[(size_t)(i0 + i) * D + lane * CPL + e], acc[e]);
        }
    }
    den += fast_exp2(s2 - mx);
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
