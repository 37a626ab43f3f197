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
// loads them straight from HBM into registers: a ring of kRing page slots
// (each 1 KiB of a page per load instruction, range-limited buffer loads
// with the nontemporal bit), so each wave keeps kRing pages in flight with
// only wave-local waits.  In a full split the wave's K pages and then its V
// pages form one load stream.  The query heads that share the KV head (GQA)
// are handled four at a time, so each K/V byte serves four rows.
//   1. scores: each K page passes from its ring slot through a small swizzled
//      LDS stage of the wave into the matrix-core operand layout; Q'K^T on
//      the matrix cores (v_mfma_f32_16x16x32_bf16), with the four query heads
//      replicated over the 16 MFMA rows so every lane ends up holding all
//      four heads' scores for its token; scaled to base 2 and parked in the
//      wave's LDS rows (slots past the sequence end are -inf);
//   2. the wave's exact max and sum over its own tokens (no online rescaling);
//      the V copies are already in flight;
//   3. P.V on the vector ALUs from the V pages in the ring, 8 head-dim
//      columns x 4 heads per lane;
//   4. the four waves' partials are merged by log-sum-exp and the split's
//      normalised output and base-2 log-sum-exp go to the workspace.
// decode_combine: per (sequence, query head), merge the splits' partials.
#include "common.hpp"
#include "decode_params.hpp"

#include <mutex>
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

constexpr int kRing = 4;   // pages each wave keeps in flight (registers)

// Cache policy of the page loads: nontemporal (the nt bit).  Every cache byte
// is read once per decode step, and in a 4.5 GiB streaming test nontemporal
// loads of shuffled 4 KiB pages ran at 6.44 TB/s against 5.98 TB/s with the
// default policy.
constexpr int kStreamLoad = 2;

// MODS: the score modifications (soft cap, per-head slope times the key's
// distance from the query at position seq_len - 1) turn each score into its
// base-2 logit before the softmax.
template <int D, bool MODS>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeParams p) {
    constexpr int T = kSplitTokens;
    constexpr int NM = D / 32;              // MFMA steps over the head dim = 16-byte loads per lane per page
    constexpr int CL = D / 8;               // lanes covering one token row with 16-byte reads
    constexpr int TPI = 64 / CL;            // tokens per wave-wide V read
    constexpr int IT = kPage / TPI;         // V reads per lane per page
    static_assert(IT == NM, "a K page and a V page take the same loads per lane");
    constexpr int WP = T / kPage / 4;       // pages per wave in a full split
    static_assert(WP % kRing == 0, "V page i must land in ring slot i % kRing");
    __shared__ __attribute__((aligned(16))) float sc[4][T / 4][4];      // per wave: its tokens x 4 heads
    __shared__ __attribute__((aligned(16))) float red_o[4][4][D];       // per wave: partial output of 4 heads
    __shared__ float red_m[4][4], red_l[4][4];
    __shared__ __attribute__((aligned(16))) uint8_t kst[4][2][kPage * D * 2];  // per wave: two K page stages

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hkv = blockIdx.x % p.Hkv;
    const int rest = blockIdx.x / p.Hkv;
    const int split = rest % p.max_splits;
    const int s = rest / p.max_splits;
    const int tok0 = split * T;
    const int page0 = tok0 / kPage;
    // Physical page of logical page page0 + i sits in lane i (i < npages <=
    // 64).  The entries of a whole split are read together with the sequence
    // length (indices clamped to the table row; entries past the sequence are
    // never used), so the first page loads wait for one memory round trip,
    // not two; the empty asm keeps the load ahead of the early exit.
    static_assert(T / kPage <= 64, "one block-table entry per lane");
    const int bt_lane = p.block_table[(size_t)s * p.max_pages + min(page0 + lane, p.max_pages - 1)];
    const int len = clamped_len(p, s);
    asm volatile("" ::"v"(bt_lane));
    if (tok0 >= len) return;
    const int ntok = min(T, len - tok0);
    const int npages = (ntok + kPage - 1) / kPage;
    const size_t head_stride = (size_t)kPage * D;             // elements per (page, kv head)
    // this wave takes pages wave, wave + 4, ...
    const int n = npages > wave ? (npages - wave + 3) / 4 : 0;
    float (*scw)[4] = sc[wave];

    // Pages go straight from HBM into registers, NM 16-byte loads per lane
    // and page, each load a contiguous 1 KiB of the page (token m*TPI +
    // lane / CL, elements (lane % CL)*8 ..+8): a row-major V page is then
    // ready for the P V products, and a K page goes through the wave's LDS
    // stage into the matrix-core operand layout (operand loads that take a
    // 64-byte piece of 16 rows each stream about 14 % slower from HBM).  Each
    // page's buffer covers only its valid tokens, so slots past the sequence
    // end read as zero whatever they hold (NaN included).
    uint32_t voff[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) voff[m] = (uint32_t)((m * TPI + lane / CL) * D * 2 + (lane % CL) * 16);
    // K stage: 16-byte chunk c of token row r sits at chunk c ^ (r % CL), so
    // the stores of whole rows and the operand reads of 16 rows at one chunk
    // both hit distinct banks
    int kput[NM], kget[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int rw = m * TPI + lane / CL, cw = lane % CL;
        kput[m] = rw * D * 2 + ((cw ^ (rw % CL)) << 4);
        const int rr = lane & 15, cr = m * 4 + (lane >> 4);
        kget[m] = rr * D * 2 + ((cr ^ (rr % CL)) << 4);
    }
    auto load_page = [&](u32x4 (&buf)[NM], const uint16_t* base, int i, const uint32_t (&off)[NM]) {
        const int phys = __builtin_amdgcn_readlane(bt_lane, wave + 4 * i);
        const uint16_t* pg = base + ((size_t)phys * p.Hkv + hkv) * head_stride;
        const int valid = min(kPage, ntok - (wave + 4 * i) * kPage);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)pg, (short)0, valid * D * 2,
                                                                            0x00020000);
#pragma unroll
        for (int m = 0; m < NM; ++m) buf[m] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[m], 0, kStreamLoad);
    };
    // the ring: kRing pages of registers, slot k always named by a constant
    u32x4 ring[kRing][NM];

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
        // In a full split (n = WP) the wave's loads form one stream: its K
        // pages 0 .. WP-1, then its V pages 0 .. WP-1, stream page j in slot
        // j % kRing, each slot reloaded with page j + kRing right after page j
        // is used, so the first V pages are in flight while the last K pages
        // are scored and while the softmax runs.  A shorter (last) split loads
        // its V pages after its K pages.
        const bool full_split = n == WP;
        static_for<kRing>([&](auto k_tag) {
            constexpr int k = decltype(k_tag)::value;
            if (k < n) load_page(ring[k], p.kp, k, voff);
        });
        float mloc[4] = {neg_inf(), neg_inf(), neg_inf(), neg_inf()};
        auto k_page = [&](auto full_tag, auto i_tag) {
            constexpr bool FULL = decltype(full_tag)::value;
            constexpr int i = decltype(i_tag)::value;
            uint8_t* stage = kst[wave][i & 1];
#pragma unroll
            for (int m = 0; m < NM; ++m) *(u32x4*)(stage + kput[m]) = ring[i % kRing][m];
            f32x4 acc = f32x4{};
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const u32x4 w = *(const u32x4*)(stage + kget[m]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[m], __builtin_bit_cast(bf16x8, w), acc, 0, 0, 0);
            }
            if (i + kRing < WP) {
                if (FULL || i + kRing < n) load_page(ring[i % kRing], p.kp, i + kRing, voff);
            } else if (FULL) {
                load_page(ring[i % kRing], p.vp, i + kRing - WP, voff);
            }
            const int t_in = (wave + 4 * i) * kPage + (lane & 15);
            if (lane < 16) {
                f32x4 v;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = t_in < ntok ? (MODS ? acc[r] : acc[r] * p.scale_log2) : neg_inf();
                *(f32x4*)(&scw[i * kPage + lane][0]) = v;
#pragma unroll
                for (int r = 0; r < 4; ++r) mloc[r] = fmaxf(mloc[r], v[r]);
            }
        };
        if (full_split) {
            static_for<WP>([&](auto i_tag) { k_page(std::true_type{}, i_tag); });
        } else {
            static_for<WP>([&](auto i_tag) {
                if (decltype(i_tag)::value < n) k_page(std::false_type{}, i_tag);
            });
            static_for<kRing>([&](auto k_tag) {
                constexpr int k = decltype(k_tag)::value;
                if (k < n) load_page(ring[k], p.vp, k, voff);
            });
        }
        // ---- score modifications: the wave's stored raw scores (register r:
        // head hc + r) become base-2 logits, and its maxima are taken again
        if constexpr (MODS) {
            const ScoreMod smod = make_score_mod(p.scale_log2, p.softcap, nullptr, 0);
            float sl2[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sl2[r] = p.alibi_slopes != nullptr && hc + r < p.group
                             ? p.alibi_slopes[hkv * p.group + hc + r] * kLog2e : 0.f;
                mloc[r] = neg_inf();
            }
            for (int t = lane; t < n * kPage; t += 64) {
                f32x4 v = *(const f32x4*)(&scw[t][0]);
                const int tok = tok0 + (wave + 4 * (t / kPage)) * kPage + t % kPage;
                const float dist = (float)(tok - (len - 1));   // key position minus the query's
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float x;
                    if (smod.cap_k != 0.f) {
                        const float rr = __builtin_amdgcn_rcpf(fast_exp2(v[r] * smod.cap_k) + 1.f);
                        x = __builtin_fmaf(-2.f * smod.cap_l2, rr, smod.cap_l2);
                    } else {
                        x = v[r] * p.scale_log2;
                    }
                    v[r] = v[r] == neg_inf() ? neg_inf() : __builtin_fmaf(sl2[r], dist, x);
                    mloc[r] = fmaxf(mloc[r], v[r]);
                }
                *(f32x4*)(&scw[t][0]) = v;
            }
        }
        // ---- 2. this wave's own max and sum over its tokens
        float sm[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) mloc[r] = wave_max(mloc[r]);
        {
            f32x4 part = f32x4{};
            for (int t = lane; t < n * kPage; t += 64) {
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
        auto v_page = [&](auto i_tag) {
            constexpr int i = decltype(i_tag)::value;
            u32x4 vv[IT];
#pragma unroll
            for (int it = 0; it < IT; ++it) vv[it] = ring[i % kRing][it];
            if (i + kRing < WP && i + kRing < n) load_page(ring[i % kRing], p.vp, i + kRing, voff);
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
        static_for<WP>([&](auto i_tag) {
            if (decltype(i_tag)::value < n) v_page(i_tag);
        });
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
                *(f32x4*)(&red_o[wave][r][lane * 8]) = f32x4{oacc[r][0], oacc[r][1], oacc[r][2], oacc[r][3]};
                *(f32x4*)(&red_o[wave][r][lane * 8 + 4]) = f32x4{oacc[r][4], oacc[r][5], oacc[r][6], oacc[r][7]};
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
                    num = __builtin_fmaf(sc_w, red_o[w][r][c], num);
                    den = __builtin_fmaf(sc_w, red_l[w][r], den);
                }
                const size_t row = ((size_t)s * p.Hq + hkv * p.group + hl) * p.max_splits + split;
                p.ws_o[row * D + c] = num / den;
                if (c == 0) p.ws_lse[row] = M + fast_log2(den);
            }
        }
        __syncthreads();  // sc / red reused by the next head chunk
    }
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
    const int len = clamped_len(p, s);
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

// Scratch of the allocation-free decode entry point: a file-scope device
// array, one copy per GPU, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in):
// it takes each device's address once, with that device current, and uses
// that address from then on.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
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
    p.max_len = max_seq_len;
    const size_t rows = (size_t)p.num_seqs * p.Hq * p.max_splits;
    p.ws_o = (float*)ws;
    p.ws_lse = (float*)((char*)ws + ((rows * d * sizeof(float) + 255) / 256) * 256);
    if (max_splits > 0) {
        const int blocks = p.num_seqs * p.Hkv * p.max_splits;
        const bool mods = p.softcap > 0.f || p.alibi_slopes != nullptr;
        if (d == 128) {
            if (mods) hipLaunchKernelGGL(HIP_KERNEL_NAME(decode_split_kernel<128, true>), dim3(blocks), dim3(256), 0, stream, p);
            else hipLaunchKernelGGL(HIP_KERNEL_NAME(decode_split_kernel<128, false>), dim3(blocks), dim3(256), 0, stream, p);
        } else {
            if (mods) hipLaunchKernelGGL(HIP_KERNEL_NAME(decode_split_kernel<64, true>), dim3(blocks), dim3(256), 0, stream, p);
            else hipLaunchKernelGGL(HIP_KERNEL_NAME(decode_split_kernel<64, false>), dim3(blocks), dim3(256), 0, stream, p);
        }
    }
    const int cblocks = (p.num_seqs * p.Hq + 3) / 4;
    if (d == 128)
        hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(cblocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(cblocks), dim3(256), 0, stream, p);
    return 0;
}

}  // namespace xattn
