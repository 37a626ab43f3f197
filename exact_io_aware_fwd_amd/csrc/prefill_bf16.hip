// bf16 prefill attention forward for gfx950.
//
// One workgroup (4 waves) owns a tile of 128 query rows of one (batch, query
// head); each wave owns 32 of those rows for the whole kernel, so its softmax
// state needs no exchange with the other waves (the per-warp split of Q that
// FlashAttention-2 introduced; "Attention Is the Bottleneck", FlashAttention-2
// section).  K/V tiles of 64 keys stream from HBM through a double-buffered
// LDS ring while the Q tile stays in registers, and the score tile never
// leaves the chip ("FlashAttention: same math, different IO").
//
// Both contractions run on the matrix cores with v_mfma_f32_32x32x16_bf16 and
// fp32 accumulation.  They are evaluated transposed, S^T = K Q^T and
// O^T = V^T P^T, because that MFMA's accumulator layout puts one query row's
// scores in a single lane pair (lane l and lane l ^ 32): the row max needs one
// cross-lane exchange per tile and the per-row rescale factor is a per-lane
// scalar.  The S^T accumulator registers are exactly the P^T operand of the
// second MFMA once converted to bf16, up to a fixed permutation of the keys
// inside each 16-key block, which the V^T tile in LDS is stored with.
//
// Softmax runs in base 2: scores are scaled by scale*log2(e) with one FMA that
// also subtracts the running max, then v_exp_f32.  The division by the row sum
// happens once at the end (delayed normalisation, FlashAttention-2 section).
#include "common.hpp"

namespace xattn {

template <int D>
struct PrefillBf16Cfg {
    static constexpr int BM = 128;          // query rows per workgroup
    static constexpr int BN = 64;           // keys per K/V tile
    static constexpr int KSTR = D + 8;      // bf16 per K row in LDS (16 B pad: rows shift banks)
    static constexpr int VSTR = BN + 8;     // bf16 per V^T row in LDS
    static constexpr int DK = D / 16;       // MFMA steps over the head dim for S
    static constexpr int CB = D / 32;       // 32-wide blocks of the head dim for O
    static constexpr int K_CHUNKS = BN * D / 8 / 256;            // 16-byte K loads per thread
    static constexpr int V_GROUPS = (BN / 4) * (D / 8);          // 4 keys x 8 columns each
    static constexpr int V_PER_THREAD = (V_GROUPS + 255) / 256;
};

// Position of 4-key group `kg` (keys 4kg..4kg+3 of the tile) inside the V^T
// rows: within each 16-key block the two middle groups trade places, matching
// the key order of the P^T operand built from the S^T accumulator.
__device__ __forceinline__ int vt_pos(int kg) {
    const int sub = kg & 3;
    const int psub = (sub == 1) ? 2 : (sub == 2 ? 1 : sub);
    return (kg >> 2) * 16 + psub * 4;
}

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(PrefillParams p) {
    using C = PrefillBf16Cfg<D>;
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][C::BN * C::KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][D * C::VSTR];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nbk = p.B * p.Hkv;
    int bk, qt, g;
    decode_work(blockIdx.x, nbk, p.num_q_tiles, p.group, bk, qt, g);
    const int b = bk / p.Hkv, hkv = bk % p.Hkv, hq = hkv * p.group + g;

    const uint16_t* __restrict__ qg = (const uint16_t*)p.q;
    const uint16_t* __restrict__ kg_ = (const uint16_t*)p.k + ((size_t)b * p.Hkv + hkv) * (size_t)p.Nk * D;
    const uint16_t* __restrict__ vg_ = (const uint16_t*)p.v + ((size_t)b * p.Hkv + hkv) * (size_t)p.Nk * D;

    const int r0 = qt * C::BM;
    const int r_last = min(r0 + C::BM, p.Nq) - 1;
    const int w0 = r0 + wave * 32;                      // first row of this wave
    const int w_last = min(w0 + 31, p.Nq - 1);          // last valid row of this wave
    const int row = w0 + (lane & 31);
    const bool row_ok = row < p.Nq;

    int lo_i, hi_i;
    row_interval(p, row, lo_i, hi_i);
    int lo_wg, tmp, hi_wg;
    row_interval(p, r0, lo_wg, tmp);
    row_interval(p, r_last, tmp, hi_wg);
    int lo_w_first, hi_w_first, lo_w_last, hi_w_last;
    row_interval(p, w0, lo_w_first, hi_w_first);
    row_interval(p, w_last, lo_w_last, hi_w_last);
    const bool wave_has_rows = w0 < p.Nq;

    // Q fragment: MFMA B operand, column = query row (lane & 31), k slots
    // (lane >> 5) * 8 .. +8 of every 16-wide step of the head dim.
    bf16x8 qf[C::DK];
    {
        const uint16_t* qrow = qg + (((size_t)b * p.Hq + hq) * (size_t)p.Nq + (row_ok ? row : 0)) * D;
#pragma unroll
        for (int kk = 0; kk < C::DK; ++kk) {
            u32x4 w = row_ok ? *(const u32x4*)(qrow + kk * 16 + (lane >> 5) * 8) : u32x4{0, 0, 0, 0};
            qf[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }

    f32x16 acc[C::CB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) acc[cb] = f32x16{};
    float m_run = neg_inf();   // running row max, base-2 scaled units
    float l_run = 0.f;         // this lane's half of the running row sum

    const int t_begin = lo_wg / C::BN;
    const int t_end = hi_wg >= lo_wg ? hi_wg / C::BN : t_begin - 1;

    // Register staging for the next K/V tile.
    u32x4 kreg[C::K_CHUNKS];
    u32x4 vreg[C::V_PER_THREAD][4];

    auto load_tile = [&](int t) {
        const int n0 = t * C::BN;
#pragma unroll
        for (int u = 0; u < C::K_CHUNKS; ++u) {
            const int c = u * 256 + tid;
            const int r = c / (D / 8), c8 = c % (D / 8);
            const int key = n0 + r;
            kreg[u] = key < p.Nk ? *(const u32x4*)(kg_ + (size_t)key * D + c8 * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int s = 0; s < C::V_PER_THREAD; ++s) {
            const int gidx = s * 256 + tid;
            const int cc = gidx % (D / 8), kgp = gidx / (D / 8);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int key = n0 + kgp * 4 + u;
                vreg[s][u] = (gidx < C::V_GROUPS && key < p.Nk)
                                 ? *(const u32x4*)(vg_ + (size_t)key * D + cc * 8)
                                 : u32x4{0, 0, 0, 0};
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int u = 0; u < C::K_CHUNKS; ++u) {
            const int c = u * 256 + tid;
            const int r = c / (D / 8), c8 = c % (D / 8);
            *(u32x4*)(&k_lds[buf][r * C::KSTR + c8 * 8]) = kreg[u];
        }
#pragma unroll
        for (int s = 0; s < C::V_PER_THREAD; ++s) {
            const int gidx = s * 256 + tid;
            if (gidx < C::V_GROUPS) {
                const int cc = gidx % (D / 8), kgp = gidx / (D / 8);
                const int pos = vt_pos(kgp);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    // columns 8cc+2w (low halves) and 8cc+2w+1 (high halves)
                    const uint32_t lo01 = __builtin_amdgcn_perm(vreg[s][1][w], vreg[s][0][w], 0x05040100u);
                    const uint32_t lo23 = __builtin_amdgcn_perm(vreg[s][3][w], vreg[s][2][w], 0x05040100u);
                    const uint32_t hi01 = __builtin_amdgcn_perm(vreg[s][1][w], vreg[s][0][w], 0x07060302u);
                    const uint32_t hi23 = __builtin_amdgcn_perm(vreg[s][3][w], vreg[s][2][w], 0x07060302u);
                    *(u32x2*)(&vt_lds[buf][(cc * 8 + 2 * w) * C::VSTR + pos]) = u32x2{lo01, lo23};
                    *(u32x2*)(&vt_lds[buf][(cc * 8 + 2 * w + 1) * C::VSTR + pos]) = u32x2{hi01, hi23};
                }
            }
        }
    };

    if (t_begin <= t_end) {
        load_tile(t_begin);
        store_tile(0);
        __syncthreads();
        for (int t = t_begin; t <= t_end; ++t) {
            const int buf = (t - t_begin) & 1;
            const bool has_next = t < t_end;
            if (has_next) load_tile(t + 1);
            const int n0 = t * C::BN;
            const bool active = wave_has_rows && n0 <= hi_w_last && n0 + C::BN - 1 >= lo_w_first;
            if (active) {
                const uint16_t* kl = k_lds[buf];
                const uint16_t* vl = vt_lds[buf];
                // ---- S^T = K Q^T, two 32-key blocks
                f32x16 s[2];
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    s[jb] = f32x16{};
#pragma unroll
                    for (int kk = 0; kk < C::DK; ++kk) {
                        const u32x4 a = *(const u32x4*)(kl + (jb * 32 + (lane & 31)) * C::KSTR + kk * 16 + (lane >> 5) * 8);
                        s[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[kk], s[jb], 0, 0, 0);
                    }
                }
                // ---- mask, only where the tile is not fully visible to this wave
                const bool full = n0 >= lo_w_last && n0 + C::BN - 1 <= hi_w_first;
                if (!full) {
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = n0 + jb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                            if (key < lo_i || key > hi_i) s[jb][r] = neg_inf();
                        }
                }
                // ---- online softmax
                float mt = neg_inf();
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[jb][r]);
                mt = fmaxf(mt, __shfl_xor(mt, 32));
                const float m_new = fmaxf(m_run, mt * p.scale_log2);
                const float m_use = m_new == neg_inf() ? 0.f : m_new;
                const float alpha = fast_exp2(m_run - m_use);
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[jb][r] = fast_exp2(__builtin_fmaf(s[jb][r], p.scale_log2, -m_use));
                // ---- P^T operands (bf16), one per 16-key block.  The row sum is
                // taken over the same bf16-rounded weights the PV product uses, so
                // the output is an exact weighted average of V rows under those
                // weights (a dot with (1, 1) adds two packed bf16 values at once).
                bf16x8 pf[4];
                float psum = 0.f;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const int jb = kb >> 1, h = (kb & 1) * 8;
                    u32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        w[e] = pack_bf16x2(s[jb][h + 2 * e], s[jb][h + 2 * e + 1]);
                        psum = sum_bf16x2(w[e], psum);
                    }
                    pf[kb] = __builtin_bit_cast(bf16x8, w);
                }
                l_run = l_run * alpha + psum;
                m_run = m_new;
                if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                    for (int cb = 0; cb < C::CB; ++cb) acc[cb] *= alpha;
                }
                // ---- O^T += V^T P^T
#pragma unroll
                for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) {
                        const u32x4 a = *(const u32x4*)(vl + (cb * 32 + (lane & 31)) * C::VSTR + kb * 16 + (lane >> 5) * 8);
                        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pf[kb], acc[cb], 0, 0, 0);
                    }
            }
            if (has_next) store_tile(buf ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogue: O = acc / l once, LSE in natural log
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (row_ok) {
        const bool any = l_tot > 0.f;
        const float inv = any ? 1.f / l_tot : 0.f;
        uint16_t* orow = (uint16_t*)p.o + (((size_t)b * p.Hq + hq) * (size_t)p.Nq + row) * D;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                u32x2 w;
                w[0] = pack_bf16x2(acc[cb][4 * gq + 0] * inv, acc[cb][4 * gq + 1] * inv);
                w[1] = pack_bf16x2(acc[cb][4 * gq + 2] * inv, acc[cb][4 * gq + 3] * inv);
                *(u32x2*)(orow + cb * 32 + 8 * gq + 4 * (lane >> 5)) = w;
            }
        if (p.lse != nullptr && lane < 32) {
            p.lse[((size_t)b * p.Hq + hq) * (size_t)p.Nq + row] =
                any ? (m_run + fast_log2(l_tot)) * kLn2 : neg_inf();
        }
    }
}

int launch_prefill_bf16(const PrefillParams& p, int d, hipStream_t stream) {
    const int blocks = p.B * p.Hq * p.num_q_tiles;
    if (d == 128)
        hipLaunchKernelGGL(prefill_bf16_kernel<128>, dim3(blocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(prefill_bf16_kernel<64>, dim3(blocks), dim3(256), 0, stream, p);
    return 0;
}

}  // namespace xattn
