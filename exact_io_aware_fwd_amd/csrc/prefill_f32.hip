// fp32 prefill attention forward for gfx950.
//
// Same tiling and online softmax as the bf16 kernel (one wave per 32 query
// rows, transposed products S^T = K Q^T and O^T = V^T P^T so a row's state
// lives in one lane pair), but every operand stays fp32 and the products use
// v_mfma_f32_32x32x2_f32.  With k = 2 per instruction the P^T operand of the
// second product is one accumulator register per lane: register r of S^T holds
// keys 8(r/4) + r%4 (lanes 0-31) and 8(r/4) + 4 + r%4 (lanes 32-63), so the
// matching V values are read from a row-major V tile with one 4-byte LDS read
// per lane.  This path is for full-precision checks rather than throughput:
// single-buffered LDS, 32-key tiles.
#include "common.hpp"

namespace xattn {

template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillParams p) {
    constexpr int BM = 128, BN = 32;
    constexpr int KSTR = D + 1;   // odd stride: 32 consecutive rows hit 32 banks
    constexpr int DK = D / 2;
    constexpr int CB = D / 32;
    __shared__ float k_lds[BN * KSTR];
    __shared__ float v_lds[BN * D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int bk, qt, g;
    decode_work(blockIdx.x, p.B * p.Hkv, p.num_q_tiles, p.group, bk, qt, g);
    const int b = bk / p.Hkv, hkv = bk % p.Hkv, hq = hkv * p.group + g;
    const float* __restrict__ kg_ = (const float*)p.k + ((size_t)b * p.Hkv + hkv) * (size_t)p.Nk * D;
    const float* __restrict__ vg_ = (const float*)p.v + ((size_t)b * p.Hkv + hkv) * (size_t)p.Nk * D;

    const int r0 = qt * BM;
    const int r_last = min(r0 + BM, p.Nq) - 1;
    const int w0 = r0 + wave * 32;
    const int w_last = min(w0 + 31, p.Nq - 1);
    const int row = w0 + (lane & 31);
    const bool row_ok = row < p.Nq;
    int lo_i, hi_i, lo_wg, hi_wg, tmp, lo_w_first, hi_w_first, lo_w_last, hi_w_last;
    row_interval(p, row, lo_i, hi_i);
    row_interval(p, r0, lo_wg, tmp);
    row_interval(p, r_last, tmp, hi_wg);
    row_interval(p, w0, lo_w_first, hi_w_first);
    row_interval(p, w_last, lo_w_last, hi_w_last);
    const bool wave_has_rows = w0 < p.Nq;

    // Q fragment (B operand): column = query row, k slot = lane >> 5.
    float qf[DK];
    {
        const float* qrow = (const float*)p.q + (((size_t)b * p.Hq + hq) * (size_t)p.Nq + (row_ok ? row : 0)) * D;
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) qf[kk] = row_ok ? qrow[kk * 2 + (lane >> 5)] : 0.f;
    }
    f32x16 acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};
    float m_run = neg_inf(), l_run = 0.f;
    const bool mods = p.softcap > 0.f || p.alibi_slopes != nullptr;
    const float slope_l2 = p.alibi_slopes != nullptr ? p.alibi_slopes[hq] * kLog2e : 0.f;
    const int qpos = row + p.Nk - p.Nq;
    const float sl = mods ? 1.f : p.scale_log2;   // scores in base-2 units after the modifications

    const TileRange tr = tile_range(lo_wg, hi_wg, p.sink_end, BN);
    for (int it = 0; it < tr.n; ++it) {
        const int n0 = tile_of(tr, it) * BN;
        __syncthreads();  // previous tile fully consumed
        for (int c = tid; c < BN * D / 4; c += 256) {
            const int r = c / (D / 4), c4 = c % (D / 4);
            const int key = n0 + r;
            f32x4 kv = key < p.Nk ? *(const f32x4*)(kg_ + (size_t)key * D + c4 * 4) : f32x4{};
            f32x4 vv = key < p.Nk ? *(const f32x4*)(vg_ + (size_t)key * D + c4 * 4) : f32x4{};
#pragma unroll
            for (int e = 0; e < 4; ++e) k_lds[r * KSTR + c4 * 4 + e] = kv[e];
            *(f32x4*)(&v_lds[r * D + c4 * 4]) = vv;
        }
        __syncthreads();
        const bool active = wave_has_rows && n0 <= hi_w_last && (n0 + BN - 1 >= lo_w_first || n0 < p.sink_end);
        if (!active) continue;
        f32x16 s = f32x16{};
#pragma unroll
        for (int kk = 0; kk < DK; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(k_lds[(lane & 31) * KSTR + kk * 2 + (lane >> 5)], qf[kk], s, 0, 0, 0);
        const bool full = n0 + BN - 1 <= hi_w_first && (n0 >= lo_w_last || n0 + BN - 1 < p.sink_end);
        // score modifications (uniform branch): x = scale q.k, then the cap
        // c tanh(x / c) and the bias slope (key - query position), into base-2
        // units; the softmax below then runs at unit scale
        if (mods) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = n0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                float x = s[r] * p.scale;
                if (p.softcap > 0.f) x = p.softcap * tanhf(x / p.softcap);
                s[r] = __builtin_fmaf(x, kLog2e, slope_l2 * (float)(key - qpos));
            }
        }
        if (!full) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = n0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (key > hi_i || (key < lo_i && key >= p.sink_end)) s[r] = neg_inf();
            }
        }
        float mt = neg_inf();
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[r]);
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt * sl);
        const float m_use = m_new == neg_inf() ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(__builtin_fmaf(s[r], sl, -m_use));
            s[r] = e;
            psum += e;
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[cb] *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v_lds[key * D + cb * 32 + (lane & 31)], s[r], acc[cb], 0, 0, 0);
            }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (row_ok) {
        const float s2 = p.sink_logits != nullptr ? p.sink_logits[hq] * kLog2e : neg_inf();
        float inv, lse_row;
        finish_row(m_run, l_tot, l_tot, s2, inv, lse_row);
        float* orow = (float*)p.o + (((size_t)b * p.Hq + hq) * (size_t)p.Nq + row) * D;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                f32x4 w = {acc[cb][4 * gq] * inv, acc[cb][4 * gq + 1] * inv, acc[cb][4 * gq + 2] * inv,
                           acc[cb][4 * gq + 3] * inv};
                *(f32x4*)(orow + cb * 32 + 8 * gq + 4 * (lane >> 5)) = w;
            }
        if (p.lse != nullptr && lane < 32)
            p.lse[((size_t)b * p.Hq + hq) * (size_t)p.Nq + row] = lse_row;
    }
}

int launch_prefill_f32(const PrefillParams& p, int d, hipStream_t stream) {
    const int blocks = p.B * p.Hq * p.num_q_tiles;
    if (d == 128)
        hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3(blocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3(blocks), dim3(256), 0, stream, p);
    return 0;
}

}  // namespace xattn
