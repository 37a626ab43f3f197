// fp32 attention backward: the same recomputation from the saved LSE as the
// bf16 backward ("Attention Is the Bottleneck", FlashAttention-2 section),
// written for full-precision checks rather than throughput.  One wave per
// query row (dQ) or per key (dK, dV); the lanes split the head dim (D / 64
// values each) and every dot product is a wave reduction.
//
//   P = exp(S - LSE),  D = rowsum(dO o O),  dS = P o (dO V^T - D) o S'
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO
// with S the (modified) score and S' = dS/dx the soft cap's chain-rule factor
// 1 - tanh^2(x / c) (1 without a cap).
#include "backward_params.hpp"
#include "common.hpp"

namespace xattn {

namespace {

__device__ __forceinline__ PrefillParams f32_mask_params(const BackwardParams& p) {
    PrefillParams m;
    m.Nq = p.Nq;
    m.Nk = p.Nk;
    m.mask_kind = p.mask_kind;
    m.window = p.window;
    m.doc_offsets = p.doc_offsets;
    m.num_docs = p.num_docs;
    m.sink_end = p.sink_end;
    return m;
}

// The modified score of one pair in base-2 units and the chain-rule factor.
// x = scale q.k; dist = key - query position.
__device__ __forceinline__ float f32_logit(const BackwardParams& p, float x, float slope, int dist, float& fac) {
    fac = 1.f;
    if (p.softcap > 0.f) {
        const float th = tanhf(x / p.softcap);
        x = p.softcap * th;
        fac = 1.f - th * th;
    }
    return (x + slope * (float)dist) * kLog2e;
}

}  // namespace

// One thread per query row: D = dO . O, -LSE log2 e and the row's key
// interval (the learned sink's gradient is reduced from D afterwards).
template <int D>
__global__ __launch_bounds__(256) void bwd_f32_prep_kernel(BackwardParams p) {
    const long long rows = (long long)p.B * p.Hq * p.Nq;
    const long long rg = (long long)blockIdx.x * 256 + threadIdx.x;
    if (rg >= rows) return;
    const float* o = (const float*)p.o + rg * D;
    const float* g = (const float*)p.dO + rg * D;
    float acc = 0.f;
    for (int c = 0; c < D; ++c) acc = __builtin_fmaf(o[c], g[c], acc);
    const int i = (int)(rg % p.Nq);
    const float L = p.lse[rg];
    p.ws_d[rg] = acc;
    p.ws_nl[rg] = L > -__builtin_inff() ? -L * kLog2e : 0.f;
    int lo, hi;
    row_interval(f32_mask_params(p), i, lo, hi);
    p.ws_lo[rg] = lo;
    p.ws_hi[rg] = hi;
}

// dQ: one wave per query row, over the row's visible keys.
template <int D>
__global__ __launch_bounds__(256) void bwd_f32_dq_kernel(BackwardParams p) {
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const long long rows = (long long)p.B * p.Hq * p.Nq;
    const long long rg = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (rg >= rows) return;   // whole wave
    const int i = (int)(rg % p.Nq);
    const int h = (int)((rg / p.Nq) % p.Hq);
    const int b = (int)(rg / ((long long)p.Nq * p.Hq));
    const int hk = h / p.group;
    const float* kg = (const float*)p.k + ((size_t)b * p.Hkv + hk) * (size_t)p.Nk * D;
    const float* vg = (const float*)p.v + ((size_t)b * p.Hkv + hk) * (size_t)p.Nk * D;
    float q[E], g[E], dq[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        q[e] = ((const float*)p.q)[rg * D + lane + 64 * e];
        g[e] = ((const float*)p.dO)[rg * D + lane + 64 * e];
        dq[e] = 0.f;
    }
    const float nl = p.ws_nl[rg], Dr = p.ws_d[rg];
    const int lo = p.ws_lo[rg], hi = p.ws_hi[rg];
    const float slope = p.alibi_slopes != nullptr ? p.alibi_slopes[h] : 0.f;
    const int qpos = i + p.Nk - p.Nq;
    for (int j = 0; j <= hi; ++j) {
        if (j < lo && j >= p.sink_end) {   // between the sink keys and the row's interval
            j = lo - 1;
            continue;
        }
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            s = __builtin_fmaf(q[e], kg[(size_t)j * D + lane + 64 * e], s);
            dp = __builtin_fmaf(g[e], vg[(size_t)j * D + lane + 64 * e], dp);
        }
        s = wave_sum(s);
        dp = wave_sum(dp);
        float fac;
        const float t = f32_logit(p, s * p.scale, slope, j - qpos, fac);
        const float ds = __builtin_amdgcn_exp2f(t + nl) * (dp - Dr) * fac;
#pragma unroll
        for (int e = 0; e < E; ++e) dq[e] = __builtin_fmaf(ds, kg[(size_t)j * D + lane + 64 * e], dq[e]);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) ((float*)p.dq)[rg * D + lane + 64 * e] = dq[e] * p.scale;
}

// dK and dV: one wave per key, over the rows of every query head of its
// group that see it.
template <int D>
__global__ __launch_bounds__(256) void bwd_f32_dkdv_kernel(BackwardParams p) {
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const long long keys = (long long)p.B * p.Hkv * p.Nk;
    const long long kg_i = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (kg_i >= keys) return;   // whole wave
    const int j = (int)(kg_i % p.Nk);
    const int hk = (int)((kg_i / p.Nk) % p.Hkv);
    const int b = (int)(kg_i / ((long long)p.Nk * p.Hkv));
    float k[E], v[E], dk[E], dv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        k[e] = ((const float*)p.k)[kg_i * D + lane + 64 * e];
        v[e] = ((const float*)p.v)[kg_i * D + lane + 64 * e];
        dk[e] = 0.f;
        dv[e] = 0.f;
    }
    for (int h = hk * p.group; h < (hk + 1) * p.group; ++h) {
        const size_t head_row = ((size_t)b * p.Hq + h) * (size_t)p.Nq;
        const float slope = p.alibi_slopes != nullptr ? p.alibi_slopes[h] : 0.f;
        for (int i = 0; i < p.Nq; ++i) {
            const size_t r = head_row + i;
            if (j > p.ws_hi[r] || (j < p.ws_lo[r] && j >= p.sink_end)) continue;   // row i does not see key j
            const float* qr = (const float*)p.q + r * D;
            const float* gr = (const float*)p.dO + r * D;
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                s = __builtin_fmaf(qr[lane + 64 * e], k[e], s);
                dp = __builtin_fmaf(gr[lane + 64 * e], v[e], dp);
            }
            s = wave_sum(s);
            dp = wave_sum(dp);
            float fac;
            const float t = f32_logit(p, s * p.scale, slope, j - (i + p.Nk - p.Nq), fac);
            const float pr = __builtin_amdgcn_exp2f(t + p.ws_nl[r]);
            const float ds = pr * (dp - p.ws_d[r]) * fac;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                dv[e] = __builtin_fmaf(pr, gr[lane + 64 * e], dv[e]);
                dk[e] = __builtin_fmaf(ds, qr[lane + 64 * e], dk[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        ((float*)p.dk)[kg_i * D + lane + 64 * e] = dk[e] * p.scale;
        ((float*)p.dv)[kg_i * D + lane + 64 * e] = dv[e];
    }
}

int launch_backward_f32(BackwardParams p, int d, void* ws, hipStream_t stream) {
    const size_t rows = (size_t)p.B * p.Hq * p.Nq;
    const size_t keys = (size_t)p.B * p.Hkv * p.Nk;
    const size_t stride = ((rows * 4 + 255) / 256) * 256;
    p.ws_nl = (float*)ws;
    p.ws_d = (float*)((char*)ws + stride);
    p.ws_lo = (int32_t*)((char*)ws + 2 * stride);
    p.ws_hi = (int32_t*)((char*)ws + 3 * stride);
    const dim3 wg(256);
    if (rows > 0) {
        const dim3 gp((unsigned)((rows + 255) / 256)), gq((unsigned)((rows + 3) / 4));
        if (d == 128) {
            hipLaunchKernelGGL(bwd_f32_prep_kernel<128>, gp, wg, 0, stream, p);
            hipLaunchKernelGGL(bwd_f32_dq_kernel<128>, gq, wg, 0, stream, p);
        } else {
            hipLaunchKernelGGL(bwd_f32_prep_kernel<64>, gp, wg, 0, stream, p);
            hipLaunchKernelGGL(bwd_f32_dq_kernel<64>, gq, wg, 0, stream, p);
        }
    }
    launch_dsink(p, stream);   // after prep (it reads D); also with no rows, where it writes 0
    if (keys > 0) {
        const dim3 gk((unsigned)((keys + 3) / 4));
        if (d == 128) hipLaunchKernelGGL(bwd_f32_dkdv_kernel<128>, gk, wg, 0, stream, p);
        else hipLaunchKernelGGL(bwd_f32_dkdv_kernel<64>, gk, wg, 0, stream, p);
    }
    return 0;
}

}  // namespace xattn
