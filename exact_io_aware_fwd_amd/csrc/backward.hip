// Attention backward (bf16, head dim 64 or 128) by recomputation from the saved
// log-sum-exp, the FlashAttention-2 backward ("Attention Is the Bottleneck",
// FlashAttention-2 section: the forward keeps only O and the per-row
// statistic; the backward recomputes the probabilities tile by tile).
//
//   P = exp(S - LSE),  D = rowsum(dO o O),  dS = P o (dO V^T - D)
//   dV = P^T dO,  dQ = scale dS K,  dK = scale dS^T Q
//
// Three passes, no atomics on the gradients:
//   prep   per query row: -LSE log2(e), D, the row's visible key interval,
//          and the learned sink's gradient -sum_i P_sink,i D_i;
//   dQ     one workgroup per (batch, query head, 128-row query tile), each
//          wave owning 32 rows as in the forward; per 32-key tile it
//          recomputes S^T = K Q^T and dP^T = V dO^T and accumulates
//          dQ^T += K^T dS^T (the forward's O^T += V^T P^T with K and dS);
//   dK/dV  one workgroup per (batch, KV head, 128-key tile), each wave owning
//          32 keys in registers; it streams 64-row query tiles of every query
//          head of the group, recomputes S = Q K^T and dP = dO V^T with the
//          keys as the accumulator columns, and accumulates dV^T += dO^T P
//          and dK^T += Q^T dS.
// Tiles that one product reads by rows and another transposed are copied to
// LDS twice, once in each padded layout, so every read is conflict-free.
#include "backward_params.hpp"
#include "prefill_tiles.hpp"

namespace xattn {

namespace {

// A operand of a 32x32x16 MFMA read by rows from a row-padded tile: row
// (lane & 31) + 32 jb, head-dim chunk 2 kk + (lane >> 5).  rl = this lane's
// base, tile + (lane & 31) * KS * 16 + (lane >> 5) * 16.
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const uint8_t* rl, int jb, int kk) {
    using C = PrefillBf16Cfg<D>;
    return __builtin_bit_cast(bf16x8, *(const u32x4*)(rl + jb * 32 * C::KS * 16 + kk * 32));
}

// A operand of a 32x32x16 MFMA read transposed from a transpose-padded tile
// (two ds_read_b64_tr_b16): column cb*32 + (lane & 31) of tile rows
// kb*16 + 8 (t / 4) + 4 (lane >> 5) + t % 4, t = 0..7, the row order of the
// B operand packed from a 32x32 accumulator's registers in order.  tl = this
// lane's base, tile + vbase.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint8_t* tl, int kb, int cb) {
    using C = PrefillBf16Cfg<D>;
    const uint8_t* vp = tl + kb * 16 * C::VS * 16 + cb * 64;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * C::VS * 16));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
}

// Order a product's LDS operand reads AHEAD MFMAs ahead of their use (R
// reads per MFMA), as the forward's tile step does.
template <int NMFMA, int R, int AHEAD>
__device__ __forceinline__ void order_operand_reads() {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD * R, 0);
#pragma unroll
    for (int i = 0; i < NMFMA - AHEAD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
#endif
}

// acc[jb] = sum_kk A(rows of the tile) x bf[kk]: a 64 x 32 product over the
// head dim (16 MFMAs).
template <int D>
__device__ __forceinline__ void rows_times(const uint8_t* rl, const bf16x8 (&bf)[D / 16], f32x16 (&acc)[2]) {
    acc[0] = f32x16{};
    acc[1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
            acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<D>(rl, jb, kk), bf[kk], acc[jb], 0, 0, 0);
    order_operand_reads<D / 8, 1, 4>();
}

// Store a d x 32 accumulator (column = this lane's row or key) as one bf16
// row of d values, times `mul`.
template <int D>
__device__ __forceinline__ void store_row(uint16_t* dst, const f32x16 (&acc)[D / 32], float mul, int lane) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            u32x2 w;
            w[0] = pack_bf16x2(acc[cb][4 * gq + 0] * mul, acc[cb][4 * gq + 1] * mul);
            w[1] = pack_bf16x2(acc[cb][4 * gq + 2] * mul, acc[cb][4 * gq + 3] * mul);
            *(u32x2*)(dst + cb * 32 + 8 * gq + 4 * (lane >> 5)) = w;
        }
}

// The B operand fragment of a row held in registers (query row for dQ, key
// for dK/dV): chunks (lane >> 5) * 8 .. + 8 of every 16-wide head-dim step.
template <int D>
__device__ __forceinline__ void load_fragment(const uint16_t* rowp, bool ok, int lane, bf16x8 (&f)[D / 16]) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        const u32x4 w = ok ? *(const u32x4*)(rowp + kk * 16 + (lane >> 5) * 8) : u32x4{0, 0, 0, 0};
        f[kk] = __builtin_bit_cast(bf16x8, w);
    }
}

__device__ __forceinline__ PrefillParams mask_params(const BackwardParams& p) {
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

}  // namespace

__global__ void bwd_zero_kernel(float* x, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) x[i] = 0.f;
}

// D / 8 threads per query row (8 columns each): D = dO . O, plus the row's
// statistics for the two gradient passes.  256 / (D / 8) rows per workgroup.
template <int D>
__device__ __forceinline__ void bwd_prep_body(BackwardParams p) {
    constexpr int TPR = D / 8;
    const int t = threadIdx.x;
    const long long rows = (long long)p.B * p.Hq * p.Nq;
    const long long rg = (long long)blockIdx.x * (256 / TPR) + t / TPR;
    float acc = 0.f;
    if (rg < rows) {
        const u32x4 a = *(const u32x4*)(p.o + rg * D + (t % TPR) * 8);
        const u32x4 g = *(const u32x4*)(p.dO + rg * D + (t % TPR) * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc += bf16_lo(a[e]) * bf16_lo(g[e]) + bf16_hi(a[e]) * bf16_hi(g[e]);
    }
#pragma unroll
    for (int o = TPR / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (rg < rows && t % TPR == 0) {
        const int i = (int)(rg % p.Nq);
        const int h = (int)((rg / p.Nq) % p.Hq);
        const float L = p.lse[rg];
        p.ws_d[rg] = acc;
        p.ws_nl[rg] = L > -__builtin_inff() ? -L * kLog2e : 0.f;
        const PrefillParams m = mask_params(p);
        int lo, hi;
        row_interval(m, i, lo, hi);
        p.ws_lo[rg] = lo;
        p.ws_hi[rg] = hi;
        if (p.dsink != nullptr && p.sink_logits != nullptr && L > -__builtin_inff())
            atomicAdd(p.dsink + h, -__builtin_amdgcn_exp2f((p.sink_logits[h] - L) * kLog2e) * acc);
    }
}

__global__ __launch_bounds__(256) void bwd_prep_kernel(BackwardParams p) { bwd_prep_body<128>(p); }
__global__ __launch_bounds__(256) void bwd_prep_d64_kernel(BackwardParams p) { bwd_prep_body<64>(p); }

// dQ: per 32-key tile, S^T = K Q^T, dP^T = V dO^T, dS = P (dP - D),
// dQ^T += K^T dS^T.  K is copied twice (row and transposed layouts), V once.
// With 32-key tiles a stage of that ring is 28 KiB and a wave needs 190
// registers, so two workgroups share a CU and two waves each SIMD (64-key
// tiles took 54 KiB per stage and 280 registers, one wave per SIMD; the
// backward of C2 went from 468 to 414 us with this change).
template <int D>
struct DqCfg {
    static constexpr int BN = 32;
    static constexpr int KS = D / 8 + 1;          // row layout: one 16-byte slot of padding per row
    static constexpr int VS = D / 8 + 4;          // transposed layout: four slots
    // whole 1 KiB copies, rounded up (d 128: 32 x 17 slots = 8.5 KiB copied
    // as 9 KiB, the slack rows never read; d 64: 4.5 KiB as 5)
    static constexpr int KLOADS = (BN * KS * 16 + 1023) / 1024;
    static constexpr int VLOADS = (BN * VS * 16 + 1023) / 1024;
    static constexpr int KTILE = KLOADS * 1024;
    static constexpr int VTILE = VLOADS * 1024;
    static constexpr int KLW = (KLOADS + 3) / 4;
    static constexpr int VLW = (VLOADS + 3) / 4;
};

// MODS: the scores went through the score modifications.  With t the
// modified score and x = scale q.k, P = exp(t - LSE) and the gradient
// P (dP - D) is with respect to t; the cap's chain-rule factor
// dt/dx = 1 - tanh^2 = 4 r (1 - r), r = 1 / (e^(2x/c) + 1), turns it into
// the gradient with respect to x (the slope bias does not depend on q or k).
template <int D, bool MODS>
__device__ __forceinline__ void bwd_dq_body(BackwardParams p) {
    using C = DqCfg<D>;
    constexpr int BM = 128;
    __shared__ __attribute__((aligned(1024))) uint8_t kr0[C::KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t kt0[C::VTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t vr0[C::KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t kr1[C::KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t kt1[C::VTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t vr1[C::KTILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bk, qt, g;
    decode_work(blockIdx.x, p.B * p.Hkv, p.num_q_tiles, p.group, bk, qt, g);
    const int b = bk / p.Hkv, hkv = bk % p.Hkv, hq = hkv * p.group + g;
    const PrefillParams m = mask_params(p);
    const ScoreMod sm = MODS ? make_score_mod(p.scale_log2, p.softcap, p.alibi_slopes, hq) : ScoreMod{};

    const int r0 = qt * BM;
    const int r_last = min(r0 + BM, p.Nq) - 1;
    const int w0 = r0 + wave * 32;
    const int w_last = min(w0 + 31, p.Nq - 1);
    const int row = w0 + (lane & 31);
    const bool row_ok = row < p.Nq;
    int lo_i, hi_i, lo_wg, hi_wg, tmp, lo_w_first, hi_w_first, lo_w_last, hi_w_last;
    row_interval(m, row, lo_i, hi_i);
    row_interval(m, r0, lo_wg, tmp);
    row_interval(m, r_last, tmp, hi_wg);
    row_interval(m, w0, lo_w_first, hi_w_first);
    row_interval(m, w_last, lo_w_last, hi_w_last);
    const bool wave_has_rows = w0 < p.Nq;

    const size_t head_row = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
    bf16x8 qf[D / 16], df[D / 16];
    load_fragment<D>(p.q + (head_row + (row_ok ? row : 0)) * D, row_ok, lane, qf);
    load_fragment<D>(p.dO + (head_row + (row_ok ? row : 0)) * D, row_ok, lane, df);
    const float nl = row_ok ? p.ws_nl[head_row + row] : -__builtin_inff();
    const float Drow = row_ok ? p.ws_d[head_row + row] : 0.f;

    f32x16 acc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};

    const uint16_t* kg_ = p.k + ((size_t)b * p.Hkv + hkv) * (size_t)p.Nk * D;
    const uint16_t* vg_ = p.v + ((size_t)b * p.Hkv + hkv) * (size_t)p.Nk * D;
    const TileRange tr = tile_range(lo_wg, hi_wg, p.sink_end, C::BN);
    uint32_t koff[C::KLW], voff[C::VLW];
    tile_src_offsets<D, C::KS, C::KLOADS>(koff, wave, lane);
    tile_src_offsets<D, C::VS, C::VLOADS>(voff, wave, lane);
    const int kbase = (lane & 31) * C::KS * 16 + (lane >> 5) * 16;
    const int vbase = (4 * (lane >> 5) + ((lane >> 2) & 3)) * C::VS * 16 + (((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2;

    auto copy = [&](int t, uint8_t* kr, uint8_t* kt, uint8_t* vr) __attribute__((always_inline)) {
        load_tile_async<D, C::KS, C::KLOADS>(kg_, t * C::BN, p.Nk, kr, koff, wave);
        load_tile_async<D, C::VS, C::VLOADS>(kg_, t * C::BN, p.Nk, kt, voff, wave);
        load_tile_async<D, C::KS, C::KLOADS>(vg_, t * C::BN, p.Nk, vr, koff, wave);
    };
    auto stage = [&](int it, const uint8_t* kr, const uint8_t* kt, const uint8_t* vr, uint8_t* krn, uint8_t* ktn,
                     uint8_t* vrn) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of this tile landed
        __syncthreads();
        if (it + 1 < tr.n) copy(tile_of(tr, it + 1), krn, ktn, vrn);
        const int n0 = tile_of(tr, it) * C::BN;
        const bool active = wave_has_rows && n0 <= hi_w_last && (n0 + C::BN - 1 >= lo_w_first || n0 < p.sink_end);
        if (!active) return;
        const bool full = n0 + C::BN - 1 <= hi_w_first && (n0 >= lo_w_last || n0 + C::BN - 1 < p.sink_end);
        // S^T = K Q^T and dP^T = V dO^T, one 32-key block each
        f32x16 s = f32x16{}, dp = f32x16{};
        const uint8_t* krl = kr + kbase;
        const uint8_t* vrl = vr + kbase;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, *(const u32x4*)(krl + kk * 32)), qf[kk], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, *(const u32x4*)(vrl + kk * 32)), df[kk], dp, 0, 0, 0);
        }
        order_operand_reads<D / 8, 1, 4>();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = n0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            float pr, fac = 1.f;
            if constexpr (MODS) {
                const float bias = sm.slope_l2 * (float)(key - (row + p.Nk - p.Nq));
                float t;
                if (sm.cap_k != 0.f) {
                    const float rr = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(s[r] * sm.cap_k) + 1.f);
                    t = __builtin_fmaf(-2.f * sm.cap_l2, rr, sm.cap_l2) + bias;
                    fac = 4.f * rr * (1.f - rr);
                } else {
                    t = __builtin_fmaf(s[r], sm.scale_l2, bias);
                }
                pr = __builtin_amdgcn_exp2f(t + nl);
            } else {
                pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], p.scale_log2, nl));
            }
            if (!full && (key > hi_i || (key < lo_i && key >= p.sink_end))) pr = 0.f;
            s[r] = MODS ? pr * (dp[r] - Drow) * fac : pr * (dp[r] - Drow);   // dS^T
        }
        bf16x8 dsf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(s[kb * 8 + 2 * e], s[kb * 8 + 2 * e + 1]);
            dsf[kb] = __builtin_bit_cast(bf16x8, w);
        }
        // dQ^T += K^T dS^T
        const uint8_t* ktl = kt + vbase;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const uint8_t* vp = ktl + kb * 16 * C::VS * 16 + cb * 64;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * C::VS * 16));
                const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}), dsf[kb], acc[cb], 0, 0, 0);
            }
        order_operand_reads<D / 16, 2, 2>();
    };

    if (tr.n > 0) {
        copy(tile_of(tr, 0), kr0, kt0, vr0);
        for (int it = 0; it < tr.n; it += 2) {
            stage(it, kr0, kt0, vr0, kr1, kt1, vr1);
            if (it + 1 < tr.n) stage(it + 1, kr1, kt1, vr1, kr0, kt0, vr0);
        }
    }
    if (row_ok) store_row<D>(p.dq + (head_row + row) * D, acc, p.scale, lane);
}

__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BackwardParams p) { bwd_dq_body<128, false>(p); }
__global__ __launch_bounds__(256, 2) void bwd_dq_mod_kernel(BackwardParams p) { bwd_dq_body<128, true>(p); }
__global__ __launch_bounds__(256, 2) void bwd_dq_d64_kernel(BackwardParams p) { bwd_dq_body<64, false>(p); }
__global__ __launch_bounds__(256, 2) void bwd_dq_d64_mod_kernel(BackwardParams p) { bwd_dq_body<64, true>(p); }

// dK and dV: each wave owns 32 keys (K and V fragments in registers) and
// streams 64-row query tiles of every query head of its group.
// MODS: as for the dQ pass; each streamed tile's query head brings its own slope.
template <int D, bool MODS>
__device__ __forceinline__ void bwd_dkdv_body(BackwardParams p) {
    using C = PrefillBf16Cfg<D>;
    constexpr int BQ = 64;    // query rows per streamed tile
    constexpr int BK = 128;   // keys per workgroup
    __shared__ __attribute__((aligned(1024))) uint8_t qr0[C::KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t qt0[C::VTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t dr0[C::KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t dt0[C::VTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t qr1[C::KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t qt1[C::VTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t dr1[C::KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t dt1[C::VTILE];
    // per tile row: -LSE log2 e, D, lo, hi (256 bytes each)
    __shared__ __attribute__((aligned(1024))) uint8_t st0[4 * BQ * 4];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[4 * BQ * 4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nbk = p.B * p.Hkv;
    const int kt_idx = blockIdx.x / nbk;     // key tiles in order: under causal masks the first are the heaviest
    const int bk = blockIdx.x % nbk;
    const int b = bk / p.Hkv, hkv = bk % p.Hkv;
    const PrefillParams m = mask_params(p);

    const int k0 = kt_idx * BK;
    const int k0w = k0 + wave * 32;
    const int key = k0w + (lane & 31);
    const bool key_ok = key < p.Nk;
    const int k_last = min(k0 + BK, p.Nk) - 1;

    const size_t kv_head = ((size_t)b * p.Hkv + hkv) * (size_t)p.Nk;
    bf16x8 kf[D / 16], vf[D / 16];
    load_fragment<D>(p.k + (kv_head + (key_ok ? key : 0)) * D, key_ok, lane, kf);
    load_fragment<D>(p.v + (kv_head + (key_ok ? key : 0)) * D, key_ok, lane, vf);
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
        dk[cb] = f32x16{};
        dv[cb] = f32x16{};
    }

    // Query rows that see any key of [k0, k_last]: from the first row whose
    // interval reaches k0 to the last whose interval starts at or before
    // k_last (every later row, when sink keys are in the tile).  Both ends
    // are monotone in the row, so two binary searches find them.
    int first = p.Nq, last = -1;
    {
        int a = 0, z = p.Nq;
        while (a < z) {
            const int mid = (a + z) >> 1;
            int l, h;
            row_interval(m, mid, l, h);
            if (h >= k0) z = mid; else a = mid + 1;
        }
        first = a;
        if (k0 < p.sink_end) {
            last = p.Nq - 1;
        } else {
            a = -1;
            z = p.Nq - 1;
            while (a < z) {
                const int mid = (a + z + 1) >> 1;
                int l, h;
                row_interval(m, mid, l, h);
                if (l <= k_last) a = mid; else z = mid - 1;
            }
            last = a;
        }
    }
    const int qt_first = first / BQ;
    const int ntq = (first <= last && k0 < p.Nk) ? last / BQ - qt_first + 1 : 0;
    const int n_iter = ntq * p.group;

    uint32_t koff[C::KLW], voff[C::VLW];
    tile_src_offsets<D, C::KS, C::KLOADS>(koff, wave, lane);
    tile_src_offsets<D, C::VS, C::VLOADS>(voff, wave, lane);
    const int kbase = (lane & 31) * C::KS * 16 + (lane >> 5) * 16;
    const int vbase = (4 * (lane >> 5) + ((lane >> 2) & 3)) * C::VS * 16 + (((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2;

    auto head_of = [&](int it) __attribute__((always_inline)) { return hkv * p.group + it / ntq; };
    auto q0_of = [&](int it) __attribute__((always_inline)) { return (qt_first + it % ntq) * BQ; };
    // copies of iteration it: Q and dO rows in both layouts, and the rows' statistics
    auto copy = [&](int it, uint8_t* qr, uint8_t* qt, uint8_t* dr, uint8_t* dt, uint8_t* st)
        __attribute__((always_inline)) {
        const size_t head_row = ((size_t)b * p.Hq + head_of(it)) * (size_t)p.Nq;
        const int q0 = q0_of(it);
        const uint16_t* qg = p.q + head_row * D;
        const uint16_t* dg = p.dO + head_row * D;
        load_tile_async<D, C::KS, C::KLOADS>(qg, q0, p.Nq, qr, koff, wave);
        load_tile_async<D, C::VS, C::VLOADS>(qg, q0, p.Nq, qt, voff, wave);
        load_tile_async<D, C::KS, C::KLOADS>(dg, q0, p.Nq, dr, koff, wave);
        load_tile_async<D, C::VS, C::VLOADS>(dg, q0, p.Nq, dt, voff, wave);
        if (wave == 0) {
            const int nrow = (p.Nq - q0) * 4;   // bytes of rows that exist; the rest read 0
            const void* srcs[4] = {p.ws_nl + head_row + q0, p.ws_d + head_row + q0, p.ws_lo + head_row + q0,
                                   p.ws_hi + head_row + q0};
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)srcs[a], (short)0, nrow, 0x00020000);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(st + a * BQ * 4), 4, lane * 4, 0, 0, 0);
            }
        }
    };

    auto stage = [&](int it, const uint8_t* qr, const uint8_t* qt, const uint8_t* dr, const uint8_t* dt,
                     const uint8_t* st, uint8_t* qrn, uint8_t* qtn, uint8_t* drn, uint8_t* dtn, uint8_t* stn)
        __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        __syncthreads();
        if (it + 1 < n_iter) copy(it + 1, qrn, qtn, drn, dtn, stn);
        const int q0 = q0_of(it);
        const int q_end = min(q0 + BQ, p.Nq) - 1;
        int lo_a, hi_a, lo_z, hi_z;
        row_interval(m, q0, lo_a, hi_a);
        row_interval(m, q_end, lo_z, hi_z);
        // does some row of the tile see some key of this wave (its keys exist)?
        if (!(k0w < p.Nk && hi_z >= k0w && (lo_a <= k0w + 31 || k0w < p.sink_end))) return;
        const bool full = q0 + BQ - 1 < p.Nq && k0w + 31 < p.Nk && hi_a >= k0w + 31 &&
                          (lo_z <= k0w || k0w + 31 < p.sink_end);
        f32x16 s[2], dp[2];
        rows_times<D>(qr + kbase, kf, s);    // S = Q K^T   (columns: this lane's key)
        // MODS: S -> modified base-2 scores (before the mask: a capped -inf
        // would come back finite) and the cap factor of each element.  Element
        // (jb, r) is row q0 + 32 jb + 8 (r / 4) + 4 (lane / 32) + r % 4.
        f32x16 fac[2];
        if constexpr (MODS) {
            const ScoreMod sm = make_score_mod(p.scale_log2, p.softcap, p.alibi_slopes, head_of(it));
            const float b0 = sm.slope_l2 * (float)(key - q0 - 4 * (lane >> 5) - p.Nk + p.Nq);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float bias = __builtin_fmaf(-sm.slope_l2, (float)(32 * jb + 8 * (r >> 2) + (r & 3)), b0);
                    if (sm.cap_k != 0.f) {
                        const float rr = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(s[jb][r] * sm.cap_k) + 1.f);
                        s[jb][r] = __builtin_fmaf(-2.f * sm.cap_l2, rr, sm.cap_l2) + bias;
                        fac[jb][r] = 4.f * rr * (1.f - rr);
                    } else {
                        s[jb][r] = __builtin_fmaf(s[jb][r], sm.scale_l2, bias);
                        fac[jb][r] = 1.f;
                    }
                }
        }
        const float sl = MODS ? 1.f : p.scale_log2;   // scores already in base-2 units under MODS
        const float* nl = (const float*)st;
        const float* dd = (const float*)(st + BQ * 4);
        if (!full) {
            // scores of invisible (row, key) pairs and of rows past Nq become
            // -inf, so their P and dS are 0 below
            const int32_t* rlo = (const int32_t*)(st + 2 * BQ * 4);
            const int32_t* rhi = (const int32_t*)(st + 3 * BQ * 4);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int rb = jb * 32 + 8 * g4 + 4 * (lane >> 5);   // first of this lane's 4 consecutive rows
                    const u32x4 a = *(const u32x4*)(rlo + rb);
                    const u32x4 z = *(const u32x4*)(rhi + rb);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool vis = q0 + rb + e < p.Nq && key <= (int32_t)z[e] &&
                                         (key >= (int32_t)a[e] || key < p.sink_end);
                        if (!vis) s[jb][4 * g4 + e] = -__builtin_inff();
                    }
                }
        }
        // the rows' statistics for the whole tile
        f32x4 nl4[8], dd4[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int rb = (q >> 2) * 32 + 8 * (q & 3) + 4 * (lane >> 5);
            nl4[q] = *(const f32x4*)(nl + rb);
            dd4[q] = *(const f32x4*)(dd + rb);
        }
        // dP = dO V^T (NM = D / 8 products), each followed by EPM of the tile's
        // 32 P = exp2(.)
        {
            constexpr int NM = D / 8, EPM = 32 / NM;
            dp[0] = f32x16{};
            dp[1] = f32x16{};
            const uint8_t* drl = dr + kbase;
            bf16x8 ra[5];
#pragma unroll
            for (int j = 0; j < 4; ++j) ra[j] = row_operand<D>(drl, j & 1, j >> 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                if (i + 4 < NM) ra[(i + 4) % 5] = row_operand<D>(drl, (i + 4) & 1, (i + 4) >> 1);
                dp[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[i % 5], vf[i >> 1], dp[i & 1], 0, 0, 0);
#pragma unroll
                for (int x = 0; x < EPM; ++x) {
                    const int el = EPM * i + x, jb = el >> 4, r = el & 15, q = 4 * jb + (r >> 2);
                    s[jb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jb][r], sl, nl4[q][r & 3]));   // P
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // dS of element e of 16-row block kb (P already in s[jb][8 (kb & 1) + e])
        auto element = [&](int kb, int e) __attribute__((always_inline)) {
            const int jb = kb >> 1, r = 8 * (kb & 1) + e, q = 4 * jb + (r >> 2);
            if constexpr (MODS) dp[jb][r] = s[jb][r] * (dp[jb][r] - dd4[q][r & 3]) * fac[jb][r];   // dS
            else dp[jb][r] = s[jb][r] * (dp[jb][r] - dd4[q][r & 3]);
        };
        bf16x8 pf[4], dsf[4];
        auto pack = [&](int kb) __attribute__((always_inline)) {
            const int jb = kb >> 1, h = (kb & 1) * 8;
            u32x4 wp, wd;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                wp[x] = pack_bf16x2(s[jb][h + 2 * x], s[jb][h + 2 * x + 1]);
                wd[x] = pack_bf16x2(dp[jb][h + 2 * x], dp[jb][h + 2 * x + 1]);
            }
            pf[kb] = __builtin_bit_cast(bf16x8, wp);
            dsf[kb] = __builtin_bit_cast(bf16x8, wd);
        };
        // product i: block kb = i / PPB, head-dim block cb = (i / 2) % CB, dV
        // (i even) or dK (i odd); PPB = 2 CB products per 16-row block, each
        // followed by EPP of the next block's 8 dS elements
        constexpr int CB = D / 32, PPB = 2 * CB, NP = 4 * PPB, EPP = 8 / PPB;
        auto operand = [&](int i) __attribute__((always_inline)) {
            return tr_operand<D>(((i & 1) ? qt : dt) + vbase, i / PPB, (i >> 1) % CB);
        };
        // Block 0's dS first; then the dV / dK products, each followed by
        // EPP elements of the next block's dS and the operand reads of the
        // product two ahead, pinned in that order by scheduling barriers.  At
        // one wave per SIMD nothing else fills the matrix core while VALU work
        // issues: with the exponentials and dS all ahead of the products (the
        // compiler's own order, also under group-barrier hints) the backward
        // of C2 took 428 us; pinned under the products, 360 us; with the
        // exponentials moved under the dP products as well, 345 us.
#pragma unroll
        for (int x = 0; x < 8; ++x) element(0, x);
        pack(0);
        bf16x8 opr[3];
        opr[0] = operand(0);
        opr[1] = operand(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int kb = i / PPB, cb = (i >> 1) % CB;
            if (i + 2 < NP) opr[(i + 2) % 3] = operand(i + 2);
            if (i & 1) dk[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opr[i % 3], dsf[kb], dk[cb], 0, 0, 0);
            else dv[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opr[i % 3], pf[kb], dv[cb], 0, 0, 0);
            if (kb < 3) {
#pragma unroll
                for (int y = 0; y < EPP; ++y) element(kb + 1, (i % PPB) * EPP + y);
                if (i % PPB == PPB - 1) pack(kb + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (n_iter > 0) {
        copy(0, qr0, qt0, dr0, dt0, st0);
        for (int it = 0; it < n_iter; it += 2) {
            stage(it, qr0, qt0, dr0, dt0, st0, qr1, qt1, dr1, dt1, st1);
            if (it + 1 < n_iter) stage(it + 1, qr1, qt1, dr1, dt1, st1, qr0, qt0, dr0, dt0, st0);
        }
    }
    if (key_ok) {
        store_row<D>(p.dk + (kv_head + key) * D, dk, p.scale, lane);
        store_row<D>(p.dv + (kv_head + key) * D, dv, 1.f, lane);
    }
}

__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BackwardParams p) { bwd_dkdv_body<128, false>(p); }
__global__ __launch_bounds__(256, 1) void bwd_dkdv_mod_kernel(BackwardParams p) { bwd_dkdv_body<128, true>(p); }
__global__ __launch_bounds__(256, 1) void bwd_dkdv_d64_kernel(BackwardParams p) { bwd_dkdv_body<64, false>(p); }
__global__ __launch_bounds__(256, 1) void bwd_dkdv_d64_mod_kernel(BackwardParams p) { bwd_dkdv_body<64, true>(p); }

size_t backward_workspace_bytes(int B, int Hq, int Nq) {
    const size_t rows = (size_t)B * Hq * Nq;
    return 4 * ((rows * 4 + 255) / 256) * 256;
}

int launch_backward(BackwardParams p, int d, void* ws, hipStream_t stream) {
    const size_t rows = (size_t)p.B * p.Hq * p.Nq;
    const bool mods = p.softcap > 0.f || p.alibi_slopes != nullptr;
    const size_t stride = ((rows * 4 + 255) / 256) * 256;
    p.ws_nl = (float*)ws;
    p.ws_d = (float*)((char*)ws + stride);
    p.ws_lo = (int32_t*)((char*)ws + 2 * stride);
    p.ws_hi = (int32_t*)((char*)ws + 3 * stride);
    // the sink gradient accumulates across rows: clear it with a kernel (not a
    // memset, so the sequence can be captured into a graph)
    if (p.dsink != nullptr && p.Hq > 0)
        hipLaunchKernelGGL(bwd_zero_kernel, dim3((p.Hq + 255) / 256), dim3(256), 0, stream, p.dsink, p.Hq);
    const dim3 wg(256), gq(p.B * p.Hq * p.num_q_tiles), gk(p.B * p.Hkv * p.num_k_tiles);
    if (rows > 0) {
        const size_t rows_per_wg = 256 / (d / 8);   // the prep pass's D / 8 threads per row
        const dim3 gp((unsigned)((rows + rows_per_wg - 1) / rows_per_wg));
        if (d == 128) {
            hipLaunchKernelGGL(bwd_prep_kernel, gp, wg, 0, stream, p);
            if (mods) hipLaunchKernelGGL(bwd_dq_mod_kernel, gq, wg, 0, stream, p);
            else hipLaunchKernelGGL(bwd_dq_kernel, gq, wg, 0, stream, p);
        } else {
            hipLaunchKernelGGL(bwd_prep_d64_kernel, gp, wg, 0, stream, p);
            if (mods) hipLaunchKernelGGL(bwd_dq_d64_mod_kernel, gq, wg, 0, stream, p);
            else hipLaunchKernelGGL(bwd_dq_d64_kernel, gq, wg, 0, stream, p);
        }
    }
    if ((long long)p.B * p.Hkv * p.num_k_tiles > 0) {
        if (d == 128) {
            if (mods) hipLaunchKernelGGL(bwd_dkdv_mod_kernel, gk, wg, 0, stream, p);
            else hipLaunchKernelGGL(bwd_dkdv_kernel, gk, wg, 0, stream, p);
        } else {
            if (mods) hipLaunchKernelGGL(bwd_dkdv_d64_mod_kernel, gk, wg, 0, stream, p);
            else hipLaunchKernelGGL(bwd_dkdv_d64_kernel, gk, wg, 0, stream, p);
        }
    }
    return 0;
}

}  // namespace xattn
