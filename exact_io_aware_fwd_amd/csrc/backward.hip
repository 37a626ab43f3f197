// Attention backward (bf16, head dim 64 or 128) by recomputation from the saved
// log-sum-exp, the FlashAttention-2 backward ("Attention Is the Bottleneck",
// FlashAttention-2 section: the forward keeps only O and the per-row
// statistic; the backward recomputes the probabilities tile by tile).
//
//   P = exp(S - LSE),  D = rowsum(dO o O),  dS = P o (dO V^T - D)
//   dV = P^T dO,  dQ = scale dS K,  dK = scale dS^T Q
//
// Two passes, no atomics:
//   dQ     one workgroup per (batch, query head, 128-row query tile), each
//          wave owning 32 rows as in the forward.  It first writes each
//          row's statistics to the workspace (-LSE log2(e), D and the row's
//          visible key interval), then per 32-key tile recomputes
//          S^T = K Q^T and dP^T = V dO^T and accumulates dQ^T += K^T dS^T
//          (the forward's O^T += V^T P^T with K and dS); with a learned
//          sink, a per-head reduction of its gradient -sum_i P_sink,i D_i
//          in a fixed order follows;
//   dK/dV  one workgroup per (batch, KV head, 128-key tile); it streams
//          64-row query tiles of every query head of the group, recomputes
//          S = Q K^T and dP = dO V^T with the keys as the accumulator
//          columns, and accumulates dV^T += dO^T P and dK^T += Q^T dS.  At
//          d = 128 two waves on one SIMD share each 32-key block (one holds
//          K and dV, the other V and dK, the weights handed over in LDS,
//          bwd_dkdv2_kernel); at d = 64 one wave owns each block.
// At d = 128 a tile that one product reads by rows and another transposed
// (Q and dO in the dK/dV pass, K in the dQ pass) is one swizzled copy that
// both reads use without bank conflicts (DualSwizzle); at d = 64 such tiles
// are copied twice, once in each padded layout.
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

// One LDS copy of a d = 128 tile that serves both row reads and transposing
// reads: 16-byte chunk c of row r is stored at chunk c ^ (4 (r % 4) + (r / 4) % 4).
// 16 consecutive rows at one chunk (a row operand) land in 16 different
// chunks, and the 4 consecutive rows x 64 bytes of a transposing read land in
// 16 different chunks, so neither read has bank conflicts (checked on a CPU
// model of the banks).  Each 1 KiB copy holds 4 whole rows, and a lane's
// source offset is the same for all of a wave's copies.  Per-lane offsets:
// ro[kk] for the row operand at head-dim step kk (32-row block jb adds 8 KiB),
// tr0/tr1[cb] for the two transposing reads of column block cb (16-row block
// kb adds 4 KiB), cpo for this wave's copies (block wave + 4 j, j KiB apart).
struct DualSwizzle {
    int ro[8], tr0[4], tr1[4];
    uint32_t cpo;
    __device__ __forceinline__ void init(int lane, int wave) {
        const int gl = 4 * (lane & 3) + ((lane >> 2) & 3);   // the chunk swizzle of this lane's rows
        const int y = (lane >> 5) ^ gl;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) ro[kk] = (lane & 31) * 256 + 32 * (kk ^ (y >> 1)) + 16 * (y & 1);
        const int a = lane >> 5, bq = (lane >> 2) & 3, e = (lane >> 4) & 1, d = (lane & 3) >> 1;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            tr0[cb] = (4 * a + bq) * 256 + 64 * (cb ^ bq) + 16 * (2 * e + (d ^ a)) + 8 * (lane & 1);
            tr1[cb] = (4 * a + bq + 8) * 256 + 64 * (cb ^ bq) + 16 * (2 * (e ^ 1) + (d ^ a)) + 8 * (lane & 1);
        }
        const int q = lane >> 4;
        cpo = (uint32_t)(q * 256 + (((lane & 15) ^ (4 * q) ^ wave) * 16));
    }
    // A operand by rows: rows (lane & 31) + 32 jb, head-dim chunk 2 kk + (lane >> 5)
    __device__ __forceinline__ bf16x8 row(const uint8_t* tile, int jb, int kk) const {
        return __builtin_bit_cast(bf16x8, *(const u32x4*)(tile + jb * 8192 + ro[kk]));
    }
    // A operand transposed, as tr_operand
    __device__ __forceinline__ bf16x8 tr(const uint8_t* tile, int kb, int cb) const {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + kb * 4096 + tr0[cb]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + kb * 4096 + tr1[cb]));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
    }
    // the same with eight waves sharing the copies (blocks wave8 + 8 j; init
    // took wave8 & 3, the block index modulo 4 that the swizzle uses)
    template <int NB>
    __device__ __forceinline__ void copy8(const uint16_t* src, int rows, uint8_t* lds, int wave8) const {
#if defined(__HIP_DEVICE_COMPILE__)
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)src, (short)0, (int)tile_range_bytes<128>(rows, NB * 4), 0x00020000);
#pragma unroll
        for (int j = 0; j < NB / 8; ++j) {
            const int blk = wave8 + 8 * j;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + blk * 1024), 16, cpo, blk * 1024, 0, 0);
        }
#endif
    }
    // this wave's copies of one tile of NB KiB (4 rows each) from rows
    // following each other in memory; rows at or past `rows` read as zero
    template <int NB>
    __device__ __forceinline__ void copy(const uint16_t* src, int rows, uint8_t* lds, int wave) const {
#if defined(__HIP_DEVICE_COMPILE__)
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)src, (short)0, (int)tile_range_bytes<128>(rows, NB * 4), 0x00020000);
#pragma unroll
        for (int j = 0; j < NB / 4; ++j) {
            const int blk = wave + 4 * j;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + blk * 1024), 16, cpo, blk * 1024, 0, 0);
        }
#endif
    }
};

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

// Store a wave's d x 32 accumulator (column = this lane's row or key, 32
// rows) as bf16 rows of d values, times `mul`, through the wave's LDS
// staging area `stg` (32 rows of 2 d + 16 bytes, the padding spreading the
// rows' writes over the banks): each lane writes its pieces of its row, then
// every store writes whole rows, 16 bytes per lane (stores of 8 bytes per
// lane straight from the accumulator, spread over 32 rows, took about 3500
// cycles per tile).  dst is row 0; rows at or past `rows` are not written.
template <int D>
__device__ __forceinline__ void store_rows_staged(uint16_t* dst, int rows, const f32x16 (&acc)[D / 32], float mul,
                                                  int lane, uint8_t* stg) {
    constexpr int RB = 2 * D + 16;   // staged row stride in bytes
    constexpr int CPR = 2 * D / 16;  // 16-byte chunks per row
    constexpr int RPS = 64 / CPR;    // rows per store
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            u32x2 w;
            w[0] = pack_bf16x2(acc[cb][4 * gq + 0] * mul, acc[cb][4 * gq + 1] * mul);
            w[1] = pack_bf16x2(acc[cb][4 * gq + 2] * mul, acc[cb][4 * gq + 3] * mul);
            *(u32x2*)(stg + (lane & 31) * RB + (cb * 32 + 8 * gq + 4 * (lane >> 5)) * 2) = w;
        }
    // the wave reads what its other lanes wrote
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < 32 / RPS; ++j) {
        const int row = j * RPS + lane / CPR, c = lane % CPR;
        const u32x4 v = *(const u32x4*)(stg + row * RB + c * 16);
        if (row < rows) *(u32x4*)(dst + (size_t)row * D + c * 8) = v;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The B operand fragment of a row held in registers (query row for dQ, key
// for dK/dV): chunks (lane >> 5) * 8 .. + 8 of every 16-wide head-dim step.
// rowp is a row that exists even where !ok (the caller's row 0 then); it is
// read either way and the fragment zeroed after, with no branch per load.
template <int D>
__device__ __forceinline__ void load_fragment(const uint16_t* rowp, bool ok, int lane, bf16x8 (&f)[D / 16]) {
    u32x4 w[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) w[kk] = *(const u32x4*)(rowp + kk * 16 + (lane >> 5) * 8);
    const uint32_t keep = ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        f[kk] = __builtin_bit_cast(bf16x8, u32x4{w[kk][0] & keep, w[kk][1] & keep, w[kk][2] & keep, w[kk][3] & keep});
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

// The learned sink's gradient, dsink[h] = -sum over (batch, row) of
// P_sink D with P_sink = exp(sink[h] - LSE), from the saved LSE and the D
// that the dQ pass (the fp32 path: its prep pass) left in the workspace.  One workgroup per query head; every thread sums its rows in a
// fixed order and the workgroup adds the partial sums in a fixed tree, so the
// result is the same bit for bit on every run (no atomics).
__global__ __launch_bounds__(256) void bwd_dsink_kernel(BackwardParams p) {
    __shared__ float part[256];
    const int h = blockIdx.x, t = threadIdx.x;
    const float s2 = p.sink_logits[h] * kLog2e;
    float acc = 0.f;
    for (int b = 0; b < p.B; ++b) {
        const size_t base = ((size_t)b * p.Hq + h) * (size_t)p.Nq;
        for (int i = t; i < p.Nq; i += 256) {
            const float L = p.lse[base + i];
            if (L > -__builtin_inff()) acc -= __builtin_amdgcn_exp2f(s2 - L * kLog2e) * p.ws_d[base + i];
        }
    }
    part[t] = acc;
    __syncthreads();
#pragma unroll
    for (int w = 128; w >= 1; w >>= 1) {
        if (t < w) part[t] += part[t + w];
        __syncthreads();
    }
    if (t == 0) p.dsink[h] = part[0];
}

void launch_dsink(const BackwardParams& p, hipStream_t stream) {
    if (p.dsink == nullptr || p.Hq == 0) return;
    hipLaunchKernelGGL(bwd_dsink_kernel, dim3(p.Hq), dim3(256), 0, stream, p);
}

// dQ: per 32-key tile, S^T = K Q^T, dP^T = V dO^T, dS = P (dP - D),
// dQ^T += K^T dS^T.  At d = 128 the K tile is one DualSwizzle copy that
// serves the row reads (S^T) and the transposing reads (dQ^T), and V is
// copied in the same layout: 16 KiB per stage, 4 copies per wave and tile.
// At d = 64 K is copied twice (row and transposed padded layouts), V once.
// With 32-key tiles a wave needs about 200 registers, so two workgroups share
// a CU and two waves each SIMD (64-key tiles took 280 registers, one wave per
// SIMD; the backward of C2 went from 468 to 414 us with 32-key tiles).
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
    constexpr bool SWZ = D == 128;
    constexpr int RT = SWZ ? C::BN * D * 2 : C::KTILE;   // row-layout tile (K and V; the only tiles with SWZ)
    constexpr int TT = SWZ ? 16 : C::VTILE;              // transposed-layout K tile (unused with SWZ)
    __shared__ __attribute__((aligned(1024))) uint8_t kr0[RT];
    __shared__ __attribute__((aligned(1024))) uint8_t kt0_[TT];
    __shared__ __attribute__((aligned(1024))) uint8_t vr0[RT];
    __shared__ __attribute__((aligned(1024))) uint8_t kr1[RT];
    __shared__ __attribute__((aligned(1024))) uint8_t kt1_[TT];
    __shared__ __attribute__((aligned(1024))) uint8_t vr1[RT];
    // each wave's dQ rows on their way out
    __shared__ __attribute__((aligned(16))) uint8_t stage_out[4 * 32 * (2 * D + 16)];
    uint8_t* kt0 = SWZ ? kr0 : kt0_;
    uint8_t* kt1 = SWZ ? kr1 : kt1_;

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

    // Every load of the prologue (the row's LSE, the Q, dO and O fragments,
    // and below the first K/V tile) is issued before the first wait on any of
    // them: issued one after another's use, their round trips added up to
    // about 7000 cycles per workgroup.
    const size_t head_row = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
    const float L = p.lse[head_row + (row_ok ? row : 0)];
    bf16x8 qf[D / 16], df[D / 16], of[D / 16];
    load_fragment<D>(p.q + (head_row + (row_ok ? row : 0)) * D, row_ok, lane, qf);
    load_fragment<D>(p.dO + (head_row + (row_ok ? row : 0)) * D, row_ok, lane, df);
    load_fragment<D>(p.o + (head_row + (row_ok ? row : 0)) * D, row_ok, lane, of);
    float nl = 0.f, Drow = 0.f;   // set below, once the first K/V copy is issued

    f32x16 acc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};

    const uint16_t* kg_ = p.k + ((size_t)b * p.Hkv + hkv) * (size_t)p.Nk * D;
    const uint16_t* vg_ = p.v + ((size_t)b * p.Hkv + hkv) * (size_t)p.Nk * D;
    const TileRange tr = tile_range(lo_wg, hi_wg, p.sink_end, C::BN);
    uint32_t koff[C::KLW], voff[C::VLW];
    int kbase = 0, vbase = 0;
    DualSwizzle dz;
    if constexpr (SWZ) {
        dz.init(lane, wave);
    } else {
        tile_src_offsets<D, C::KS, C::KLOADS>(koff, wave, lane);
        tile_src_offsets<D, C::VS, C::VLOADS>(voff, wave, lane);
        kbase = (lane & 31) * C::KS * 16 + (lane >> 5) * 16;
        vbase = (4 * (lane >> 5) + ((lane >> 2) & 3)) * C::VS * 16 + (((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2;
    }

    auto copy = [&](int t, uint8_t* kr, uint8_t* kt, uint8_t* vr) __attribute__((always_inline)) {
        if constexpr (SWZ) {
            // keys past Nk read as zero
            dz.template copy<C::BN / 4>(kg_ + (size_t)t * C::BN * D, p.Nk - t * C::BN, kr, wave);
            dz.template copy<C::BN / 4>(vg_ + (size_t)t * C::BN * D, p.Nk - t * C::BN, vr, wave);
            (void)kt;
        } else {
            load_tile_async<D, C::KS, C::KLOADS>(kg_, t * C::BN, p.Nk, kr, koff, wave);
            load_tile_async<D, C::VS, C::VLOADS>(kg_, t * C::BN, p.Nk, kt, voff, wave);
            load_tile_async<D, C::KS, C::KLOADS>(vg_, t * C::BN, p.Nk, vr, koff, wave);
        }
    };
    auto stage = [&](int it, const uint8_t* kr, const uint8_t* kt, const uint8_t* vr, uint8_t* krn, uint8_t* ktn,
                     uint8_t* vrn) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of this tile landed
        __syncthreads();
        // Two workgroups share a CU (dispatched num_cus apart); they take the
        // higher wave priority in turn, tile by tile, as the forward does
        // (C2 backward 307-310 -> 304-306 us in alternated timings).
        if (((it + (int)blockIdx.x / p.num_cus) & 1) != 0) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        if (it + 1 < tr.n) copy(tile_of(tr, it + 1), krn, ktn, vrn);
        const int n0 = tile_of(tr, it) * C::BN;
        const bool active = wave_has_rows && n0 <= hi_w_last && (n0 + C::BN - 1 >= lo_w_first || n0 < p.sink_end);
        if (!active) return;
        const bool full = n0 + C::BN - 1 <= hi_w_first && (n0 >= lo_w_last || n0 + C::BN - 1 < p.sink_end);
        // S^T = K Q^T and dP^T = V dO^T, one 32-key block each
        f32x16 s = f32x16{}, dp = f32x16{};
        const uint8_t* krl = kr + kbase;
        const uint8_t* vrl = vr + kbase;
        auto rowop = [&](const uint8_t* tile, const uint8_t* tl, int kk) __attribute__((always_inline)) {
            if constexpr (SWZ) return dz.row(tile, 0, kk);
            else return __builtin_bit_cast(bf16x8, *(const u32x4*)(tl + kk * 32));
        };
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rowop(kr, krl, kk), qf[kk], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rowop(vr, vrl, kk), df[kk], dp, 0, 0, 0);
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
                bf16x8 a;
                if constexpr (SWZ) {
                    a = dz.tr(kt, kb, cb);
                } else {
                    const uint8_t* vp = ktl + kb * 16 * C::VS * 16 + cb * 64;
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * C::VS * 16));
                    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
                    a = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
                }
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsf[kb], acc[cb], 0, 0, 0);
            }
        order_operand_reads<D / 16, 2, 2>();
    };

    if (tr.n > 0) copy(tile_of(tr, 0), kr0, kt0, vr0);
    // The row's statistics, which the dK/dV pass and the sink gradient read
    // from the workspace: D = dO . O (this lane and lane ^ 32 hold the two
    // halves of the row), -LSE log2 e (0 for a row that sees nothing) and
    // the row's visible key interval.  Every row belongs to one workgroup
    // of this pass, so nothing else computes them.
    {
        float dsum = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf((float)df[kk][e], (float)of[kk][e], dsum);
        dsum += __shfl_xor(dsum, 32);
        const float Lr = row_ok ? L : -__builtin_inff();
        const float nlw = Lr > -__builtin_inff() ? -Lr * kLog2e : 0.f;
        nl = row_ok ? nlw : -__builtin_inff();
        Drow = row_ok ? dsum : 0.f;
        if (row_ok && lane < 32) {
            p.ws_d[head_row + row] = dsum;
            p.ws_nl[head_row + row] = nlw;
            p.ws_lo[head_row + row] = lo_i;
            p.ws_hi[head_row + row] = hi_i;
        }
    }
    if (tr.n > 0) {
        for (int it = 0; it < tr.n; it += 2) {
            stage(it, kr0, kt0, vr0, kr1, kt1, vr1);
            if (it + 1 < tr.n) stage(it + 1, kr1, kt1, vr1, kr0, kt0, vr0);
        }
    }
    if (wave_has_rows)
        store_rows_staged<D>(p.dq + (head_row + w0) * D, p.Nq - w0, acc, p.scale, lane,
                             stage_out + wave * 32 * (2 * D + 16));
}

__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BackwardParams p) { bwd_dq_body<128, false>(p); }
__global__ __launch_bounds__(256, 2) void bwd_dq_mod_kernel(BackwardParams p) { bwd_dq_body<128, true>(p); }
__global__ __launch_bounds__(256, 2) void bwd_dq_d64_kernel(BackwardParams p) { bwd_dq_body<64, false>(p); }
__global__ __launch_bounds__(256, 2) void bwd_dq_d64_mod_kernel(BackwardParams p) { bwd_dq_body<64, true>(p); }

// dK and dV at d = 64: each wave owns 32 keys (K and V fragments in
// registers) and streams 64-row query tiles of every query head of its group;
// every Q and dO tile is copied twice, in the row and the transposed padded
// layouts.  (At d = 128 the two-wave pass below runs instead.)
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
    // each wave's dK and dV rows on their way out
    __shared__ __attribute__((aligned(16))) uint8_t stage_out[4 * 32 * (2 * D + 16)];

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

    // Query rows that see any key of [k0, k_last] (in closed form but for
    // document masks: two scalar binary searches here took about 4500 cycles
    // of a workgroup that runs alone on its CU)
    int first = p.Nq, last = -1;
    if (k0 < p.Nk) query_rows_seeing(m, k0, k_last, first, last);
    const int qt_first = first / BQ;
    const int ntq = (first <= last && k0 < p.Nk) ? last / BQ - qt_first + 1 : 0;
    const int n_iter = ntq * p.group;

    uint32_t koff[C::KLW], voff[C::VLW];
    tile_src_offsets<D, C::KS, C::KLOADS>(koff, wave, lane);
    tile_src_offsets<D, C::VS, C::VLOADS>(voff, wave, lane);
    const int kbase = (lane & 31) * C::KS * 16 + (lane >> 5) * 16;
    const int vbase = (4 * (lane >> 5) + ((lane >> 2) & 3)) * C::VS * 16 + (((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2;
    // A operands: rows of a Q or dO tile (32-row block jb, head-dim step kk),
    // and a Q or dO tile transposed (16-row block kb, 32-column block cb)
    auto rowop = [&](const uint8_t* tile, int jb, int kk) __attribute__((always_inline)) {
        return row_operand<D>(tile + kbase, jb, kk);
    };
    auto trop = [&](const uint8_t* tile, int kb, int cb) __attribute__((always_inline)) {
        return tr_operand<D>(tile + vbase, kb, cb);
    };

    auto head_of = [&](int it) __attribute__((always_inline)) { return hkv * p.group + it / ntq; };
    auto q0_of = [&](int it) __attribute__((always_inline)) { return (qt_first + it % ntq) * BQ; };
    // copies of iteration it: Q and dO rows in both layouts, and the rows' statistics
    auto copy = [&](int it, uint8_t* qr, uint8_t* qt, uint8_t* dr, uint8_t* dt, uint8_t* st)
        __attribute__((always_inline)) {
        const size_t head_row = ((size_t)b * p.Hq + head_of(it)) * (size_t)p.Nq;
        const int q0 = q0_of(it);
        const uint16_t* qg = p.q + head_row * D;
        const uint16_t* dg = p.dO + head_row * D;
        // rows past Nq read as zero
        load_tile_async<D, C::KS, C::KLOADS>(qg, q0, p.Nq, qr, koff, wave);
        load_tile_async<D, C::VS, C::VLOADS>(qg, q0, p.Nq, qt, voff, wave);
        load_tile_async<D, C::KS, C::KLOADS>(dg, q0, p.Nq, dr, koff, wave);
        load_tile_async<D, C::VS, C::VLOADS>(dg, q0, p.Nq, dt, voff, wave);
        const int nrow = min(p.Nq - q0, BQ) * 4;   // bytes of the tile's rows that exist; the rest read 0
        const void* srcs[4] = {p.ws_nl + head_row + q0, p.ws_d + head_row + q0, p.ws_lo + head_row + q0,
                               p.ws_hi + head_row + q0};
        if (wave == 0) {
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
        // S = Q K^T (columns: this lane's key)
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
                s[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rowop(qr, jb, kk), kf[kk], s[jb], 0, 0, 0);
        order_operand_reads<D / 8, 1, 4>();
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
            bf16x8 ra[5];
#pragma unroll
            for (int j = 0; j < 4; ++j) ra[j] = rowop(dr, j & 1, j >> 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                if (i + 4 < NM) ra[(i + 4) % 5] = rowop(dr, (i + 4) & 1, (i + 4) >> 1);
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
            return trop((i & 1) ? qt : dt, i / PPB, (i >> 1) % CB);
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
    if (k0w < p.Nk) {
        uint8_t* stg = stage_out + wave * 32 * (2 * D + 16);
        store_rows_staged<D>(p.dk + (kv_head + k0w) * D, p.Nk - k0w, dk, p.scale, lane, stg);
        store_rows_staged<D>(p.dv + (kv_head + k0w) * D, p.Nk - k0w, dv, 1.f, lane, stg);
    }
}


// dK and dV at d = 128 with two waves per 32-key block, on one SIMD: wave A
// (0-3) holds the block's K fragments and dV, wave B (4-7) its V fragments
// and dK.  No product is computed twice, and each wave needs about half the
// registers of one wave doing all four products, so two fit on a SIMD.  B
// runs one query tile behind A, so the two waves' matrix and vector phases
// alternate: at tile t,
//   phase 1  A: S(t) = Q K^T                  B: dS(t-1) = P (dP - D)
//   phase 2  A: P(t) = exp2(...), to LDS      B: dP(t) = dO V^T
//   phase 3  A: dV^T += dO^T P(t)             B: dK^T += Q^T dS(t-1)
// with P (times the cap factor under score modifications) handed from A
// to B in LDS.  B still reads tile t-1 at tile t, so the ring has three
// stages.
template <bool MODS>
__device__ __forceinline__ void bwd_dkdv2_body(BackwardParams p) {
    constexpr int D = 128;
    constexpr int BQ = 64;    // query rows per streamed tile
    constexpr int BK = 128;   // keys per workgroup
    constexpr int RT = BQ * D * 2;
    constexpr int RB = 2 * D + 16;   // staged output row stride (bytes)
    constexpr int PW = 32 * RB / 4;  // floats per key block in pbuf (the staging size: pbuf stages rows too)
    __shared__ __attribute__((aligned(1024))) uint8_t qr0[RT];
    __shared__ __attribute__((aligned(1024))) uint8_t dr0[RT];
    __shared__ __attribute__((aligned(1024))) uint8_t qr1[RT];
    __shared__ __attribute__((aligned(1024))) uint8_t dr1[RT];
    __shared__ __attribute__((aligned(1024))) uint8_t qr2[RT];
    __shared__ __attribute__((aligned(1024))) uint8_t dr2[RT];
    // per tile row: -LSE log2 e, D, lo, hi (256 bytes each)
    __shared__ __attribute__((aligned(1024))) uint8_t st0[4 * BQ * 4];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[4 * BQ * 4];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[4 * BQ * 4];
    // A's weights for B: 32 per lane and key block, element e of lane l at
    // e / 4 * 256 + l * 4 + e % 4; after the loop, A's dV rows on their way out
    __shared__ __attribute__((aligned(16))) float pbuf[4 * PW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_a = wave < 4;
    const int kw = wave & 3;
    const int nbk = p.B * p.Hkv;
    const int kt_idx = blockIdx.x / nbk;     // key tiles in order: under causal masks the first are the heaviest
    const int bk = blockIdx.x % nbk;
    const int b = bk / p.Hkv, hkv = bk % p.Hkv;
    const PrefillParams m = mask_params(p);

    const int k0 = kt_idx * BK;
    const int k0w = k0 + kw * 32;
    const int key = k0w + (lane & 31);
    const bool key_ok = key < p.Nk;
    const int k_last = min(k0 + BK, p.Nk) - 1;

    const size_t kv_head = ((size_t)b * p.Hkv + hkv) * (size_t)p.Nk;
    // A: K fragments, B: V fragments.  A key past Nk reads key 0's row and
    // keeps it: its column of S is masked to -inf, so its P and dS are 0, and
    // its dK and dV rows are never stored.  Not zeroing it lets the loads stay
    // in flight while the first tile's copies are issued (the first wait is
    // the first tile's).
    bf16x8 xf[D / 16];
    load_fragment<D>((is_a ? p.k : p.v) + (kv_head + (key_ok ? key : 0)) * D, true, lane, xf);
    f32x16 acc[D / 32];  // A: dV^T, B: dK^T
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};

    int first = p.Nq, last = -1;
    if (k0 < p.Nk) query_rows_seeing(m, k0, k_last, first, last);
    const int qt_first = first / BQ;
    const int ntq = (first <= last && k0 < p.Nk) ? last / BQ - qt_first + 1 : 0;
    const int n_iter = ntq * p.group;

    DualSwizzle dz;
    dz.init(lane, kw);
    auto head_of = [&](int it) __attribute__((always_inline)) { return hkv * p.group + it / ntq; };
    auto q0_of = [&](int it) __attribute__((always_inline)) { return (qt_first + it % ntq) * BQ; };
    auto copy = [&](int it, uint8_t* qr, uint8_t* dr, uint8_t* st) __attribute__((always_inline)) {
        const size_t head_row = ((size_t)b * p.Hq + head_of(it)) * (size_t)p.Nq;
        const int q0 = q0_of(it);
        // rows past Nq read as zero
        dz.template copy8<BQ / 4>(p.q + (head_row + q0) * D, p.Nq - q0, qr, wave);
        dz.template copy8<BQ / 4>(p.dO + (head_row + q0) * D, p.Nq - q0, dr, wave);
        if (wave == 0) {
            const int nrow = min(p.Nq - q0, BQ) * 4;   // bytes of the tile's rows that exist; the rest read 0
            const void* srcs[4] = {p.ws_nl + head_row + q0, p.ws_d + head_row + q0, p.ws_lo + head_row + q0,
                                   p.ws_hi + head_row + q0};
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)srcs[a], (short)0, nrow, 0x00020000);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(st + a * BQ * 4), 4, lane * 4, 0, 0, 0);
            }
        }
    };
    // does some row of tile it see some key of this block (its keys exist)?
    auto tile_active = [&](int it, bool& full) __attribute__((always_inline)) {
        const int q0 = q0_of(it);
        const int q_end = min(q0 + BQ, p.Nq) - 1;
        int lo_a, hi_a, lo_z, hi_z;
        row_interval(m, q0, lo_a, hi_a);
        row_interval(m, q_end, lo_z, hi_z);
        full = q0 + BQ - 1 < p.Nq && k0w + 31 < p.Nk && hi_a >= k0w + 31 && (lo_z <= k0w || k0w + 31 < p.sink_end);
        return k0w < p.Nk && hi_z >= k0w && (lo_a <= k0w + 31 || k0w < p.sink_end);
    };
    float* pw = pbuf + kw * PW;

    // B: dS of the tile behind (dP in xr, statistics st) from A's weights, packed into pr
    auto b_ds = [&](const uint8_t* st, f32x16 (&xr)[2], bf16x8 (&pr)[4]) __attribute__((always_inline)) {
        const float* dd = (const float*)(st + BQ * 4);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int jb = q >> 2, r0 = 4 * (q & 3);
            const int rb = jb * 32 + 8 * (q & 3) + 4 * (lane >> 5);
            const f32x4 dd4 = *(const f32x4*)(dd + rb);
            const f32x4 pa = *(const f32x4*)(pw + q * 256 + lane * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) xr[jb][r0 + e] = pa[e] * (xr[jb][r0 + e] - dd4[e]);   // dS
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int jb = kb >> 1, h = (kb & 1) * 8;
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(xr[jb][h + 2 * e], xr[jb][h + 2 * e + 1]);
            pr[kb] = __builtin_bit_cast(bf16x8, w);
        }
    };
    // B: dK^T += Q^T dS of the tile behind (packed in pr; its Q tile qr)
    auto b_dk = [&](const uint8_t* qr, const bf16x8 (&pr)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dz.tr(qr, kb, cb), pr[kb], acc[cb], 0, 0, 0);
    };

    // The roles run loops of their own (the same copies and barriers in the
    // same order), so each role's values count against its own registers only.
    auto head = [&](int it, uint8_t* qrn, uint8_t* drn, uint8_t* stn) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        __syncthreads();   // tile it landed; A's weights of the tile behind are in LDS
        if (it + 1 < n_iter) copy(it + 1, qrn, drn, stn);
    };
    // A: tile it in ring stage (qr, dr, st); the next tile's copies go to (qrn, drn, stn)
    auto stage_a = [&](int it, const uint8_t* qr, const uint8_t* dr, const uint8_t* st, uint8_t* qrn, uint8_t* drn,
                       uint8_t* stn) __attribute__((always_inline)) {
        head(it, qrn, drn, stn);
        bool full;
        const bool active = tile_active(it, full);
        const int q0 = q0_of(it);
        f32x16 xr[2];     // S, then P
        bf16x8 pr[4];     // P packed per 16-row block
        // phase 1: S = Q K^T
        if (active) {
            xr[0] = f32x16{};
            xr[1] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
                    xr[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dz.row(qr, jb, kk), xf[kk], xr[jb], 0, 0, 0);
            order_operand_reads<D / 8, 1, 4>();
        }
        __syncthreads();   // B has read the weights of the tile behind
        // phase 2: the weights, into LDS for B; phase 3: dV^T += dO^T P
        if (active) {
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
                            const float rr = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(xr[jb][r] * sm.cap_k) + 1.f);
                            xr[jb][r] = __builtin_fmaf(-2.f * sm.cap_l2, rr, sm.cap_l2) + bias;
                            fac[jb][r] = 4.f * rr * (1.f - rr);
                        } else {
                            xr[jb][r] = __builtin_fmaf(xr[jb][r], sm.scale_l2, bias);
                            fac[jb][r] = 1.f;
                        }
                    }
            }
            const float sl = MODS ? 1.f : p.scale_log2;   // scores already in base-2 units under MODS
            if (!full) {
                // scores of invisible (row, key) pairs and of rows past Nq
                // become -inf, so their P (and B's dS) are 0
                const int32_t* rlo = (const int32_t*)(st + 2 * BQ * 4);
                const int32_t* rhi = (const int32_t*)(st + 3 * BQ * 4);
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int rb = jb * 32 + 8 * g4 + 4 * (lane >> 5);
                        const u32x4 a = *(const u32x4*)(rlo + rb);
                        const u32x4 z = *(const u32x4*)(rhi + rb);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const bool vis = q0 + rb + e < p.Nq && key <= (int32_t)z[e] &&
                                             (key >= (int32_t)a[e] || key < p.sink_end);
                            if (!vis) xr[jb][4 * g4 + e] = -__builtin_inff();
                        }
                    }
            }
            const float* nl = (const float*)st;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int rb = (q >> 2) * 32 + 8 * (q & 3) + 4 * (lane >> 5);
                const f32x4 nl4 = *(const f32x4*)(nl + rb);
                const int jb = q >> 2, r0 = 4 * (q & 3);
                f32x4 hand;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xr[jb][r0 + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(xr[jb][r0 + e], sl, nl4[e]));   // P
                    hand[e] = MODS ? xr[jb][r0 + e] * fac[jb][r0 + e] : xr[jb][r0 + e];
                }
                *(f32x4*)(pw + q * 256 + lane * 4) = hand;
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int jb = kb >> 1, h = (kb & 1) * 8;
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(xr[jb][h + 2 * e], xr[jb][h + 2 * e + 1]);
                pr[kb] = __builtin_bit_cast(bf16x8, w);
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int cb = 0; cb < D / 32; ++cb)
                    acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dz.tr(dr, kb, cb), pr[kb], acc[cb], 0, 0, 0);
        }
    };
    // B: tile it in (dr, st), the tile behind in (qrp, stp); dP of the tile
    // behind in xr, its dS packed into pr
    bool b_pending = false;   // the tile behind needs its dS and dK
    auto stage_b = [&](int it, const uint8_t* dr, const uint8_t* qrp, const uint8_t* stp, uint8_t* qrn,
                       uint8_t* drn, uint8_t* stn, f32x16 (&xr)[2], bf16x8 (&pr)[4]) __attribute__((always_inline)) {
        head(it, qrn, drn, stn);
        bool full;
        const bool active = tile_active(it, full);
        // phase 1: dS of the tile behind
        if (b_pending) b_ds(stp, xr, pr);
        __syncthreads();   // B has read the weights of the tile behind
        // phase 2: dP = dO V^T of this tile
        if (active) {
            xr[0] = f32x16{};
            xr[1] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
                    xr[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dz.row(dr, jb, kk), xf[kk], xr[jb], 0, 0, 0);
            order_operand_reads<D / 8, 1, 4>();
        }
        // phase 3: dK^T += Q^T dS of the tile behind
        if (b_pending) b_dk(qrp, pr);
        b_pending = active;
    };

    if (is_a) {
        if (n_iter > 0) {
            copy(0, qr0, dr0, st0);
            for (int it = 0; it < n_iter; it += 3) {
                stage_a(it, qr0, dr0, st0, qr1, dr1, st1);
                if (it + 1 < n_iter) stage_a(it + 1, qr1, dr1, st1, qr2, dr2, st2);
                if (it + 2 < n_iter) stage_a(it + 2, qr2, dr2, st2, qr0, dr0, st0);
            }
        }
        __syncthreads();   // A's weights of the last tile are in LDS
    } else {
        f32x16 xr[2];
        bf16x8 pr[4];
        if (n_iter > 0) {
            copy(0, qr0, dr0, st0);
            for (int it = 0; it < n_iter; it += 3) {
                stage_b(it, dr0, qr2, st2, qr1, dr1, st1, xr, pr);
                if (it + 1 < n_iter) stage_b(it + 1, dr1, qr0, st0, qr2, dr2, st2, xr, pr);
                if (it + 2 < n_iter) stage_b(it + 2, dr2, qr1, st1, qr0, dr0, st0, xr, pr);
            }
        }
        __syncthreads();   // A's weights of the last tile are in LDS
        // dS and dK of the last tile (ring stage (n_iter - 1) % 3)
        if (b_pending) {
            const int ls = (n_iter - 1) % 3;
            b_ds(ls == 0 ? st0 : (ls == 1 ? st1 : st2), xr, pr);
            b_dk(ls == 0 ? qr0 : (ls == 1 ? qr1 : qr2), pr);
        }
    }
    __syncthreads();   // every wave is done with the ring and pbuf: both stage their rows there
    if (k0w < p.Nk) {
        if (is_a) {
            store_rows_staged<D>(p.dv + (kv_head + k0w) * D, p.Nk - k0w, acc, 1.f, lane, (uint8_t*)pw);
        } else {
            uint8_t* stg = kw == 0 ? dr0 : (kw == 1 ? dr1 : (kw == 2 ? dr2 : qr0));
            store_rows_staged<D>(p.dk + (kv_head + k0w) * D, p.Nk - k0w, acc, p.scale, lane, stg);
        }
    }
}

__global__ __launch_bounds__(512, 1) void bwd_dkdv2_kernel(BackwardParams p) { bwd_dkdv2_body<false>(p); }
__global__ __launch_bounds__(512, 1) void bwd_dkdv2_mod_kernel(BackwardParams p) { bwd_dkdv2_body<true>(p); }
__global__ __launch_bounds__(256, 1) void bwd_dkdv_d64_kernel(BackwardParams p) { bwd_dkdv_body<64, false>(p); }
__global__ __launch_bounds__(256, 1) void bwd_dkdv_d64_mod_kernel(BackwardParams p) { bwd_dkdv_body<64, true>(p); }

size_t backward_workspace_bytes(int B, int Hq, int Nq) {
    const size_t rows = (size_t)B * Hq * Nq;
    return 4 * ((rows * 4 + 255) / 256) * 256;
}

int launch_backward(BackwardParams p, int d, void* ws, hipStream_t stream) {
    const size_t rows = (size_t)p.B * p.Hq * p.Nq;
    p.num_cus = device_cus();
    const bool mods = p.softcap > 0.f || p.alibi_slopes != nullptr;
    const size_t stride = ((rows * 4 + 255) / 256) * 256;
    p.ws_nl = (float*)ws;
    p.ws_d = (float*)((char*)ws + stride);
    p.ws_lo = (int32_t*)((char*)ws + 2 * stride);
    p.ws_hi = (int32_t*)((char*)ws + 3 * stride);
    const dim3 wg(256), gq(p.B * p.Hq * p.num_q_tiles), gk(p.B * p.Hkv * p.num_k_tiles);
    if (rows > 0) {
        // the dQ pass also writes every row's statistics for the passes after it
        if (d == 128) {
            if (mods) hipLaunchKernelGGL(bwd_dq_mod_kernel, gq, wg, 0, stream, p);
            else hipLaunchKernelGGL(bwd_dq_kernel, gq, wg, 0, stream, p);
        } else {
            if (mods) hipLaunchKernelGGL(bwd_dq_d64_mod_kernel, gq, wg, 0, stream, p);
            else hipLaunchKernelGGL(bwd_dq_d64_kernel, gq, wg, 0, stream, p);
        }
    }
    launch_dsink(p, stream);   // after the dQ pass (it reads D); also with no rows, where it writes 0
    if ((long long)p.B * p.Hkv * p.num_k_tiles > 0) {
        if (d == 128) {
            const dim3 wg2(512);
            if (mods) hipLaunchKernelGGL(bwd_dkdv2_mod_kernel, gk, wg2, 0, stream, p);
            else hipLaunchKernelGGL(bwd_dkdv2_kernel, gk, wg2, 0, stream, p);
        } else {
            if (mods) hipLaunchKernelGGL(bwd_dkdv_d64_mod_kernel, gk, wg, 0, stream, p);
            else hipLaunchKernelGGL(bwd_dkdv_d64_kernel, gk, wg, 0, stream, p);
        }
    }
    return 0;
}

}  // namespace xattn
