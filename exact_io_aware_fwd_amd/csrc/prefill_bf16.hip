// bf16 prefill attention forward for gfx950.
//
// One workgroup (4 waves) owns a tile of 128 query rows of one (batch, query
// head); each wave owns 32 of those rows for the whole kernel, so its softmax
// state needs no exchange with the other waves (the per-warp split of Q that
// FlashAttention-2 introduced; "Attention Is the Bottleneck", FlashAttention-2
// section).  K/V tiles of 64 keys (32 under the window and document masks at
// d = 128) stream from HBM through a double-buffered LDS ring while the Q
// tile stays in registers, and the score tile never leaves the chip
// ("FlashAttention: same math, different IO").
//
// Both contractions run on the matrix cores with v_mfma_f32_32x32x16_bf16 and
// fp32 accumulation.  They are evaluated transposed, S^T = K Q^T and
// O^T = V^T P^T, because that MFMA's accumulator layout puts one query row's
// scores in a single lane pair (lane l and lane l ^ 32): the row max needs at
// most one cross-lane exchange per tile and the per-row rescale factor is a
// per-lane scalar.  The S^T accumulator registers are exactly the P^T operand of the
// second MFMA once converted to bf16, up to a fixed permutation of the keys
// inside each 16-key block, which the V^T tile in LDS is stored with.
//
// Softmax runs in base 2: scores are scaled by scale*log2(e) with one FMA that
// also subtracts the running max, then v_exp_f32.  The division by the row sum
// happens once at the end (delayed normalisation, FlashAttention-2 section).
#include "exp2_poly.hpp"
#include "prefill_tiles.hpp"

namespace xattn {

// Softmax weights are kept relative to a stale row max until a tile's max
// exceeds it by more than 2^8; only then is the accumulator rescaled (the
// conditional rescaling of FlashAttention-4, "Attention Is the Bottleneck").
// Weights stay below 256, well inside fp32 and bf16 range, and the result is
// unchanged because O and the row sums share the same reference.
constexpr float kRescaleThreshold = 8.f;

template <int D>
struct PrefillBf16State {
    bf16x8 qf[D / 16];
    f32x16 acc[D / 32];
    float m_run;
    float l_run;   // this lane's half of the row sum of the bf16 weights: normalises O
    float l_f32;   // same sum over the unrounded fp32 weights: gives the LSE
    // the whole row's sum of the bf16 weights (every lane of the row pair)
    __device__ __forceinline__ float l_total() const { return l_run + __shfl_xor(l_run, 32); }
    __device__ __forceinline__ void init() {
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};
        m_run = -__builtin_inff();
        l_run = 0.f;
        l_f32 = 0.f;
    }
};

// Order one product's LDS operand reads against its MFMAs: the first
// AHEAD * R reads, then each MFMA followed by the next R reads, then the last
// AHEAD MFMAs.  Left to itself the compiler issues each operand read about
// two MFMAs ahead, and its latency then shows between the MFMAs; holding the
// reads this far ahead (AHEAD 4 for K, 2 for V^T, measured) cut the causal
// prefill's cycles by 5-6 %.  The V^T reads keep AHEAD 2 inside
// interleave_weights_products below; the backward's products use this order.
template <int NMFMA, int R, int AHEAD>
__device__ __forceinline__ void order_reads_ahead() {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD * R, 0);   // DS reads
#pragma unroll
    for (int i = 0; i < NMFMA - AHEAD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
#endif
}

// Order the weights-and-products part of a tile: the first V^T reads and the
// first 16-key block's weights (PRE VALU ops: exponentials, sums and bf16
// packing), then each MFMA followed by the next two V^T reads and VALU_PER
// ops of the following blocks' weights, so the exponentials of block kb+1
// issue while block kb's products run on the matrix core (measured: C2
// causal prefill 189 K -> 184 K cycles, nothing else changed).
template <int NMFMA, int PRE, int VALU_PER>
__device__ __forceinline__ void interleave_weights_products() {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);           // DS reads
    __builtin_amdgcn_sched_group_barrier(0x002, PRE, 0);         // VALU
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // one MFMA
        if (i < NMFMA - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        if (i < NMFMA - NMFMA / 4) __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER, 0);
    }
#endif
}

// (mask & a) | (~mask & b).  Written as one v_bfi_b32: the plain C form of
// this select over the 32 scores of a lane was combined by the compiler into
// three-input logic ops that read a neighbouring score's register (wrong
// results, seen in the generated code of this kernel).
__device__ __forceinline__ float bit_select(uint32_t mask, float a, float b) {
    float out;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(out) : "v"(mask), "v"(a), "v"(b));
    return out;
}

// Where a lane's MFMA operands sit in a K / V tile in LDS.
//
// PaddedTiles: rows padded to KS / VS 16-byte slots.  k / v point at this
// lane's own base; every other operand address is a compile-time offset.
template <int D>
struct PaddedTiles {
    using C = PrefillBf16Cfg<D>;
    const uint8_t* k;
    const uint8_t* v;
    // K operand: rows (lane & 31) + 32 jb, 16-byte chunk 2 kk + (lane >> 5)
    __device__ __forceinline__ const uint8_t* k_at(int jb, int kk) const { return k + jb * 32 * C::KS * 16 + kk * 32; }
    // V^T operand (two transposing reads, the second 8 rows below the first)
    __device__ __forceinline__ const uint8_t* v_at(int kb, int cb) const { return v + kb * 16 * C::VS * 16 + cb * 64; }
    static constexpr int kVHalf = 8 * C::VS * 16;
};

// SwizzledTiles (d = 128): unpadded 256-byte rows, 16-byte chunk c of row r
// stored at chunk c ^ (r % 16) in K tiles and c ^ 4 (r % 4) in V tiles.  A
// 1 KiB direct copy then covers 4 whole rows (one page of a paged cache per
// copy), and both operand reads stay free of bank conflicts: the 16 lanes of
// a K row read hit 16 different chunks, and the 4 rows x 4 chunks of a
// transposing V read land in 16 different chunks.  The lane-dependent part of
// each address is a per-lane table (8 K and 4 V offsets).
struct SwizzledTiles {
    const uint8_t* k;
    const uint8_t* v;
    int ko[8];
    int vo[4];
    __device__ __forceinline__ void init(int lane) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            ko[kk] = (lane & 31) * 256 + (((2 * kk + (lane >> 5)) ^ (lane & 15)) * 16);
        const int t = (lane >> 2) & 3, i = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
            vo[cb] = (4 * (lane >> 5) + t) * 256 + (4 * (cb ^ t) + i) * 16 + 8 * (lane & 1);
    }
    __device__ __forceinline__ const uint8_t* k_at(int jb, int kk) const { return k + jb * 32 * 256 + ko[kk]; }
    __device__ __forceinline__ const uint8_t* v_at(int kb, int cb) const { return v + kb * 16 * 256 + vo[cb]; }
    static constexpr int kVHalf = 8 * 256;
};

// S^T = K Q^T for one key tile resident in LDS (laid out as T says): NJB
// 32-key blocks (2 for the 64-key tiles, 1 for 32-key tiles), 8 MFMAs each.
template <int D, int NJB, class T>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[NJB], const PrefillBf16State<D>& st, const T& tl) {
    using C = PrefillBf16Cfg<D>;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) s[jb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::DK; ++kk)
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            const u32x4 a = *(const u32x4*)tl.k_at(jb, kk);
            s[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), st.qf[kk], s[jb], 0, 0, 0);
        }
}

// Score modifications, mask and the row max of a score tile, with the
// conditional rescale; returns the reference the weights are taken against.
// MODS: the raw q.k scores become base-2 logits here and scale_log2 becomes 1.
template <int D, bool MODS, int NJB>
__device__ __forceinline__ float prepare_tile(PrefillBf16State<D>& st, f32x16 (&s)[NJB], int n0, bool full, int lo_i,
                                              int hi_i, int sink_end, float& scale_log2, int lane, const ScoreMod& sm,
                                              int qpos) {
    using C = PrefillBf16Cfg<D>;
    // ---- score modifications: raw q.k -> base-2 logit (unit scale below).
    // Score 16 jb + r of this lane is key n0 + 4 (lane / 32) + 32 jb +
    // 8 (r / 4) + r % 4 (see the mask below).  They come before the mask, so
    // a masked key still ends at -inf.
    if constexpr (MODS) {
        const float b0 = sm.slope_l2 * (float)(n0 + 4 * (lane >> 5) - qpos);
        if (sm.cap_k != 0.f) {
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = fast_exp2(s[jb][r] * sm.cap_k);
                    const float capped = __builtin_fmaf(-2.f * sm.cap_l2, __builtin_amdgcn_rcpf(e + 1.f), sm.cap_l2);
                    s[jb][r] = capped + __builtin_fmaf(sm.slope_l2, (float)(32 * jb + 8 * (r >> 2) + (r & 3)), b0);
                }
        } else {
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[jb][r] = __builtin_fmaf(s[jb][r], sm.scale_l2,
                                              __builtin_fmaf(sm.slope_l2, (float)(32 * jb + 8 * (r >> 2) + (r & 3)), b0));
        }
        scale_log2 = 1.f;
    }
    // ---- mask, only where the tile is not fully visible to this wave
    if (!full) {
        // Score i = 16 jb + r of this lane is key base + c_i with the
        // compile-time offset c_i = 8 (i / 4) + i % 4, increasing in i.  So
        // each bound of the visible set (key <= hi_i; key >= lo_i or key <
        // sink_end) keeps a run of consecutive i, counted by below(x) =
        // #{i : c_i < x}, and the visible set is one 32-bit mask per lane.
        const int base = n0 + 4 * (lane >> 5);
        auto below = [](int x) {
            x = min(max(x, 0), 64);
            return 4 * (x >> 3) + min(x & 7, 4);
        };
        auto low_bits = [](int k) { return k >= 32 ? 0xffffffffu : (1u << k) - 1u; };
        uint32_t vis = low_bits(below(hi_i - base + 1));
        vis &= ~low_bits(below(lo_i - base)) | low_bits(below(sink_end - base));
        const float ninf = neg_inf();
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t keep = (uint32_t)((int)(vis << (31 - (16 * jb + r))) >> 31);   // bit i, sign-extended
                s[jb][r] = bit_select(keep, s[jb][r], ninf);
            }
    }
    // Row max: each lane reduces its own half of the row (two independent
    // chains, a dependent VALU op waits a second issue slot).  Weights stay
    // relative to the running max m_run unless some half-row exceeds it by
    // more than the threshold; only then are the two halves combined (the one
    // cross-lane exchange) and the accumulator rescaled to the new row max.
    float ma = neg_inf(), mb = neg_inf();
    if constexpr (NJB == 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            ma = fmaxf(ma, s[0][r]);
            mb = fmaxf(mb, s[1][r]);
        }
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            ma = fmaxf(ma, s[0][r]);
            mb = fmaxf(mb, s[0][r + 8]);
        }
    }
    const float mh = fmaxf(ma, mb) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mh > st.m_run + kRescaleThreshold)) {
        const float mt = fmaxf(mh, __shfl_xor(mh, 32));
        // A row that has still seen no key (both maxima -inf) keeps alpha = 0
        // from the 0 reference instead of exp2(-inf - -inf) = NaN; its acc and
        // sums are 0 anyway.
        const float m_new = fmaxf(st.m_run, mt);
        const float alpha = fast_exp2(st.m_run - (m_new == neg_inf() ? 0.f : m_new));
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) st.acc[cb] *= alpha;
        st.l_run *= alpha;
        st.l_f32 *= alpha;
        st.m_run = m_new;
    }
    return st.m_run == neg_inf() ? 0.f : st.m_run;
}

// Weights, P^T operands and O^T += V^T P^T, one 16-key block kb at a time.
// O is normalised by the sum of the same bf16-rounded weights the PV
// product uses, so it is an exact weighted average of V rows under those
// weights (a dot with (1, 1) adds two packed bf16 values at once); the LSE
// uses the fp32 sum, free of the weights' rounding.
//
// The V^T operand comes from the row-major V tile through two transposing
// reads (ds_read_b64_tr_b16): in each 16-lane group, source lane 4k+q
// points at 4 columns c0+4q.. of key row k, and lane i receives column
// c0+i of those 4 rows.  Rows are picked so the 8 keys a lane holds are the
// ones its P^T operand slots hold.
//
// SOFT: the first SOFT of the 8 weights a lane computes per 16-key block take
// the software 2^x (soft_exp2, FMA units), the rest v_exp_f32.
template <int D, int SOFT, int NJB, class T>
__device__ __forceinline__ void softmax_pv(PrefillBf16State<D>& st, f32x16 (&s)[NJB], const T& tl, float scale_log2,
                                           float m_use) {
    using C = PrefillBf16Cfg<D>;
    float fs[4] = {0.f, 0.f, 0.f, 0.f};
    float ps[2] = {0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2 * NJB; ++kb) {
        const int jb = kb >> 1, h = (kb & 1) * 8;
#pragma unroll
        for (int r = h; r < h + 8; ++r) {
            const float x = __builtin_fmaf(s[jb][r], scale_log2, -m_use);
            s[jb][r] = r - h < SOFT ? soft_exp2(x) : fast_exp2(x);
            fs[(r & 1) + 2 * jb] += s[jb][r];
        }
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w[e] = pack_bf16x2(s[jb][h + 2 * e], s[jb][h + 2 * e + 1]);
            ps[e & 1] = sum_bf16x2(w[e], ps[e & 1]);
        }
        const bf16x8 pf = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
            const uint8_t* vp = tl.v_at(kb, cb);
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + T::kVHalf));
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
            const u32x4 a = {lo2[0], lo2[1], hi2[0], hi2[1]};
            st.acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pf, st.acc[cb], 0, 0, 0);
        }
    }
    st.l_run += ps[0] + ps[1];
    st.l_f32 += (fs[0] + fs[1]) + (fs[2] + fs[3]);
}

// S^T = K Q^T, mask, online softmax and O^T += V^T P^T for one wave and one
// key tile resident in LDS, laid out as T says.  MODS: the scores first go
// through the score modifications sm (qpos: this lane's query position).
// SOFT: weights from the software 2^x, as in softmax_pv.  NJB: 32-key blocks
// per tile (2: 64-key tiles; 1: 32-key tiles, swizzled layout only).
template <int D, bool MODS = false, int SOFT = 0, int NJB = 2, class T>
__device__ __forceinline__ void tile_step(PrefillBf16State<D>& st, const T& tl, int n0,
                                          bool full, int lo_i, int hi_i, int sink_end, float scale_log2, int lane,
                                          const ScoreMod& sm = ScoreMod{}, int qpos = 0) {
    using C = PrefillBf16Cfg<D>;
    f32x16 s[NJB];
    qk_tile<D, NJB>(s, st, tl);
    order_reads_ahead<NJB * C::DK, 1, 4>();
    const float m_use = prepare_tile<D, MODS, NJB>(st, s, n0, full, lo_i, hi_i, sink_end, scale_log2, lane, sm, qpos);
    softmax_pv<D, SOFT, NJB>(st, s, tl, scale_log2, m_use);
    interleave_weights_products<2 * NJB * C::CB, 40, 6>();
}

// SINKS: the window mask keeps sink tokens visible (the second key interval);
// without it the tile loop and the mask compile to the one-interval form.
// MODS: the score modifications are on (a kernel of its own, so the plain
// kernel's code does not change).
// Issue this wave's copies of one ROWS-key tile (64 or 32) in the SwizzledTiles layout
// (d = 128) from K or V rows that follow each other in memory: copy jj fills
// tile rows 16 jj + 4 wave .. + 3, and lane l brings the source chunk that
// lands swizzled at 16-byte slot l % 16 of row 4 wave + l / 16 (`lane_off`,
// the same for every tile; jj only moves the source by 16 rows).  The buffer
// resource starts at key n0 and covers the keys that exist, so rows past Nk
// read as zeros.
template <int ROWS = 64>
__device__ __forceinline__ void load_swz_tile_async(const uint16_t* __restrict__ base, int n0, int Nk, uint8_t* lds,
                                                    uint32_t lane_off, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int D = 128;
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + (size_t)n0 * D), (short)0, (int)tile_range_bytes<D>(Nk - n0, ROWS), 0x00020000);
#pragma unroll
    for (int jj = 0; jj < ROWS / 16; ++jj)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (4 * jj + wave) * 1024), 16, lane_off,
                                                 jj * 16 * D * 2, 0, 0);
#endif
}

template <int D, bool SINKS, bool MODS, int SOFT = 0, int NJB = 2>
__device__ __forceinline__ void prefill_bf16_body(PrefillParams p) {
    using C = PrefillBf16Cfg<D>;
    constexpr int BNK = NJB * 32;   // keys per K/V tile
    static_assert(NJB == 2 || D == 128, "32-key tiles exist only in the swizzled layout (d = 128)");
    // Head dim 128 keeps its K/V tiles unpadded and swizzled (16 KiB each,
    // 4 + 4 copies per wave and tile); head dim 64 keeps the padded tiles.
    constexpr bool SWZ = D == 128;
    constexpr int KT = SWZ ? BNK * D * 2 : C::KTILE;
    constexpr int VT = SWZ ? BNK * D * 2 : C::VTILE;
    const int sink_end = SINKS ? p.sink_end : 0;
    // two stages of the K/V ring, as separate arrays so each access names its buffer
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[KT];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[VT];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[KT];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[VT];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, lets loads use scalar control
    const int nbk = p.B * p.Hkv;
    int bk, unit, g;
    decode_work(blockIdx.x, nbk, p.q_tile_pairs > 0 ? p.q_tile_pairs : p.num_q_tiles, p.group, bk, unit, g);
    const int b = bk / p.Hkv, hkv = bk % p.Hkv, hq = hkv * p.group + g;
    const ScoreMod sm = MODS ? make_score_mod(p.scale_log2, p.softcap, p.alibi_slopes, hq) : ScoreMod{};

    const uint16_t* __restrict__ qg = (const uint16_t*)p.q;
    const uint16_t* __restrict__ kg_ = (const uint16_t*)p.k + ((size_t)b * p.Hkv + hkv) * (size_t)p.Nk * D;
    const uint16_t* __restrict__ vg_ = (const uint16_t*)p.v + ((size_t)b * p.Hkv + hkv) * (size_t)p.Nk * D;

    // Under a causal mask a row tile's work grows with its index.  A
    // workgroup then takes two row tiles, a heavy one and its mirror (tiles
    // num_q_tiles-1-u and u), so every workgroup does about the same work and
    // the grid drains evenly instead of ending on a round of light tiles.
    // Pairs go in ascending u, so an odd middle tile (alone) comes last.
    const bool paired = p.q_tile_pairs > 0;
    const int u = paired ? p.q_tile_pairs - 1 - unit : unit;
    const int nsub = paired && p.num_q_tiles - 1 - u != u ? 2 : 1;
    for (int sub = 0; sub < nsub; ++sub) {
        const int qt = paired && sub == 0 ? p.num_q_tiles - 1 - u : u;
        if (sub > 0) __syncthreads();   // every wave is done with the ring before it is refilled
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

        PrefillBf16State<D> st;
        // Q fragment: MFMA B operand, column = query row (lane & 31), k slots
        // (lane >> 5) * 8 .. +8 of every 16-wide step of the head dim.
        {
            const uint16_t* qrow = qg + (((size_t)b * p.Hq + hq) * (size_t)p.Nq + (row_ok ? row : 0)) * D;
    #pragma unroll
            for (int kk = 0; kk < C::DK; ++kk) {
                u32x4 w = row_ok ? *(const u32x4*)(qrow + kk * 16 + (lane >> 5) * 8) : u32x4{0, 0, 0, 0};
                st.qf[kk] = __builtin_bit_cast(bf16x8, w);
            }
        }
        st.init();   // running row max -inf (base-2 scaled units), sums and O 0

        const TileRange tr = tile_range(lo_wg, hi_wg, sink_end, BNK);

        uint32_t koff[C::KLW], voff[C::VLW];
        if constexpr (!SWZ) {
            tile_src_offsets<D, C::KS, C::KLOADS>(koff, wave, lane);
            tile_src_offsets<D, C::VS, C::VLOADS>(voff, wave, lane);
        }
        // this lane's operand bases inside a K / V tile (padded layout)
        const int kbase = (lane & 31) * C::KS * 16 + (lane >> 5) * 16;
        const int vbase = (4 * (lane >> 5) + ((lane >> 2) & 3)) * C::VS * 16 + (((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2;
        // swizzled layout: this lane's copy source offsets and operand offsets
        const int rip = 4 * wave + (lane >> 4);
        [[maybe_unused]] const uint32_t kso = (uint32_t)(rip * 256 + (((lane & 15) ^ rip) * 16));
        [[maybe_unused]] const uint32_t vso = (uint32_t)(rip * 256 + (((lane & 15) ^ (4 * ((lane >> 4) & 3))) * 16));
        SwizzledTiles stl;
        if constexpr (SWZ) stl.init(lane);
        auto copy_tile = [&](int t, uint8_t* kd, uint8_t* vd) __attribute__((always_inline)) {
            if constexpr (SWZ) {
                load_swz_tile_async<BNK>(kg_, t * BNK, p.Nk, kd, kso, wave);
                load_swz_tile_async<BNK>(vg_, t * BNK, p.Nk, vd, vso, wave);
            } else {
                load_tile_async<D, C::KS, C::KLOADS>(kg_, t * C::BN, p.Nk, kd, koff, wave);
                load_tile_async<D, C::VS, C::VLOADS>(vg_, t * C::BN, p.Nk, vd, voff, wave);
            }
        };

        // One stage of the ring: wait for this tile's copies, make them visible to
        // every wave (which also proves every wave is done with the other stage),
        // start copying the next tile into the other stage, then compute.
        // Iteration it runs tile tile_of(tr, it).
        auto stage = [&](int it, const uint8_t* kc, const uint8_t* vc, uint8_t* kn, uint8_t* vn) {
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of tile t landed
            __syncthreads();
            // Two workgroups share each CU, and on a SIMD the older wave wins
            // the issue arbitration when priorities tie.  With one round of
            // workgroups (C2) the second-dispatched half then ran 35 % slower
            // per tile and ended about 14 us after the first half (workgroup
            // timestamps).  Handing the higher priority to the two halves in
            // turn, tile by tile, evens them out: C2 181 K -> 174 K cycles.
            // The phase is the dispatch round (workgroups num_cus apart share
            // a CU first), which for C2 is the grid's half; for the
            // multi-round configs it took C3b from 167-171 to 164-165 us.
            if (((it + (int)blockIdx.x / p.num_cus) & 1) != 0) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
            // (issuing these copies one or two at a time between the S^T
            // products, or after them, was 3-6 % slower than this burst)
            if (it + 1 < tr.n) copy_tile(tile_of(tr, it + 1), kn, vn);
            const int n0 = tile_of(tr, it) * BNK;
            const bool active = wave_has_rows && n0 <= hi_w_last && (n0 + BNK - 1 >= lo_w_first || n0 < sink_end);
            if (active) {
                const bool full = n0 + BNK - 1 <= hi_w_first && (n0 >= lo_w_last || n0 + BNK - 1 < sink_end);
                if constexpr (SWZ) {
                    stl.k = kc;
                    stl.v = vc;
                    tile_step<D, MODS, SOFT, NJB>(st, stl, n0, full, lo_i, hi_i, sink_end, p.scale_log2, lane, sm,
                                             row + p.Nk - p.Nq);
                } else {
                    tile_step<D, MODS>(st, PaddedTiles<D>{kc + kbase, vc + vbase}, n0, full, lo_i, hi_i, sink_end,
                                       p.scale_log2, lane, sm, row + p.Nk - p.Nq);
                }
            }
        };

        if (tr.n > 0) {
            copy_tile(tile_of(tr, 0), k_lds0, v_lds0);
            for (int it = 0; it < tr.n; it += 2) {
                stage(it, k_lds0, v_lds0, k_lds1, v_lds1);
                if (it + 1 < tr.n) stage(it + 1, k_lds1, v_lds1, k_lds0, v_lds0);
            }
        }
        f32x16* acc = st.acc;
        const float lf_tot = st.l_f32 + __shfl_xor(st.l_f32, 32);

        // ---- epilogue: O = acc / l once, LSE in natural log (with the sink, if any)
        const float l_tot = st.l_total();
        if (row_ok) {
            const float s2 = p.sink_logits != nullptr ? p.sink_logits[hq] * kLog2e : neg_inf();
            float inv, lse_row;
            finish_row(st.m_run, l_tot, lf_tot, s2, inv, lse_row);
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
            if (p.lse != nullptr && lane < 32) p.lse[((size_t)b * p.Hq + hq) * (size_t)p.Nq + row] = lse_row;
        }
    }
}

template <int D, bool SINKS>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(PrefillParams p) {
    prefill_bf16_body<D, SINKS, false>(p);
}

template <int D, bool SINKS>
__global__ __launch_bounds__(256, 2) void prefill_bf16_mod_kernel(PrefillParams p) {
    prefill_bf16_body<D, SINKS, true>(p);
}

// d = 128 with 32-key K/V tiles, for the sliding-window and document masks.
// Under those masks a wave's visible keys start and end inside a tile at both
// ends of its range, and the finer tiles compute fewer masked-off scores
// (window 1024 at 8192 keys and the 32768-key document mask: about 2.5 %
// faster than the 64-key tiles, measured alternately on one GPU).  Causal
// rows end inside a tile only at the diagonal, where the 64-key tiles'
// fewer barriers and copies per key win (the 2048-key causal config about
// 1-3 % slower with 32-key tiles).  8 KiB per K or V tile, 162 registers.
template <bool SINKS>
__global__ __launch_bounds__(256, 2) void prefill_bf16_k32_kernel(PrefillParams p) {
    prefill_bf16_body<128, SINKS, false, 0, 1>(p);
}

// d = 128 with SOFT of each lane's 8 weights per 16-key block from the
// software 2^x (kernels of their own, so the plain kernel's code does not
// change)
template <bool SINKS, int SOFT>
__global__ __launch_bounds__(256, 2) void prefill_bf16_soft_kernel(PrefillParams p) {
    prefill_bf16_body<128, SINKS, false, SOFT>(p);
}

// ------------------------------------------------------------------------
// Chunked prefill over the paged KV cache.  The tile compute is tile_step
// above; what changes is where rows come from.  Query rows are the chunk's
// tokens (token-major), and a 64-key K/V tile is four 16-token pages that
// the block table scatters over the page pool.  Rows at or past the
// sequence's end must read as zeros, so a page tail's contents (any bit
// pattern, NaN included) never reach P V: their keys are masked and their
// values are 0.  Head dim 128 uses page-aligned tiles (paged_prefill_swz_kernel
// below).  Head dim 64 keeps the padded tiles: the copies gather rows with
// per-lane 64-bit addresses (global_load_lds_dwordx4: lane l's 16 bytes still
// land at LDS base + 16 l), and rows past the end read this all-zero row.
__device__ __attribute__((aligned(16))) uint16_t kZeroRow[128];

// (row, chunk) of the padded tile layout that each of this wave's direct
// loads fills for this lane (see tile_src_offsets), packed as row << 8 | chunk.
template <int D, int S, int NL>
__device__ __forceinline__ void tile_rows_chunks(uint32_t (&rc)[(NL + 3) / 4], int wave, int lane) {
#pragma unroll
    for (int j = 0; j < (NL + 3) / 4; ++j) {
        const int slot = (wave + 4 * j) * 64 + lane;
        const int r = slot / S;
        int c = slot % S;
        c = c < D / 8 ? c : D / 8 - 1;
        rc[j] = (uint32_t)((r << 8) | c);
    }
}

// Issue this wave's copies of one 64-key tile.  pb0..pb3: element offsets in
// the page pool of the tile's four pages for this KV head; `rows` = keys of
// the tile that exist (rows at or past it read the zero row).
template <int D, int NL>
__device__ __forceinline__ void load_paged_tile_async(const uint16_t* __restrict__ pool, size_t pb0, size_t pb1,
                                                      size_t pb2, size_t pb3, int rows, uint8_t* lds,
                                                      const uint32_t (&rc)[(NL + 3) / 4], int wave) {
#pragma unroll
    for (int j = 0; j < (NL + 3) / 4; ++j) {
        const int blk = wave + 4 * j;
        if (NL % 4 == 0 || blk < NL) {
            const int r = (int)(rc[j] >> 8), c = (int)(rc[j] & 255);
            const size_t pb = r < 32 ? (r < 16 ? pb0 : pb1) : (r < 48 ? pb2 : pb3);
            const uint16_t* src = r < rows ? pool + pb + (size_t)((r & 15) * D + c * 8) : kZeroRow + c * 8;
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(lds + blk * 1024), 16, 0, 0);
        }
    }
}

// Sequence of work slot `slot`: sequences sorted by their work, heaviest
// first.  Workgroups are issued in slot order on every die, so the longest
// chunks start first and the grid does not end on one long sequence
// (longest-processing-time-first order; on 16 chunks of 256-2048 tokens over
// 88,889 cached tokens, 1.5-3 % faster than index order, with
// identical results).  Work = the visible (query, key) pairs of a causal chunk,
// nq (L - (nq - 1) / 2).  Ties keep index order.  Every thread of the
// workgroup calls this; beyond kSortSeqs sequences the index order stays.
constexpr int kSortSeqs = 256;
__device__ __forceinline__ int seq_by_work(const PagedPrefillParams& pp, int slot) {
    __shared__ float work_s[kSortSeqs];
    __shared__ int order_s[kSortSeqs];
    const int S = pp.num_seqs;
    if (S > kSortSeqs) return slot;
    const int t = threadIdx.x;
    if (t < S) {
        const float nq = (float)(pp.q_offsets[t + 1] - pp.q_offsets[t]);
        work_s[t] = nq * ((float)pp.seq_lens[t] - 0.5f * (nq - 1.f));
    }
    __syncthreads();
    if (t < S) {
        const float w = work_s[t];
        int rank = 0;   // sequences ahead of t
        for (int u = 0; u < S; ++u) {
            const float x = work_s[u];
            rank += (x > w || (x == w && u < t)) ? 1 : 0;
        }
        order_s[rank] = t;
    }
    __syncthreads();
    return order_s[slot];
}

template <int D, bool SINKS, bool MODS>
__device__ __forceinline__ void paged_prefill_bf16_body(PagedPrefillParams pp) {
    using C = PrefillBf16Cfg<D>;
    const int sink_end = SINKS ? pp.sink_end : 0;
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[C::KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[C::VTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[C::KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[C::VTILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bk, qt, g;
    decode_work_pair_major(blockIdx.x, pp.num_seqs * pp.Hkv, pp.num_q_tiles, pp.group, bk, qt, g);
    const int seq = __builtin_amdgcn_readfirstlane(seq_by_work(pp, bk / pp.Hkv));
    const int hkv = bk % pp.Hkv, hq = hkv * pp.group + g;
    const ScoreMod sm = MODS ? make_score_mod(pp.scale_log2, pp.softcap, pp.alibi_slopes, hq) : ScoreMod{};
    const int q0 = pp.q_offsets[seq];
    const int nq = pp.q_offsets[seq + 1] - q0;   // chunk length
    const int L = min(max(pp.seq_lens[seq], 0), pp.max_len);   // cached keys, the chunk included
    const int r0 = qt * C::BM;
    if (r0 >= nq) return;                        // whole workgroup: this chunk is shorter

    // the sequence as one attention problem: Nq = chunk, Nk = cache length,
    // bottom-right alignment (row_interval puts query i at i + Nk - Nq)
    PrefillParams p;
    p.Nq = nq;
    p.Nk = L;
    p.mask_kind = pp.mask_kind;
    p.window = pp.window;
    p.doc_offsets = nullptr;
    p.num_docs = 0;
    p.sink_end = sink_end;
    p.q_tile_pairs = 0;

    const int r_last = min(r0 + C::BM, nq) - 1;
    const int w0 = r0 + wave * 32;
    const int w_last = min(w0 + 31, nq - 1);
    const int row = w0 + (lane & 31);
    const bool row_ok = row < nq;

    int lo_i, hi_i;
    row_interval(p, row, lo_i, hi_i);
    int lo_wg, tmp, hi_wg;
    row_interval(p, r0, lo_wg, tmp);
    row_interval(p, r_last, tmp, hi_wg);
    int lo_w_first, hi_w_first, lo_w_last, hi_w_last;
    row_interval(p, w0, lo_w_first, hi_w_first);
    row_interval(p, w_last, lo_w_last, hi_w_last);
    const bool wave_has_rows = w0 < nq;

    const size_t row_stride = (size_t)pp.Hq * D;   // token-major rows
    PrefillBf16State<D> st;
    {
        const uint16_t* qrow = pp.q + (size_t)(q0 + (row_ok ? row : 0)) * row_stride + (size_t)hq * D;
#pragma unroll
        for (int kk = 0; kk < C::DK; ++kk) {
            u32x4 w = row_ok ? *(const u32x4*)(qrow + kk * 16 + (lane >> 5) * 8) : u32x4{0, 0, 0, 0};
            st.qf[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }
    st.init();

    const TileRange tr = tile_range(lo_wg, hi_wg, sink_end, C::BN);

    uint32_t krc[C::KLW], vrc[C::VLW];
    tile_rows_chunks<D, C::KS, C::KLOADS>(krc, wave, lane);
    tile_rows_chunks<D, C::VS, C::VLOADS>(vrc, wave, lane);
    const int kbase = (lane & 31) * C::KS * 16 + (lane >> 5) * 16;
    const int vbase = (4 * (lane >> 5) + ((lane >> 2) & 3)) * C::VS * 16 + (((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2;

    const int32_t* bt = pp.block_table + (size_t)seq * pp.max_pages;
    const int last_page = max((L + 15) / 16 - 1, 0);
    const size_t head_off = (size_t)hkv * 16 * D;
    const size_t page_elems = (size_t)pp.Hkv * 16 * D;
    // Block-table entries of a tile's four pages.  Indices past the
    // sequence's last page are clamped to it (those rows read the zero row,
    // so the entry is never used), which keeps every read inside the table.
    struct Pages { int32_t e0, e1, e2, e3; };
    auto entries = [&](int t) __attribute__((always_inline)) {
        const int lp = t * (C::BN / 16);
        Pages pg;
        pg.e0 = bt[min(lp + 0, last_page)];
        pg.e1 = bt[min(lp + 1, last_page)];
        pg.e2 = bt[min(lp + 2, last_page)];
        pg.e3 = bt[min(lp + 3, last_page)];
        return pg;
    };
    auto copy_tile = [&](int t, const Pages& pg, uint8_t* kd, uint8_t* vd) __attribute__((always_inline)) {
        const size_t pb0 = (size_t)__builtin_amdgcn_readfirstlane(pg.e0) * page_elems + head_off;
        const size_t pb1 = (size_t)__builtin_amdgcn_readfirstlane(pg.e1) * page_elems + head_off;
        const size_t pb2 = (size_t)__builtin_amdgcn_readfirstlane(pg.e2) * page_elems + head_off;
        const size_t pb3 = (size_t)__builtin_amdgcn_readfirstlane(pg.e3) * page_elems + head_off;
        const int rows = L - t * C::BN;
        load_paged_tile_async<D, C::KLOADS>(pp.k_pages, pb0, pb1, pb2, pb3, rows, kd, krc, wave);
        load_paged_tile_async<D, C::VLOADS>(pp.v_pages, pb0, pb1, pb2, pb3, rows, vd, vrc, wave);
    };

    // Stage it: wait for its tile's copies (and the next tile's block-table
    // entries, read one stage ahead so their latency hides under a tile of
    // compute), copy the next tile, read the entries of the one after, compute.
    Pages next;
    auto stage = [&](int it, const uint8_t* kc, const uint8_t* vc, uint8_t* kn, uint8_t* vn) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of this tile landed
        __syncthreads();
        if (it + 1 < tr.n) {
            copy_tile(tile_of(tr, it + 1), next, kn, vn);
            if (it + 2 < tr.n) next = entries(tile_of(tr, it + 2));
        }
        const int n0 = tile_of(tr, it) * C::BN;
        const bool active = wave_has_rows && n0 <= hi_w_last && (n0 + C::BN - 1 >= lo_w_first || n0 < sink_end);
        if (active) {
            const bool full = n0 + C::BN - 1 <= hi_w_first && (n0 >= lo_w_last || n0 + C::BN - 1 < sink_end);
            tile_step<D, MODS>(st, PaddedTiles<D>{kc + kbase, vc + vbase}, n0, full, lo_i, hi_i, sink_end,
                               pp.scale_log2, lane, sm, row + L - nq);
        }
    };

    if (tr.n > 0) {
        const int t0 = tile_of(tr, 0);
        copy_tile(t0, entries(t0), k_lds0, v_lds0);
        if (tr.n > 1) next = entries(tile_of(tr, 1));
        for (int it = 0; it < tr.n; it += 2) {
            stage(it, k_lds0, v_lds0, k_lds1, v_lds1);
            if (it + 1 < tr.n) stage(it + 1, k_lds1, v_lds1, k_lds0, v_lds0);
        }
    }
    const float lf_tot = st.l_f32 + __shfl_xor(st.l_f32, 32);
    const float l_tot = st.l_total();
    if (row_ok) {
        const float s2 = pp.sink_logits != nullptr ? pp.sink_logits[hq] * kLog2e : neg_inf();
        float inv, lse_row;
        finish_row(st.m_run, l_tot, lf_tot, s2, inv, lse_row);
        uint16_t* orow = pp.o + (size_t)(q0 + row) * row_stride + (size_t)hq * D;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                u32x2 w;
                w[0] = pack_bf16x2(st.acc[cb][4 * gq + 0] * inv, st.acc[cb][4 * gq + 1] * inv);
                w[1] = pack_bf16x2(st.acc[cb][4 * gq + 2] * inv, st.acc[cb][4 * gq + 3] * inv);
                *(u32x2*)(orow + cb * 32 + 8 * gq + 4 * (lane >> 5)) = w;
            }
        if (pp.lse != nullptr && lane < 32)
            pp.lse[(size_t)(q0 + row) * pp.Hq + hq] = lse_row;
    }
}

template <int D, bool SINKS>
__global__ __launch_bounds__(256, 2) void paged_prefill_bf16_kernel(PagedPrefillParams pp) {
    paged_prefill_bf16_body<D, SINKS, false>(pp);
}

template <int D, bool SINKS>
__global__ __launch_bounds__(256, 2) void paged_prefill_bf16_mod_kernel(PagedPrefillParams pp) {
    paged_prefill_bf16_body<D, SINKS, true>(pp);
}

// Chunked prefill at d = 128 with page-aligned tiles (SwizzledTiles): each
// 1 KiB copy reads 4 rows of one page through a buffer resource made for that
// page, whose range ends at the sequence's last key, so rows past it read as
// zero in hardware and a lane's source offset is the same for every tile.
// (The padded layout's copies cross page boundaries and needed per-lane
// 64-bit page selects and zero-row selects: about 170 VALU instructions per
// tile and wave.)
template <bool SINKS, bool MODS>
__device__ __forceinline__ void paged_prefill_swz_body(PagedPrefillParams pp) {
    constexpr int D = 128;
    using C = PrefillBf16Cfg<D>;
    constexpr int TILE = C::BN * D * 2;   // 16 KiB
    const int sink_end = SINKS ? pp.sink_end : 0;
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bk, qt, g;
    decode_work_pair_major(blockIdx.x, pp.num_seqs * pp.Hkv, pp.num_q_tiles, pp.group, bk, qt, g);
    const int seq = __builtin_amdgcn_readfirstlane(seq_by_work(pp, bk / pp.Hkv));
    const int hkv = bk % pp.Hkv, hq = hkv * pp.group + g;
    const ScoreMod sm = MODS ? make_score_mod(pp.scale_log2, pp.softcap, pp.alibi_slopes, hq) : ScoreMod{};
    // per-sequence values, made wave-uniform so everything built from them
    // (tile ranges, the per-page buffer resources) stays in scalar registers
    const int q0 = __builtin_amdgcn_readfirstlane(pp.q_offsets[seq]);
    const int nq = __builtin_amdgcn_readfirstlane(pp.q_offsets[seq + 1]) - q0;   // chunk length
    const int L = __builtin_amdgcn_readfirstlane(min(max(pp.seq_lens[seq], 0), pp.max_len));   // cached keys, the chunk included
    const int r0 = qt * C::BM;
    if (r0 >= nq) return;                        // whole workgroup: this chunk is shorter

    PrefillParams p;
    p.Nq = nq;
    p.Nk = L;
    p.mask_kind = pp.mask_kind;
    p.window = pp.window;
    p.doc_offsets = nullptr;
    p.num_docs = 0;
    p.sink_end = sink_end;
    p.q_tile_pairs = 0;

    const int r_last = min(r0 + C::BM, nq) - 1;
    const int w0 = r0 + wave * 32;
    const int w_last = min(w0 + 31, nq - 1);
    const int row = w0 + (lane & 31);
    const bool row_ok = row < nq;

    int lo_i, hi_i;
    row_interval(p, row, lo_i, hi_i);
    int lo_wg, tmp, hi_wg;
    row_interval(p, r0, lo_wg, tmp);
    row_interval(p, r_last, tmp, hi_wg);
    int lo_w_first, hi_w_first, lo_w_last, hi_w_last;
    row_interval(p, w0, lo_w_first, hi_w_first);
    row_interval(p, w_last, lo_w_last, hi_w_last);
    const bool wave_has_rows = w0 < nq;

    const size_t row_stride = (size_t)pp.Hq * D;   // token-major rows
    PrefillBf16State<D> st;
    {
        const uint16_t* qrow = pp.q + (size_t)(q0 + (row_ok ? row : 0)) * row_stride + (size_t)hq * D;
#pragma unroll
        for (int kk = 0; kk < C::DK; ++kk) {
            u32x4 w = row_ok ? *(const u32x4*)(qrow + kk * 16 + (lane >> 5) * 8) : u32x4{0, 0, 0, 0};
            st.qf[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }
    st.init();

    const TileRange tr = tile_range(lo_wg, hi_wg, sink_end, C::BN);

    // Copy jj (0..3) of this wave fills tile rows 16 jj + 4 wave .. + 3, i.e.
    // rows 4 wave .. + 3 of the tile's page jj; lane l brings physical chunk
    // l % 16 of row 4 wave + l / 16, which holds the swizzled logical chunk.
    const int rip = 4 * wave + (lane >> 4);
    [[maybe_unused]] const uint32_t kvo = (uint32_t)(rip * 256 + (((lane & 15) ^ rip) * 16));
    [[maybe_unused]] const uint32_t vvo = (uint32_t)(rip * 256 + (((lane & 15) ^ (4 * ((lane >> 4) & 3))) * 16));
    SwizzledTiles tl;
    tl.init(lane);

    const int32_t* bt = pp.block_table + (size_t)seq * pp.max_pages;
    const int last_page = max((L + 15) / 16 - 1, 0);
    // this KV head's rows in page 0 of the pool, and the bytes from one page
    // to the next (a 32-bit count: Hkv * 16 rows * 256 bytes)
    [[maybe_unused]] const uint8_t* kpool = (const uint8_t*)(pp.k_pages + (size_t)hkv * 16 * D);
    [[maybe_unused]] const uint8_t* vpool = (const uint8_t*)(pp.v_pages + (size_t)hkv * 16 * D);
    [[maybe_unused]] const uint32_t page_bytes = (uint32_t)pp.Hkv * (16u * D * 2u);
    struct Pages { int32_t e0, e1, e2, e3; };
    auto entries = [&](int t) __attribute__((always_inline)) {
        const int lp = t * (C::BN / 16);
        Pages pg;
        pg.e0 = bt[min(lp + 0, last_page)];
        pg.e1 = bt[min(lp + 1, last_page)];
        pg.e2 = bt[min(lp + 2, last_page)];
        pg.e3 = bt[min(lp + 3, last_page)];
        return pg;
    };
    // Page entries are valid page indices (non-negative), so a page's byte
    // offset is one unsigned 32 x 32 -> 64-bit product.  A tile whose 64 keys
    // all exist (every tile but a sequence's last) takes whole-page ranges;
    // only the last tile clamps each page's range to its rows that exist.
    auto copy_pages = [&](const int32_t (&e)[4], const int (&rows)[4], uint8_t* kd, uint8_t* vd)
        __attribute__((always_inline)) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const uint64_t off = (uint64_t)(uint32_t)e[jj] * page_bytes;
            __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kpool + off), (short)0, rows[jj] * D * 2, 0x00020000);
            __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vpool + off), (short)0, rows[jj] * D * 2, 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kd + (4 * jj + wave) * 1024), 16, kvo, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vd + (4 * jj + wave) * 1024), 16, vvo, 0, 0, 0);
        }
#endif
    };
    auto copy_tile = [&](int t, const Pages& pg, uint8_t* kd, uint8_t* vd) __attribute__((always_inline)) {
#if defined(__HIP_DEVICE_COMPILE__)
        const int32_t e[4] = {__builtin_amdgcn_readfirstlane(pg.e0), __builtin_amdgcn_readfirstlane(pg.e1),
                              __builtin_amdgcn_readfirstlane(pg.e2), __builtin_amdgcn_readfirstlane(pg.e3)};
        const int left = L - t * C::BN;   // keys from this tile's first to the sequence's end (uniform)
        if (left >= C::BN) {
            const int rows[4] = {16, 16, 16, 16};
            copy_pages(e, rows, kd, vd);
        } else {
            // rows of each page that exist (uniform, so the resources stay scalar)
            int rows[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) rows[jj] = __builtin_amdgcn_readfirstlane(min(max(left - 16 * jj, 0), 16));
            copy_pages(e, rows, kd, vd);
        }
#endif
    };

    Pages next;
    auto stage = [&](int it, const uint8_t* kc, const uint8_t* vc, uint8_t* kn, uint8_t* vn) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of this tile landed
        __syncthreads();
        if (it + 1 < tr.n) {
            copy_tile(tile_of(tr, it + 1), next, kn, vn);
            if (it + 2 < tr.n) next = entries(tile_of(tr, it + 2));
        }
        const int n0 = tile_of(tr, it) * C::BN;
        const bool active = wave_has_rows && n0 <= hi_w_last && (n0 + C::BN - 1 >= lo_w_first || n0 < sink_end);
        if (active) {
            const bool full = n0 + C::BN - 1 <= hi_w_first && (n0 >= lo_w_last || n0 + C::BN - 1 < sink_end);
            tl.k = kc;
            tl.v = vc;
            tile_step<D, MODS>(st, tl, n0, full, lo_i, hi_i, sink_end, pp.scale_log2, lane, sm, row + L - nq);
        }
    };

    if (tr.n > 0) {
        const int t0 = tile_of(tr, 0);
        copy_tile(t0, entries(t0), k_lds0, v_lds0);
        if (tr.n > 1) next = entries(tile_of(tr, 1));
        for (int it = 0; it < tr.n; it += 2) {
            stage(it, k_lds0, v_lds0, k_lds1, v_lds1);
            if (it + 1 < tr.n) stage(it + 1, k_lds1, v_lds1, k_lds0, v_lds0);
        }
    }
    const float lf_tot = st.l_f32 + __shfl_xor(st.l_f32, 32);
    const float l_tot = st.l_total();
    if (row_ok) {
        const float s2 = pp.sink_logits != nullptr ? pp.sink_logits[hq] * kLog2e : neg_inf();
        float inv, lse_row;
        finish_row(st.m_run, l_tot, lf_tot, s2, inv, lse_row);
        uint16_t* orow = pp.o + (size_t)(q0 + row) * row_stride + (size_t)hq * D;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                u32x2 w;
                w[0] = pack_bf16x2(st.acc[cb][4 * gq + 0] * inv, st.acc[cb][4 * gq + 1] * inv);
                w[1] = pack_bf16x2(st.acc[cb][4 * gq + 2] * inv, st.acc[cb][4 * gq + 3] * inv);
                *(u32x2*)(orow + cb * 32 + 8 * gq + 4 * (lane >> 5)) = w;
            }
        if (pp.lse != nullptr && lane < 32)
            pp.lse[(size_t)(q0 + row) * pp.Hq + hq] = lse_row;
    }
}

template <bool SINKS>
__global__ __launch_bounds__(256, 2) void paged_prefill_swz_kernel(PagedPrefillParams pp) {
    paged_prefill_swz_body<SINKS, false>(pp);
}

template <bool SINKS>
__global__ __launch_bounds__(256, 2) void paged_prefill_swz_mod_kernel(PagedPrefillParams pp) {
    paged_prefill_swz_body<SINKS, true>(pp);
}

int launch_paged_prefill_bf16(const PagedPrefillParams& p, int d, hipStream_t stream) {
    const int blocks = p.num_seqs * p.Hq * p.num_q_tiles;
    const bool sinks = p.sink_end > 0;
    const bool mods = p.softcap > 0.f || p.alibi_slopes != nullptr;
    const dim3 g(blocks), wg(256);
    if (d == 128) {
        if (mods) {
            if (sinks) hipLaunchKernelGGL(HIP_KERNEL_NAME(paged_prefill_swz_mod_kernel<true>), g, wg, 0, stream, p);
            else hipLaunchKernelGGL(HIP_KERNEL_NAME(paged_prefill_swz_mod_kernel<false>), g, wg, 0, stream, p);
        } else {
            if (sinks) hipLaunchKernelGGL(HIP_KERNEL_NAME(paged_prefill_swz_kernel<true>), g, wg, 0, stream, p);
            else hipLaunchKernelGGL(HIP_KERNEL_NAME(paged_prefill_swz_kernel<false>), g, wg, 0, stream, p);
        }
    } else {
        if (mods) {
            if (sinks) hipLaunchKernelGGL(HIP_KERNEL_NAME(paged_prefill_bf16_mod_kernel<64, true>), g, wg, 0, stream, p);
            else hipLaunchKernelGGL(HIP_KERNEL_NAME(paged_prefill_bf16_mod_kernel<64, false>), g, wg, 0, stream, p);
        } else {
            if (sinks) hipLaunchKernelGGL(HIP_KERNEL_NAME(paged_prefill_bf16_kernel<64, true>), g, wg, 0, stream, p);
            else hipLaunchKernelGGL(HIP_KERNEL_NAME(paged_prefill_bf16_kernel<64, false>), g, wg, 0, stream, p);
        }
    }
    return 0;
}

int prefill_bf16_rows_per_block() { return PrefillBf16Cfg<128>::BM; }

// Compute units of the current device (read once per process).
int device_cus() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
        else
            return 256;
    }
    return cus;
}

int launch_prefill_bf16(const PrefillParams& p0, int d, hipStream_t stream) {
    PrefillParams p = p0;
    // Causal row tiles are paired (see the kernel) when the unpaired grid is
    // at most two rounds of the workgroup slots (two per CU): with more rounds
    // the heaviest-first order already drains the grid evenly, and measured
    // pairing was then slower (C3a +6 % cycles; C2 -2 %).
    const long long unpaired = (long long)p.B * p.Hq * p.num_q_tiles;
    const bool pair = p.mask_kind == kMaskCausal && p.num_q_tiles > 1 && unpaired <= 2LL * 2 * device_cus();
    p.num_cus = device_cus();
    p.q_tile_pairs = pair ? (p.num_q_tiles + 1) / 2 : 0;
    const int blocks = p.B * p.Hq * (p.q_tile_pairs > 0 ? p.q_tile_pairs : p.num_q_tiles);
    const bool sinks = p.sink_end > 0;
    const bool mods = p.softcap > 0.f || p.alibi_slopes != nullptr;
    const dim3 g(blocks), wg(256);
    if (d == 128 && p.soft_exp2 != 0) {  // accepted only without score modifications
        if (p.soft_exp2 == 2) {
            if (sinks) hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_bf16_soft_kernel<true, 2>), g, wg, 0, stream, p);
            else hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_bf16_soft_kernel<false, 2>), g, wg, 0, stream, p);
        } else {
            if (sinks) hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_bf16_soft_kernel<true, 4>), g, wg, 0, stream, p);
            else hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_bf16_soft_kernel<false, 4>), g, wg, 0, stream, p);
        }
    } else if (d == 128) {
        if (mods) {
            if (sinks) hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_bf16_mod_kernel<128, true>), g, wg, 0, stream, p);
            else hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_bf16_mod_kernel<128, false>), g, wg, 0, stream, p);
        } else if (p.mask_kind == kMaskWindow || p.mask_kind == kMaskDocument) {
            if (sinks) hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_bf16_k32_kernel<true>), g, wg, 0, stream, p);
            else hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_bf16_k32_kernel<false>), g, wg, 0, stream, p);
        } else {
            if (sinks) hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_bf16_kernel<128, true>), g, wg, 0, stream, p);
            else hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_bf16_kernel<128, false>), g, wg, 0, stream, p);
        }
    } else {
        if (mods) {
            if (sinks) hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_bf16_mod_kernel<64, true>), g, wg, 0, stream, p);
            else hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_bf16_mod_kernel<64, false>), g, wg, 0, stream, p);
        } else {
            if (sinks) hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_bf16_kernel<64, true>), g, wg, 0, stream, p);
            else hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_bf16_kernel<64, false>), g, wg, 0, stream, p);
        }
    }
    return 0;
}

}  // namespace xattn
