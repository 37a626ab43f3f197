// LDS tile layouts and direct HBM -> LDS tile copies shared by the bf16
// attention kernels (forward prefill, chunked prefill, backward).
#pragma once

#include "common.hpp"

namespace xattn {

template <int D>
struct PrefillBf16Cfg {
    static constexpr int BM = 128;               // query rows per workgroup (4 waves x 32)
    static constexpr int BN = 64;                // keys per K/V tile
    static constexpr int CHUNKS = D / 8;         // 16-byte chunks per K/V row
    // Row strides in LDS, in 16-byte slots (LDS serves 256 bytes per cycle).
    // One slot of padding per K row puts 16 consecutive rows on 16 different
    // 16-byte bank groups (the K operand reads one chunk of 16 consecutive
    // rows).  Four slots per V row put 4 consecutive rows x 64 bytes on
    // distinct banks (the transposed V reads of 32 lanes: 4 key rows x 32
    // columns).
    static constexpr int KS = CHUNKS + 1;
    static constexpr int VS = CHUNKS + 4;
    static constexpr int KTILE = BN * KS * 16;   // bytes per K tile in LDS
    static constexpr int VTILE = BN * VS * 16;
    static constexpr int KLOADS = KTILE / 1024;  // 1 KiB direct loads per K tile
    static constexpr int VLOADS = VTILE / 1024;
    static constexpr int KLW = (KLOADS + 3) / 4; // per wave (rounded up)
    static constexpr int VLW = (VLOADS + 3) / 4;
    static constexpr int DK = D / 16;            // MFMA steps over the head dim for S
    static constexpr int CB = D / 32;            // 32-wide blocks of the head dim for O
    static_assert(KTILE % 1024 == 0 && VTILE % 1024 == 0, "tiles must be whole 1 KiB blocks");
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Per-lane byte offsets into one K or V tile in global memory for this wave's
// direct loads.  Load i of the tile fills LDS bytes [1024 i, 1024 i + 1024):
// lane l lands on 16-byte slot 64 i + l, i.e. row (64 i + l) / S, chunk
// (64 i + l) % S of the padded layout.  Padding slots fetch the row's last
// chunk again (never read back).
template <int D, int S, int NL>
__device__ __forceinline__ void tile_src_offsets(uint32_t (&off)[(NL + 3) / 4], int wave, int lane) {
#pragma unroll
    for (int j = 0; j < (NL + 3) / 4; ++j) {
        const int slot = (wave + 4 * j) * 64 + lane;
        const int r = slot / S;
        int c = slot % S;
        c = c < D / 8 ? c : D / 8 - 1;
        off[j] = (uint32_t)((r * D + c * 8) * 2);
    }
}

// Byte range of a tile's buffer resource: the rows that exist from the
// tile's first row on (rows = Nk - n0, possibly <= 0), but never more than the
// tile's own `tile_rows`, so the 32-bit range cannot overflow however long the
// sequence is (rows * D * 2 would pass 2^31 at 2^23 rows of d = 128).
template <int D>
__host__ __device__ constexpr uint32_t tile_range_bytes(int rows, int tile_rows) {
    return (uint32_t)(rows <= 0 ? 0 : (rows < tile_rows ? rows : tile_rows)) * (uint32_t)(D * 2);
}

// The range arithmetic near and past the old 32-bit overflow (2^23 and 2^24
// rows of d = 128), at the largest accepted length (2^28) and for a tile past
// the end, checked at every build.
static_assert(tile_range_bytes<128>((1 << 23) - 1, 64) == 64u * 256u, "range at 2^23 - 1 rows");
static_assert(tile_range_bytes<128>(1 << 23, 64) == 64u * 256u, "range at 2^23 rows");
static_assert(tile_range_bytes<128>(1 << 24, 64) == 64u * 256u, "range at 2^24 rows");
static_assert(tile_range_bytes<128>(1 << 28, 64) == 64u * 256u, "range at 2^28 rows");
static_assert(tile_range_bytes<128>(37, 64) == 37u * 256u, "a ragged last tile");
static_assert(tile_range_bytes<64>(64, 64) == 64u * 128u, "an exact tile, d = 64");
static_assert(tile_range_bytes<128>(0, 64) == 0u && tile_range_bytes<128>(-5, 64) == 0u, "no rows");

// Issue this wave's share of the direct HBM -> LDS copies of one tile
// (buffer_load_dwordx4 ... lds).  The buffer resource starts at key n0 and
// covers only the keys that exist, so rows past Nk read as zeros.  The NL
// 1 KiB copies of rows padded to S 16-byte slots reach ceil(NL * 64 / S) rows
// (a tile that is not a whole number of copies fetches a few rows past its
// end, which nothing reads back).
template <int D, int S, int NL>
__device__ __forceinline__ void load_tile_async(const uint16_t* __restrict__ base, int n0, int Nk, uint8_t* lds,
                                                const uint32_t (&off)[(NL + 3) / 4], int wave) {
    // the host pass instantiates kernel templates too, and the buffer
    // resource type and builtins exist only for the device target
#if defined(__HIP_DEVICE_COMPILE__)
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + (size_t)n0 * D), (short)0, (int)tile_range_bytes<D>(Nk - n0, (NL * 64 + S - 1) / S), 0x00020000);
#pragma unroll
    for (int j = 0; j < (NL + 3) / 4; ++j) {
        const int blk = wave + 4 * j;
        if (NL % 4 == 0 || blk < NL)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + blk * 1024), 16, off[j], 0, 0, 0);
    }
#endif
}

}  // namespace xattn
