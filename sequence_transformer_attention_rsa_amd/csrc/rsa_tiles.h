// rsa_tiles.h -- staging 64-row bf16 tiles from HBM into LDS, row-major or
// transposed, by the 256 threads of a workgroup (gfx950).
//
// Loads go to registers first (so they can be issued one tile ahead) and are
// written to LDS after the buffer is free. Row r of a tile is read from
// rowptr(r), which returns nullptr for rows outside the range (stored as
// zeros: an unwritten LDS row could hold a NaN pattern that an MFMA would
// spread through a zero weight).
#pragma once

#include "rsa_device.h"

namespace rsa {

constexpr int kTileRows = 64;
constexpr int kTileThreads = 256;

// Position of row x (0..15) of a 16-row group inside a transposed tile. A
// 32x32 accumulator gives lane half h the rows 4h+{0..3} and 8+4h+{0..3} of
// each 16-row MFMA step; storing them adjacently lets one 16-byte LDS read
// fetch a lane's whole fragment.
__device__ __forceinline__ constexpr int t_slot(int x) { return 8 * ((x >> 2) & 1) + (x & 3) + 4 * (x >> 3); }

// [64 rows][D] bf16 -> LDS row-major with pitch D + 8 elements (16-byte
// fragment reads of 8 consecutive rows hit distinct banks).
template <int D>
struct RowTile {
    static constexpr int P = D + 8;
    static constexpr int ELEMS = kTileRows * P;
    static constexpr int CH = kTileRows * D / 8 / kTileThreads;   // 16-byte chunks per thread
    static_assert(CH * kTileThreads * 8 == kTileRows * D, "row tile staging");
    u32x4 r[CH];

    template <class RowPtr>
    __device__ __forceinline__ void load(RowPtr rowptr) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = threadIdx.x + i * kTileThreads;
            const int row = c / (D / 8), col = c % (D / 8);
            const uint16_t* src = rowptr(row);
            u32x4 x = {0u, 0u, 0u, 0u};
            if (src) x = *reinterpret_cast<const u32x4*>(src + col * 8);
            r[i] = x;
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = threadIdx.x + i * kTileThreads;
            const int row = c / (D / 8), col = c % (D / 8);
            *reinterpret_cast<u32x4*>(lds + row * P + col * 8) = r[i];
        }
    }
    // 16-byte fragment: row `row`, elements e0 .. e0 + 7.
    __device__ __forceinline__ static u32x4 frag(const uint16_t* lds, int row, int e0) {
        return *reinterpret_cast<const u32x4*>(lds + row * P + e0);
    }
};

// [64 rows][D] bf16 -> LDS transposed [D][64 + 8]: element (row, d) at
// d * P + 16 * (row / 16) + t_slot(row % 16).
template <int D>
struct TransTile {
    static constexpr int P = kTileRows + 8;
    static constexpr int ELEMS = D * P;
    static constexpr int U = (D / 2) * (kTileRows / 8) / kTileThreads;   // (d pair, 8 rows) units per thread
    static_assert(U * kTileThreads * 16 == kTileRows * D, "transposed tile staging");
    uint32_t w[U][8];

    template <class RowPtr>
    __device__ __forceinline__ void load(RowPtr rowptr) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int u = threadIdx.x + i * kTileThreads;
            const int dp = u % (D / 2), rg = u / (D / 2);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint16_t* src = rowptr(rg * 8 + e);
                w[i][e] = src ? *reinterpret_cast<const uint32_t*>(src + 2 * dp) : 0u;
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int u = threadIdx.x + i * kTileThreads;
            const int dp = u % (D / 2), rg = u / (D / 2);
            const uint32_t* x = w[i];
            const int s0 = 16 * (rg >> 1) + t_slot(8 * (rg & 1));       // rows rg*8 + 0..3
            const int s1 = 16 * (rg >> 1) + t_slot(8 * (rg & 1) + 4);   // rows rg*8 + 4..7
            const u32x2 lo0 = {(x[0] & 0xffffu) | (x[1] << 16), (x[2] & 0xffffu) | (x[3] << 16)};
            const u32x2 lo1 = {(x[4] & 0xffffu) | (x[5] << 16), (x[6] & 0xffffu) | (x[7] << 16)};
            const u32x2 hi0 = {(x[0] >> 16) | (x[1] & 0xffff0000u), (x[2] >> 16) | (x[3] & 0xffff0000u)};
            const u32x2 hi1 = {(x[4] >> 16) | (x[5] & 0xffff0000u), (x[6] >> 16) | (x[7] & 0xffff0000u)};
            uint16_t* r0 = lds + (2 * dp) * P;
            uint16_t* r1 = r0 + P;
            *reinterpret_cast<u32x2*>(r0 + s0) = lo0;
            *reinterpret_cast<u32x2*>(r0 + s1) = lo1;
            *reinterpret_cast<u32x2*>(r1 + s0) = hi0;
            *reinterpret_cast<u32x2*>(r1 + s1) = hi1;
        }
    }
    // 16-byte fragment for the A operand of a contraction over tile rows:
    // lane (d row i, half h), 16-row step `step` -> rows of slots 8h .. 8h+7.
    __device__ __forceinline__ static u32x4 frag(const uint16_t* lds, int i, int step, int h) {
        return *reinterpret_cast<const u32x4*>(lds + i * P + 16 * step + 8 * h);
    }
};

// B operand of a 16-row contraction step taken from a packed 32x32
// accumulator (pk[blk][8] holds bf16 pairs of registers 2i, 2i+1).
__device__ __forceinline__ u32x4 acc_frag(const uint32_t (&pk)[2][8], int step) {
    const int blk = step >> 1, half = step & 1;
    const u32x4 f = {pk[blk][4 * half], pk[blk][4 * half + 1], pk[blk][4 * half + 2], pk[blk][4 * half + 3]};
    return f;
}

// Occupancy of a 64-key tile in ring order: bit 0 = some key valid, bit 1 =
// all 64 keys exist and are valid. `contiguous` means the chunk length is a
// multiple of 64, so the tile is one aligned run of the sequence.
__device__ __forceinline__ uint8_t key_tile_flags(const uint8_t* mrow, int n, int N, int Lc, bool contiguous,
                                                  int v0, int vend) {
    const int cnt = min(kTileRows, vend - v0);
    if (mrow == nullptr) return cnt == kTileRows ? 3 : 1;
    bool any = false, all = (cnt == kTileRows);
    if (contiguous) {
        const u32x4* m4 = reinterpret_cast<const u32x4*>(mrow + ring_pos(v0, n, N, Lc));
#pragma unroll
        for (int i = 0; i < kTileRows / 16; ++i) {
            const u32x4 w = m4[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                any |= (w[e] != 0u);
                all &= !has_zero_byte(w[e]);
            }
        }
    } else {
        for (int i = 0; i < cnt; ++i) {
            const bool ok = mrow[ring_pos(v0 + i, n, N, Lc)] != 0;
            any |= ok;
            all &= ok;
        }
    }
    return (any ? 1 : 0) | (all ? 2 : 0);
}

// Valid-key bits of a 64-key tile in ring order (lane i <-> key v0 + i).
__device__ __forceinline__ uint64_t key_tile_bits(const uint8_t* mrow, int n, int N, int Lc, bool contiguous,
                                                  int v0, int vend) {
    const int lane = threadIdx.x % kWave;
    const int vk = v0 + lane;
    bool ok = vk < vend;
    if (ok && mrow) ok = mrow[contiguous ? ring_pos(v0, n, N, Lc) + lane : ring_pos(vk, n, N, Lc)] != 0;
    return __ballot(ok);
}

}  // namespace rsa
