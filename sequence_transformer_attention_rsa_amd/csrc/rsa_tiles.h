// rsa_tiles.h -- 64-row bf16 tiles in LDS and the fragments the 32x32 MFMA
// kernels read from them (gfx950).
#pragma once

#include "rsa_device.h"

namespace rsa {

constexpr int kTileRows = 64;

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

// Causal visibility of a key tile (ring indices v0 .. v0 + cnt - 1 of rank n)
// to the query positions [qlo, qhi]: 0 = every key lies after every query
// (hidden), 3 = every key at or before every query (visible), 1 = mixed.
// The causal variant is not on the pages: the query at position i sees key
// j only if j <= i (the standard autoregressive mask). Within one chunk the
// ring indices map to consecutive positions, so a tile is split into at most
// a few chunk segments.
__device__ __forceinline__ uint32_t causal_tile_class(int v0, int cnt, int n, int N, int Lc, bool contiguous, int qlo,
                                                      int qhi) {
    int kmin, kmax;
    if (contiguous) {
        kmin = ring_pos(v0, n, N, Lc);
        kmax = kmin + cnt - 1;
    } else {
        kmin = 0x7fffffff;
        kmax = -1;
        for (int v = v0; v < v0 + cnt;) {
            const int seg_end = min(v0 + cnt, (v / Lc + 1) * Lc);
            const int a = ring_pos(v, n, N, Lc);
            kmin = min(kmin, a);
            kmax = max(kmax, a + (seg_end - 1 - v));
            v = seg_end;
        }
    }
    if (kmin > qhi) return 0u;
    return kmax <= qlo ? 3u : 1u;
}

// Occupancy table of a workgroup's key tiles in LDS: the two bits of
// key_tile_flags per tile, four tiles per byte. build() is called by all
// `nthreads` threads (a multiple of the wave size) and must be followed by a
// barrier before get(). Thread i classifies tile i (so every thread's mask
// reads are in flight at once), and four neighbouring lanes combine their
// flags into one byte.
struct TileTable {
    uint8_t* bytes;

    __device__ __forceinline__ uint32_t get(int t) const { return (bytes[t >> 2] >> (2 * (t & 3))) & 3u; }

    template <class Flags>
    __device__ __forceinline__ void build(int ntile, int nthreads, Flags flags) const {
        for (int t0 = 0; t0 < ntile; t0 += nthreads) {   // the same trip count in every thread
            const int t = t0 + (int)threadIdx.x;
            const uint32_t f = t < ntile ? (uint32_t)flags(t) : 0u;
            const uint32_t b = f | (__shfl_down(f, 1) << 2) | (__shfl_down(f, 2) << 4) | (__shfl_down(f, 3) << 6);
            if ((threadIdx.x & 3) == 0 && t < ntile) bytes[t >> 2] = (uint8_t)b;
        }
    }
};

// Valid-key bits of a 64-key tile in ring order (lane i <-> key v0 + i).
__device__ __forceinline__ uint64_t key_tile_bits(const uint8_t* mrow, int n, int N, int Lc, bool contiguous,
                                                  int v0, int vend) {
    const int lane = threadIdx.x % kWave;
    const int vk = v0 + lane;
    bool ok = vk < vend;
    if (ok && mrow) ok = mrow[contiguous ? ring_pos(v0, n, N, Lc) + lane : ring_pos(vk, n, N, Lc)] != 0;
    return __ballot(ok);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ---- Direct HBM -> LDS copies issued from inline assembly.
//
// The compiler tracks copies made with __builtin_amdgcn_global_load_lds and
// inserts a wait for them before any LDS read it cannot prove disjoint, and
// the memory counter is in-order, so waiting for any later load (a register
// spill, a mask byte) waits for every copy in flight too. Copies issued from
// inline assembly are invisible to that tracking: the kernels that use them
// wait for them explicitly with vm_wait<N>() (at most N of this wave's
// memory loads still outstanding) before the barrier that publishes a tile.
// The copy reads 16 (or 4) bytes at sbase + voff per lane and writes them to
// LDS at m0 + 16 (or 4) * lane; sbase and m0 must be wave-uniform. One wait
// state separates the write of m0 from the copy that reads it.

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// m0 is reserved to the compiler, which ignores it in a clobber list (and
// warns); the kernels that issue these copies have no compiler-generated use
// of m0, and none may be added to them (e.g. the builtin copy). The build
// checks this on the device assembly of every kernel (build.py,
// m0_violations) and fails if such a use appears.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_copy16(const void* sbase, uint32_t voff, uint32_t lds) {
    __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     ::"v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ void dma_copy4(const void* sbase, uint32_t voff, uint32_t lds) {
    __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                     ::"v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N), leaving the other counters alone (N < 64; the count
// is split over bits 3:0 and 15:14 of the immediate).
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads() (which
// waits for every load in flight, prefetches included). LDS visibility is
// the caller's business (vm_wait for copies; ds reads complete before their
// results are used). The empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void bare_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// [64 rows][D] bf16 tile copied from HBM straight into LDS with
// global_load_lds (16 bytes per lane, no registers, no VALU): each
// wave-instruction fills one contiguous 1 KB block, so rows are unpadded and
// the 16-byte chunk c of row r is stored at r * 2D + 16 * (c ^ swz(r)) bytes;
// the XOR is chosen through each lane's source address. LDS has 64 banks of
// 4 bytes; a 16-byte read is served 16 lanes per cycle, an 8-byte read 32
// lanes per cycle. The fragment reads put 16 consecutive rows (lanes) on one
// logical chunk, the transposing ds_read_b64_tr_b16 puts four consecutive
// rows on four consecutive chunks (eight 8-byte pieces per row over 32
// lanes). swz(r) is chosen so that both touch 64 different banks:
//   D = 64 (two rows per 256 bytes): rows of one parity among 16 consecutive
//     rows get eight different swz values, and the two rows of one parity in
//     an aligned group of four differ in swz bit 2 (disjoint aligned chunk
//     quads);
//   D = 128 (one row per 256 bytes): 16 consecutive rows get 16 different
//     swz values, four consecutive rows four different swz bits 2-3.
// One copy of a tile then serves both operand orientations.
template <int D, int WAVES = 4>
struct DirectTile {
    static constexpr int ROW_BYTES = 2 * D;
    static constexpr int BYTES = kTileRows * ROW_BYTES;
    static constexpr int CPR = D / 8;                     // 16-byte chunks per row
    static constexpr int RPI = 1024 / ROW_BYTES;          // rows per wave-instruction
    static constexpr int IPW = kTileRows / RPI / WAVES;   // instructions per wave
    static_assert(IPW * RPI * WAVES == kTileRows, "tile copy split");

    __device__ __forceinline__ static constexpr int swz(int r) {
        if constexpr (CPR == 8)
            return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r ^ (r >> 3)) & 1);
        else
            return ((r & 3) << 2) | ((r >> 2) & 3);
    }
    static_assert(CPR == 8 || CPR == 16, "tile rows of 64 or 128 bf16");

    // Issue the copies; rowptr(r) must return a readable row for every r
    // (callers point rows outside the range at any valid row).
    template <class RowPtr>
    __device__ __forceinline__ static void load(uint8_t* lds, RowPtr rowptr) {
        const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
            const int blk = wave * IPW + u;
            const int r = blk * RPI + lane / CPR;
            const int c = (lane % CPR) ^ swz(r);
            const uint16_t* src = rowptr(r) + 8 * c;
            __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                             (__attribute__((address_space(3))) void*)(lds + blk * 1024), 16, 0, 0);
        }
    }

    // Per-lane byte offsets of the untracked copy of a tile whose rows are
    // contiguous in global memory (row pitch ROW_BYTES): row r of the tile
    // comes from base + r * ROW_BYTES. The same for every tile.
    __device__ __forceinline__ static void row_offsets(uint32_t (&voff)[IPW]) {
        const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
            const int r = (wave * IPW + u) * RPI + lane / CPR;
            voff[u] = (uint32_t)(r * ROW_BYTES + 16 * ((lane % CPR) ^ swz(r)));
        }
    }

    // Untracked copy of 64 contiguous rows starting at `base` (wave-uniform);
    // IPW copies per wave, waited for with vm_wait.
    __device__ __forceinline__ static void load_rows(uint8_t* lds, const uint16_t* base, const uint32_t (&voff)[IPW]) {
        load_rows(lds, base, voff, wave_lds_offset());
    }

    // Byte offset of this wave's blocks within a tile (wave-uniform), for
    // callers that compute it once outside their tile loop.
    __device__ __forceinline__ static uint32_t wave_lds_offset() {
        return (uint32_t)(__builtin_amdgcn_readfirstlane(threadIdx.x / kWave) * IPW * 1024);
    }

    __device__ __forceinline__ static void load_rows(uint8_t* lds, const uint16_t* base, const uint32_t (&voff)[IPW],
                                                     uint32_t wave_lds) {
        const uint32_t l0 = lds_addr(lds) + wave_lds;
#pragma unroll
        for (int u = 0; u < IPW; ++u) dma_copy16(base, voff[u], l0 + (uint32_t)(u * 1024));
    }

    // 16-byte chunk c of row r (ds_read_b128).
    __device__ __forceinline__ static u32x4 chunk(const uint8_t* lds, int r, int c) {
        return *reinterpret_cast<const u32x4*>(lds + r * ROW_BYTES + 16 * (c ^ swz(r)));
    }

    // Transposed fragment: the A operand of a 32x32x16 MFMA that contracts
    // over 16 tile rows starting at `row0`, for 32 columns starting at `col0`.
    // Lane (column col0 + lane % 32, half h) receives rows
    // row0 + 4h + {0..3} and row0 + 8 + 4h + {0..3} of its column -- the
    // register order of a 32x32 accumulator used as the B operand.
    // ds_read_b64_tr_b16: in each 16-lane group, lane 4*rho + c supplies
    // elements 4c..4c+3 of row rho of a 4 x 16 block; lane i receives column i.
    __device__ __forceinline__ static u32x4 tfrag(const uint8_t* lds, int row0, int col0) {
        return tfrag_rows<false>(lds, row0, col0);
    }

    // The same fragment with rows in sequence: lane half h receives rows
    // row0 + 8h + {0..7}, the order of a 16-byte row-major operand load.
    __device__ __forceinline__ static u32x4 tfrag_seq(const uint8_t* lds, int row0, int col0) {
        return tfrag_rows<true>(lds, row0, col0);
    }

    template <bool SEQ>
    __device__ __forceinline__ static u32x4 tfrag_rows(const uint8_t* lds, int row0, int col0) {
        const int lane = threadIdx.x % kWave;
        const int i = lane & 15, ig = (lane >> 4) & 1, h = lane >> 5;
        const int rho = i >> 2, c4 = i & 3;
        const int e = col0 + 16 * ig + 4 * c4;          // first element of this lane's 4
        const int c = e >> 3, half = (e >> 2) & 1;
        u32x4 f;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int r = row0 + (SEQ ? 8 * h + 4 * k : 8 * k + 4 * h) + rho;
            const uint8_t* addr = lds + r * ROW_BYTES + 16 * (c ^ swz(r)) + 8 * half;
            const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)addr);
            const u32x2 w = __builtin_bit_cast(u32x2, x);
            f[2 * k] = w[0];
            f[2 * k + 1] = w[1];
        }
        return f;
    }
};

}  // namespace rsa
