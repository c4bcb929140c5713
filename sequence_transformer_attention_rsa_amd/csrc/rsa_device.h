// rsa_device.h -- device-side building blocks shared by the RSA kernels
// (gfx950 / CDNA4: 64-lane wavefronts, MFMA matrix cores, LDS).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kXcds = 8;          // MI355X: 8 accelerator complex dies, one L2 each
constexpr int kCUs = 256;         // MI355X: compute units
constexpr float kLn2 = 0.69314718055994530942f;

// ---------------------------------------------------------------- MFMA ---
// 32x32 accumulator layout (all 32x32 MFMA shapes): lane l holds column
// n = l % 32; register r holds row m = 8*(r/4) + 4*(l/32) + (r%4).
// Operand layout: A lane l holds row m = l % 32, B lane l holds column
// n = l % 32; the contraction index is spread over (l / 32, register) in the
// same way for A and B, so any data placed consistently in both contracts
// correctly.
__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_32x32x2_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row index held by accumulator register r of a lane in half h = lane / 32.
__device__ __forceinline__ constexpr int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// ----------------------------------------------------------- bf16 packs ---
// Two fp32 values to one dword of two bf16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a dword of two bf16, in fp32 (one dot2 instruction).
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, acc, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------ ring math ---
// Sequence position of the v-th key that rank n visits: ring step t = v / Lc
// brings chunk c = (n - t) mod N, whose keys are visited in ascending order.
__device__ __forceinline__ int ring_pos(int v, int n, int N, int Lc) {
    const int t = v / Lc;
    int c = n - t;
    c += (c < 0) ? N : 0;
    return c * Lc + (v - t * Lc);
}

// -------------------------------------------------------------- dropout ---
// Philox-4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
// As Easy as 1, 2, 3", SC'11): counter (c0..c3), key (k0, k1); ten rounds of
// hi0:lo0 = M0 * c0, hi1:lo1 = M1 * c2, counter <- (hi1 ^ c1 ^ k0, lo1,
// hi0 ^ c3 ^ k1, lo0), with the key increased by the Weyl constants between
// rounds. Each 32x32 -> 64 product is one v_mad_u64_u32.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    const u32x4 x = {c0, c1, c2, c3};
    return x;
}

// Dropout of the softmax weights. The keep decision of the weight of query
// position i and key position j in head bh is byte (j mod 4) of word
// ((j / 8) mod 4) of Philox-4x32-10 at counter ((j / 32) * 2 + bit 2 of j,
// i, bh, offset), key (seed low, seed high) words; the weight is kept iff
// that byte is >= p8 (drop probability p8 / 256) and then scaled by
// 256 / (256 - p8). One counter covers the 16 keys of a 32-key block that
// share bit 2 of j -- the keys one lane of a 32x32 accumulator holds.
struct Dropout {
    uint32_t p8;       // 0: no dropout
    uint32_t seed_lo, seed_hi, offset;
    float scale;       // 256 / (256 - p8)
    float keep;        // (256 - p8) / 256, exact
};

// The 16 bytes of the counter of (key block jb = j / 32, half hh = bit 2 of j, query i, head bh).
__device__ __forceinline__ u32x4 dropout_bytes(const Dropout& dr, int jb, int hh, int i, int bh) {
    return philox4x32_10((uint32_t)((jb << 1) | hh), (uint32_t)i, (uint32_t)bh, dr.offset, dr.seed_lo, dr.seed_hi);
}

// Keep decision of one weight (query position i, key position j, head bh).
__device__ __forceinline__ bool dropout_keep(const Dropout& dr, int i, int j, int bh) {
    const u32x4 x = dropout_bytes(dr, j >> 5, (j >> 2) & 1, i, bh);
    return ((x[(j >> 3) & 3] >> (8 * (j & 3))) & 0xffu) >= dr.p8;
}

// Mask for a dword of two bf16 weights whose keep bytes are the low two
// bytes of w: each 16-bit half all ones if kept, zero if dropped.
__device__ __forceinline__ uint32_t keep_mask_bf16x2(uint32_t w, uint32_t p8) {
    return ((w & 0xffu) >= p8 ? 0x0000ffffu : 0u) | (((w >> 8) & 0xffu) >= p8 ? 0xffff0000u : 0u);
}

// ------------------------------------------------------------- dispatch ---
// Workgroups are dealt to the XCDs round-robin by id. Renumber them so that
// each XCD receives a contiguous range of logical work items: neighbouring
// items (query tiles of one head) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int id, int n) {
    const int xcd = id % kXcds, local = id / kXcds;
    const int per = n / kXcds, rem = n % kXcds;
    return (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Tile t and head bh of workgroup id, for launches of nt tiles per head.
// When the heads split evenly over the XCDs, XCD x (ids x, x + 8, ...) takes
// heads x, x + 8, ...: a head's tiles share one L2, and every XCD gets the
// same mix of batch rows, whose key padding differs. Within an XCD the tiles
// go head by head, or, with rank_major (causal launches, whose tile t = 0 is
// the heaviest), the t-th tile of each of its heads before the (t + 1)-th of
// any, so that the heavy tiles start first. Other head counts: xcd_remap
// order, head by head.
__device__ __forceinline__ void head_order(int id, int nt, int BH, bool rank_major, int& t, int& bh) {
    if (BH % kXcds == 0) {
        const int xcd = id % kXcds, local = id / kXcds, hx = BH / kXcds;
        t = rank_major ? local / hx : local % nt;
        bh = xcd + kXcds * (rank_major ? local % hx : local / nt);
    } else {
        const int lid = xcd_remap(id, nt * BH);
        t = lid % nt;
        bh = lid / nt;
    }
}

__device__ __forceinline__ bool wave_any(bool p) { return __any(p); }

__device__ __forceinline__ float shfl_xor32(float x) { return __shfl_xor(x, 32); }

// True if some byte of w is zero.
__device__ __forceinline__ bool has_zero_byte(uint32_t w) {
    return ((w - 0x01010101u) & ~w & 0x80808080u) != 0;
}

}  // namespace rsa
