// rsa_layer.hip -- the token-local steps of the sequence-parallel layer
// around RSA on gfx950: a bf16 MFMA matrix product with fused prologue and
// epilogue variants (head split of Q/K/V, head merge of the attention output,
// bias, GeLU, residual sum), and a layer normalisation over the hidden size.
//
// Review page of "Sequence Parallelism: Making 4D Parallelism Possible"
// (ABSTRACT): each device holds one chunk of the sequence, and every step of
// the Transformer layer other than the attention acts on one token at a
// time, so these run on a chunk without any exchange. The tensor-parallelism
// page ("一文捋順千億模型訓練技術", section 二, 1D tensor parallelism, parts
// (2) and (3)) describes the two fully connected layers with GeLU and the
// independent attention heads.

#include <atomic>

#include "rsa_internal.h"
#include "rsa_tiles.h"

namespace rsa {
namespace {

constexpr int kThreads = 256;
constexpr int kGT = 128;                         // output tile: 128 rows x 128 columns
constexpr int kGK = 64;                          // contraction step
using GTile = DirectTile<64>;                    // [64 rows][64 bf16], 8 KB, swizzled
constexpr int kStageBytes = 4 * GTile::BYTES;    // A rows 0-63, 64-127; W rows 0-63, 64-127
constexpr int kGemmBuf = 2;                      // stage buffers: one step in flight
constexpr int kStagePitch = kGT * 4 + 16;        // fp32 epilogue row, bytes (16 B pad)
constexpr int kGemmLds = (kGemmBuf * kStageBytes > kGT * kStagePitch) ? kGemmBuf * kStageBytes
                                                                       : kGT * kStagePitch;

// A operand layouts: [M, K] rows, or the attention output [B, H, L, d] read
// as [B*L, H*d] (head merge). Output layouts: [M, N] rows, or Q/K/V
// [B, H, L, d] from column blocks [0, E), [E, 2E), [2E, 3E) (head split).
enum { kProRows = 0, kProHeads = 1 };
enum { kEpiRows = 0, kEpiQkv = 1 };

struct GemmParams {
    const uint16_t* a;
    const uint16_t* w;      // [N, K]
    const float* bias;      // [N] or nullptr
    const uint16_t* res;    // [M, N] or nullptr
    uint16_t* out0;         // [M, N], or Q
    uint16_t* out1;         // K
    uint16_t* out2;         // V
    int M, N, K;
    int L, H, d, E;         // token/head layout of the head variants
    int mt, nt;             // tile counts
};

// erfc(x) from the Chebyshev fit published in Press, Teukolsky, Vetterling
// and Flannery, Numerical Recipes (section 6.2, the routine erfcc): with
// t = 1 / (1 + |x|/2), erfc(|x|) = t exp(-x^2 + P(t)) for a degree-9
// polynomial P, fractional error below 1.2e-7 for every x, and
// erfc(-|x|) = 2 - erfc(|x|). Branch-free, so one code path serves every
// lane; in fp32 the rounding of x^2 adds up to ~1.6e-5 relative error at
// |x| ~ 9, far below the bf16 rounding of the output.
__device__ __forceinline__ float erfc_fit(float x) {
    const float ax = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, ax, 1.0f));
    float q = 0.17087277f;
    q = fmaf(q, t, -0.82215223f);
    q = fmaf(q, t, 1.48851587f);
    q = fmaf(q, t, -1.13520398f);
    q = fmaf(q, t, 0.27886807f);
    q = fmaf(q, t, -0.18628806f);
    q = fmaf(q, t, 0.09678418f);
    q = fmaf(q, t, 0.37409196f);
    q = fmaf(q, t, 1.00002368f);
    q = fmaf(q, t, -1.26551223f);
    const float r = t * __builtin_amdgcn_exp2f(fmaf(-ax, ax, q) * 1.44269504088896341f);
    return x >= 0.0f ? r : 2.0f - r;
}

// GeLU(z) = z Phi(z) = z/2 erfc(-z / sqrt 2): the complementary form keeps
// full fp32 accuracy for negative z, where 1 + erf(z / sqrt 2) would cancel.
__device__ __forceinline__ float gelu(float z) { return 0.5f * z * erfc_fit(-z * 0.70710678118654752f); }

// out = act(A W^T + bias) + res for one 128x128 tile. Four waves, each a
// 64x64 quarter as 2x2 MFMA blocks. The MFMA computes the transposed block
// (W rows as its A operand) so that each lane holds one output row and
// registers run along the columns: the epilogue then writes four
// consecutive fp32 columns per lane into an LDS staging tile, from which
// the whole workgroup stores 16-byte chunks of rows.
// GELU: apply GeLU before the residual sum (a template argument, so that
// the products without it carry none of its code or registers).
template <int PRO, int EPI, bool GELU>
__global__ __launch_bounds__(kThreads) void rsa_gemm_bf16(GemmParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kGemmLds];

    const int lid = xcd_remap(blockIdx.x, p.mt * p.nt);
    const int m0 = (lid / p.nt) * kGT, n0 = (lid % p.nt) * kGT;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int j = lane & 31, h = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = p.K / kGK;

    // Per-lane source offsets of this workgroup's copies (the same for every
    // contraction step; the step moves the scalar base). Rows past M read row
    // M - 1 (their results are never stored).
    uint32_t va[2][GTile::IPW], vw[2][GTile::IPW];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < GTile::IPW; ++u) {
            const int r = (wave * GTile::IPW + u) * GTile::RPI + lane / GTile::CPR;
            const uint32_t sw = 16u * (uint32_t)((lane % GTile::CPR) ^ GTile::swz(r));
            const int m = min(m0 + 64 * t + r, p.M - 1);
            if constexpr (PRO == kProRows) {
                va[t][u] = (uint32_t)(m - m0) * (uint32_t)(2 * p.K) + sw;
            } else {
                const int b = m / p.L, l = m - b * p.L;
                va[t][u] = ((uint32_t)(b * p.H) * (uint32_t)p.L + (uint32_t)l) * (uint32_t)(2 * p.d) + sw;
            }
            vw[t][u] = (uint32_t)(64 * t + r) * (uint32_t)(2 * p.K) + sw;
        }

    auto load = [&](int s, int bi) {
        uint8_t* sb = smem + bi * kStageBytes;
        const uint16_t* abase;
        if constexpr (PRO == kProRows) {
            abase = p.a + (size_t)m0 * p.K + (size_t)s * kGK;
        } else {
            const int k0 = s * kGK, hh = k0 / p.d;
            abase = p.a + (size_t)hh * p.L * p.d + (k0 - hh * p.d);
        }
        const uint16_t* wbase = p.w + (size_t)n0 * p.K + (size_t)s * kGK;
        const uint32_t l0 = lds_addr(sb) + (uint32_t)(__builtin_amdgcn_readfirstlane(wave) * GTile::IPW * 1024);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int u = 0; u < GTile::IPW; ++u) {
                dma_copy16(abase, va[t][u], l0 + (uint32_t)(t * GTile::BYTES + u * 1024));
                dma_copy16(wbase, vw[t][u], l0 + (uint32_t)((2 + t) * GTile::BYTES + u * 1024));
            }
    };
    constexpr int kCopies = 4 * GTile::IPW;   // this wave's copies per step

    f32x16 acc[2][2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ni][mi][r] = 0.0f;

    for (int s = 0; s < kGemmBuf - 1 && s < nk; ++s) load(s, s);
    for (int s = 0; s < nk; ++s) {
        // step s landed (the steps after it that were issued may stay in
        // flight); after the barrier every wave is done with step s - 1,
        // whose buffer takes step s + kGemmBuf - 1
        const int ahead = min(kGemmBuf - 2, nk - 1 - s);
        if (kGemmBuf >= 4 && ahead >= 2)
            vm_wait<2 * kCopies>();
        else if (kGemmBuf >= 3 && ahead >= 1)
            vm_wait<kCopies>();
        else
            vm_wait<0>();
        bare_barrier();
        if (s + kGemmBuf - 1 < nk) load(s + kGemmBuf - 1, (s + kGemmBuf - 1) % kGemmBuf);
        const uint8_t* sb = smem + (s % kGemmBuf) * kStageBytes;
        const uint8_t* at = sb + wm * GTile::BYTES;
        const uint8_t* wt = sb + (2 + wn) * GTile::BYTES;
        // fragments of sub-step ks + 1 are read while the MFMAs of ks run
        u32x4 af[2][2], wf[2][2];
        auto frags = [&](int ks, int slot) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                af[slot][x] = GTile::chunk(at, 32 * x + j, 2 * ks + h);
                wf[slot][x] = GTile::chunk(wt, 32 * x + j, 2 * ks + h);
            }
        };
        frags(0, 0);
#pragma unroll
        for (int ks = 0; ks < kGK / 16; ++ks) {
            if (ks + 1 < kGK / 16) frags(ks + 1, (ks + 1) & 1);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
                    acc[ni][mi] = mfma_32x32x16_bf16(wf[ks & 1][ni], af[ks & 1][mi], acc[ni][mi]);
        }
    }
    bare_barrier();   // every wave's last reads of the stage buffers are done

    // bias and activation in registers, fp32 tile to LDS
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int nl = 64 * wn + 32 * ni + 8 * r4 + 4 * h;   // first of 4 columns
            f32x4 bv = {0.0f, 0.0f, 0.0f, 0.0f};
            if (p.bias) bv = *reinterpret_cast<const f32x4*>(p.bias + n0 + nl);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                f32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float z = acc[ni][mi][4 * r4 + e] + bv[e];
                    o[e] = GELU ? gelu(z) : z;
                }
                const int ml = 64 * wm + 32 * mi + j;
                *reinterpret_cast<f32x4*>(smem + ml * kStagePitch + nl * 4) = o;
            }
        }
    __syncthreads();

    // 16-byte output chunks: 128 rows x 16 chunks of 8 columns
    uint16_t* dst = p.out0;
    int ncol0 = n0;
    if constexpr (EPI == kEpiQkv) {
        const int which = n0 / p.E;   // a tile never straddles Q, K and V (E % 128 == 0)
        dst = which == 0 ? p.out0 : (which == 1 ? p.out1 : p.out2);
        ncol0 = n0 - which * p.E;
    }
#pragma unroll 2
    for (int it = 0; it < kGT * 16 / kThreads; ++it) {
        const int idx = it * kThreads + threadIdx.x;
        const int row = idx >> 4, c = idx & 15;
        const int m = m0 + row;
        if (m >= p.M) continue;
        const uint8_t* src = smem + row * kStagePitch + c * 32;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 16);
        float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if (p.res) {
            const u32x4 rv = *reinterpret_cast<const u32x4*>(p.res + (size_t)m * p.N + n0 + 8 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] += bf16_lo(rv[e]);
                x[2 * e + 1] += bf16_hi(rv[e]);
            }
        }
        const u32x4 pk = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                          pack_bf16x2(x[6], x[7])};
        size_t off;
        if constexpr (EPI == kEpiQkv) {
            const int nn = ncol0 + 8 * c, hh = nn / p.d, dd = nn - hh * p.d;
            const int b = m / p.L, l = m - b * p.L;
            off = ((size_t)(b * p.H + hh) * p.L + l) * p.d + dd;
        } else {
            off = (size_t)m * p.N + n0 + 8 * c;
        }
        *reinterpret_cast<u32x4*>(dst + off) = pk;
    }
}

// ---- 256-row tiles, eight waves ------------------------------------------
// The same product with 256 rows and NT = 256 or 192 columns per tile. At
// NT = 256 each contraction step copies (256 + 256) x 64 bf16 for
// 2 x 256 x 256 x 64 flops, half the L2-to-LDS bytes per flop of the
// 128x128 tile, and each wave (a 128 x 64 strip, 4x2 MFMA blocks) reads 6
// fragments per 8 MFMAs instead of 4 per 4. NT = 192 (waves of 64 x 96,
// 2x3 blocks, 5 fragments per 6 MFMAs) exists for the widths that 256
// columns divide into a poor number of workgroups: N = 768 gives 256
// workgroups of 256 x 192 for 256 CUs, where 256 x 256 tiles would leave a
// quarter of the CUs idle. Two stage buffers fill 128 or 112 KB of LDS
// (one workgroup per CU, two waves per SIMD).
// The epilogue finishes each value in registers (bias, GeLU, residual read
// as 8-byte pieces), rounds once to bf16 and stages each wave's strip in
// its own part of LDS (NT = 256: 128-byte rows with 16-byte chunks
// XOR-swizzled by row; NT = 192: 192-byte rows at a 208-byte pitch), from
// which the wave stores whole row segments.
constexpr int kBigThreads = 512;
constexpr int kBT = 256;
using BTile = DirectTile<64, 8>;                 // one copy instruction per wave per 64-row tile

template <int NT>
struct BigShape {
    static_assert(NT == 256 || NT == 192, "256 or 192 columns");
    static constexpr int WTILES = NT / 64;                        // W tiles per stage
    static constexpr int STAGE = (4 + WTILES) * BTile::BYTES;     // A: tiles 0-3, W: tiles 4 ..
    static constexpr int WM = NT == 256 ? 128 : 64;               // wave strip rows
    static constexpr int WN = NT == 256 ? 64 : 96;                // wave strip columns
    static constexpr int MWAVES = kBT / WM;                       // waves along the rows
    static constexpr int MI = WM / 32, NI = WN / 32;              // MFMA blocks per wave
    static constexpr int CW = WN / 8;                             // 16-byte chunks per strip row
    static constexpr int PITCH = NT == 256 ? 128 : 208;           // strip row pitch, bytes
    static constexpr int LDS = 2 * STAGE;
    static_assert(MWAVES * (NT / WN) == kBigThreads / kWave, "wave grid");
    static_assert(8 * WM * PITCH <= LDS, "epilogue strips fit in the stage buffers");
    static_assert(WM * CW % kWave == 0, "whole store iterations");
    // byte offset of 16-byte chunk c of strip row ml
    __device__ __forceinline__ static int pos(int ml, int c) {
        return NT == 256 ? ml * PITCH + 16 * (c ^ (ml & 7)) : ml * PITCH + 16 * c;
    }
};

template <int PRO, int EPI, int NT, bool GELU>
__global__ __launch_bounds__(kBigThreads) void rsa_gemm_bf16_256(GemmParams p) {
    using S = BigShape<NT>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[S::LDS];

    const int lid = xcd_remap(blockIdx.x, p.mt * p.nt);
    const int m0 = (lid / p.nt) * kBT, n0 = (lid % p.nt) * NT;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int j = lane & 31, h = lane >> 5;
    const int wm = wave % S::MWAVES, wn = wave / S::MWAVES;   // rows WM wm .., columns WN wn ..
    const int nk = p.K / kGK;

    uint32_t va[4], vw[S::WTILES];
    {
        const int r = wave * BTile::RPI + lane / BTile::CPR;   // tile row this lane copies
        const uint32_t sw = 16u * (uint32_t)((lane % BTile::CPR) ^ BTile::swz(r));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int m = min(m0 + 64 * t + r, p.M - 1);
            if constexpr (PRO == kProRows) {
                va[t] = (uint32_t)(m - m0) * (uint32_t)(2 * p.K) + sw;
            } else {
                const int b = m / p.L, l = m - b * p.L;
                va[t] = ((uint32_t)(b * p.H) * (uint32_t)p.L + (uint32_t)l) * (uint32_t)(2 * p.d) + sw;
            }
            if (t < S::WTILES) vw[t] = (uint32_t)(64 * t + r) * (uint32_t)(2 * p.K) + sw;
        }
    }
    auto load = [&](int s, int bi) {
        uint8_t* sb = smem + bi * S::STAGE;
        const uint16_t* abase;
        if constexpr (PRO == kProRows) {
            abase = p.a + (size_t)m0 * p.K + (size_t)s * kGK;
        } else {
            const int k0 = s * kGK, hh = k0 / p.d;
            abase = p.a + (size_t)hh * p.L * p.d + (k0 - hh * p.d);
        }
        const uint16_t* wbase = p.w + (size_t)n0 * p.K + (size_t)s * kGK;
        const uint32_t l0 = lds_addr(sb) + (uint32_t)(__builtin_amdgcn_readfirstlane(wave) * 1024);
#pragma unroll
        for (int t = 0; t < 4; ++t) dma_copy16(abase, va[t], l0 + (uint32_t)(t * BTile::BYTES));
#pragma unroll
        for (int t = 0; t < S::WTILES; ++t) dma_copy16(wbase, vw[t], l0 + (uint32_t)((4 + t) * BTile::BYTES));
    };

    f32x16 acc[S::NI][S::MI];
#pragma unroll
    for (int ni = 0; ni < S::NI; ++ni)
#pragma unroll
        for (int mi = 0; mi < S::MI; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ni][mi][r] = 0.0f;

    auto compute = [&](int bi) {
        const uint8_t* sb = smem + bi * S::STAGE;
        const uint8_t* wt = sb + 4 * BTile::BYTES;
        // fragments of sub-step ks + 1 are read while the MFMAs of ks run
        u32x4 af[2][S::MI], wf[2][S::NI];
        auto frags = [&](int ks, int slot) {
#pragma unroll
            for (int mi = 0; mi < S::MI; ++mi) {
                const int r = S::WM * wm + 32 * mi;     // tile row of this block
                af[slot][mi] = BTile::chunk(sb + (r >> 6) * BTile::BYTES, (r & 63) + j, 2 * ks + h);
            }
#pragma unroll
            for (int ni = 0; ni < S::NI; ++ni) {
                const int c = S::WN * wn + 32 * ni;     // tile column of this block
                wf[slot][ni] = BTile::chunk(wt + (c >> 6) * BTile::BYTES, (c & 63) + j, 2 * ks + h);
            }
        };
        frags(0, 0);
#pragma unroll
        for (int ks = 0; ks < kGK / 16; ++ks) {
            if (ks + 1 < kGK / 16) frags(ks + 1, (ks + 1) & 1);
#pragma unroll
            for (int ni = 0; ni < S::NI; ++ni)
#pragma unroll
                for (int mi = 0; mi < S::MI; ++mi)
                    acc[ni][mi] = mfma_32x32x16_bf16(wf[ks & 1][ni], af[ks & 1][mi], acc[ni][mi]);
        }
    };
    load(0, 0);
    for (int s = 0; s < nk; ++s) {
        vm_wait<0>();   // step s landed
        bare_barrier(); // ... for every wave; every wave is done with step s - 1
        if (s + 1 < nk) load(s + 1, (s + 1) & 1);
        compute(s & 1);
    }
    bare_barrier();   // every wave's last reads of the stage buffers are done

    uint8_t* st = smem + wave * (S::WM * S::PITCH);   // this wave's WM x WN bf16 strip
#pragma unroll
    for (int ni = 0; ni < S::NI; ++ni)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int nl = 32 * ni + 8 * r4 + 4 * h;             // strip column of 4
            const int n = n0 + S::WN * wn + nl;
            f32x4 bv = {0.0f, 0.0f, 0.0f, 0.0f};
            if (p.bias) bv = *reinterpret_cast<const f32x4*>(p.bias + n);
#pragma unroll
            for (int mi = 0; mi < S::MI; ++mi) {
                const int ml = 32 * mi + j;                       // strip row
                const int m = m0 + S::WM * wm + ml;
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float z = acc[ni][mi][4 * r4 + e] + bv[e];
                    o[e] = GELU ? gelu(z) : z;
                }
                if (p.res && m < p.M) {
                    const u32x2 rv = *reinterpret_cast<const u32x2*>(p.res + (size_t)m * p.N + n);
                    o[0] += bf16_lo(rv[0]);
                    o[1] += bf16_hi(rv[0]);
                    o[2] += bf16_lo(rv[1]);
                    o[3] += bf16_hi(rv[1]);
                }
                const u32x2 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                *reinterpret_cast<u32x2*>(st + S::pos(ml, nl >> 3) + 8 * h) = pk;
            }
        }
    __syncthreads();

    uint16_t* dst = p.out0;
    int ncol0 = n0 + S::WN * wn;
    if constexpr (EPI == kEpiQkv) {
        const int which = n0 / p.E;   // a tile never straddles Q, K and V (E % NT == 0)
        dst = which == 0 ? p.out0 : (which == 1 ? p.out1 : p.out2);
        ncol0 -= which * p.E;
    }
#pragma unroll 4
    for (int it = 0; it < S::WM * S::CW / kWave; ++it) {
        const int idx = kWave * it + lane;
        const int ml = idx / S::CW, c = idx % S::CW;      // strip row, 16-byte chunk
        const int m = m0 + S::WM * wm + ml;
        if (m >= p.M) continue;
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + S::pos(ml, c));
        size_t off;
        if constexpr (EPI == kEpiQkv) {
            const int nn = ncol0 + 8 * c, hh = nn / p.d, dd = nn - hh * p.d;
            const int b = m / p.L, l = m - b * p.L;
            off = ((size_t)(b * p.H + hh) * p.L + l) * p.d + dd;
        } else {
            off = (size_t)m * p.N + ncol0 + 8 * c;
        }
        *reinterpret_cast<u32x4*>(dst + off) = v;
    }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// y = (x - mean) / sqrt(var + eps) * gamma + beta over each row of E bf16
// values; one wave per RPW consecutive rows (all their loads issued before
// the first reduction, gamma and beta read once per wave), CPL 16-byte
// chunks per lane and row, statistics in fp32 (the mean first, then the
// mean squared deviation from it).
template <int CPL, int RPW>
__global__ __launch_bounds__(kThreads) void rsa_layernorm_bf16(const uint16_t* __restrict__ x,
                                                               const float* __restrict__ gamma,
                                                               const float* __restrict__ beta,
                                                               uint16_t* __restrict__ y, int rows, int E,
                                                               float eps) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const long long row0 = ((long long)blockIdx.x * (kThreads / kWave) + wave) * RPW;
    if (row0 >= rows) return;
    const int nch = E / 8;
    float v[RPW][CPL][8];
    float mean[RPW], rstd[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const bool ok = row0 + i < rows;   // rows past the end: zeros, never stored
        const uint16_t* xr = x + (row0 + i) * E;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ch = lane + kWave * c;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (ok && ch < nch) w = *reinterpret_cast<const u32x4*>(xr + 8 * ch);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[i][c][2 * e] = bf16_lo(w[e]);
                v[i][c][2 * e + 1] = bf16_hi(w[e]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) s += v[i][c][2 * e] + v[i][c][2 * e + 1];
        mean[i] = wave_sum(s) / (float)E;
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        float q = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if (lane + kWave * c < nch) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float dv = v[i][c][e] - mean[i];
                    q += dv * dv;
                }
            }
        }
        rstd[i] = 1.0f / sqrtf(wave_sum(q) / (float)E + eps);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = lane + kWave * c;
        if (ch >= nch) continue;
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + 8 * ch);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + 8 * ch + 4);
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(beta + 8 * ch);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(beta + 8 * ch + 4);
        const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
        const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            if (row0 + i >= rows) continue;
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = pack_bf16x2((v[i][c][2 * e] - mean[i]) * rstd[i] * g[2 * e] + b[2 * e],
                                   (v[i][c][2 * e + 1] - mean[i]) * rstd[i] * g[2 * e + 1] + b[2 * e + 1]);
            *reinterpret_cast<u32x4*>(y + (row0 + i) * E + 8 * ch) = o;
        }
    }
}

// Compute units of the current device (cached per device; threads that
// race on the first call store the same value).
int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int PRO, int EPI, bool GELU>
hipError_t launch_gemm_t(const GemmParams& p0, hipStream_t stream) {
    GemmParams p = p0;
    // 256-row tiles where the widths allow them (a Q/K/V block must not
    // straddle a tile), else 128x128. Between 256 and 192 columns, the one
    // with the shorter schedule: rounds of one workgroup per CU times the
    // tile's share of a 256x256 tile's work (ties go to 256).
    auto fits = [&](int nt) { return p.N % nt == 0 && (EPI != kEpiQkv || p.E % nt == 0); };
    const long long mt = (p.M + kBT - 1) / kBT, cus = device_cus();
    auto cost = [&](int nt) { return (mt * (p.N / nt) + cus - 1) / cus * nt; };
    int nt = 0;
    if (fits(256)) nt = 256;
    if (fits(192) && (nt == 0 || cost(192) < cost(256))) nt = 192;
    if (nt != 0) {
        p.mt = (int)mt;
        p.nt = p.N / nt;
        if (nt == 256)
            hipLaunchKernelGGL((rsa_gemm_bf16_256<PRO, EPI, 256, GELU>), dim3((unsigned)(p.mt * p.nt)), dim3(kBigThreads),
                               0, stream, p);
        else
            hipLaunchKernelGGL((rsa_gemm_bf16_256<PRO, EPI, 192, GELU>), dim3((unsigned)(p.mt * p.nt)), dim3(kBigThreads),
                               0, stream, p);
    } else {
        p.mt = (p.M + kGT - 1) / kGT;
        p.nt = p.N / kGT;
        hipLaunchKernelGGL((rsa_gemm_bf16<PRO, EPI, GELU>), dim3((unsigned)(p.mt * p.nt)), dim3(kThreads), 0, stream,
                           p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(const LinearCall& c, hipStream_t stream) {
    GemmParams p{};
    p.a = static_cast<const uint16_t*>(c.a);
    p.w = static_cast<const uint16_t*>(c.w);
    p.bias = c.bias;
    p.res = static_cast<const uint16_t*>(c.residual);
    p.out0 = static_cast<uint16_t*>(c.out0);
    p.out1 = static_cast<uint16_t*>(c.out1);
    p.out2 = static_cast<uint16_t*>(c.out2);
    p.M = c.M;
    p.N = c.N;
    p.K = c.K;
    p.L = c.L;
    p.H = c.H;
    p.d = c.d;
    p.E = c.N / 3;
    // GeLU is offered on the row layout only (the first MLP product)
    if (c.layout != kLinearRows && c.act) return hipErrorInvalidValue;
    if (c.layout == kLinearQkv) return launch_gemm_t<kProRows, kEpiQkv, false>(p, stream);
    if (c.layout == kLinearHeadsIn) return launch_gemm_t<kProHeads, kEpiRows, false>(p, stream);
    if (c.act) return launch_gemm_t<kProRows, kEpiRows, true>(p, stream);
    return launch_gemm_t<kProRows, kEpiRows, false>(p, stream);
}

hipError_t launch_layernorm(const void* x, const float* gamma, const float* beta, int rows, int E, float eps,
                            void* y, hipStream_t stream) {
    const uint16_t* xi = static_cast<const uint16_t*>(x);
    uint16_t* yo = static_cast<uint16_t*>(y);
    const int cpl = (E / 8 + kWave - 1) / kWave;
    // rows per wave so that each lane holds 64 values of x
    auto blocks = [&](int rpw) { return (unsigned)((rows + 4 * rpw - 1) / (4 * rpw)); };
    if (cpl <= 1)
        hipLaunchKernelGGL((rsa_layernorm_bf16<1, 8>), dim3(blocks(8)), dim3(kThreads), 0, stream, xi, gamma, beta,
                           yo, rows, E, eps);
    else if (cpl <= 2)
        hipLaunchKernelGGL((rsa_layernorm_bf16<2, 4>), dim3(blocks(4)), dim3(kThreads), 0, stream, xi, gamma, beta,
                           yo, rows, E, eps);
    else if (cpl <= 4)
        hipLaunchKernelGGL((rsa_layernorm_bf16<4, 2>), dim3(blocks(2)), dim3(kThreads), 0, stream, xi, gamma, beta,
                           yo, rows, E, eps);
    else
        hipLaunchKernelGGL((rsa_layernorm_bf16<8, 1>), dim3(blocks(1)), dim3(kThreads), 0, stream, xi, gamma, beta,
                           yo, rows, E, eps);
    return hipGetLastError();
}

}  // namespace rsa
