// rsa_bwd.hip -- Ring Self-Attention backward for gfx950 (bf16 in/out, fp32
// accumulate).
//
// The review page of "Sequence Parallelism: Making 4D Parallelism Possible"
// (proposed-method section) says gradients also travel the ring. For the
// loss <O, dO> of O = softmax(S) V with S = Q K^T / sqrt(d) the gradients are
//
//   P = exp(S - lse),  D_i = dO_i . O_i,  dP = dO V^T,  dS = P o (dP - D),
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),  dV = P^T dO.
//
// Three kernels, all deterministic (no atomics):
//   rsa_bwd_pre   row statistics: -D_i (times 1 - p with dropout) and
//                 -lse_i * log2(e)                                  (HBM-bound)
//   rsa_bwd_dq    query-stationary: a rank's query tile meets the key chunks
//                 in ring order (as in the forward) and accumulates dQ;
//                 recomputes S, P and dP (3 contractions); when one call
//                 asks for the statistics and dQ together it forms the
//                 statistics itself and rsa_bwd_pre is not launched
//   rsa_bwd_dkdv  key-stationary: a key chunk meets every query chunk in the
//                 order the ring delivers them (query chunk (c + t) mod N at
//                 step t) and accumulates dK and dV -- the sum over query
//                 chunks that the ring performs across devices (4
//                 contractions)
//
// As in the forward, tiles are copied from HBM straight into swizzled LDS
// (global_load_lds), fragments contracted over tile rows come from the
// transposing LDS read, every 32x32 accumulator is reused as the B operand of
// the next contraction, P = exp2(s * log2(e)/sqrt(d) - lse * log2(e)) is one
// FMA and one exp, and the dP accumulator starts at -D so dS = P * acc.

#include <type_traits>

#include "rsa_device.h"
#include "rsa_internal.h"
#include "rsa_tiles.h"

namespace rsa {
namespace {

constexpr int kThreads = 256;
constexpr int kKT = kTileRows;   // rows per LDS tile
constexpr float kLog2e = 1.4426950408889634f;

struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;
    const uint8_t* mask;
    float* stats;   // [2][B*H*L]: -D, then -lse * log2(e)
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    int H, L, N, Lc, BH, nt;   // nt: 128-row tiles per head
    float sl2;                 // log2(e) / sqrt(d)
    float scale;               // 1 / sqrt(d)
    int causal;                // the query at position i sees keys at positions <= i only
    Dropout drop;              // the forward's dropout (drop.p8 == 0: none)
    float dmul;                // -D is stored times dmul (1, or 1 - p with dropout)
    int pre_in_dq;             // the dQ kernel computes and stores the row statistics itself
};

// Sequence position of the u-th query row that key chunk c meets: ring step
// t = u / Lc brings query chunk (c + t) mod N.
__device__ __forceinline__ int ring_pos_rev(int u, int c, int N, int Lc) {
    const int t = u / Lc;
    int n = c + t;
    n -= (n >= N) ? N : 0;
    return n * Lc + (u - t * Lc);
}

// --------------------------------------------------------- row statistics ---
// dO . O over 8 elements (one 16-byte chunk of each row), in the order both
// the preprocess and the dQ kernel that can replace it use.
__device__ __forceinline__ float dot8_bf16(const u32x4& a, const u32x4& g) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += bf16_lo(a[e]) * bf16_lo(g[e]) + bf16_hi(a[e]) * bf16_hi(g[e]);
    return acc;
}

template <int D>
__global__ __launch_bounds__(kThreads) void rsa_bwd_pre(const uint16_t* __restrict__ o,
                                                        const uint16_t* __restrict__ dout,
                                                        const float* __restrict__ lse, float* __restrict__ stats,
                                                        long long rows, float dmul) {
    constexpr int TPR = D / 8;   // lanes per row, 8 elements each
    const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long row = t / TPR;
    const int c = (int)(t % TPR);
    float acc = 0.0f;
    if (row < rows) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(o + row * D + 8 * c);
        const u32x4 g = *reinterpret_cast<const u32x4*>(dout + row * D + 8 * c);
        acc = dot8_bf16(a, g);
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && c == 0) {
        stats[row] = -acc * dmul;
        const float l = lse[row];
        stats[rows + row] = l == -INFINITY ? -INFINITY : -l * kLog2e;   // a row without keys gets P = 0
    }
}

// Copy one fp32 per row for the 64 rows of a tile (rows r -> src + rowoff(r))
// into LDS: one global_load_lds of 4 bytes per lane, issued by one wave.
template <class RowOff>
__device__ __forceinline__ void load_rowvec(uint8_t* lds, const float* src, RowOff rowoff) {
    const int lane = threadIdx.x % kWave;
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(src + rowoff(lane)),
                                     (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// ------------------------------------------------------------------ dQ ---
// Query-stationary, mirror of the forward: 4 waves x 32 query rows; per key
// tile S^T = K Q^T and dP^T = V dO^T (lane <-> query), then
// dQ^T += K^T dS^T with K^T from the transposing read of the same K tile.
// DROP: with dropout, dS = P o (Z o dP - D) for the forward's keep factors Z
// (kept: 1 / (1 - p), dropped: 0). The row statistic then holds -D (1 - p),
// where the dP accumulator starts: dS (1 - p) = P acc for a kept weight and
// P (-D (1 - p)) for a dropped one, and the common factor 1 / (1 - p) is
// applied to dQ at the end. The dropout instances run at two waves per SIMD
// (at three, the keep-decision generator pushed 14 registers into scratch).
// FULL (with or without dropout): no key mask and chunk-aligned tiles, so
// every key tile is whole: no occupancy table is built or consulted, and the
// two 32-key halves of a tile are unrolled (their LDS offsets become
// constants of the read instructions). With the causal mask (FULL and CAUSAL, chunks a multiple
// of 128 rows so that a workgroup's rows lie in one chunk) the visible tiles
// are walked directly: in ring order the row's own chunk comes first, whose
// tiles up to the workgroup's last row are visible (the last two of them
// partly, masked per element), then the earlier chunks, whole; the later
// chunks are hidden.
template <int D, bool CONTIG, bool CAUSAL, bool DROP = false, bool FULL = false, bool KSPLIT = false>
__global__ __launch_bounds__(kThreads, D == 64 ? (DROP ? 2 : 3) : 1) void rsa_bwd_dq(BwdParams p) {
    static_assert(!FULL || CONTIG, "whole tiles need chunk-aligned, unmasked ranges");
    static_assert(!KSPLIT || (!CAUSAL && !DROP), "key-split instances: plain launches");
    using T = DirectTile<D>;
    constexpr int BUF = 2 * T::BYTES;   // K, V
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * BUF];
    __shared__ uint8_t tflag_bytes[FULL ? 4 : kFwdMaxTiles / 4];
    const TileTable tflag{tflag_bytes};

    // causal: the last query tiles see the most keys; dispatch them first
    int qt, bh;
    head_order(blockIdx.x, p.nt, p.BH, CAUSAL, qt, bh);
    if (CAUSAL) qt = p.nt - 1 - qt;
    const int b = bh / p.H;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int j = lane & 31, h = lane >> 5;
    // KSPLIT (small grids): 64 rows per workgroup; waves 0 and 1 take rows
    // 0-31 and 32-63 against keys 0-31 of every tile, waves 2 and 3 the same
    // rows against keys 32-63, and their dQ parts are added at the end
    constexpr int ROWS = KSPLIT ? 64 : 128;
    const int khalf = KSPLIT ? wave >> 1 : 0;
    const int row0 = qt * ROWS;
    const int row = row0 + (KSPLIT ? wave & 1 : wave) * 32 + j;
    const bool row_ok = row < p.L;
    const int n = row0 / p.Lc;
    const int ntile = (p.L + kKT - 1) / kKT;
    if (ntile > kFwdMaxTiles) return;   // the host never launches such a length

    const size_t hoff = (size_t)bh * p.L * D;
    const uint16_t* kh = p.k + hoff;
    const uint16_t* vh = p.v + hoff;
    const uint8_t* mrow = p.mask ? p.mask + (size_t)b * p.L : nullptr;
    const size_t rows_all = (size_t)p.BH * p.L;

    const int qhi = min(row0 + ROWS, p.L) - 1;
    if constexpr (!FULL) {
        tflag.build(ntile, kThreads, [&](int t) {
            const uint32_t f = key_tile_flags(mrow, n, p.N, p.Lc, CONTIG, t * kKT, p.L);
            return CAUSAL ? f & causal_tile_class(t * kKT, min(kKT, p.L - t * kKT), n, p.N, p.Lc, CONTIG, row0, qhi)
                          : f;
        });
    }

    u32x4 qf[D / 16], gf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        u32x4 a = {0u, 0u, 0u, 0u}, g = {0u, 0u, 0u, 0u};
        if (row_ok) {
            a = *reinterpret_cast<const u32x4*>(p.q + hoff + (size_t)row * D + 16 * ks + 8 * h);
            g = *reinterpret_cast<const u32x4*>(p.dout + hoff + (size_t)row * D + 16 * ks + 8 * h);
        }
        qf[ks] = a;
        gf[ks] = g;
    }
    // tail rows get P = 0 through nl2 = -inf
    float nD, nl2;
    if (p.pre_in_dq) {
        // The preprocess for this lane's row, here: this lane holds chunks
        // 2 ks + h of dO (16 bytes each); their dot products with O are
        // combined in the order of the preprocess's lane reduction (chunks c
        // and c + TPR/2 first, ..., the two lane halves last), so the
        // statistics are the same bits.
        float part[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            u32x4 a = {0u, 0u, 0u, 0u};
            if (row_ok) a = *reinterpret_cast<const u32x4*>(p.o + hoff + (size_t)row * D + 16 * ks + 8 * h);
            part[ks] = dot8_bf16(a, gf[ks]);
        }
#pragma unroll
        for (int m = D / 32; m >= 1; m >>= 1)
#pragma unroll
            for (int ks = 0; ks < m; ++ks) part[ks] = part[ks] + part[ks + m];
        const float other = __shfl_xor(part[0], 32);
        const float dsum = h == 0 ? part[0] + other : other + part[0];
        const float l = row_ok ? p.lse[(size_t)bh * p.L + row] : -INFINITY;
        nD = row_ok ? -dsum * p.dmul : 0.0f;
        nl2 = l == -INFINITY ? -INFINITY : -l * kLog2e;
        if (row_ok && h == 0 && khalf == 0) {
            p.stats[(size_t)bh * p.L + row] = nD;
            p.stats[rows_all + (size_t)bh * p.L + row] = nl2;
        }
    } else {
        nD = row_ok ? p.stats[(size_t)bh * p.L + row] : 0.0f;
        nl2 = row_ok ? p.stats[rows_all + (size_t)bh * p.L + row] : -INFINITY;
    }
    const float nD0 = nD;   // the dP accumulator's start

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

    // the row data above has landed (waited for here, so that the compiler
    // keeps no wait for it inside the tile loop); tile flags visible
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    uint32_t voff[T::IPW];
    T::row_offsets(voff);
    auto load = [&](int t, int bi) {
        const int v0 = t * kKT;
        uint8_t* kb = smem + bi * BUF;
        if constexpr (CONTIG) {
            const size_t pos0 = (size_t)ring_pos(v0, n, p.N, p.Lc) * D;
            T::load_rows(kb, kh + pos0, voff);
            T::load_rows(kb + T::BYTES, vh + pos0, voff);
        } else {
            auto off = [&](int r) -> size_t {
                const int vk = v0 + r;
                return vk < p.L ? (size_t)ring_pos(vk, n, p.N, p.Lc) * D : 0;
            };
            T::load(kb, [&](int r) { return kh + off(r); });
            T::load(kb + T::BYTES, [&](int r) { return vh + off(r); });
        }
    };
    // FULL and CAUSAL: tiles 0 .. lo/64 + 1 of the own chunk (lo = the
    // workgroup's first row within it), then tiles tpc .. (n + 1) tpc - 1
    const int tpc = p.Lc / kKT;
    const int tdiag = (row0 - n * p.Lc) / kKT;               // first partly visible tile
    const int tend = (FULL && CAUSAL) ? (n + 1) * tpc : ntile;
    auto next_tile = [&](int t) {
        ++t;
        if constexpr (FULL && CAUSAL) {
            if (t == tdiag + 2) t = tpc;
        } else if constexpr (!FULL) {
            while (t < ntile && !(tflag.get(t) & 1)) ++t;
        }
        return t;
    };

    // Two LDS buffers: the copy of tile t+1 is issued right after the barrier
    // that opens tile t and lands while t is computed. (Three buffers, the
    // copy of t+2 in flight until t+1 opens, need 100 KB of LDS per
    // workgroup at d = 64, leave one workgroup per CU and measured 3.7x
    // slower.)
    int t = next_tile(-1);
    auto body = [&](auto cb_c) -> bool {
        constexpr int CB = decltype(cb_c)::value;
        vm_wait<0>();
        bare_barrier();   // every wave's part of tile t landed, tile t-1 consumed
        const int tn = next_tile(t);
        if (tn < tend) load(tn, CB ^ 1);
        const uint8_t* kb = smem + CB * BUF;
        const uint8_t* vb = kb + T::BYTES;
        // key acc_row(r, h) = 8 (r / 4) + 4 h + r % 4 of a 32-key half: after one
        // shift by 4 h every bit position is a constant
        const bool partial = FULL ? (CAUSAL && t >= tdiag && t < tpc) : !(tflag.get(t) & 2);
        const uint64_t bits =
            (!FULL && partial) ? key_tile_bits(mrow, n, p.N, p.Lc, CONTIG, t * kKT, p.L) >> (4 * h) : ~0ull;
        // causal: key i of a chunk-aligned tile sits at position kp0 + i
        const int kp0 = (CAUSAL && CONTIG) ? ring_pos(t * kKT, n, p.N, p.Lc) : 0;
        auto half = [&](int kb2) __attribute__((always_inline)) {
            // ---- S^T = K Q^T and dP^T - D = V dO^T - D for keys 32 kb2 .. +32
            f32x16 s, dp;
            {
                u32x4 kfr[D / 16], vfr[D / 16];
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    kfr[ks] = T::chunk(kb, 32 * kb2 + j, 2 * ks + h);
                    vfr[ks] = T::chunk(vb, 32 * kb2 + j, 2 * ks + h);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s[r] = 0.0f;
                    dp[r] = nD0;
                }
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    s = mfma_32x32x16_bf16(kfr[ks], qf[ks], s);
                    dp = mfma_32x32x16_bf16(vfr[ks], gf[ks], dp);
                }
            }
            if constexpr (DROP) {
                // register r holds key 8 (r / 4) + 4 h + r % 4 of this 32-key
                // half: byte r % 4 of word r / 4 of its keep bytes
                if constexpr (CONTIG) {
                    const int jb = (ring_pos(t * kKT, n, p.N, p.Lc) >> 5) + kb2;
                    const u32x4 x = dropout_bytes(p.drop, jb, h, row, bh);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dp[r] = ((x[r >> 2] >> (8 * (r & 3))) & 0xffu) >= p.drop.p8 ? dp[r] : nD;
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int vk = t * kKT + 32 * kb2 + acc_row(r, h);
                        const bool keep = vk >= p.L || dropout_keep(p.drop, row, ring_pos(vk, n, p.N, p.Lc), bh);
                        dp[r] = keep ? dp[r] : nD;
                    }
                }
            }
            if constexpr (!FULL || CAUSAL) {
                if (!FULL && bits != ~0ull) {
                    const uint32_t hb = (uint32_t)(bits >> (32 * kb2));
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (!((hb >> (8 * (r >> 2) + (r & 3))) & 1u)) s[r] = -INFINITY;
                }
                if (CAUSAL && partial) {   // keys after this lane's row
                    const int rel = row - kp0 - 32 * kb2 - 4 * h;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int i = 8 * (r >> 2) + (r & 3);
                        bool hide;
                        if constexpr (CONTIG) {
                            hide = i > rel;
                        } else {
                            const int vk = t * kKT + 32 * kb2 + 4 * h + i;
                            hide = vk < p.L && ring_pos(vk, n, p.N, p.Lc) > row;
                        }
                        if (hide) s[r] = -INFINITY;
                    }
                }
            }
            uint32_t pk[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p0 = fast_exp2(fmaf(s[2 * i], p.sl2, nl2));
                const float p1 = fast_exp2(fmaf(s[2 * i + 1], p.sl2, nl2));
                pk[i] = pack_bf16x2(p0 * dp[2 * i], p1 * dp[2 * i + 1]);
            }
            // ---- dQ^T += K^T dS^T over these 32 keys (K^T: transposing read)
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
                const u32x4 bfrag = {pk[4 * hs], pk[4 * hs + 1], pk[4 * hs + 2], pk[4 * hs + 3]};
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    acc[db] = mfma_32x32x16_bf16(T::tfrag(kb, 32 * kb2 + 16 * hs, 32 * db), bfrag, acc[db]);
            }
        };
        if constexpr (KSPLIT) {
            half(khalf);
        } else if constexpr (FULL) {
            half(0);
            half(1);
        } else {
            // two 32-key halves in turn, to bound the live registers
#pragma unroll 1
            for (int kb2 = 0; kb2 < 2; ++kb2) half(kb2);
        }
        t = tn;
        return t >= tend;
    };

    if (t < tend) {
        using C0 = std::integral_constant<int, 0>;
        using C1 = std::integral_constant<int, 1>;
        load(t, 0);
        while (true) {
            if (body(C0{})) break;
            if (body(C1{})) break;
        }
    }

    if constexpr (KSPLIT) {
        // waves 2 and 3 hand their part of dQ to waves 0 and 1
        constexpr int XS = (D / 32) * 16;   // floats per lane: its dQ part
        static_assert(2 * kWave * XS * sizeof(float) <= sizeof(smem), "merge area inside the tile buffers");
        float* xs = reinterpret_cast<float*>(smem) + ((wave & 1) * kWave + lane) * XS;
        __syncthreads();   // every wave is done with the tile buffers
        if (khalf == 1) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    *reinterpret_cast<f32x4*>(xs + 16 * db + 4 * r4) =
                        f32x4{acc[db][4 * r4], acc[db][4 * r4 + 1], acc[db][4 * r4 + 2], acc[db][4 * r4 + 3]};
        }
        __syncthreads();
        if (khalf == 1) return;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(xs + 16 * db + 4 * r4);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[db][4 * r4 + e] += x[e];
            }
    }

    if (row_ok) {
        uint16_t* out = p.dq + hoff + (size_t)row * D;
        const float qs = DROP ? p.scale * p.drop.scale : p.scale;   // dropout: the kept weights' 1 / (1 - p)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const u32x2 w = {pack_bf16x2(acc[db][4 * r4] * qs, acc[db][4 * r4 + 1] * qs),
                                 pack_bf16x2(acc[db][4 * r4 + 2] * qs, acc[db][4 * r4 + 3] * qs)};
                *reinterpret_cast<u32x2*>(out + 32 * db + 8 * r4 + 4 * h) = w;
            }
    }
}

// ---------------------------------------------------------------- dK dV ---
// Key-stationary: 4 waves x 32 keys, K and V fragments in registers. Per
// query tile (64 rows, in ring delivery order): S = Q K^T and dP - D =
// dO V^T (lane <-> key, registers <-> query rows), P and dS elementwise, then
// dV^T += dO^T P and dK^T += Q^T dS, with Q^T and dO^T from the transposing
// read of the same Q and dO tiles.
// (The causal instance runs at two waves per SIMD: its per-element mask of
// the diagonal tiles pushes three waves' worth of registers into spills,
// which measured 21% slower.)
// DROP: dropout of the forward's weights. The lanes of this kernel hold keys
// and its registers query rows, the transpose of the forward's layout, so
// the keep bytes are exchanged through LDS: per query tile each lane draws
// the two counters of one query row (the wave's 32 keys are one 32-key
// block, two halves), writes their 32 bytes into the wave's table, and each
// lane then reads its key's byte for its 32 rows. dV accumulates P over the
// kept weights and dK the dS (1 - p) of the dQ kernel; both take the factor
// 1 / (1 - p) at the end.
template <int D, bool CONTIG, bool CAUSAL, bool DROP = false>
__global__ __launch_bounds__(kThreads, D == 64 ? ((CAUSAL || DROP) ? 2 : 3) : 1) void rsa_bwd_dkdv(BwdParams p) {
    using T = DirectTile<D>;
    constexpr int NBUF = 3;
    constexpr int ROWV = 2 * kKT * 4;             // -D and -lse*log2(e) for 64 rows
    constexpr int BUF = 2 * T::BYTES + ROWV;      // Q, dO, row statistics
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NBUF * BUF];
    // per wave: keep words [half hh][word w][row u]
    __shared__ __attribute__((aligned(16))) uint32_t keep_tab[DROP ? 4 * 2 * 4 * kKT : 1];

    // causal: the first key tiles are seen by the most rows (tile 0 first)
    int kt, bh;
    head_order(blockIdx.x, p.nt, p.BH, CAUSAL, kt, bh);
    const int b = bh / p.H;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int j = lane & 31, h = lane >> 5;
    const int key0 = kt * 128;
    const int key = key0 + wave * 32 + j;
    const bool key_in = key < p.L;
    const bool key_ok = key_in && (p.mask == nullptr || p.mask[(size_t)b * p.L + key] != 0);
    const int c = key0 / p.Lc;   // key chunk of the tile's first key
    const size_t hoff = (size_t)bh * p.L * D;
    const size_t rows_all = (size_t)p.BH * p.L;
    const float* nDh = p.stats + (size_t)bh * p.L;
    const float* nLh = p.stats + rows_all + (size_t)bh * p.L;

    if (!__syncthreads_or(key_ok)) {
        // no valid key in this tile: its gradients are exactly zero
        if (key_in) {
            const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = h; e < D / 8; e += 2) {
                *reinterpret_cast<u32x4*>(p.dk + hoff + (size_t)key * D + 8 * e) = z;
                *reinterpret_cast<u32x4*>(p.dv + hoff + (size_t)key * D + 8 * e) = z;
            }
        }
        return;
    }

    u32x4 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        u32x4 a = {0u, 0u, 0u, 0u}, g = {0u, 0u, 0u, 0u};
        if (key_in) {
            a = *reinterpret_cast<const u32x4*>(p.k + hoff + (size_t)key * D + 16 * ks + 8 * h);
            g = *reinterpret_cast<const u32x4*>(p.v + hoff + (size_t)key * D + 16 * ks + 8 * h);
        }
        kf[ks] = a;
        vf[ks] = g;
    }

    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk[db][r] = 0.0f;
            dv[db][r] = 0.0f;
        }

    // Query tiles in ring delivery order. Causal with chunk-aligned tiles:
    // rows before this workgroup's first key see none of its keys, and in
    // delivery order (query chunk c, c + 1, ..., N - 1, 0, ..., c - 1) the
    // visible rows form one run, from the tile holding row key0 to the end
    // of chunk N - 1. Otherwise every tile is visited.
    int tbeg = 0, ntq = (p.L + kKT - 1) / kKT;
    if (CONTIG && CAUSAL) {
        tbeg = (key0 - c * p.Lc) / kKT;
        ntq = (p.N - c) * (p.Lc / kKT);
    }
    const int key_last = min(key0 + 127, p.L - 1);
    // The K and V fragments have landed (waited for here, so that the
    // compiler keeps no wait for them inside the tile loop).
    __builtin_amdgcn_s_waitcnt(0);
    uint32_t voff[T::IPW];
    T::row_offsets(voff);
    const uint32_t roff = (uint32_t)(4 * lane);
    // Copy query tile t into buffer bi. Rows past the sequence read row 0
    // (finite data) and get -lse*log2(e) = -inf, so their P is 0.
    auto load = [&](int t, int bi) {
        const int u0 = t * kKT;
        uint8_t* qb = smem + bi * BUF;
        uint8_t* gb = qb + T::BYTES;
        uint8_t* rb = gb + T::BYTES;
        if constexpr (CONTIG) {
            const int pos0 = ring_pos_rev(u0, c, p.N, p.Lc);
            T::load_rows(qb, p.q + hoff + (size_t)pos0 * D, voff);
            T::load_rows(gb, p.dout + hoff + (size_t)pos0 * D, voff);
            if (wave == 0) dma_copy4(nDh + pos0, roff, lds_addr(rb));
            if (wave == 1) dma_copy4(nLh + pos0, roff, lds_addr(rb + kKT * 4));
        } else {
            auto pos = [&](int r) -> int {
                const int u = u0 + r;
                return u < p.L ? ring_pos_rev(u, c, p.N, p.Lc) : 0;
            };
            T::load(qb, [&](int r) { return p.q + hoff + (size_t)pos(r) * D; });
            T::load(gb, [&](int r) { return p.dout + hoff + (size_t)pos(r) * D; });
            if (wave == 0) load_rowvec(rb, nDh, pos);
            if (wave == 1) load_rowvec(rb + kKT * 4, nLh, pos);
        }
    };
    // Rows past the sequence get P = 0. Run by wave 1, which issued the copy
    // of these values, after its own wait for that copy (so its write lands
    // last).
    auto fix_tail = [&](int t, int bi) {
        if (CONTIG || t >= ntq || t * kKT + kKT <= p.L || wave != 1) return;
        float* nl = reinterpret_cast<float*>(smem + bi * BUF + 2 * T::BYTES) + kKT;
        if (t * kKT + lane >= p.L) nl[lane] = -INFINITY;
    };

    // This wave's copies per query tile: Q and dO tiles, plus one row vector
    // for waves 0 and 1. Wait until only one tile's copies remain in flight.
    auto wait_tile_copies_but_one = [&]() {
        if (wave < 2)
            vm_wait<2 * T::IPW + 1>();
        else
            vm_wait<2 * T::IPW>();
    };

    auto body = [&](auto cb_c, int t) -> bool {
        constexpr int CB = decltype(cb_c)::value;
        constexpr int FB = (CB + 2) % NBUF;
        const uint8_t* qb = smem + CB * BUF;
        const uint8_t* gb = qb + T::BYTES;
        const float* nDs = reinterpret_cast<const float*>(gb + T::BYTES);
        const float* nLs = nDs + kKT;
        if (t + 2 < ntq) load(t + 2, FB);
        // causal: does some row of this tile come before some key of the
        // workgroup (then rows are masked per element)?
        const int pos0c = (CAUSAL && CONTIG) ? ring_pos_rev(t * kKT, c, p.N, p.Lc) : 0;
        const bool cmask = CAUSAL && (!CONTIG || pos0c < key_last);
        uint32_t* ktab = keep_tab + (DROP ? wave * (2 * 4 * kKT) : 0);
        if constexpr (DROP) {
            // lane l draws the keep bytes of query row l of the tile for the
            // wave's 32-key block (both halves) and writes them to its table
            const int u = t * kKT + lane;
            if (u < p.L) {
                const int qpos = CONTIG ? ring_pos_rev(t * kKT, c, p.N, p.Lc) + lane : ring_pos_rev(u, c, p.N, p.Lc);
                const int jb = (key0 >> 5) + wave;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const u32x4 x = dropout_bytes(p.drop, jb, hh, qpos, bh);
#pragma unroll
                    for (int w = 0; w < 4; ++w) ktab[(hh * 4 + w) * kKT + lane] = x[w];
                }
            }
        }
        // two 32-query halves in turn, to bound the live registers
#pragma unroll
        for (int qb2 = 0; qb2 < 2; ++qb2) {
            // ---- S = Q K^T and dP - D = dO V^T - D for queries 32 qb2 .. +32
            f32x16 s, dp;
            {
                u32x4 qfr[D / 16], gfr[D / 16];
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    qfr[ks] = T::chunk(qb, 32 * qb2 + j, 2 * ks + h);
                    gfr[ks] = T::chunk(gb, 32 * qb2 + j, 2 * ks + h);
                }
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {   // dP accumulators start at -D of their rows
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(nDs + 32 * qb2 + 8 * r4 + 4 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dp[4 * r4 + e] = d4[e];
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    s = mfma_32x32x16_bf16(qfr[ks], kf[ks], s);
                    dp = mfma_32x32x16_bf16(gfr[ks], vf[ks], dp);
                }
            }
            u32x4 qtf[2][D / 32], gtf[2][D / 32];
#pragma unroll
            for (int hs = 0; hs < 2; ++hs)
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    qtf[hs][db] = T::tfrag(qb, 32 * qb2 + 16 * hs, 32 * db);
                    gtf[hs][db] = T::tfrag(gb, 32 * qb2 + 16 * hs, 32 * db);
                }
            if (cmask) {   // causal: rows before this lane's key see nothing of it
                const int rel = key - pos0c - 32 * qb2 - 4 * h;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int u = 8 * (r >> 2) + (r & 3);   // row 32 qb2 + 4 h + u of the tile
                    bool hide;
                    if constexpr (CONTIG) {
                        hide = rel > u;
                    } else {
                        const int uu = t * kKT + 32 * qb2 + 4 * h + u;
                        hide = uu < p.L && key > ring_pos_rev(uu, c, p.N, p.Lc);
                    }
                    if (hide) s[r] = -INFINITY;
                }
            }
            uint32_t pp[8], pd[8];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(nLs + 32 * qb2 + 8 * r4 + 4 * h);
                float pv[4], dsv[4];
                if constexpr (DROP) {
                    // keep bytes of rows 32 qb2 + 8 r4 + 4 h + {0..3} for this lane's key
                    const u32x4 kw = *reinterpret_cast<const u32x4*>(
                        ktab + (((j >> 2) & 1) * 4 + ((j >> 3) & 3)) * kKT + 32 * qb2 + 8 * r4 + 4 * h);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(nDs + 32 * qb2 + 8 * r4 + 4 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * r4 + e;
                        const bool keep = ((kw[e] >> (8 * (j & 3))) & 0xffu) >= p.drop.p8;
                        const float pr = fast_exp2(fmaf(s[r], p.sl2, l4[e]));
                        pv[e] = keep ? pr : 0.0f;
                        dsv[e] = pr * (keep ? dp[r] : d4[e]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * r4 + e;
                        pv[e] = fast_exp2(fmaf(s[r], p.sl2, l4[e]));
                        dsv[e] = pv[e] * dp[r];
                    }
                }
                pp[2 * r4] = pack_bf16x2(pv[0], pv[1]);
                pp[2 * r4 + 1] = pack_bf16x2(pv[2], pv[3]);
                pd[2 * r4] = pack_bf16x2(dsv[0], dsv[1]);
                pd[2 * r4 + 1] = pack_bf16x2(dsv[2], dsv[3]);
            }
            // ---- dV^T += dO^T P and dK^T += Q^T dS over these 32 queries
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
                const u32x4 bp = {pp[4 * hs], pp[4 * hs + 1], pp[4 * hs + 2], pp[4 * hs + 3]};
                const u32x4 bd = {pd[4 * hs], pd[4 * hs + 1], pd[4 * hs + 2], pd[4 * hs + 3]};
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    dv[db] = mfma_32x32x16_bf16(gtf[hs][db], bp, dv[db]);
                    dk[db] = mfma_32x32x16_bf16(qtf[hs][db], bd, dk[db]);
                }
            }
        }
        if (t + 1 >= ntq) return true;
        // tile t+1 landed (this wave's copies of t+2 may stay in flight)
        if (t + 2 < ntq)
            wait_tile_copies_but_one();
        else
            vm_wait<0>();
        fix_tail(t + 1, (CB + 1) % NBUF);
        bare_barrier();   // tile t+1 visible; buffer CB free for tile t+3
        return false;
    };

    load(tbeg, 0);
    if (ntq > tbeg + 1) {
        load(tbeg + 1, 1);
        wait_tile_copies_but_one();
    } else {
        vm_wait<0>();
    }
    fix_tail(tbeg, 0);
    bare_barrier();
    {
        using C0 = std::integral_constant<int, 0>;
        using C1 = std::integral_constant<int, 1>;
        using C2 = std::integral_constant<int, 2>;
        int t = tbeg;
        while (true) {
            if (body(C0{}, t++)) break;
            if (body(C1{}, t++)) break;
            if (body(C2{}, t++)) break;
        }
    }

    if (key_in) {
        // a padded key's lane accumulated only into its own columns; it is 0
        const float zs = DROP ? p.drop.scale : 1.0f;   // dropout: the kept weights' 1 / (1 - p)
        const float sk = key_ok ? p.scale * zs : 0.0f;
        const float sv = key_ok ? zs : 0.0f;
        uint16_t* okk = p.dk + hoff + (size_t)key * D;
        uint16_t* ovv = p.dv + hoff + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int dcol = 32 * db + 8 * r4 + 4 * h;
                u32x2 wk = {pack_bf16x2(dk[db][4 * r4] * sk, dk[db][4 * r4 + 1] * sk),
                            pack_bf16x2(dk[db][4 * r4 + 2] * sk, dk[db][4 * r4 + 3] * sk)};
                u32x2 wv = {pack_bf16x2(dv[db][4 * r4] * sv, dv[db][4 * r4 + 1] * sv),
                            pack_bf16x2(dv[db][4 * r4 + 2] * sv, dv[db][4 * r4 + 3] * sv)};
                if (!key_ok) {   // inf * 0 would be NaN
                    wk = u32x2{0u, 0u};
                    wv = u32x2{0u, 0u};
                }
                *reinterpret_cast<u32x2*>(okk + dcol) = wk;
                *reinterpret_cast<u32x2*>(ovv + dcol) = wv;
            }
    }
}

BwdParams make_params(const BackwardCall& c) {
    BwdParams p{};
    p.q = static_cast<const uint16_t*>(c.q);
    p.k = static_cast<const uint16_t*>(c.k);
    p.v = static_cast<const uint16_t*>(c.v);
    p.o = static_cast<const uint16_t*>(c.out);
    p.dout = static_cast<const uint16_t*>(c.dout);
    p.lse = c.lse;
    p.mask = c.mask;
    p.stats = c.stats;
    p.dq = static_cast<uint16_t*>(c.dq);
    p.dk = static_cast<uint16_t*>(c.dk);
    p.dv = static_cast<uint16_t*>(c.dv);
    p.H = c.H;
    p.L = c.L;
    p.N = c.N;
    p.Lc = c.L / c.N;
    p.BH = c.B * c.H;
    p.nt = (c.L + 127) / 128;
    p.scale = (float)(1.0 / __builtin_sqrt((double)c.d));
    p.causal = c.causal ? 1 : 0;
    p.sl2 = (float)(1.4426950408889634 / __builtin_sqrt((double)c.d));
    p.drop.p8 = c.drop_p8;
    p.drop.seed_lo = (uint32_t)c.drop_seed;
    p.drop.seed_hi = (uint32_t)(c.drop_seed >> 32);
    p.drop.offset = c.drop_offset;
    p.drop.scale = (float)(256.0 / (256.0 - (double)c.drop_p8));
    p.drop.keep = (float)((256.0 - (double)c.drop_p8) / 256.0);
    p.dmul = c.drop_p8 != 0 ? p.drop.keep : 1.0f;
    p.pre_in_dq = 0;
    return p;
}

template <int D>
hipError_t launch_t(const BackwardCall& c, int stages, hipStream_t stream) {
    BwdParams p = make_params(c);
    const long long rows = (long long)p.BH * c.L;
    const bool contig = (p.Lc % kKT) == 0;
    // Both stages in one call: the dQ kernel, which holds each row's dO
    // anyway, forms the row statistics itself (one launch less).
    p.pre_in_dq = (stages & kBwdStagePre) && (stages & kBwdStageDq) ? 1 : 0;
    if ((stages & kBwdStagePre) && !p.pre_in_dq) {
        const long long threads = rows * (D / 8);
        hipLaunchKernelGGL((rsa_bwd_pre<D>), dim3((unsigned)((threads + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                           stream, p.o, p.dout, p.lse, p.stats, rows, p.dmul);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const unsigned blocks = (unsigned)((long long)p.nt * p.BH);
    if (p.drop.p8 != 0u) {
        if (stages & kBwdStageDq) {
            if (contig && !p.causal && p.mask == nullptr)
                hipLaunchKernelGGL((rsa_bwd_dq<D, true, false, true, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
            else if (contig && !p.causal)
                hipLaunchKernelGGL((rsa_bwd_dq<D, true, false, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
            else if (!p.causal)
                hipLaunchKernelGGL((rsa_bwd_dq<D, false, false, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
            else if (contig)
                hipLaunchKernelGGL((rsa_bwd_dq<D, true, true, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
            else
                hipLaunchKernelGGL((rsa_bwd_dq<D, false, true, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (stages & kBwdStageDkDv) {
            if (contig && !p.causal)
                hipLaunchKernelGGL((rsa_bwd_dkdv<D, true, false, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
            else if (!p.causal)
                hipLaunchKernelGGL((rsa_bwd_dkdv<D, false, false, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
            else if (contig)
                hipLaunchKernelGGL((rsa_bwd_dkdv<D, true, true, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
            else
                hipLaunchKernelGGL((rsa_bwd_dkdv<D, false, true, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if (stages & kBwdStageDq) {
        if (D == 64 && contig && !p.causal && blocks <= 2 * kCUs) {
            // few workgroups (at most two per CU): 64 rows per workgroup,
            // each tile's keys split between two wave pairs
            if constexpr (D == 64) {
                BwdParams pq = p;
                pq.nt = (c.L + 63) / 64;
                const dim3 grid((unsigned)((long long)pq.nt * p.BH));
                if (p.mask == nullptr)
                    hipLaunchKernelGGL((rsa_bwd_dq<D, true, false, false, true, true>), grid, dim3(kThreads), 0, stream,
                                       pq);
                else
                    hipLaunchKernelGGL((rsa_bwd_dq<D, true, false, false, false, true>), grid, dim3(kThreads), 0,
                                       stream, pq);
            }
        } else if (contig && !p.causal && p.mask == nullptr)
            hipLaunchKernelGGL((rsa_bwd_dq<D, true, false, false, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
        else if (contig && p.causal && p.mask == nullptr && p.Lc % 128 == 0)
            hipLaunchKernelGGL((rsa_bwd_dq<D, true, true, false, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
        else if (contig && !p.causal)
            hipLaunchKernelGGL((rsa_bwd_dq<D, true, false>), dim3(blocks), dim3(kThreads), 0, stream, p);
        else if (!p.causal)
            hipLaunchKernelGGL((rsa_bwd_dq<D, false, false>), dim3(blocks), dim3(kThreads), 0, stream, p);
        else if (contig)
            hipLaunchKernelGGL((rsa_bwd_dq<D, true, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((rsa_bwd_dq<D, false, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (stages & kBwdStageDkDv) {
        if (contig && !p.causal)
            hipLaunchKernelGGL((rsa_bwd_dkdv<D, true, false>), dim3(blocks), dim3(kThreads), 0, stream, p);
        else if (!p.causal)
            hipLaunchKernelGGL((rsa_bwd_dkdv<D, false, false>), dim3(blocks), dim3(kThreads), 0, stream, p);
        else if (contig)
            hipLaunchKernelGGL((rsa_bwd_dkdv<D, true, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((rsa_bwd_dkdv<D, false, true>), dim3(blocks), dim3(kThreads), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_backward(const BackwardCall& c, int stages, hipStream_t stream) {
    if (!c.bf16) return launch_backward_f32(c, stages, stream);
    if (c.d == 64) return launch_t<64>(c, stages, stream);
    return launch_t<128>(c, stages, stream);
}

}  // namespace rsa
