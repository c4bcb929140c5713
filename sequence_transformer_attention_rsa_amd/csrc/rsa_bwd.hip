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
//   rsa_bwd_pre   D_i = rowsum(dO o O)                         (HBM-bound)
//   rsa_bwd_dq    query-stationary: a rank's query tile meets the key chunks
//                 in ring order (as in the forward) and accumulates dQ;
//                 recomputes S, P, dP from lse (3 contractions)
//   rsa_bwd_dkdv  key-stationary: a key chunk meets every query chunk in the
//                 order the ring delivers them (query chunk (c + t) mod N at
//                 step t) and accumulates dK and dV -- the sum over query
//                 chunks that the ring performs across devices (4
//                 contractions)
// Layout tricks as in the forward: every 32x32 accumulator is reused as the
// B operand of the next contraction; operands contracted over tile rows are
// staged transposed in LDS.

#include "rsa_device.h"
#include "rsa_internal.h"
#include "rsa_tiles.h"

namespace rsa {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;
    const uint8_t* mask;
    float* delta;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    int H, L, N, Lc, BH, nt;   // nt: 128-row tiles per head
    float sl2;                 // log2(e) / sqrt(d)
    float scale;               // 1 / sqrt(d)
    int contiguous;            // Lc % 64 == 0
};

// Sequence position of the u-th query row that key chunk c meets: ring step
// t = u / Lc brings query chunk (c + t) mod N.
__device__ __forceinline__ int ring_pos_rev(int u, int c, int N, int Lc) {
    const int t = u / Lc;
    int n = c + t;
    n -= (n >= N) ? N : 0;
    return n * Lc + (u - t * Lc);
}

// log2-domain lse, +inf for rows without a valid key so that P = 0 there.
__device__ __forceinline__ float lse_log2(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// ------------------------------------------------------------ D = rowsum ---
template <int D>
__global__ __launch_bounds__(kThreads) void rsa_bwd_pre(const uint16_t* __restrict__ o,
                                                        const uint16_t* __restrict__ dout, float* __restrict__ delta,
                                                        long long rows) {
    constexpr int TPR = D / 8;   // lanes per row, 8 elements each
    const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long row = t / TPR;
    const int c = (int)(t % TPR);
    float acc = 0.0f;
    if (row < rows) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(o + row * D + 8 * c);
        const u32x4 g = *reinterpret_cast<const u32x4*>(dout + row * D + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += bf16_lo(a[e]) * bf16_lo(g[e]) + bf16_hi(a[e]) * bf16_hi(g[e]);
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && c == 0) delta[row] = acc;
}

// ------------------------------------------------------------------ dQ ---
template <int D>
struct DqSmem {
    static constexpr int K_OFF = 0;
    static constexpr int V_OFF = K_OFF + RowTile<D>::ELEMS;
    static constexpr int KT_OFF = V_OFF + RowTile<D>::ELEMS;
    static constexpr int BUF = KT_OFF + TransTile<D>::ELEMS;
};

template <int D>
__global__ __launch_bounds__(kThreads) void rsa_bwd_dq(BwdParams p) {
    using S = DqSmem<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * S::BUF];
    __shared__ uint8_t tflag[kFwdMaxTiles];

    const int lid = xcd_remap(blockIdx.x, p.nt * p.BH);
    const int qt = lid % p.nt, bh = lid / p.nt, b = bh / p.H;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int j = lane & 31, h = lane >> 5;
    const int row0 = qt * 128;
    const int row = row0 + wave * 32 + j;
    const bool row_ok = row < p.L;
    const int n = row0 / p.Lc;
    const int ntile = (p.L + kTileRows - 1) / kTileRows;
    if (ntile > kFwdMaxTiles) return;   // the host never launches such a length

    const size_t hoff = (size_t)bh * p.L * D;
    const uint16_t* kh = p.k + hoff;
    const uint16_t* vh = p.v + hoff;
    const uint8_t* mrow = p.mask ? p.mask + (size_t)b * p.L : nullptr;
    const bool contig = p.contiguous != 0;

    for (int t = threadIdx.x; t < ntile; t += kThreads)
        tflag[t] = key_tile_flags(mrow, n, p.N, p.Lc, contig, t * kTileRows, p.L);

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
    const float lse2 = row_ok ? lse_log2(p.lse[(size_t)bh * p.L + row]) : INFINITY;
    const float Di = row_ok ? p.delta[(size_t)bh * p.L + row] : 0.0f;

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

    __syncthreads();

    RowTile<D> kst, vst;
    TransTile<D> ktst;
    auto load = [&](int t) {
        const int v0 = t * kTileRows;
        const int pos0 = contig ? ring_pos(v0, n, p.N, p.Lc) : 0;
        auto kptr = [&](int r) -> const uint16_t* {
            const int vk = v0 + r;
            if (vk >= p.L) return nullptr;
            return kh + (size_t)(contig ? pos0 + r : ring_pos(vk, n, p.N, p.Lc)) * D;
        };
        auto vptr = [&](int r) -> const uint16_t* {
            const int vk = v0 + r;
            if (vk >= p.L) return nullptr;
            return vh + (size_t)(contig ? pos0 + r : ring_pos(vk, n, p.N, p.Lc)) * D;
        };
        kst.load(kptr);
        vst.load(vptr);
        ktst.load(kptr);
    };
    auto store = [&](uint16_t* buf) {
        kst.store(buf + S::K_OFF);
        vst.store(buf + S::V_OFF);
        ktst.store(buf + S::KT_OFF);
    };

    int t = 0;
    while (t < ntile && !(tflag[t] & 1)) ++t;
    int buf = 0;
    if (t < ntile) {
        load(t);
        store(smem);
    }
    while (t < ntile) {
        int tn = t + 1;
        while (tn < ntile && !(tflag[tn] & 1)) ++tn;
        if (tn < ntile) load(tn);
        __syncthreads();
        const uint16_t* base = smem + buf * S::BUF;
        const uint16_t* ks_ = base + S::K_OFF;
        const uint16_t* vs_ = base + S::V_OFF;
        const uint16_t* kts = base + S::KT_OFF;

        f32x16 s[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[kb][r] = 0.0f;
                dp[kb][r] = 0.0f;
            }
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                s[kb] = mfma_32x32x16_bf16(RowTile<D>::frag(ks_, 32 * kb + j, 16 * ks + 8 * h), qf[ks], s[kb]);
                dp[kb] = mfma_32x32x16_bf16(RowTile<D>::frag(vs_, 32 * kb + j, 16 * ks + 8 * h), gf[ks], dp[kb]);
            }
        }
        if (!(tflag[t] & 2)) {
            const uint64_t bits = key_tile_bits(mrow, n, p.N, p.Lc, contig, t * kTileRows, p.L);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (!((bits >> (32 * kb + acc_row(r, h))) & 1ull)) s[kb][r] = -INFINITY;
        }
        uint32_t pk[2][8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p0 = fast_exp2(fmaf(s[kb][2 * i], p.sl2, -lse2));
                const float p1 = fast_exp2(fmaf(s[kb][2 * i + 1], p.sl2, -lse2));
                pk[kb][i] = pack_bf16x2(p0 * (dp[kb][2 * i] - Di), p1 * (dp[kb][2 * i + 1] - Di));
            }
#pragma unroll
        for (int stp = 0; stp < 4; ++stp) {
            const u32x4 bfrag = acc_frag(pk, stp);
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                acc[db] = mfma_32x32x16_bf16(TransTile<D>::frag(kts, 32 * db + j, stp, h), bfrag, acc[db]);
        }
        if (tn < ntile) store(smem + (buf ^ 1) * S::BUF);
        buf ^= 1;
        t = tn;
    }

    if (row_ok) {
        uint16_t* out = p.dq + hoff + (size_t)row * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const u32x2 w = {pack_bf16x2(acc[db][4 * r4] * p.scale, acc[db][4 * r4 + 1] * p.scale),
                                 pack_bf16x2(acc[db][4 * r4 + 2] * p.scale, acc[db][4 * r4 + 3] * p.scale)};
                *reinterpret_cast<u32x2*>(out + 32 * db + 8 * r4 + 4 * h) = w;
            }
    }
}

// ---------------------------------------------------------------- dK dV ---
template <int D>
struct DkvSmem {
    static constexpr int Q_OFF = 0;
    static constexpr int G_OFF = Q_OFF + RowTile<D>::ELEMS;
    static constexpr int QT_OFF = G_OFF + RowTile<D>::ELEMS;
    static constexpr int GT_OFF = QT_OFF + TransTile<D>::ELEMS;
    static constexpr int ROWS_OFF = GT_OFF + TransTile<D>::ELEMS;   // lse2[64], D[64] as fp32
    static constexpr int BUF = ROWS_OFF + 2 * kTileRows * 2;
};

template <int D>
__global__ __launch_bounds__(kThreads) void rsa_bwd_dkdv(BwdParams p) {
    using S = DkvSmem<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * S::BUF];

    const int lid = xcd_remap(blockIdx.x, p.nt * p.BH);
    const int kt = lid % p.nt, bh = lid / p.nt, b = bh / p.H;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int j = lane & 31, h = lane >> 5;
    const int key0 = kt * 128;
    const int key = key0 + wave * 32 + j;
    const bool key_in = key < p.L;
    const bool key_ok = key_in && (p.mask == nullptr || p.mask[(size_t)b * p.L + key] != 0);
    const int c = key0 / p.Lc;   // key chunk of the tile's first key
    const size_t hoff = (size_t)bh * p.L * D;
    const bool contig = p.contiguous != 0;

    if (!__syncthreads_or(key_ok)) {
        // no valid key in this tile: its gradients are exactly zero
        if (key_in) {
            const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < D / 8; e += 1) {
                if ((e & 1) != h) continue;
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

    const int ntq = (p.L + kTileRows - 1) / kTileRows;
    RowTile<D> qst, gst;
    TransTile<D> qtst, gtst;
    float rowval = 0.0f;   // threads 0..63: lse2 of row tid; 64..127: D of row tid - 64
    auto load = [&](int t) {
        const int u0 = t * kTileRows;
        const int pos0 = contig ? ring_pos_rev(u0, c, p.N, p.Lc) : 0;
        auto rpos = [&](int r) -> int {
            const int u = u0 + r;
            if (u >= p.L) return -1;
            return contig ? pos0 + r : ring_pos_rev(u, c, p.N, p.Lc);
        };
        auto qptr = [&](int r) -> const uint16_t* {
            const int pos = rpos(r);
            return pos < 0 ? nullptr : p.q + hoff + (size_t)pos * D;
        };
        auto gptr = [&](int r) -> const uint16_t* {
            const int pos = rpos(r);
            return pos < 0 ? nullptr : p.dout + hoff + (size_t)pos * D;
        };
        qst.load(qptr);
        gst.load(gptr);
        qtst.load(qptr);
        gtst.load(gptr);
        if (threadIdx.x < 2 * kTileRows) {
            const int r = threadIdx.x % kTileRows;
            const int pos = rpos(r);
            if (threadIdx.x < kTileRows)
                rowval = pos < 0 ? INFINITY : lse_log2(p.lse[(size_t)bh * p.L + pos]);
            else
                rowval = pos < 0 ? 0.0f : p.delta[(size_t)bh * p.L + pos];
        }
    };
    auto store = [&](uint16_t* buf) {
        qst.store(buf + S::Q_OFF);
        gst.store(buf + S::G_OFF);
        qtst.store(buf + S::QT_OFF);
        gtst.store(buf + S::GT_OFF);
        if (threadIdx.x < 2 * kTileRows) reinterpret_cast<float*>(buf + S::ROWS_OFF)[threadIdx.x] = rowval;
    };

    load(0);
    store(smem);
    int buf = 0;
    for (int t = 0; t < ntq; ++t) {
        if (t + 1 < ntq) load(t + 1);
        __syncthreads();
        const uint16_t* base = smem + buf * S::BUF;
        const uint16_t* qs = base + S::Q_OFF;
        const uint16_t* gs = base + S::G_OFF;
        const uint16_t* qts = base + S::QT_OFF;
        const uint16_t* gts = base + S::GT_OFF;
        const float* lse2s = reinterpret_cast<const float*>(base + S::ROWS_OFF);
        const float* ds_ = lse2s + kTileRows;

        // S = Q K^T and dP = dO V^T for 64 queries (two 32-row blocks):
        // lane <-> key column, registers <-> query rows.
        f32x16 s[2], dp[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[qb][r] = 0.0f;
                dp[qb][r] = 0.0f;
            }
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                s[qb] = mfma_32x32x16_bf16(RowTile<D>::frag(qs, 32 * qb + j, 16 * ks + 8 * h), kf[ks], s[qb]);
                dp[qb] = mfma_32x32x16_bf16(RowTile<D>::frag(gs, 32 * qb + j, 16 * ks + 8 * h), vf[ks], dp[qb]);
            }
        }
        uint32_t pp[2][8], pd[2][8];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int qr = 32 * qb + 8 * r4 + 4 * h;   // query rows qr .. qr+3 of registers 4*r4 ..
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + qr);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(ds_ + qr);
                float pv[4], dsv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * r4 + e;
                    const float pe = key_ok ? fast_exp2(fmaf(s[qb][r], p.sl2, -l4[e])) : 0.0f;
                    pv[e] = pe;
                    dsv[e] = pe * (dp[qb][r] - d4[e]);
                }
                pp[qb][2 * r4] = pack_bf16x2(pv[0], pv[1]);
                pp[qb][2 * r4 + 1] = pack_bf16x2(pv[2], pv[3]);
                pd[qb][2 * r4] = pack_bf16x2(dsv[0], dsv[1]);
                pd[qb][2 * r4 + 1] = pack_bf16x2(dsv[2], dsv[3]);
            }
        // dV^T += dO^T P and dK^T += Q^T dS, contracted over the 64 queries
#pragma unroll
        for (int stp = 0; stp < 4; ++stp) {
            const u32x4 bp = acc_frag(pp, stp);
            const u32x4 bd = acc_frag(pd, stp);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                dv[db] = mfma_32x32x16_bf16(TransTile<D>::frag(gts, 32 * db + j, stp, h), bp, dv[db]);
                dk[db] = mfma_32x32x16_bf16(TransTile<D>::frag(qts, 32 * db + j, stp, h), bd, dk[db]);
            }
        }
        if (t + 1 < ntq) store(smem + (buf ^ 1) * S::BUF);
        buf ^= 1;
    }

    if (key_in) {
        uint16_t* okk = p.dk + hoff + (size_t)key * D;
        uint16_t* ovv = p.dv + hoff + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int dcol = 32 * db + 8 * r4 + 4 * h;
                const u32x2 wk = {pack_bf16x2(dk[db][4 * r4] * p.scale, dk[db][4 * r4 + 1] * p.scale),
                                  pack_bf16x2(dk[db][4 * r4 + 2] * p.scale, dk[db][4 * r4 + 3] * p.scale)};
                const u32x2 wv = {pack_bf16x2(dv[db][4 * r4], dv[db][4 * r4 + 1]),
                                  pack_bf16x2(dv[db][4 * r4 + 2], dv[db][4 * r4 + 3])};
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
    p.delta = c.delta;
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
    p.sl2 = (float)(1.4426950408889634 / __builtin_sqrt((double)c.d));
    p.contiguous = (p.Lc % kTileRows) == 0;
    return p;
}

template <int D>
hipError_t launch_t(const BackwardCall& c, int stages, hipStream_t stream) {
    const BwdParams p = make_params(c);
    const long long rows = (long long)p.BH * c.L;
    if (stages & kBwdStagePre) {
        const long long threads = rows * (D / 8);
        hipLaunchKernelGGL((rsa_bwd_pre<D>), dim3((unsigned)((threads + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                           stream, p.o, p.dout, p.delta, rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const unsigned blocks = (unsigned)((long long)p.nt * p.BH);
    if (stages & kBwdStageDq) {
        hipLaunchKernelGGL((rsa_bwd_dq<D>), dim3(blocks), dim3(kThreads), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (stages & kBwdStageDkDv) {
        hipLaunchKernelGGL((rsa_bwd_dkdv<D>), dim3(blocks), dim3(kThreads), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

size_t backward_workspace_bytes(int B, int H, int L, int d) {
    (void)d;
    return (size_t)B * H * L * sizeof(float);
}

hipError_t launch_backward(const BackwardCall& c, int stages, hipStream_t stream) {
    if (c.d == 64) return launch_t<64>(c, stages, stream);
    return launch_t<128>(c, stages, stream);
}

}  // namespace rsa
