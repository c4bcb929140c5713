// rsa_bwd_f32.hip -- Ring Self-Attention backward for fp32 inputs (fp32 in,
// fp32 out, fp32 products on the 32x32x2 fp32 MFMA).
//
// The same gradients and ring orders as the bf16 backward (rsa_bwd.hip;
// review page of "Sequence Parallelism: Making 4D Parallelism Possible",
// proposed-method section: gradients also pass through the ring):
//
//   P = exp(S - lse),  D_i = dO_i . O_i,  dP = dO V^T,  dS = P o (dP - D),
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),  dV = P^T dO,
//
// in three kernels: row statistics (-D and -lse * log2 e), a query-stationary
// dQ kernel that meets the key chunks in the ring order of each rank, and a
// key-stationary dK/dV kernel that meets the query chunks in the order the
// ring delivers them to the key chunk. Nothing is rounded below fp32. Tiles
// are staged through registers into LDS rows of pitch d + 1 floats, so that
// both the per-lane row reads (lane <-> tile row) and the per-lane column
// reads (lane <-> feature) are free of bank conflicts; one tile at a time.

#include "rsa_device.h"
#include "rsa_internal.h"

namespace rsa {
namespace {

constexpr int kThreads = 256;
constexpr int kKT = 64;   // rows per LDS tile
constexpr float kLog2e = 1.4426950408889634f;

struct BwdF32Params {
    const float* q;
    const float* k;
    const float* v;
    const float* o;
    const float* dout;
    const float* lse;
    const uint8_t* mask;
    float* stats;   // [2][B*H*L]: -D, then -lse * log2(e)
    float* dq;
    float* dk;
    float* dv;
    int H, L, N, Lc, BH, nt;   // nt: 128-row tiles per head
    float sl2;                 // log2(e) / sqrt(d)
    float scale;               // 1 / sqrt(d)
    int causal;
    Dropout drop;              // the forward's dropout (drop.p8 == 0: none)
};

// Sequence position of the u-th query row that key chunk c meets: ring step
// t = u / Lc brings query chunk (c + t) mod N.
__device__ __forceinline__ int ring_pos_rev_f32(int u, int c, int N, int Lc) {
    const int t = u / Lc;
    int n = c + t;
    n -= (n >= N) ? N : 0;
    return n * Lc + (u - t * Lc);
}

template <int D>
__global__ __launch_bounds__(kThreads) void rsa_bwd_pre_f32(const float* __restrict__ o,
                                                            const float* __restrict__ dout,
                                                            const float* __restrict__ lse, float* __restrict__ stats,
                                                            long long rows) {
    constexpr int TPR = D / 4;   // lanes per row, 4 elements each
    const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long row = t / TPR;
    const int c = (int)(t % TPR);
    float acc = 0.0f;
    if (row < rows) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(o + row * D + 4 * c);
        const f32x4 g = *reinterpret_cast<const f32x4*>(dout + row * D + 4 * c);
        acc = a[0] * g[0] + a[1] * g[1] + a[2] * g[2] + a[3] * g[3];
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && c == 0) {
        stats[row] = -acc;
        const float l = lse[row];
        stats[rows + row] = l == -INFINITY ? -INFINITY : -l * kLog2e;
    }
}

// Copy 64 rows of two [*, D] fp32 tensors into LDS (pitch D + 1); row r
// comes from element offset rowoff(r), or is zero where rowoff(r) < 0.
template <int D, class RowOff>
__device__ __forceinline__ void stage_pair(float* sa, float* sb, const float* a, const float* b, RowOff rowoff) {
    constexpr int KP = D + 1;
    constexpr int CH = (kKT * D / 4) / kThreads;
    static_assert(CH * kThreads * 4 == kKT * D, "fp32 staging");
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = threadIdx.x + i * kThreads;
        const int r = c / (D / 4), col = c % (D / 4);
        const long long off = rowoff(r);
        f32x4 xa = {0.0f, 0.0f, 0.0f, 0.0f}, xb = {0.0f, 0.0f, 0.0f, 0.0f};
        if (off >= 0) {
            xa = *reinterpret_cast<const f32x4*>(a + off + 4 * col);
            xb = *reinterpret_cast<const f32x4*>(b + off + 4 * col);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sa[r * KP + 4 * col + e] = xa[e];
            sb[r * KP + 4 * col + e] = xb[e];
        }
    }
}

// dQ: 4 waves x 32 query rows of one head; per 64-key tile (ring order of
// the tile's first row's rank) S^T = K Q^T and dP^T = V dO^T (lane <->
// query), dS, then dQ^T += K^T dS^T.
template <int D>
__global__ __launch_bounds__(kThreads) void rsa_bwd_dq_f32(BwdF32Params p) {
    constexpr int KP = D + 1;
    __shared__ float ks[kKT * KP];
    __shared__ float vs[kKT * KP];

    const int lid = xcd_remap(blockIdx.x, p.nt * p.BH);
    const int qt = lid % p.nt, bh = lid / p.nt, b = bh / p.H;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int j = lane & 31, h = lane >> 5;
    const int row0 = qt * 128;
    const int row = row0 + wave * 32 + j;
    const bool row_ok = row < p.L;
    const int n = row0 / p.Lc;   // ring rank of the tile's first row
    const size_t hoff = (size_t)bh * p.L * D;
    const float* kh = p.k + hoff;
    const float* vh = p.v + hoff;
    const uint8_t* mrow = p.mask ? p.mask + (size_t)b * p.L : nullptr;
    const size_t rows_all = (size_t)p.BH * p.L;

    float qf[D / 2], gf[D / 2];   // Q^T and dO^T fragments: lane (j, h) holds [row][2 s + h]
#pragma unroll
    for (int s = 0; s < D / 2; ++s) {
        qf[s] = row_ok ? p.q[hoff + (size_t)row * D + 2 * s + h] : 0.0f;
        gf[s] = row_ok ? p.dout[hoff + (size_t)row * D + 2 * s + h] : 0.0f;
    }
    const float nD = row_ok ? p.stats[(size_t)bh * p.L + row] : 0.0f;
    const float nl2 = row_ok ? p.stats[rows_all + (size_t)bh * p.L + row] : -INFINITY;

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

    const int ntile = (p.L + kKT - 1) / kKT;
    for (int t = 0; t < ntile; ++t) {
        __syncthreads();   // the previous tile is consumed
        stage_pair<D>(ks, vs, kh, vh, [&](int r) -> long long {
            const int vk = t * kKT + r;
            return vk < p.L ? (long long)ring_pos(vk, n, p.N, p.Lc) * D : -1;
        });
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = 0.0f;
                dp[r] = nD;
            }
#pragma unroll
            for (int kq = 0; kq < D / 2; ++kq) {
                s = mfma_32x32x2_f32(ks[(32 * kb + j) * KP + 2 * kq + h], qf[kq], s);
                dp = mfma_32x32x2_f32(vs[(32 * kb + j) * KP + 2 * kq + h], gf[kq], dp);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kr = 32 * kb + acc_row(r, h);   // key row of the tile
                const int vk = t * kKT + kr;
                bool vis = vk < p.L;
                if (vis) {
                    const int pos = ring_pos(vk, n, p.N, p.Lc);
                    vis = (mrow == nullptr || mrow[pos] != 0) && !(p.causal && pos > row);
                }
                const float pr = vis ? fast_exp2(fmaf(s[r], p.sl2, nl2)) : 0.0f;
                float dpz = dp[r];   // dP - D, or with dropout Z dP - D
                if (p.drop.p8 != 0u && vis) {
                    const bool keep = dropout_keep(p.drop, row, ring_pos(vk, n, p.N, p.Lc), bh);
                    dpz = keep ? fmaf(dp[r] - nD, p.drop.scale, nD) : nD;
                }
                const float ds = pr * dpz;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) acc[db] = mfma_32x32x2_f32(ks[kr * KP + 32 * db + j], ds, acc[db]);
            }
        }
    }

    if (!row_ok) return;
    float* out = p.dq + hoff + (size_t)row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 w = {acc[db][4 * r4] * p.scale, acc[db][4 * r4 + 1] * p.scale, acc[db][4 * r4 + 2] * p.scale,
                             acc[db][4 * r4 + 3] * p.scale};
            *reinterpret_cast<f32x4*>(out + 32 * db + 8 * r4 + 4 * h) = w;
        }
}

// dK, dV: 4 waves x 32 keys of one head (K, V fragments in registers); per
// 64-row query tile in ring delivery order, S = Q K^T and dP = dO V^T (lane
// <-> key), P and dS, then dV^T += dO^T P and dK^T += Q^T dS.
template <int D>
__global__ __launch_bounds__(kThreads) void rsa_bwd_dkdv_f32(BwdF32Params p) {
    constexpr int KP = D + 1;
    __shared__ float qs[kKT * KP];
    __shared__ float gs[kKT * KP];
    __shared__ float st_d[kKT], st_l[kKT];
    __shared__ int st_pos[kKT];

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
    const size_t rows_all = (size_t)p.BH * p.L;
    const float* nDh = p.stats + (size_t)bh * p.L;
    const float* nLh = p.stats + rows_all + (size_t)bh * p.L;

    float kf[D / 2], vf[D / 2];   // K^T and V^T fragments: lane (j, h) holds [key][2 s + h]
#pragma unroll
    for (int s = 0; s < D / 2; ++s) {
        kf[s] = key_in ? p.k[hoff + (size_t)key * D + 2 * s + h] : 0.0f;
        vf[s] = key_in ? p.v[hoff + (size_t)key * D + 2 * s + h] : 0.0f;
    }
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk[db][r] = 0.0f;
            dv[db][r] = 0.0f;
        }

    const int ntq = (p.L + kKT - 1) / kKT;
    for (int t = 0; t < ntq; ++t) {
        __syncthreads();
        auto pos_of = [&](int r) -> int {
            const int u = t * kKT + r;
            return u < p.L ? ring_pos_rev_f32(u, c, p.N, p.Lc) : -1;
        };
        stage_pair<D>(qs, gs, p.q + hoff, p.dout + hoff, [&](int r) -> long long {
            const int pos = pos_of(r);
            return pos >= 0 ? (long long)pos * D : -1;
        });
        if (threadIdx.x < kKT) {
            const int pos = pos_of(threadIdx.x);
            st_pos[threadIdx.x] = pos;
            st_d[threadIdx.x] = pos >= 0 ? nDh[pos] : 0.0f;
            st_l[threadIdx.x] = pos >= 0 ? nLh[pos] : -INFINITY;   // rows past the sequence: P = 0
        }
        __syncthreads();
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            f32x16 s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = 0.0f;
                dp[r] = 0.0f;
            }
#pragma unroll
            for (int ks = 0; ks < D / 2; ++ks) {
                s = mfma_32x32x2_f32(qs[(32 * qb + j) * KP + 2 * ks + h], kf[ks], s);
                dp = mfma_32x32x2_f32(gs[(32 * qb + j) * KP + 2 * ks + h], vf[ks], dp);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int u = 32 * qb + acc_row(r, h);   // query row of the tile
                const bool vis = !(p.causal && key > st_pos[u]);
                float pr = vis ? fast_exp2(fmaf(s[r], p.sl2, st_l[u])) : 0.0f;
                float ds = pr * (dp[r] + st_d[u]);
                if (p.drop.p8 != 0u && vis && st_pos[u] >= 0) {   // dV takes P Z, dS = P (Z dP - D)
                    const bool keep = dropout_keep(p.drop, st_pos[u], key, bh);
                    ds = pr * (keep ? fmaf(dp[r], p.drop.scale, st_d[u]) : st_d[u]);
                    pr = keep ? pr * p.drop.scale : 0.0f;
                }
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    dv[db] = mfma_32x32x2_f32(gs[u * KP + 32 * db + j], pr, dv[db]);
                    dk[db] = mfma_32x32x2_f32(qs[u * KP + 32 * db + j], ds, dk[db]);
                }
            }
        }
    }

    if (!key_in) return;
    // a padded key's column gathered weights of a key no row may see: zero
    const float sk = key_ok ? p.scale : 0.0f;
    const float sv = key_ok ? 1.0f : 0.0f;
    float* okk = p.dk + hoff + (size_t)key * D;
    float* ovv = p.dv + hoff + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            f32x4 wk = {dk[db][4 * r4] * sk, dk[db][4 * r4 + 1] * sk, dk[db][4 * r4 + 2] * sk, dk[db][4 * r4 + 3] * sk};
            f32x4 wv = {dv[db][4 * r4] * sv, dv[db][4 * r4 + 1] * sv, dv[db][4 * r4 + 2] * sv, dv[db][4 * r4 + 3] * sv};
            if (!key_ok) {   // inf * 0 would be NaN
                wk = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                wv = wk;
            }
            *reinterpret_cast<f32x4*>(okk + 32 * db + 8 * r4 + 4 * h) = wk;
            *reinterpret_cast<f32x4*>(ovv + 32 * db + 8 * r4 + 4 * h) = wv;
        }
}

template <int D>
hipError_t launch_t(const BackwardCall& c, int stages, hipStream_t stream) {
    BwdF32Params p{};
    p.q = static_cast<const float*>(c.q);
    p.k = static_cast<const float*>(c.k);
    p.v = static_cast<const float*>(c.v);
    p.o = static_cast<const float*>(c.out);
    p.dout = static_cast<const float*>(c.dout);
    p.lse = c.lse;
    p.mask = c.mask;
    p.stats = c.stats;
    p.dq = static_cast<float*>(c.dq);
    p.dk = static_cast<float*>(c.dk);
    p.dv = static_cast<float*>(c.dv);
    p.H = c.H;
    p.L = c.L;
    p.N = c.N;
    p.Lc = c.L / c.N;
    p.BH = c.B * c.H;
    p.nt = (c.L + 127) / 128;
    p.scale = (float)(1.0 / __builtin_sqrt((double)D));
    p.sl2 = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
    p.causal = c.causal ? 1 : 0;
    p.drop.p8 = c.drop_p8;
    p.drop.seed_lo = (uint32_t)c.drop_seed;
    p.drop.seed_hi = (uint32_t)(c.drop_seed >> 32);
    p.drop.offset = c.drop_offset;
    p.drop.scale = (float)(256.0 / (256.0 - (double)c.drop_p8));
    p.drop.keep = (float)((256.0 - (double)c.drop_p8) / 256.0);
    const long long rows = (long long)p.BH * c.L;
    if (stages & kBwdStagePre) {
        const long long threads = rows * (D / 4);
        hipLaunchKernelGGL((rsa_bwd_pre_f32<D>), dim3((unsigned)((threads + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, p.o, p.dout, p.lse, p.stats, rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const unsigned blocks = (unsigned)((long long)p.nt * p.BH);
    if (stages & kBwdStageDq) {
        hipLaunchKernelGGL((rsa_bwd_dq_f32<D>), dim3(blocks), dim3(kThreads), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (stages & kBwdStageDkDv) {
        hipLaunchKernelGGL((rsa_bwd_dkdv_f32<D>), dim3(blocks), dim3(kThreads), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_backward_f32(const BackwardCall& c, int stages, hipStream_t stream) {
    if (c.d == 64) return launch_t<64>(c, stages, stream);
    return launch_t<128>(c, stages, stream);
}

}  // namespace rsa
