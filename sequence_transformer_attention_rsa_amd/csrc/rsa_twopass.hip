// rsa_twopass.hip -- Ring Self-Attention forward in the pages' own two-stage
// form (review page of "Sequence Parallelism: Making 4D Parallelism
// Possible", ABSTRACT and proposed-method section: the key chunks circulate
// first and each rank forms its full score rows, then the value chunks
// circulate and are weighted by the softmax of those rows). bf16 in/out.
//
// Three kernels, score rows materialised in HBM:
//   rsa_2p_scores   S[b,h,i,j] = q_i . k_j (fp32; -inf for padded keys),
//                   every (query, key) pair: the union over ranks and ring
//                   steps of the blocks Q_n K_c^T
//   rsa_2p_softmax  per row: P = exp(S / sqrt(d) - lse) rounded to bf16,
//                   written in place over the first half of the row; lse
//   rsa_2p_pv       O = P V on the 32x32x16 bf16 MFMA (V^T through the
//                   transposing LDS read)
// The score rows cost 4 L^2 bytes per head written and read back, so this
// form is bound by HBM bandwidth where the fused kernel is bound by the
// matrix cores; it exists to measure that difference (and the memory it
// needs: the fused kernel never holds a row of scores).

#include "rsa_device.h"
#include "rsa_internal.h"
#include "rsa_tiles.h"

namespace rsa {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t ld32(const uint16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

// S = Q K^T for a 128-query x 128-key tile: wave w owns queries
// q0 + 32 w .. +32 (A operand, lane <-> query row), the four 32-key blocks
// are B operands (lane <-> key column), so the accumulator rows are queries
// and its lanes are consecutive keys: each store is 128 contiguous bytes.
template <int D>
__global__ __launch_bounds__(kThreads) void rsa_2p_scores(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint8_t* __restrict__ mask, float* __restrict__ S,
                                                          int H, int L, int nt) {
    const int bh = blockIdx.y, b = bh / H;
    const int qt = blockIdx.x / nt, kt = blockIdx.x % nt;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int j = lane & 31, h = lane >> 5;
    const size_t hoff = (size_t)bh * L * D;
    const int qrow = qt * 128 + wave * 32 + j;
    u32x4 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (qrow < L) x = *reinterpret_cast<const u32x4*>(q + hoff + (size_t)qrow * D + 16 * ks + 8 * h);
        qf[ks] = x;
    }
    float* Sh = S + (size_t)bh * L * L;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const int key = kt * 128 + 32 * kb + j;
        const bool key_in = key < L;
        const bool valid = key_in && (mask == nullptr || mask[(size_t)b * L + key] != 0);
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            u32x4 kf = {0u, 0u, 0u, 0u};
            if (key_in) kf = *reinterpret_cast<const u32x4*>(k + hoff + (size_t)key * D + 16 * ks + 8 * h);
            acc = mfma_32x32x16_bf16(qf[ks], kf, acc);
        }
        if (key_in) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = qt * 128 + wave * 32 + acc_row(r, h);
                if (row < L) Sh[(size_t)row * L + key] = valid ? acc[r] : -INFINITY;
            }
        }
    }
}

// One workgroup per score row, the row held in registers: thread t owns
// the element pairs (2p, 2p+1) for p = t + 256 i, i < PAIRS (L <= 512 PAIRS).
// Row max, then the sum of exp2, then P in bf16 over the first 2L bytes of
// the row (pair p lands on fp32 element p, so every read of the row is done,
// two barriers earlier, before the first write), and lse.
template <int PAIRS>
__global__ __launch_bounds__(kThreads) void rsa_2p_softmax(float* __restrict__ S, float* __restrict__ lse, int L,
                                                           float sl2) {
    __shared__ float red[2][kThreads / kWave];
    const size_t ri = blockIdx.x;
    float* row = S + ri * (size_t)L;
    float e[2 * PAIRS];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < PAIRS; ++i) {
        const int x = 2 * ((int)threadIdx.x + kThreads * i);
        e[2 * i] = x < L ? row[x] : -INFINITY;
        e[2 * i + 1] = x + 1 < L ? row[x + 1] : -INFINITY;
        mx = fmaxf(mx, fmaxf(e[2 * i], e[2 * i + 1]));
    }
    for (int off = kWave / 2; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (threadIdx.x % kWave == 0) red[0][threadIdx.x / kWave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    const float base = mx == -INFINITY ? 0.0f : mx * sl2;
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 2 * PAIRS; ++i) {
        e[i] = fast_exp2(fmaf(e[i], sl2, -base));
        sum += e[i];
    }
    for (int off = kWave / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    if (threadIdx.x % kWave == 0) red[1][threadIdx.x / kWave] = sum;
    __syncthreads();
    const float l = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    uint32_t* prow = reinterpret_cast<uint32_t*>(row);
#pragma unroll
    for (int i = 0; i < PAIRS; ++i) {
        const int p = (int)threadIdx.x + kThreads * i;
        if (2 * p < L) prow[p] = pack_bf16x2(e[2 * i] * inv, e[2 * i + 1] * inv);
    }
    if (threadIdx.x == 0 && lse) lse[ri] = l > 0.0f ? (base + __log2f(l)) * (1.0f / kLog2e) : -INFINITY;
}

// Rows longer than the register-held kernel covers: one workgroup per row,
// two passes over it in chunks of 512 elements. Pass 1 keeps a running
// (maximum, sum of exp2) per thread, merged across the workgroup; pass 2
// writes the bf16 weights in place. Chunk c's weights land on fp32 elements
// [256 c, 256 c + 256), which lie in chunks already read; a barrier per chunk
// keeps a lagging thread's reads ahead of every overwrite.
__global__ __launch_bounds__(kThreads) void rsa_2p_softmax_long(float* __restrict__ S, float* __restrict__ lse,
                                                                int L, float sl2) {
    __shared__ float red_m[kThreads / kWave], red_s[kThreads / kWave];
    const size_t ri = blockIdx.x;
    float* row = S + ri * (size_t)L;
    // running maximum (raw units) and sum of exp2((v - m) * sl2)
    float m = -INFINITY, sum = 0.0f;
    for (int x = threadIdx.x; x < L; x += kThreads) {
        const float v = row[x];
        if (v > m) {
            sum = (m == -INFINITY ? 0.0f : sum * fast_exp2((m - v) * sl2)) + 1.0f;
            m = v;
        } else if (v != -INFINITY) {
            sum += fast_exp2((v - m) * sl2);
        }
    }
    auto merge = [&](float om, float os) {
        const float nm = fmaxf(m, om);
        if (nm == -INFINITY) return;
        sum = (m == -INFINITY ? 0.0f : sum * fast_exp2((m - nm) * sl2)) +
              (om == -INFINITY ? 0.0f : os * fast_exp2((om - nm) * sl2));
        m = nm;
    };
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const float om = __shfl_xor(m, off), os = __shfl_xor(sum, off);
        merge(om, os);
    }
    if (threadIdx.x % kWave == 0) {
        red_m[threadIdx.x / kWave] = m;
        red_s[threadIdx.x / kWave] = sum;
    }
    __syncthreads();
    m = red_m[0];
    sum = red_s[0];
    for (int w = 1; w < kThreads / kWave; ++w) merge(red_m[w], red_s[w]);
    const float base = m == -INFINITY ? 0.0f : m * sl2;
    const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
    uint32_t* prow = reinterpret_cast<uint32_t*>(row);
    for (int c0 = 0; c0 < L; c0 += 2 * kThreads) {
        const int x = c0 + 2 * (int)threadIdx.x;
        const float v0 = x < L ? row[x] : -INFINITY;
        const float v1 = x + 1 < L ? row[x + 1] : -INFINITY;
        __syncthreads();   // every thread's reads of this chunk precede the writes below
        if (x < L) prow[x / 2] = pack_bf16x2(fast_exp2(fmaf(v0, sl2, -base)) * inv, fast_exp2(fmaf(v1, sl2, -base)) * inv);
        __syncthreads();   // writes land before a lagging thread reads the next chunk
    }
    if (threadIdx.x == 0 && lse) lse[ri] = sum > 0.0f ? (base + __log2f(sum)) * (1.0f / kLog2e) : -INFINITY;
}

// O^T = V^T P^T for 128 queries (4 waves x 32, lane <-> query), keys in
// 64-row tiles: V through LDS (transposing read, keys in sequence), P
// straight from the materialised rows (pitch 4L bytes): lane half h loads
// keys 16 s + 8 h .. + 8 of its query as 16 contiguous bytes. The four loads
// of a tile are issued before the V tile is waited for.
template <int D>
__global__ __launch_bounds__(kThreads) void rsa_2p_pv(const float* __restrict__ S, const uint16_t* __restrict__ v,
                                                      uint16_t* __restrict__ out, int L, int nqt) {
    using VT = DirectTile<D>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[VT::BYTES];
    const int bh = blockIdx.x / nqt, qt = blockIdx.x % nqt;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int j = lane & 31, h = lane >> 5;
    const int qrow = qt * 128 + wave * 32 + j;
    const bool qin = qrow < L;
    const size_t hoff = (size_t)bh * L * D;
    const uint16_t* prow = reinterpret_cast<const uint16_t*>(S + ((size_t)bh * L + (qin ? qrow : 0)) * L);
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    const int ntile = (L + kTileRows - 1) / kTileRows;
    for (int t = 0; t < ntile; ++t) {
        const int k0 = t * kTileRows;
        u32x4 pf[4];
#pragma unroll
        for (int stp = 0; stp < 4; ++stp) {
            const int kk = k0 + 16 * stp + 8 * h;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qin && kk + 8 <= L) {
                // rows start 4-byte aligned only: 4-byte loads
                x = u32x4{ld32(prow + kk), ld32(prow + kk + 2), ld32(prow + kk + 4), ld32(prow + kk + 6)};
            } else if (qin && kk < L) {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                for (int e = 0; kk + e < L; ++e) w[e >> 1] |= (uint32_t)prow[kk + e] << (16 * (e & 1));
                x = u32x4{w[0], w[1], w[2], w[3]};
            }
            pf[stp] = x;
        }
        __syncthreads();   // previous V tile consumed
        VT::load(smem, [&](int r) { return v + hoff + (size_t)(k0 + r < L ? k0 + r : 0) * D; });
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
#pragma unroll
        for (int stp = 0; stp < 4; ++stp)
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                o[db] = mfma_32x32x16_bf16(VT::tfrag_seq(smem, 16 * stp, 32 * db), pf[stp], o[db]);
    }
    if (!qin) return;
    uint16_t* orow = out + hoff + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const u32x2 w = {pack_bf16x2(o[db][4 * r4], o[db][4 * r4 + 1]), pack_bf16x2(o[db][4 * r4 + 2], o[db][4 * r4 + 3])};
            *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * r4 + 4 * h) = w;
        }
}

template <int D>
hipError_t launch_t(const ForwardCall& c, hipStream_t stream) {
    const int BH = c.B * c.H;
    const int nt = (c.L + 127) / 128;
    float* S = c.part;
    hipLaunchKernelGGL((rsa_2p_scores<D>), dim3((unsigned)(nt * nt), (unsigned)BH), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(c.q), static_cast<const uint16_t*>(c.k), c.mask, S, c.H, c.L, nt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float sl2 = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
    const dim3 rows((unsigned)((long long)BH * c.L));
    const int pairs = (c.L + 2 * kThreads - 1) / (2 * kThreads);
    if (pairs <= 1) hipLaunchKernelGGL(rsa_2p_softmax<1>, rows, dim3(kThreads), 0, stream, S, c.lse, c.L, sl2);
    else if (pairs <= 2) hipLaunchKernelGGL(rsa_2p_softmax<2>, rows, dim3(kThreads), 0, stream, S, c.lse, c.L, sl2);
    else if (pairs <= 4) hipLaunchKernelGGL(rsa_2p_softmax<4>, rows, dim3(kThreads), 0, stream, S, c.lse, c.L, sl2);
    else if (pairs <= 8) hipLaunchKernelGGL(rsa_2p_softmax<8>, rows, dim3(kThreads), 0, stream, S, c.lse, c.L, sl2);
    else if (pairs <= 16) hipLaunchKernelGGL(rsa_2p_softmax<16>, rows, dim3(kThreads), 0, stream, S, c.lse, c.L, sl2);
    else if (pairs <= 32) hipLaunchKernelGGL(rsa_2p_softmax<32>, rows, dim3(kThreads), 0, stream, S, c.lse, c.L, sl2);
    else hipLaunchKernelGGL(rsa_2p_softmax_long, rows, dim3(kThreads), 0, stream, S, c.lse, c.L, sl2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((rsa_2p_pv<D>), dim3((unsigned)(BH * nt)), dim3(kThreads), 0, stream, S,
                       static_cast<const uint16_t*>(c.v), static_cast<uint16_t*>(c.out), c.L, nt);
    return hipGetLastError();
}

}  // namespace


hipError_t launch_forward_twopass(const ForwardCall& c, hipStream_t stream) {
    if (c.d == 64) return launch_t<64>(c, stream);
    return launch_t<128>(c, stream);
}

}  // namespace rsa
