// rsa_fwd.hip -- fused Ring Self-Attention forward for gfx950.
//
// What is computed (review page of "Sequence Parallelism: Making 4D
// Parallelism Possible", ABSTRACT and proposed-method section): rank n's
// query chunk meets the key chunks in ring order c = (n - t) mod N and the
// value chunks in the same order, producing softmax(Q K^T / sqrt(d) + M) V
// over the full key length. The pages' version materialises each rank's
// score rows before the value stage; here both stages run in one pass with
// an online softmax, so a rank's share needs O(rows * d) working memory
// instead of O(rows * L).
//
// Kernel shape (one workgroup = 4 waves = 128 query rows of one head):
//   * each wave owns 32 query rows; its Q fragment stays in registers;
//   * keys stream through LDS in tiles of 64, double-buffered: K row-major,
//     V transposed (bf16) so both contractions read 16-byte fragments;
//   * S^T = K Q^T on the 32x32x16 bf16 MFMA (fp32 inputs: 32x32x2 fp32).
//     In the 32x32 accumulator layout a lane owns one query column, so the
//     row max and row sum are in-lane plus one exchange between wave halves,
//     and the accumulator is the B operand of O^T = V^T P^T unchanged;
//   * online softmax in base 2 (scale and log2(e) folded into one FMA), with
//     a lazy rescale: the running base only moves when a tile's maximum
//     exceeds it by more than 8 (weights stay <= 2^8), which is exact after
//     the final normalisation;
//   * P is rounded to bf16 for the MFMA and the row sum adds those same
//     rounded values, so sum_j P_ij = 1 holds for the weights actually used;
//   * tiles whose keys are all padding are skipped (a per-workgroup
//     occupancy table built in LDS), so masked chunks cost nothing;
//   * in split mode (one rank's share), each workgroup covers a contiguous
//     group of ring steps and writes unnormalised partials that a merge
//     kernel combines exactly.

#include <type_traits>

#include "rsa_device.h"
#include "rsa_internal.h"

namespace rsa {
namespace {

constexpr int kThreads = 256;
constexpr int kKT = kFwdKeyTile;   // keys per tile
constexpr int kQW = 32;            // query rows per wave

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    const uint8_t* mask;
    void* out;
    float* lse;
    float* part_o;    // [groups][B*H][Lq][d]   unnormalised output
    float* part_ml;   // [groups][B*H][Lq][2]   (base in log2 units, row sum)
    int H, L, N, Lc, Lq, q_pos0, BH, groups, spg, nqt;
    float sl2;        // log2(e) / sqrt(d)
    float tau_raw;    // lazy-rescale threshold in raw score units (8 / sl2)
    int contiguous;   // Lc % kKT == 0: a tile never straddles two chunks
};

template <bool BF16, int D>
struct Cfg {
    using E = typename std::conditional<BF16, uint16_t, float>::type;
    // LDS: K row-major [kKT][KP]; V transposed [D][VP] (bf16) or row-major [kKT][D] (fp32)
    static constexpr int KP = BF16 ? D + 8 : D + 1;
    static constexpr int VP = BF16 ? kKT + 8 : D;
    static constexpr int K_ELEMS = kKT * KP;
    static constexpr int V_ELEMS = BF16 ? D * VP : kKT * D;
    static constexpr int BUF = K_ELEMS + V_ELEMS;
    // staging per thread: 16-byte K chunks; V units (bf16: one d pair x 8 keys)
    static constexpr int K_CHUNKS = BF16 ? (kKT * D / 8) / kThreads : (kKT * D / 4) / kThreads;
    static constexpr int V_UNITS = BF16 ? (D / 2 * (kKT / 8)) / kThreads : K_CHUNKS;
    static constexpr int QF = BF16 ? D / 16 : D / 2;   // Q fragments per lane (k-steps of S^T)
    static constexpr int DB = D / 32;                  // 32-row blocks of O^T
    static_assert(K_CHUNKS * kThreads * (BF16 ? 8 : 4) == kKT * D, "K staging");
    static_assert(!BF16 || V_UNITS * kThreads * 16 == kKT * D, "V staging");
};

template <bool BF16, int D>
struct Stage {
    u32x4 k[Cfg<BF16, D>::K_CHUNKS];
    uint32_t vb[BF16 ? Cfg<BF16, D>::V_UNITS : 1][8];      // bf16: 8 keys x (2 d) per unit
    u32x4 vf[BF16 ? 1 : Cfg<BF16, D>::K_CHUNKS];           // fp32: 16-byte chunks
};

// Global -> registers for the tile starting at virtual key v0.
template <bool BF16, int D>
__device__ __forceinline__ void load_tile(const FwdParams& p, const typename Cfg<BF16, D>::E* kh,
                                          const typename Cfg<BF16, D>::E* vh, int n, int v0, int vend,
                                          Stage<BF16, D>& st) {
    using C = Cfg<BF16, D>;
    const int tid = threadIdx.x;
    const int pos0 = p.contiguous ? ring_pos(v0, n, p.N, p.Lc) : 0;
    constexpr int EPC = BF16 ? 8 : 4;   // elements per 16-byte chunk
#pragma unroll
    for (int i = 0; i < C::K_CHUNKS; ++i) {
        const int c = tid + i * kThreads;
        const int row = c / (D / EPC), col = c % (D / EPC);
        const int vk = v0 + row;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (vk < vend) {
            const int pos = p.contiguous ? pos0 + row : ring_pos(vk, n, p.N, p.Lc);
            x = *reinterpret_cast<const u32x4*>(kh + (size_t)pos * D + col * EPC);
        }
        st.k[i] = x;
    }
    if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < C::V_UNITS; ++i) {
            const int u = tid + i * kThreads;
            const int dp = u % (D / 2), kg = u / (D / 2);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int vk = v0 + kg * 8 + e;
                uint32_t x = 0u;
                if (vk < vend) {
                    const int pos = p.contiguous ? pos0 + kg * 8 + e : ring_pos(vk, n, p.N, p.Lc);
                    x = *reinterpret_cast<const uint32_t*>(vh + (size_t)pos * D + 2 * dp);
                }
                st.vb[i][e] = x;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < C::K_CHUNKS; ++i) {
            const int c = tid + i * kThreads;
            const int row = c / (D / 4), col = c % (D / 4);
            const int vk = v0 + row;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (vk < vend) {
                const int pos = p.contiguous ? pos0 + row : ring_pos(vk, n, p.N, p.Lc);
                x = *reinterpret_cast<const u32x4*>(vh + (size_t)pos * D + col * 4);
            }
            st.vf[i] = x;
        }
    }
}

// Position of key x (0..15) of a 16-key group inside the transposed V tile.
// The S^T accumulator gives lane half h the keys 4h+{0..3} and 8+4h+{0..3}
// of each 16-key MFMA step; storing them adjacently lets one 16-byte LDS
// read fetch a lane's whole V^T fragment.
__device__ __forceinline__ constexpr int vt_slot(int x) { return 8 * ((x >> 2) & 1) + (x & 3) + 4 * (x >> 3); }

// Registers -> LDS buffer.
template <bool BF16, int D>
__device__ __forceinline__ void store_tile(typename Cfg<BF16, D>::E* buf, const Stage<BF16, D>& st) {
    using C = Cfg<BF16, D>;
    const int tid = threadIdx.x;
    auto* ks = buf;
    auto* vs = buf + C::K_ELEMS;
    if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < C::K_CHUNKS; ++i) {
            const int c = tid + i * kThreads;
            const int row = c / (D / 8), col = c % (D / 8);
            *reinterpret_cast<u32x4*>(ks + row * C::KP + col * 8) = st.k[i];
        }
#pragma unroll
        for (int i = 0; i < C::V_UNITS; ++i) {
            const int u = tid + i * kThreads;
            const int dp = u % (D / 2), kg = u / (D / 2);
            const uint32_t* w = st.vb[i];
            const int base = 16 * (kg >> 1) + vt_slot(8 * (kg & 1));   // keys kg*8 + 0..3
            const int base2 = 16 * (kg >> 1) + vt_slot(8 * (kg & 1) + 4);  // keys kg*8 + 4..7
            const u32x2 lo0 = {(w[0] & 0xffffu) | (w[1] << 16), (w[2] & 0xffffu) | (w[3] << 16)};
            const u32x2 lo1 = {(w[4] & 0xffffu) | (w[5] << 16), (w[6] & 0xffffu) | (w[7] << 16)};
            const u32x2 hi0 = {(w[0] >> 16) | (w[1] & 0xffff0000u), (w[2] >> 16) | (w[3] & 0xffff0000u)};
            const u32x2 hi1 = {(w[4] >> 16) | (w[5] & 0xffff0000u), (w[6] >> 16) | (w[7] & 0xffff0000u)};
            uint16_t* r0 = vs + (2 * dp) * C::VP;
            uint16_t* r1 = r0 + C::VP;
            *reinterpret_cast<u32x2*>(r0 + base) = lo0;
            *reinterpret_cast<u32x2*>(r0 + base2) = lo1;
            *reinterpret_cast<u32x2*>(r1 + base) = hi0;
            *reinterpret_cast<u32x2*>(r1 + base2) = hi1;
        }
    } else {
#pragma unroll
        for (int i = 0; i < C::K_CHUNKS; ++i) {
            const int c = tid + i * kThreads;
            const int row = c / (D / 4), col = c % (D / 4);
            float* dst = ks + row * C::KP + col * 4;
            dst[0] = __uint_as_float(st.k[i][0]);
            dst[1] = __uint_as_float(st.k[i][1]);
            dst[2] = __uint_as_float(st.k[i][2]);
            dst[3] = __uint_as_float(st.k[i][3]);
            *reinterpret_cast<u32x4*>(vs + row * D + col * 4) = st.vf[i];
        }
    }
}

// Occupancy of tile t of the workgroup's key range: bit 0 = some key valid,
// bit 1 = all kKT keys exist and are valid.
__device__ __forceinline__ uint8_t tile_flags(const FwdParams& p, const uint8_t* mrow, int n, int v0, int vend) {
    const int cnt = min(kKT, vend - v0);
    if (mrow == nullptr) return cnt == kKT ? 3 : 1;
    bool any = false, all = (cnt == kKT);
    if (p.contiguous) {
        const int pos0 = ring_pos(v0, n, p.N, p.Lc);
        const u32x4* m4 = reinterpret_cast<const u32x4*>(mrow + pos0);
#pragma unroll
        for (int i = 0; i < kKT / 16; ++i) {
            const u32x4 w = m4[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                any |= (w[e] != 0u);
                all &= !has_zero_byte(w[e]);
            }
        }
    } else {
        for (int i = 0; i < cnt; ++i) {
            const bool ok = mrow[ring_pos(v0 + i, n, p.N, p.Lc)] != 0;
            any |= ok;
            all &= ok;
        }
    }
    return (any ? 1 : 0) | (all ? 2 : 0);
}

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void rsa_fwd_kernel(FwdParams p) {
    using C = Cfg<BF16, D>;
    using E = typename C::E;
    __shared__ __attribute__((aligned(16))) E smem[2 * C::BUF];
    __shared__ uint8_t tflag[kFwdMaxTiles];

    const int total = p.nqt * p.BH * p.groups;
    const int lid = xcd_remap(blockIdx.x, total);
    const int qt = lid % p.nqt;
    const int rest = lid / p.nqt;
    const int g = rest % p.groups;
    const int bh = rest / p.groups;
    const int b = bh / p.H;

    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int j = lane & 31, h = lane >> 5;
    const int row0 = qt * (4 * kQW);
    const int row = row0 + wave * kQW + j;   // this lane's query row (within q)
    const bool row_ok = row < p.Lq;
    const int n = (p.q_pos0 + row0) / p.Lc;  // ring rank of the tile's first row

    const int step0 = g * p.spg;
    const int step1 = min(p.N, step0 + p.spg);
    const int vbeg = step0 * p.Lc, vend = step1 * p.Lc;
    const int ntile = (vend - vbeg + kKT - 1) / kKT;

    const E* qh = static_cast<const E*>(p.q) + (size_t)bh * p.Lq * D;
    const E* kh = static_cast<const E*>(p.k) + (size_t)bh * p.L * D;
    const E* vh = static_cast<const E*>(p.v) + (size_t)bh * p.L * D;
    const uint8_t* mrow = p.mask ? p.mask + (size_t)b * p.L : nullptr;
    if (ntile > kFwdMaxTiles) return;   // the host never launches such a range

    for (int t = threadIdx.x; t < ntile; t += kThreads)
        tflag[t] = tile_flags(p, mrow, n, vbeg + t * kKT, vend);

    // Q^T fragments (B operand of S^T = K Q^T): lane (j, h) holds row `row`,
    // contraction elements 16*ks + 8*h .. +8 (bf16) or 2*ks + h (fp32).
    u32x4 qf_b[BF16 ? C::QF : 1];
    float qf_f[BF16 ? 1 : C::QF];
    if constexpr (BF16) {
#pragma unroll
        for (int ks = 0; ks < C::QF; ++ks) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (row_ok) x = *reinterpret_cast<const u32x4*>(qh + (size_t)row * D + 16 * ks + 8 * h);
            qf_b[ks] = x;
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < C::QF; ++ks) qf_f[ks] = row_ok ? qh[(size_t)row * D + 2 * ks + h] : 0.0f;
    }

    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    float m_b = -INFINITY;   // running base, raw score units
    float l = 0.0f;          // running row sum over this lane half's keys

    __syncthreads();   // tile flags visible

    int t = 0;
    while (t < ntile && !(tflag[t] & 1)) ++t;
    Stage<BF16, D> st;
    int buf = 0;
    if (t < ntile) {
        load_tile<BF16, D>(p, kh, vh, n, vbeg + t * kKT, vend, st);
        store_tile<BF16, D>(smem, st);
    }

    while (t < ntile) {
        int tn = t + 1;
        while (tn < ntile && !(tflag[tn] & 1)) ++tn;
        if (tn < ntile) load_tile<BF16, D>(p, kh, vh, n, vbeg + tn * kKT, vend, st);
        __syncthreads();   // buffer `buf` complete; the other one is free

        const E* ks_ = smem + buf * C::BUF;
        const E* vs_ = ks_ + C::K_ELEMS;
        const int v0 = vbeg + t * kKT;

        // ---- scores S^T = K Q^T for 64 keys (two 32-key blocks)
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
            if constexpr (BF16) {
#pragma unroll
                for (int kq = 0; kq < C::QF; ++kq) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(ks_ + (32 * kb + j) * C::KP + 16 * kq + 8 * h);
                    s[kb] = mfma_32x32x16_bf16(a, qf_b[kq], s[kb]);
                }
            } else {
#pragma unroll
                for (int kq = 0; kq < C::QF; ++kq) {
                    const float a = ks_[(32 * kb + j) * C::KP + 2 * kq + h];
                    s[kb] = mfma_32x32x2_f32(a, qf_f[kq], s[kb]);
                }
            }
        }

        // ---- key mask and range tail (only tiles that are not fully valid)
        if (!(tflag[t] & 2)) {
            const int vk = v0 + lane;
            bool ok = vk < vend;
            if (ok && mrow) ok = mrow[p.contiguous ? ring_pos(v0, n, p.N, p.Lc) + lane : ring_pos(vk, n, p.N, p.Lc)] != 0;
            const uint64_t bits = __ballot(ok);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (!((bits >> (32 * kb + acc_row(r, h))) & 1ull)) s[kb][r] = -INFINITY;
        }

        // ---- online softmax (base 2, lazy rescale)
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = fmaxf(mx, shfl_xor32(mx));
        if (wave_any(mx > m_b + p.tau_raw)) {
            const float m_new = fmaxf(m_b, mx);
            const float alpha = fast_exp2((m_b - m_new) * p.sl2);
            m_b = m_new;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        }
        const float nb = -m_b * p.sl2;

        if constexpr (BF16) {
            uint32_t pk[2][8];   // P^T as bf16 pairs, same register order as s
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float p0 = fast_exp2(fmaf(s[kb][2 * i], p.sl2, nb));
                    const float p1 = fast_exp2(fmaf(s[kb][2 * i + 1], p.sl2, nb));
                    pk[kb][i] = pack_bf16x2(p0, p1);
                    l = add_bf16x2(pk[kb][i], l);
                }
            // ---- O^T += V^T P^T, four 16-key steps
#pragma unroll
            for (int stp = 0; stp < 4; ++stp) {
                const int kb = stp >> 1, half = stp & 1;
                const u32x4 bfrag = {pk[kb][4 * half], pk[kb][4 * half + 1], pk[kb][4 * half + 2], pk[kb][4 * half + 3]};
#pragma unroll
                for (int db = 0; db < C::DB; ++db) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(vs_ + (32 * db + j) * C::VP + 16 * stp + 8 * h);
                    o[db] = mfma_32x32x16_bf16(a, bfrag, o[db]);
                }
            }
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pr = fast_exp2(fmaf(s[kb][r], p.sl2, nb));
                    l += pr;
                    const int key = 32 * kb + acc_row(r, h);
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
                        o[db] = mfma_32x32x2_f32(vs_[key * D + 32 * db + j], pr, o[db]);
                }
        }

        if (tn < ntile) store_tile<BF16, D>(smem + (buf ^ 1) * C::BUF, st);
        buf ^= 1;
        t = tn;
    }

    // ---- epilogue
    const float l_row = l + shfl_xor32(l);
    if (p.groups == 1) {
        const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
        if (row_ok) {
            E* orow = static_cast<E*>(p.out) + ((size_t)bh * p.Lq + row) * D;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int dcol = 32 * db + 8 * r4 + 4 * h;
                    const float a0 = o[db][4 * r4] * inv, a1 = o[db][4 * r4 + 1] * inv;
                    const float a2 = o[db][4 * r4 + 2] * inv, a3 = o[db][4 * r4 + 3] * inv;
                    if constexpr (BF16) {
                        const u32x2 w = {pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
                        *reinterpret_cast<u32x2*>(orow + dcol) = w;
                    } else {
                        const f32x4 w = {a0, a1, a2, a3};
                        *reinterpret_cast<f32x4*>(orow + dcol) = w;
                    }
                }
            if (p.lse && h == 0)
                p.lse[(size_t)bh * p.Lq + row] =
                    l_row > 0.0f ? (m_b * p.sl2 + __log2f(l_row)) * kLn2 : -INFINITY;
        }
    } else if (row_ok) {
        const size_t prow = ((size_t)g * p.BH + bh) * p.Lq + row;
        float* po = p.part_o + prow * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 w = {o[db][4 * r4], o[db][4 * r4 + 1], o[db][4 * r4 + 2], o[db][4 * r4 + 3]};
                *reinterpret_cast<f32x4*>(po + 32 * db + 8 * r4 + 4 * h) = w;
            }
        if (h == 0) {
            p.part_ml[2 * prow] = l_row > 0.0f ? m_b * p.sl2 : -INFINITY;
            p.part_ml[2 * prow + 1] = l_row;
        }
    }
}

// Exact merge of ring-step-group partials: with base m_g (log2 units) and
// row sum l_g per group, M = max_g m_g, w_g = 2^(m_g - M),
// O = sum_g w_g O_g / sum_g w_g l_g.
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void rsa_merge_kernel(const float* __restrict__ part_o,
                                                             const float* __restrict__ part_ml, int groups,
                                                             int rows, void* out, float* lse) {
    using E = typename Cfg<BF16, D>::E;
    constexpr int TPR = D / 4;   // threads per row, 4 columns each
    const int tid = blockIdx.x * kThreads + threadIdx.x;
    const int rrow = tid / TPR, c4 = tid % TPR;
    if (rrow >= rows) return;
    float M = -INFINITY;
    for (int gi = 0; gi < groups; ++gi) {
        const float lg = part_ml[2 * ((size_t)gi * rows + rrow) + 1];
        if (lg > 0.0f) M = fmaxf(M, part_ml[2 * ((size_t)gi * rows + rrow)]);
    }
    float lsum = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (M != -INFINITY) {
        for (int gi = 0; gi < groups; ++gi) {
            const size_t pr = (size_t)gi * rows + rrow;
            const float lg = part_ml[2 * pr + 1];
            if (!(lg > 0.0f)) continue;
            const float w = fast_exp2(part_ml[2 * pr] - M);
            lsum += w * lg;
            const f32x4 x = *reinterpret_cast<const f32x4*>(part_o + pr * D + 4 * c4);
            acc += w * x;
        }
    }
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    E* orow = static_cast<E*>(out) + (size_t)rrow * D + 4 * c4;
    if constexpr (BF16) {
        const u32x2 w = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
        *reinterpret_cast<u32x2*>(orow) = w;
    } else {
        *reinterpret_cast<f32x4*>(orow) = acc * inv;
    }
    if (lse && c4 == 0) lse[rrow] = lsum > 0.0f ? (M + __log2f(lsum)) * kLn2 : -INFINITY;
}

template <bool BF16, int D>
hipError_t launch_t(const ForwardCall& c, hipStream_t stream) {
    FwdParams p{};
    p.q = c.q;
    p.k = c.k;
    p.v = c.v;
    p.mask = c.mask;
    p.out = c.out;
    p.lse = c.lse;
    p.H = c.H;
    p.L = c.L;
    p.N = c.N;
    p.Lc = c.L / c.N;
    p.Lq = c.Lq;
    p.q_pos0 = c.q_pos0;
    p.BH = c.B * c.H;
    p.groups = c.groups;
    p.spg = (c.N + c.groups - 1) / c.groups;
    p.nqt = (c.Lq + 4 * kQW - 1) / (4 * kQW);
    const double sl2 = 1.4426950408889634 / __builtin_sqrt((double)D);
    p.sl2 = (float)sl2;
    p.tau_raw = (float)(8.0 / sl2);
    p.contiguous = (p.Lc % kKT) == 0;
    if (c.groups > 1) {
        p.part_o = c.part;
        p.part_ml = c.part + (size_t)c.groups * p.BH * c.Lq * D;
    }
    const long long total = (long long)p.nqt * p.BH * p.groups;
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL((rsa_fwd_kernel<BF16, D>), dim3((unsigned)total), dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || c.groups == 1) return e;
    const int rows = p.BH * c.Lq;
    const long long threads = (long long)rows * (D / 4);
    hipLaunchKernelGGL((rsa_merge_kernel<BF16, D>), dim3((unsigned)((threads + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, p.part_o, p.part_ml, c.groups, rows, c.out, c.lse);
    return hipGetLastError();
}

}  // namespace

size_t forward_partial_bytes(int B, int H, int Lq, int d, int groups) {
    if (groups <= 1) return 0;
    return (size_t)groups * B * H * Lq * (size_t)(d + 2) * sizeof(float);
}

int forward_rank_groups(int B, int H, int L, int d, int N) {
    // Enough workgroups to cover the 256 CUs about twice, while keeping the
    // partials small next to K and V: at most 8 groups, and each group's key
    // range within the occupancy table.
    const int Lc = L / N;
    const long long qtiles = (long long)B * H * ((Lc + 4 * kQW - 1) / (4 * kQW));
    int g = 1;
    while (g < 8 && g < N && qtiles * g < 512) g *= 2;
    g = g < N ? g : N;
    while (((long long)((N + g - 1) / g) * Lc + kKT - 1) / kKT > kFwdMaxTiles && g < N) ++g;
    (void)d;
    return g;
}

hipError_t launch_forward(const ForwardCall& c, hipStream_t stream) {
    if (c.bf16) {
        if (c.d == 64) return launch_t<true, 64>(c, stream);
        return launch_t<true, 128>(c, stream);
    }
    if (c.d == 64) return launch_t<false, 64>(c, stream);
    return launch_t<false, 128>(c, stream);
}

}  // namespace rsa
