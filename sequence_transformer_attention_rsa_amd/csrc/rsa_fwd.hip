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
// Kernel shape (bf16; one workgroup = 4 waves = 128 query rows of one head):
//   * each wave owns 32 query rows; its Q fragment stays in registers;
//   * keys stream through LDS in tiles of 64, double-buffered, copied
//     straight from HBM by global_load_lds (no registers, no VALU) into an
//     XOR-swizzled row-major layout; V^T fragments come from the transposing
//     LDS read, so no transpose is ever stored;
//   * S^T = K Q^T on the 32x32x16 bf16 MFMA. In the 32x32 accumulator layout
//     a lane owns one query column, so the row max and row sum are in-lane
//     plus one exchange between wave halves, and the accumulator is the B
//     operand of O^T = V^T P^T unchanged;
//   * online softmax in base 2 (scale and log2(e) folded into one FMA), with
//     a lazy rescale: the weights are formed against the running base, and
//     only when some lane's sum of its 32 weights of the tile exceeds 2^12
//     (its running row sum grew by more than that) does the wave take the
//     row maximum, move the base and form them again
//     (the fp32 kernel moves the base when a tile's maximum exceeds it by
//     more than 8 in log2 units); exact after the final normalisation;
//   * tiles are dropped from the occupancy table when the causal variant
//     hides all their keys, and masked per element on the diagonal;
//   * P is rounded to bf16 for the MFMA and the row sum adds those same
//     rounded values, so sum_j P_ij = 1 holds for the weights actually used;
//   * tiles whose keys are all padding are skipped (a per-workgroup
//     occupancy table built in LDS), so masked chunks cost nothing; launches
//     without any mask on chunk-aligned tiles build no table at all;
//   * in split mode (one rank's share), each workgroup covers a group of
//     ring steps (every G-th step on chunk-aligned bf16 tiles, so padded
//     chunks spread over the groups; a contiguous run otherwise) and writes
//     unnormalised partials that a merge kernel combines exactly.
// fp32 inputs use a simpler kernel of the same structure on the 32x32x2
// fp32 MFMA.

#include <type_traits>

#include "rsa_device.h"
#include "rsa_internal.h"
#include "rsa_tiles.h"

namespace rsa {
namespace {

constexpr int kThreads = 256;
constexpr int kKT = kFwdKeyTile;   // keys per tile
constexpr int kQW = 32;            // query rows per wave
static_assert(4 * kQW == kFwdQueryTile, "query rows per workgroup");
// Initial running base (raw score units) of both kernels: finite and far
// below any score, so that a row's first visible key forces a rescale (in the
// bf16 kernel every valid weight formed against it overflows to +inf), padded
// keys (-inf) give weight 0, and a rescale of a row that has seen no key yet
// keeps a factor of exactly 1.
constexpr float kNoBase = -1.0e30f;
// Largest sum of one lane's 32 weights of a tile before the running base is
// moved up (each weight then stays <= 2^12, far from fp32 and bf16 limits).
constexpr float kMaxTileSum = 4096.0f;

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
    int strided;      // bf16, groups > 1, contiguous: group g takes ring steps g, g + groups, ...
    int causal;       // the query at position i sees keys at positions <= i only
    Dropout drop;     // dropout of the normalised weights (drop.p8 == 0: none)
};

// fp32 forward (fp32 inputs and output): the same ring-ordered online
// softmax on the 32x32x2 fp32 MFMA. K is staged row-major with pitch d+1
// (a lane reads one element of its own key row: conflict-free), V row-major
// (a lane reads one element of its own d column).
template <int D>
struct F32Cfg {
    static constexpr int KP = D + 1;
    static constexpr int K_ELEMS = kKT * KP;
    static constexpr int V_ELEMS = kKT * D;
    static constexpr int BUF = K_ELEMS + V_ELEMS;
    static constexpr int CH = (kKT * D / 4) / kThreads;   // 16-byte chunks per thread and tensor
    static_assert(CH * kThreads * 4 == kKT * D, "fp32 staging");
};

template <int D>
__global__ __launch_bounds__(kThreads) void rsa_fwd_f32(FwdParams p) {
    using C = F32Cfg<D>;
    __shared__ __attribute__((aligned(16))) float smem[2 * C::BUF];
    __shared__ uint8_t tflag_bytes[kFwdMaxTiles / 4];
    const TileTable tflag{tflag_bytes};

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

    const float* qh = static_cast<const float*>(p.q) + (size_t)bh * p.Lq * D;
    const float* kh = static_cast<const float*>(p.k) + (size_t)bh * p.L * D;
    const float* vh = static_cast<const float*>(p.v) + (size_t)bh * p.L * D;
    const uint8_t* mrow = p.mask ? p.mask + (size_t)b * p.L : nullptr;
    if (ntile > kFwdMaxTiles) return;   // the host never launches such a range
    const bool contig = p.contiguous != 0;

    const int qlo = p.q_pos0 + row0, qhi = p.q_pos0 + min(row0 + 4 * kQW, p.Lq) - 1;
    tflag.build(ntile, kThreads, [&](int t) {
        const int v0 = vbeg + t * kKT;
        const uint32_t f = key_tile_flags(mrow, n, p.N, p.Lc, contig, v0, vend);
        return p.causal ? f & causal_tile_class(v0, min(kKT, vend - v0), n, p.N, p.Lc, contig, qlo, qhi) : f;
    });

    // Q^T fragments (B operand of S^T = K Q^T): lane (j, h) holds Q[row][2 ks + h]
    float qf[D / 2];
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) qf[ks] = row_ok ? qh[(size_t)row * D + 2 * ks + h] : 0.0f;

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    // running base (raw score units): the finite sentinel kNoBase until the
    // row meets a visible key, so that a rescale forced by another lane of
    // the wave never forms -inf - (-inf) for a row that has seen none yet
    float m_b = kNoBase;
    float l = 0.0f;          // running row sum over this lane half's keys

    __syncthreads();   // tile flags visible

    u32x4 kst[C::CH], vst[C::CH];
    auto load = [&](int t) {
        const int v0 = vbeg + t * kKT;
        const int pos0 = contig ? ring_pos(v0, n, p.N, p.Lc) : 0;
#pragma unroll
        for (int i = 0; i < C::CH; ++i) {
            const int c = threadIdx.x + i * kThreads;
            const int r = c / (D / 4), col = c % (D / 4);
            const int vk = v0 + r;
            u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
            if (vk < vend) {
                const size_t pos = contig ? pos0 + r : ring_pos(vk, n, p.N, p.Lc);
                xk = *reinterpret_cast<const u32x4*>(kh + pos * D + 4 * col);
                xv = *reinterpret_cast<const u32x4*>(vh + pos * D + 4 * col);
            }
            kst[i] = xk;
            vst[i] = xv;
        }
    };
    auto store = [&](float* buf) {
#pragma unroll
        for (int i = 0; i < C::CH; ++i) {
            const int c = threadIdx.x + i * kThreads;
            const int r = c / (D / 4), col = c % (D / 4);
            float* dst = buf + r * C::KP + 4 * col;
            dst[0] = __uint_as_float(kst[i][0]);
            dst[1] = __uint_as_float(kst[i][1]);
            dst[2] = __uint_as_float(kst[i][2]);
            dst[3] = __uint_as_float(kst[i][3]);
            *reinterpret_cast<u32x4*>(buf + C::K_ELEMS + r * D + 4 * col) = vst[i];
        }
    };

    int t = 0;
    while (t < ntile && !(tflag.get(t) & 1)) ++t;
    int buf = 0;
    if (t < ntile) {
        load(t);
        store(smem);
    }
    while (t < ntile) {
        int tn = t + 1;
        while (tn < ntile && !(tflag.get(tn) & 1)) ++tn;
        if (tn < ntile) load(tn);
        __syncthreads();   // buffer `buf` complete; the other one is free

        const float* ks_ = smem + buf * C::BUF;
        const float* vs_ = ks_ + C::K_ELEMS;
        const int v0 = vbeg + t * kKT;

        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
            for (int kq = 0; kq < D / 2; ++kq) s[kb] = mfma_32x32x2_f32(ks_[(32 * kb + j) * C::KP + 2 * kq + h], qf[kq], s[kb]);
        }
        if (!(tflag.get(t) & 2)) {
            const uint64_t bits = key_tile_bits(mrow, n, p.N, p.Lc, contig, v0, vend);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (!((bits >> (32 * kb + acc_row(r, h))) & 1ull)) s[kb][r] = -INFINITY;
            if (p.causal) {   // keys after this lane's query position
                const int qpos = p.q_pos0 + row;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int vk = v0 + 32 * kb + acc_row(r, h);
                        if (vk < vend && ring_pos(vk, n, p.N, p.Lc) > qpos) s[kb][r] = -INFINITY;
                    }
            }
        }
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
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        }
        const float nb = -m_b * p.sl2;
        // O^T += V^T P^T: one MFMA per accumulator register; step r contracts
        // key acc_row(r, h) of lane half h
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float pr = fast_exp2(fmaf(s[kb][r], p.sl2, nb));
                l += pr;   // the row sum counts every weight, kept or dropped
                const int key = 32 * kb + acc_row(r, h);
                if (p.drop.p8 != 0u) {
                    const int vk = v0 + key;
                    if (vk < vend && !dropout_keep(p.drop, p.q_pos0 + row, ring_pos(vk, n, p.N, p.Lc), bh)) pr = 0.0f;
                }
#pragma unroll
                for (int db = 0; db < D / 32; ++db) o[db] = mfma_32x32x2_f32(vs_[key * D + 32 * db + j], pr, o[db]);
            }

        if (tn < ntile) store(smem + (buf ^ 1) * C::BUF);
        buf ^= 1;
        t = tn;
    }

    const float l_row = l + shfl_xor32(l);
    if (!row_ok) return;
    const float ks = p.drop.p8 != 0u ? p.drop.scale : 1.0f;   // kept weights scaled by 1 / (1 - p)
    if (p.groups == 1) {
        const float inv = l_row > 0.0f ? ks / l_row : 0.0f;
        float* orow = static_cast<float*>(p.out) + ((size_t)bh * p.Lq + row) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 w = {o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv, o[db][4 * r4 + 2] * inv,
                                 o[db][4 * r4 + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * r4 + 4 * h) = w;
            }
        if (p.lse && h == 0)
            p.lse[(size_t)bh * p.Lq + row] = l_row > 0.0f ? (m_b * p.sl2 + __log2f(l_row)) * kLn2 : -INFINITY;
    } else {
        const size_t prow = ((size_t)g * p.BH + bh) * p.Lq + row;
        float* po = p.part_o + prow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 w = {o[db][4 * r4] * ks, o[db][4 * r4 + 1] * ks, o[db][4 * r4 + 2] * ks,
                                 o[db][4 * r4 + 3] * ks};
                *reinterpret_cast<f32x4*>(po + 32 * db + 8 * r4 + 4 * h) = w;
            }
        if (h == 0) {
            p.part_ml[2 * prow] = l_row > 0.0f ? m_b * p.sl2 : -INFINITY;
            p.part_ml[2 * prow + 1] = l_row;
        }
    }
}

// bf16 forward. Two LDS buffers: after the barrier that opens tile t (at
// d = 64 without causal mask or dropout: after tile t's score MFMAs), the
// copy of tile t+1 is issued into the buffer that held tile t-1 and lands
// while tile t is computed. Chunk-aligned key ranges use copies the
// compiler does not track (see rsa_tiles.h), so nothing but the explicit
// vm_wait before each barrier waits for them. Registers are held to 128 so
// that four waves run per SIMD at d = 64 (two at d = 128): with several
// workgroups per CU, one wave's MFMAs run while another's softmax occupies
// the vector ALU. (A variant that overlapped the next tile's score MFMAs
// with this tile's softmax inside one wave needed more registers, ran at
// fewer waves per SIMD and was slower; so was three buffers at three waves.)
// FULL: no key mask and chunk-aligned tiles, so every key tile of the range
// is whole: the occupancy table is not built and the loop takes every tile
// without looking it up. With the causal mask (FULL and CAUSAL: one group,
// chunks and the rows' first position multiples of 128, so that a
// workgroup's rows lie in one chunk) the visible tiles are walked directly:
// in ring order the rows' own chunk comes first, whose tiles up to the
// workgroup's last row are visible (the last two of them partly, masked per
// element), then the earlier chunks, whole; the later chunks are hidden.
// DROP: dropout of the normalised weights (the row sums count every weight;
// dropped ones are zeroed in the packed bf16 operand of the PV product and
// the output is scaled by 1 / (1 - p) at the end). The dropout instances run
// at three waves per SIMD: the keep-decision generator does not fit 128
// registers (11-16 of them went to scratch at four waves).
template <int D, bool CONTIG, int QB, bool CAUSAL, bool FULL = false, bool DROP = false, bool KSPLIT = false>
__global__ __launch_bounds__(256 / QB, (D == 64 && QB == 1) ? (DROP ? 3 : 4) : 2)
void rsa_fwd_bf16(FwdParams p) {
    static_assert(!FULL || CONTIG, "whole tiles need chunk-aligned ranges");
    static_assert(!DROP || QB == 1, "dropout instances: one query block per wave");
    static_assert(!KSPLIT || (QB == 1 && !CAUSAL && !DROP), "key-split instances: plain launches");
    // QB 32-row query blocks per wave; 128 query rows per workgroup either
    // way (4 waves x 32 rows, or 2 waves x 64 rows: each K and V^T fragment
    // read from LDS then feeds two MFMAs).
    constexpr int WAVES = 4 / QB;
    constexpr int NTH = WAVES * kWave;
    using KTile = DirectTile<D, WAVES>;
    using VTile = DirectTile<D, WAVES>;
    constexpr int BUF = KTile::BYTES + VTile::BYTES;
    constexpr int NBUF = 2;   // 4 x (2 x 16 KB + 4 KB) of LDS per CU at d = 64
    // KSPLIT (small grids): 64 rows per workgroup, waves 0 and 1 take rows
    // 0-31 and 32-63 against keys 0-31 of every tile, waves 2 and 3 the same
    // rows against keys 32-63; the two halves merge at the end
    constexpr int ROWS = KSPLIT ? 2 * 32 : 4 * 32;
    constexpr int NKB = KSPLIT ? 1 : 2;   // 32-key blocks of a tile per wave
    // d = 64 without causal mask or dropout: the copy of the next tile is
    // issued after this tile's score MFMAs rather than before them, so that
    // the first fragment reads and MFMAs of a tile do not queue behind the
    // copy instructions (2% at L = 8192; the other instances measured
    // slower that way)
    constexpr bool LATE_COPY = D == 64 && !CAUSAL && !DROP;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NBUF * BUF];
    __shared__ uint8_t tflag_bytes[FULL ? 4 : kFwdMaxTiles / 4];
    const TileTable tflag{tflag_bytes};

    int qt, g, bh;
    if (p.groups == 1) {
        // causal: the last query tiles of a head see the most keys; dispatch
        // them first so that the light ones fill the tail
        head_order(blockIdx.x, p.nqt, p.BH, CAUSAL, qt, bh);
        if (CAUSAL) qt = p.nqt - 1 - qt;
        g = 0;
    } else {
        const int lid = xcd_remap(blockIdx.x, p.nqt * p.BH * p.groups);
        qt = CAUSAL ? p.nqt - 1 - lid % p.nqt : lid % p.nqt;
        const int rest = lid / p.nqt;
        g = rest % p.groups;
        bh = rest / p.groups;
    }
    const int b = bh / p.H;

    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int j = lane & 31, h = lane >> 5;
    const int row0 = qt * ROWS;
    const int wrow0 = row0 + (KSPLIT ? (wave & 1) : wave) * 32 * QB;
    const int khalf = KSPLIT ? wave >> 1 : 0;   // this wave's 32-key half of each tile
    const int n = (p.q_pos0 + row0) / p.Lc;

    const int step0 = g * p.spg;
    const int step1 = min(p.N, step0 + p.spg);
    const int vbeg = step0 * p.Lc, vend = step1 * p.Lc;
    // Ring indices of this workgroup's key tiles. One group, or tiles that
    // straddle chunks: the ring steps [step0, step1) in order. Several groups
    // on chunk-aligned tiles: group g takes every groups-th ring step (g,
    // g + groups, ...), so the padded chunks, which a rank meets one after
    // another, spread evenly over the groups (the merge is exact for any
    // grouping of the steps).
    const bool strided = CONTIG && p.strided;
    const int tpc = p.Lc / kKT;   // tiles per chunk (chunk-aligned tiles)
    const int ntile = strided ? (p.N - g + p.groups - 1) / p.groups * tpc : (vend - vbeg + kKT - 1) / kKT;
    auto tile_v0 = [&](int t) { return strided ? (g + p.groups * (t / tpc)) * p.Lc + (t % tpc) * kKT : vbeg + t * kKT; };
    auto tile_end = [&](int v0) { return strided ? v0 + kKT : vend; };

    const uint16_t* qh = static_cast<const uint16_t*>(p.q) + (size_t)bh * p.Lq * D;
    const uint16_t* kh = static_cast<const uint16_t*>(p.k) + (size_t)bh * p.L * D;
    const uint16_t* vh = static_cast<const uint16_t*>(p.v) + (size_t)bh * p.L * D;
    const uint8_t* mrow = p.mask ? p.mask + (size_t)b * p.L : nullptr;
    if (ntile > kFwdMaxTiles) return;   // the host never launches such a range

    const int qlo = p.q_pos0 + row0, qhi = p.q_pos0 + min(row0 + ROWS, p.Lq) - 1;
    if constexpr (!FULL) {
        tflag.build(ntile, NTH, [&](int t) {
            const int v0 = tile_v0(t), ve = tile_end(v0);
            const uint32_t f = key_tile_flags(mrow, n, p.N, p.Lc, CONTIG, v0, ve);
            return CAUSAL ? f & causal_tile_class(v0, min(kKT, ve - v0), n, p.N, p.Lc, CONTIG, qlo, qhi) : f;
        });
    }

    u32x4 qf[QB][D / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = wrow0 + 32 * qb + j;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (row < p.Lq) x = *reinterpret_cast<const u32x4*>(qh + (size_t)row * D + 16 * ks + 8 * h);
            qf[qb][ks] = x;
        }
    }
    f32x16 o[QB][D / 32];
    // running base m_b (raw score units) and nb = -m_b * log2(e)/sqrt(d);
    // running row sums l0, l1 (two dot-product chains); lim = l0 + l1 +
    // kMaxTileSum, the sum beyond which a tile's weights are too large
    float m_b[QB], nb[QB], l0[QB], l1[QB], lim[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.0f;
        m_b[qb] = kNoBase;
        nb[qb] = -kNoBase * p.sl2;
        l0[qb] = 0.0f;
        l1[qb] = 0.0f;
        lim[qb] = kMaxTileSum;
    }

    // The Q fragments have landed (waited for here, so that the compiler
    // keeps no wait for them inside the tile loop); tile flags visible.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    uint32_t voff[KTile::IPW];
    KTile::row_offsets(voff);
    const uint32_t wave_lds = KTile::wave_lds_offset();
    auto load = [&](int t, int bi) {
        const int v0 = tile_v0(t);
        uint8_t* kbuf = smem + bi * BUF;
        uint8_t* vbuf = kbuf + KTile::BYTES;
        if constexpr (CONTIG) {
            const int pos0 = ring_pos(v0, n, p.N, p.Lc);
            KTile::load_rows(kbuf, kh + (size_t)pos0 * D, voff, wave_lds);
            VTile::load_rows(vbuf, vh + (size_t)pos0 * D, voff, wave_lds);
        } else {
            auto rowoff = [&](int r) -> size_t {
                const int vk = v0 + r;
                return vk < vend ? (size_t)ring_pos(vk, n, p.N, p.Lc) * D : 0;
            };
            KTile::load(kbuf, [&](int r) { return kh + rowoff(r); });
            VTile::load(vbuf, [&](int r) { return vh + rowoff(r); });
        }
    };
    // FULL and CAUSAL: tiles 0 .. lo/64 + 1 of the own chunk (lo = the
    // workgroup's first row position within it), then tpc .. (n + 1) tpc - 1
    const int tdiag = (qlo - n * p.Lc) / kKT;   // first partly visible tile
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

    int t = next_tile(-1);
    auto body = [&](auto cb_c) -> bool {
        constexpr int CB = decltype(cb_c)::value;
        vm_wait<0>();
        bare_barrier();   // every wave's part of tile t landed, tile t-1 consumed
        const int tn = next_tile(t);
        if (!LATE_COPY && tn < tend) load(tn, CB ^ 1);
        const uint8_t* kbuf = smem + CB * BUF;
        const uint8_t* vbuf = kbuf + KTile::BYTES;

        // ---- S^T = K Q^T for 64 keys (two 32-key blocks). All K fragments
        // are requested before the first MFMA so their LDS latency overlaps.
        f32x16 s[QB][2];
        {
            u32x4 kf[2][D / 16];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int kq = 0; kq < D / 16; ++kq) kf[kb][kq] = KTile::chunk(kbuf, 32 * (kb + khalf) + j, 2 * kq + h);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.0f;
            // the 2 * QB accumulation chains interleaved: a dependent MFMA
            // waits for the whole latency of its predecessor
#pragma unroll
            for (int kq = 0; kq < D / 16; ++kq)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        s[qb][kb] = mfma_32x32x16_bf16(kf[kb][kq], qf[qb][kq], s[qb][kb]);
        }
        if (LATE_COPY && tn < tend) load(tn, CB ^ 1);
        // ---- key mask and range tail (tiles not fully valid)
        const bool part = FULL ? (CAUSAL && t >= tdiag && t < tpc) : !(tflag.get(t) & 2);
        if (part) {
            if constexpr (!FULL) {
                // key acc_row(r, h) = 8 (r / 4) + 4 h + r % 4 of block kb: after
                // one shift by 4 h every bit position is a constant (no
                // per-register masks held in registers)
                const int tv0 = tile_v0(t);
                const uint64_t bits = key_tile_bits(mrow, n, p.N, p.Lc, CONTIG, tv0, tile_end(tv0)) >> (4 * h + 32 * khalf);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (!((bits >> (32 * kb + 8 * (r >> 2) + (r & 3))) & 1ull)) {
#pragma unroll
                            for (int qb = 0; qb < QB; ++qb) s[qb][kb][r] = -INFINITY;
                        }
            }
            if constexpr (CAUSAL) {
                // keys after this lane's query position; within a chunk-aligned
                // tile key 32 kb + acc_row(r, h) sits at position kp0 plus that,
                // so one offset per lane leaves constant comparisons
                const int v0 = tile_v0(t);
                const int kp0 = CONTIG ? ring_pos(v0, n, p.N, p.Lc) : 0;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int qpos = p.q_pos0 + wrow0 + 32 * qb + j;
                    const int rel = qpos - kp0 - 4 * h;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int i = 32 * kb + 8 * (r >> 2) + (r & 3);
                            bool hide;
                            if constexpr (CONTIG) {
                                hide = i > rel;
                            } else {
                                const int vk = v0 + i + 4 * h;
                                hide = vk < vend && ring_pos(vk, n, p.N, p.Lc) > qpos;
                            }
                            if (hide) s[qb][kb][r] = -INFINITY;
                        }
                }
            }
        }
        // ---- online softmax (base 2). The weights are formed against the
        // running base first; only when some lane's tile sum exceeds
        // kMaxTileSum (always, while the base is still kNoBase) does the wave
        // take the row maximum, move the base up, rescale and form them again.
        // the row sums after this tile: the dot-product chains continue from
        // l0 and l1, and the tile's weights were too large if the sum passed lim
        uint32_t pk[QB][2][8];
        float tl0[QB], tl1[QB], tsum[QB];
        auto weights = [&](int qb) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float p0 = fast_exp2(fmaf(s[qb][kb][2 * i], p.sl2, nb[qb]));
                    const float p1 = fast_exp2(fmaf(s[qb][kb][2 * i + 1], p.sl2, nb[qb]));
                    pk[qb][kb][i] = pack_bf16x2(p0, p1);
                }
            float a0 = l0[qb], a1 = l1[qb];
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                a0 = add_bf16x2(pk[qb][0][i], a0);
                a1 = add_bf16x2(pk[qb][0][i + 1], a1);
                if constexpr (NKB == 2) {
                    a0 = add_bf16x2(pk[qb][1][i], a0);
                    a1 = add_bf16x2(pk[qb][1][i + 1], a1);
                }
            }
            tl0[qb] = a0;
            tl1[qb] = a1;
            tsum[qb] = a0 + a1;
        };
        bool over = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            weights(qb);
            over |= tsum[qb] > lim[qb];
        }
        if (wave_any(over)) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float a = __builtin_fmaxf(s[qb][0][0], s[qb][0][1]);
#pragma unroll
                for (int r = 2; r < 16; r += 2) a = __builtin_fmaxf(a, __builtin_fmaxf(s[qb][0][r], s[qb][0][r + 1]));
                if constexpr (NKB == 2) {
#pragma unroll
                    for (int r = 0; r < 16; r += 2) a = __builtin_fmaxf(a, __builtin_fmaxf(s[qb][1][r], s[qb][1][r + 1]));
                }
                const float m_new = fmaxf(m_b[qb], fmaxf(a, shfl_xor32(a)));
                const float alpha = fast_exp2((m_b[qb] - m_new) * p.sl2);
                m_b[qb] = m_new;
                nb[qb] = -m_new * p.sl2;
                l0[qb] *= alpha;
                l1[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
                weights(qb);
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            l0[qb] = tl0[qb];
            l1[qb] = tl1[qb];
            lim[qb] = tsum[qb] + kMaxTileSum;
        }
        if constexpr (DROP) {
            // zero the dropped weights: dword i of block kb holds keys
            // 8 (i / 2) + 4 h + 2 (i % 2) + {0, 1} of the block, whose keep
            // bytes are bytes 2 (i % 2) + {0, 1} of word i / 2
            const int qpos = p.q_pos0 + wrow0 + j;
            const int tv0 = tile_v0(t);
            if constexpr (CONTIG) {
                const int jb0 = ring_pos(tv0, n, p.N, p.Lc) >> 5;   // tiles are 64-key aligned here
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const u32x4 x = dropout_bytes(p.drop, jb0 + kb, h, qpos, bh);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        pk[0][kb][i] &= keep_mask_bf16x2(x[i >> 1] >> (16 * (i & 1)), p.drop.p8);
                }
            } else {
                const int ve = tile_end(tv0);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        uint32_t m = 0xffffffffu;
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int vk = tv0 + 32 * kb + acc_row(2 * i + e, h);
                            if (vk < ve && !dropout_keep(p.drop, qpos, ring_pos(vk, n, p.N, p.Lc), bh))
                                m &= e ? 0x0000ffffu : 0xffff0000u;
                        }
                        pk[0][kb][i] &= m;
                    }
            }
        }
        // ---- O^T += V^T P^T, 16-key steps over this wave's keys
#pragma unroll
        for (int stp = 0; stp < 2 * NKB; ++stp) {
            u32x4 vf[D / 32];
#pragma unroll
            for (int db = 0; db < D / 32; ++db) vf[db] = VTile::tfrag(vbuf, 16 * stp + 32 * khalf, 32 * db);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const u32x4 bfrag = acc_frag(pk[qb], stp);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) o[qb][db] = mfma_32x32x16_bf16(vf[db], bfrag, o[qb][db]);
            }
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
        // The exact merge of the two key halves (as for ring-step groups):
        // waves 2 and 3 hand their base, lane row sum and O to waves 0 and 1
        // through LDS; then waves 0 and 1 finish the rows.
        constexpr int XS = (D / 32) * 16 + 4;   // floats per lane: O, base, row sum (16-byte rows)
        static_assert(2 * kWave * XS * sizeof(float) <= sizeof(smem), "merge area inside the tile buffers");
        float* xs = reinterpret_cast<float*>(smem) + ((wave & 1) * kWave + lane) * XS;
        const float lsum = l0[0] + l1[0];
        __syncthreads();   // every wave is done with the tile buffers
        if (khalf == 1) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    *reinterpret_cast<f32x4*>(xs + 16 * db + 4 * r4) =
                        f32x4{o[0][db][4 * r4], o[0][db][4 * r4 + 1], o[0][db][4 * r4 + 2], o[0][db][4 * r4 + 3]};
            xs[XS - 4] = m_b[0];
            xs[XS - 3] = lsum;
        }
        __syncthreads();
        if (khalf == 1) return;
        const float m1 = xs[XS - 4], ls1 = xs[XS - 3];
        const float mm = fmaxf(m_b[0], m1);
        const float a0 = fast_exp2((m_b[0] - mm) * p.sl2), a1 = fast_exp2((m1 - mm) * p.sl2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(xs + 16 * db + 4 * r4);
#pragma unroll
                for (int e = 0; e < 4; ++e) o[0][db][4 * r4 + e] = a0 * o[0][db][4 * r4 + e] + a1 * x[e];
            }
        m_b[0] = mm;
        l0[0] = a0 * lsum + a1 * ls1;
        l1[0] = 0.0f;
    }

    // ---- epilogue
    const float ks = DROP ? p.drop.scale : 1.0f;   // kept weights scaled by 1 / (1 - p)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = wrow0 + 32 * qb + j;
        const float lsum = l0[qb] + l1[qb];
        const float l_row = lsum + shfl_xor32(lsum);
        if (row >= p.Lq) continue;
        if (p.groups == 1) {
            const float inv = l_row > 0.0f ? ks / l_row : 0.0f;
            uint16_t* orow = static_cast<uint16_t*>(p.out) + ((size_t)bh * p.Lq + row) * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const f32x16& a = o[qb][db];
                    const u32x2 w = {pack_bf16x2(a[4 * r4] * inv, a[4 * r4 + 1] * inv),
                                     pack_bf16x2(a[4 * r4 + 2] * inv, a[4 * r4 + 3] * inv)};
                    *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * r4 + 4 * h) = w;
                }
            if (p.lse && h == 0)
                p.lse[(size_t)bh * p.Lq + row] =
                    l_row > 0.0f ? (m_b[qb] * p.sl2 + __log2f(l_row)) * kLn2 : -INFINITY;
        } else {
            const size_t prow = ((size_t)g * p.BH + bh) * p.Lq + row;
            float* po = p.part_o + prow * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const f32x16& a = o[qb][db];
                    const f32x4 w = {a[4 * r4] * ks, a[4 * r4 + 1] * ks, a[4 * r4 + 2] * ks, a[4 * r4 + 3] * ks};
                    *reinterpret_cast<f32x4*>(po + 32 * db + 8 * r4 + 4 * h) = w;
                }
            if (h == 0) {
                p.part_ml[2 * prow] = l_row > 0.0f ? m_b[qb] * p.sl2 : -INFINITY;
                p.part_ml[2 * prow + 1] = l_row;
            }
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
    using E = typename std::conditional<BF16, uint16_t, float>::type;
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
    p.strided = (BF16 && c.groups > 1 && p.contiguous) ? 1 : 0;
    p.causal = c.causal ? 1 : 0;
    p.drop.p8 = c.drop_p8;
    p.drop.seed_lo = (uint32_t)c.drop_seed;
    p.drop.seed_hi = (uint32_t)(c.drop_seed >> 32);
    p.drop.offset = c.drop_offset;
    p.drop.scale = (float)(256.0 / (256.0 - (double)c.drop_p8));
    p.drop.keep = (float)((256.0 - (double)c.drop_p8) / 256.0);
    if (c.groups > 1) {
        p.part_o = c.part;
        p.part_ml = c.part + (size_t)c.groups * p.BH * c.Lq * D;
    }
    const long long total = (long long)p.nqt * p.BH * p.groups;
    if (total <= 0) return hipSuccess;
    if constexpr (BF16) {
        // 32 query rows per wave: 64 (QB = 2, two waves per workgroup) halves the
        // LDS reads per MFMA but needs 256 VGPRs and two waves per SIMD, and
        // measured 12% slower at d = 64.
        constexpr int QB = 1;
        const dim3 block(kWave * 4 / QB);
        if (p.drop.p8 != 0u) {
            if (p.contiguous && !p.causal && p.mask == nullptr)
                hipLaunchKernelGGL((rsa_fwd_bf16<D, true, QB, false, true, true>), dim3((unsigned)total), block, 0,
                                   stream, p);
            else if (p.contiguous && !p.causal)
                hipLaunchKernelGGL((rsa_fwd_bf16<D, true, QB, false, false, true>), dim3((unsigned)total), block, 0,
                                   stream, p);
            else if (!p.causal)
                hipLaunchKernelGGL((rsa_fwd_bf16<D, false, QB, false, false, true>), dim3((unsigned)total), block, 0,
                                   stream, p);
            else if (p.contiguous)
                hipLaunchKernelGGL((rsa_fwd_bf16<D, true, QB, true, false, true>), dim3((unsigned)total), block, 0,
                                   stream, p);
            else
                hipLaunchKernelGGL((rsa_fwd_bf16<D, false, QB, true, false, true>), dim3((unsigned)total), block, 0,
                                   stream, p);
        } else if (D == 64 && p.contiguous && !p.causal && c.groups == 1 && total <= 2 * kCUs) {
            // few workgroups (at most two per CU): split each tile's keys
            // between two wave pairs, 64 rows per workgroup, so that twice
            // as many waves run
            if constexpr (D == 64) {
                p.nqt = (c.Lq + 63) / 64;
                const dim3 grid((unsigned)((long long)p.nqt * p.BH));
                if (p.mask == nullptr)
                    hipLaunchKernelGGL((rsa_fwd_bf16<D, true, QB, false, true, false, true>), grid, block, 0, stream, p);
                else
                    hipLaunchKernelGGL((rsa_fwd_bf16<D, true, QB, false, false, false, true>), grid, block, 0, stream,
                                       p);
            }
        } else if (p.contiguous && !p.causal && p.mask == nullptr)
            hipLaunchKernelGGL((rsa_fwd_bf16<D, true, QB, false, true>), dim3((unsigned)total), block, 0, stream, p);
        else if (p.contiguous && p.causal && p.mask == nullptr && c.groups == 1 && p.Lc % 128 == 0 &&
                 c.q_pos0 % 128 == 0 && c.Lq % 128 == 0)
            hipLaunchKernelGGL((rsa_fwd_bf16<D, true, QB, true, true>), dim3((unsigned)total), block, 0, stream, p);
        else if (p.contiguous && !p.causal)
            hipLaunchKernelGGL((rsa_fwd_bf16<D, true, QB, false>), dim3((unsigned)total), block, 0, stream, p);
        else if (!p.causal)
            hipLaunchKernelGGL((rsa_fwd_bf16<D, false, QB, false>), dim3((unsigned)total), block, 0, stream, p);
        else if (p.contiguous)
            hipLaunchKernelGGL((rsa_fwd_bf16<D, true, QB, true>), dim3((unsigned)total), block, 0, stream, p);
        else
            hipLaunchKernelGGL((rsa_fwd_bf16<D, false, QB, true>), dim3((unsigned)total), block, 0, stream, p);
    } else {
        hipLaunchKernelGGL((rsa_fwd_f32<D>), dim3((unsigned)total), dim3(kThreads), 0, stream, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || c.groups == 1) return e;
    const int rows = p.BH * c.Lq;
    const long long threads = (long long)rows * (D / 4);
    hipLaunchKernelGGL((rsa_merge_kernel<BF16, D>), dim3((unsigned)((threads + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, p.part_o, p.part_ml, c.groups, rows, c.out, c.lse);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const ForwardCall& c, hipStream_t stream) {
    if (c.bf16) {
        if (c.d == 64) return launch_t<true, 64>(c, stream);
        return launch_t<true, 128>(c, stream);
    }
    if (c.d == 64) return launch_t<false, 64>(c, stream);
    return launch_t<false, 128>(c, stream);
}

}  // namespace rsa
