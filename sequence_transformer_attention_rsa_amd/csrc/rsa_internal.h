// rsa_internal.h -- host-side launch interface between the C ABI and the
// kernels. Not installed; the public interface is include/rsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rsa {

// Keys per tile of the forward kernels, and the most tiles one workgroup's
// key range may hold (the tile-occupancy table lives in LDS, two bits per
// tile: 4 KB for 16384 tiles = 1048576 keys).
constexpr int kFwdKeyTile = 64;
constexpr int kFwdMaxTiles = 16384;
// Query rows per forward workgroup (4 waves x 32 rows).
constexpr int kFwdQueryTile = 128;

struct ForwardCall {
    const void* q;          // [B,H,Lq,d]
    const void* k;          // [B,H,L,d]
    const void* v;          // [B,H,L,d]
    const uint8_t* mask;    // [B,L] or nullptr
    void* out;              // [B,H,Lq,d]
    float* lse;             // [B,H,Lq] or nullptr
    float* part;            // split partials (groups > 1), see forward_workspace_bytes
    int B, H, L, d, N;
    int Lq;                 // query rows per head held by q / out
    int q_pos0;             // sequence position of q's row 0
    int groups;             // ring-step groups computed in parallel (1 = no split)
    bool bf16;
    bool causal;            // the query at position i sees keys at positions <= i only
    uint32_t drop_p8;       // dropout of the softmax weights, probability drop_p8 / 256 (0: none)
    uint32_t drop_offset;
    uint64_t drop_seed;
};

// Bytes of split partials for `groups` ring-step groups.
size_t forward_partial_bytes(int B, int H, int Lq, int d, int groups);

// Ring-step groups the one-rank-share path uses for these sizes.
int forward_rank_groups(int B, int H, int L, int d, int N);

hipError_t launch_forward(const ForwardCall& c, hipStream_t stream);

// Two-stage forward with the score rows materialised: fp32 scores
// [B,H,L,L] in `part` (rewritten in place as bf16 weights), then P V. The
// softmax pass holds a row in one workgroup's registers up to 16384 keys and
// makes two passes over longer rows; the workspace bounds L in practice.
constexpr int kTwoPassMaxL = kFwdKeyTile * kFwdMaxTiles;
size_t twopass_workspace_bytes(int B, int H, int L);
hipError_t launch_forward_twopass(const ForwardCall& c, hipStream_t stream);

struct BackwardCall {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const void* dout;
    const float* lse;
    const uint8_t* mask;
    float* stats;           // row statistics [2][B,H,L] fp32: -D, -lse*log2(e)
    void* dq;
    void* dk;
    void* dv;
    int B, H, L, d, N;
    bool bf16;              // bf16 tensors; fp32 otherwise
    bool causal;
    uint32_t drop_p8;       // dropout as in ForwardCall (the forward's settings)
    uint32_t drop_offset;
    uint64_t drop_seed;
};

size_t backward_workspace_bytes(int B, int H, int L, int d);

// Every check of rsa_backward_ex except the workspace's: NULL pointers,
// sizes, dtype, flags and alignment, before any HIP call. Returns an
// rsa_status.
int check_backward_call(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, const uint8_t* key_mask, int B, int H, int L, int d, int N, int dtype,
                        int flags, const void* dq, const void* dk, const void* dv);

// Backward stages (bit mask): row statistics; dq; dk and dv.
constexpr int kBwdStagePre = 1;
constexpr int kBwdStageDq = 2;
constexpr int kBwdStageDkDv = 4;
constexpr int kBwdStageAll = kBwdStagePre | kBwdStageDq | kBwdStageDkDv;

hipError_t launch_backward(const BackwardCall& c, int stages, hipStream_t stream);
// fp32 tensors (rsa_bwd_f32.hip); launch_backward dispatches to it.
hipError_t launch_backward_f32(const BackwardCall& c, int stages, hipStream_t stream);

// Token-local steps of the layer around the attention (rsa_layer.hip).
// Matrix product out = act(a w^T + bias) + residual, bf16 operands, fp32
// accumulation; N % 128 == 0 and K % 64 == 0.
constexpr int kLinearRows = 0;      // a [M,K], out0 [M,N]
constexpr int kLinearQkv = 1;       // a [M,K] = x [B*L,E]; out0/1/2 = Q/K/V [B,H,L,d] (N = 3E)
constexpr int kLinearHeadsIn = 2;   // a = attention output [B,H,L,d] read as [B*L,H*d]; out0 [M,N]

struct LinearCall {
    const void* a;
    const void* w;          // [N,K]
    const float* bias;      // [N] or nullptr
    const void* residual;   // [M,N] or nullptr
    void* out0;
    void* out1;
    void* out2;
    int M, N, K;
    int act;                // 0: none, 1: GeLU
    int layout;             // kLinear*
    int L, H, d;            // token/head layout for kLinearQkv and kLinearHeadsIn
};

hipError_t launch_linear(const LinearCall& c, hipStream_t stream);
hipError_t launch_layernorm(const void* x, const float* gamma, const float* beta, int rows, int E, float eps,
                            void* y, hipStream_t stream);

}  // namespace rsa
