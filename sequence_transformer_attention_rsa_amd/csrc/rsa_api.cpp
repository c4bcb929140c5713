// rsa_api.cpp -- the C ABI declared in include/rsa.h: argument validation
// (before any HIP call), workspace sizing and dispatch to the kernels.

#include "rsa.h"

#include <hip/hip_runtime_api.h>

#include "rsa_internal.h"

namespace {

constexpr int kMaxL = rsa::kFwdKeyTile * rsa::kFwdMaxTiles;   // longest key range per launch

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_sizes(int B, int H, int L, int d, int N, int dtype) {
    if (B <= 0 || H <= 0 || L <= 0 || d <= 0 || N <= 0 || L % N != 0) return RSA_ERR_SHAPE;
    if (d != 64 && d != 128) return RSA_ERR_UNSUPPORTED;
    if (dtype != RSA_F32 && dtype != RSA_BF16) return RSA_ERR_UNSUPPORTED;
    // element offsets are 64-bit; block and row counts must fit the launch grid
    const long long rows = (long long)B * H * L;
    if (rows > (1ll << 30)) return RSA_ERR_UNSUPPORTED;
    return RSA_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? RSA_OK : RSA_ERR_HIP; }

int check_backward(int B, int H, int L, int d, int N, int dtype) {
    int st = check_sizes(B, H, L, d, N, dtype);
    if (st != RSA_OK) return st;
    if (dtype != RSA_BF16) return RSA_ERR_UNSUPPORTED;
    if (L > kMaxL) return RSA_ERR_UNSUPPORTED;
    return RSA_OK;
}

rsa::BackwardCall backward_call(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                const float* lse, const uint8_t* mask, int B, int H, int L, int d, int N) {
    rsa::BackwardCall c{};
    c.q = q;
    c.k = k;
    c.v = v;
    c.out = out;
    c.dout = dout;
    c.lse = lse;
    c.mask = mask;
    c.B = B;
    c.H = H;
    c.L = L;
    c.d = d;
    c.N = N;
    return c;
}

}  // namespace

extern "C" {

int rsa_forward(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                int B, int H, int L, int d, int N, int dtype,
                void* stream, void* out, float* lse) {
    if (!q || !k || !v || !out) return RSA_ERR_NULL;
    int st = check_sizes(B, H, L, d, N, dtype);
    if (st != RSA_OK) return st;
    if (L > kMaxL) return RSA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(key_mask, 16) || !aligned(lse, 4))
        return RSA_ERR_ALIGN;
    rsa::ForwardCall c{};
    c.q = q;
    c.k = k;
    c.v = v;
    c.mask = key_mask;
    c.out = out;
    c.lse = lse;
    c.part = nullptr;
    c.B = B;
    c.H = H;
    c.L = L;
    c.d = d;
    c.N = N;
    c.Lq = L;
    c.q_pos0 = 0;
    c.groups = 1;
    c.bf16 = dtype == RSA_BF16;
    return launch_status(rsa::launch_forward(c, static_cast<hipStream_t>(stream)));
}

size_t rsa_forward_rank_workspace_bytes(int B, int H, int L, int d, int N) {
    if (check_sizes(B, H, L, d, N, RSA_BF16) != RSA_OK) return 0;
    const int g = rsa::forward_rank_groups(B, H, L, d, N);
    const size_t bytes = rsa::forward_partial_bytes(B, H, L / N, d, g);
    return bytes > 0 ? bytes : 256;   // a token buffer when no split is needed
}

int rsa_forward_rank(const void* q_local, const void* k, const void* v, const uint8_t* key_mask,
                     int B, int H, int L, int d, int N, int rank, int dtype,
                     void* workspace, size_t workspace_bytes,
                     void* stream, void* out_local, float* lse_local) {
    if (!q_local || !k || !v || !out_local) return RSA_ERR_NULL;
    int st = check_sizes(B, H, L, d, N, dtype);
    if (st != RSA_OK) return st;
    if (rank < 0 || rank >= N) return RSA_ERR_SHAPE;
    if (!aligned(q_local, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out_local, 16) ||
        !aligned(key_mask, 16) || !aligned(lse_local, 4) || !aligned(workspace, 16))
        return RSA_ERR_ALIGN;
    const int g = rsa::forward_rank_groups(B, H, L, d, N);
    const size_t need = rsa::forward_partial_bytes(B, H, L / N, d, g);
    if (!workspace || workspace_bytes < need) return RSA_ERR_WORKSPACE;
    const int spg = (N + g - 1) / g;
    if ((long long)spg * (L / N) > kMaxL) return RSA_ERR_UNSUPPORTED;
    rsa::ForwardCall c{};
    c.q = q_local;
    c.k = k;
    c.v = v;
    c.mask = key_mask;
    c.out = out_local;
    c.lse = lse_local;
    c.part = static_cast<float*>(workspace);
    c.B = B;
    c.H = H;
    c.L = L;
    c.d = d;
    c.N = N;
    c.Lq = L / N;
    c.q_pos0 = rank * (L / N);
    c.groups = g;
    c.bf16 = dtype == RSA_BF16;
    return launch_status(rsa::launch_forward(c, static_cast<hipStream_t>(stream)));
}

size_t rsa_forward_twopass_workspace_bytes(int B, int H, int L, int d, int N) {
    if (check_sizes(B, H, L, d, N, RSA_BF16) != RSA_OK) return 0;
    return rsa::twopass_workspace_bytes(B, H, L);
}

int rsa_forward_twopass(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                        int B, int H, int L, int d, int N, int dtype,
                        void* workspace, size_t workspace_bytes,
                        void* stream, void* out, float* lse) {
    if (!q || !k || !v || !out) return RSA_ERR_NULL;
    int st = check_sizes(B, H, L, d, N, dtype);
    if (st != RSA_OK) return st;
    if (dtype != RSA_BF16 || L > rsa::kTwoPassMaxL || (long long)B * H > 65535) return RSA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(key_mask, 16) || !aligned(lse, 4) || !aligned(workspace, 16))
        return RSA_ERR_ALIGN;
    if (!workspace || workspace_bytes < rsa::twopass_workspace_bytes(B, H, L)) return RSA_ERR_WORKSPACE;
    rsa::ForwardCall c{};
    c.q = q;
    c.k = k;
    c.v = v;
    c.mask = key_mask;
    c.out = out;
    c.lse = lse;
    c.part = static_cast<float*>(workspace);
    c.B = B;
    c.H = H;
    c.L = L;
    c.d = d;
    c.N = N;
    c.Lq = L;
    c.q_pos0 = 0;
    c.groups = 1;
    c.bf16 = true;
    return launch_status(rsa::launch_forward_twopass(c, static_cast<hipStream_t>(stream)));
}

size_t rsa_backward_workspace_bytes(int B, int H, int L, int d, int N, int dtype) {
    if (check_sizes(B, H, L, d, N, dtype) != RSA_OK) return 0;
    return rsa::backward_workspace_bytes(B, H, L, d);
}

int rsa_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, const uint8_t* key_mask,
                 int B, int H, int L, int d, int N, int dtype,
                 void* workspace, size_t workspace_bytes,
                 void* stream, void* dq, void* dk, void* dv) {
    if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv) return RSA_ERR_NULL;
    int st = check_backward(B, H, L, d, N, dtype);
    if (st != RSA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(key_mask, 16) ||
        !aligned(lse, 4) || !aligned(workspace, 16))
        return RSA_ERR_ALIGN;
    if (!workspace || workspace_bytes < rsa::backward_workspace_bytes(B, H, L, d)) return RSA_ERR_WORKSPACE;
    rsa::BackwardCall c = backward_call(q, k, v, out, dout, lse, key_mask, B, H, L, d, N);
    c.stats = static_cast<float*>(workspace);
    c.dq = dq;
    c.dk = dk;
    c.dv = dv;
    return launch_status(rsa::launch_backward(c, rsa::kBwdStageAll, static_cast<hipStream_t>(stream)));
}

int rsa_backward_preprocess(const void* out, const void* dout, const float* lse, int B, int H, int L, int d,
                            int dtype, void* stream, float* rowstats) {
    if (!out || !dout || !lse || !rowstats) return RSA_ERR_NULL;
    int st = check_backward(B, H, L, d, 1, dtype);
    if (st != RSA_OK) return st;
    if (!aligned(out, 16) || !aligned(dout, 16) || !aligned(lse, 4) || !aligned(rowstats, 4)) return RSA_ERR_ALIGN;
    rsa::BackwardCall c = backward_call(nullptr, nullptr, nullptr, out, dout, lse, nullptr, B, H, L, d, 1);
    c.stats = rowstats;
    return launch_status(rsa::launch_backward(c, rsa::kBwdStagePre, static_cast<hipStream_t>(stream)));
}

int rsa_backward_dq(const void* q, const void* k, const void* v, const void* dout, const float* rowstats,
                    const uint8_t* key_mask, int B, int H, int L, int d, int N, int dtype,
                    void* stream, void* dq) {
    if (!q || !k || !v || !dout || !rowstats || !dq) return RSA_ERR_NULL;
    int st = check_backward(B, H, L, d, N, dtype);
    if (st != RSA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) || !aligned(dq, 16) ||
        !aligned(key_mask, 16) || !aligned(rowstats, 4))
        return RSA_ERR_ALIGN;
    rsa::BackwardCall c = backward_call(q, k, v, nullptr, dout, nullptr, key_mask, B, H, L, d, N);
    c.stats = const_cast<float*>(rowstats);
    c.dq = dq;
    return launch_status(rsa::launch_backward(c, rsa::kBwdStageDq, static_cast<hipStream_t>(stream)));
}

int rsa_backward_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* rowstats,
                      const uint8_t* key_mask, int B, int H, int L, int d, int N, int dtype,
                      void* stream, void* dk, void* dv) {
    if (!q || !k || !v || !dout || !rowstats || !dk || !dv) return RSA_ERR_NULL;
    int st = check_backward(B, H, L, d, N, dtype);
    if (st != RSA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) || !aligned(dk, 16) ||
        !aligned(dv, 16) || !aligned(key_mask, 16) || !aligned(rowstats, 4))
        return RSA_ERR_ALIGN;
    rsa::BackwardCall c = backward_call(q, k, v, nullptr, dout, nullptr, key_mask, B, H, L, d, N);
    c.stats = const_cast<float*>(rowstats);
    c.dk = dk;
    c.dv = dv;
    return launch_status(rsa::launch_backward(c, rsa::kBwdStageDkDv, static_cast<hipStream_t>(stream)));
}

const char* rsa_status_string(int status) {
    switch (status) {
        case RSA_OK: return "RSA_OK";
        case RSA_ERR_NULL: return "RSA_ERR_NULL: a required pointer is NULL";
        case RSA_ERR_SHAPE: return "RSA_ERR_SHAPE: sizes must be positive, L % N == 0 and 0 <= rank < N";
        case RSA_ERR_UNSUPPORTED: return "RSA_ERR_UNSUPPORTED: d must be 64 or 128, dtype RSA_F32 or RSA_BF16, sizes within range";
        case RSA_ERR_ALIGN: return "RSA_ERR_ALIGN: tensor pointers must be 16-byte aligned (lse 4-byte)";
        case RSA_ERR_WORKSPACE: return "RSA_ERR_WORKSPACE: workspace missing or too small";
        case RSA_ERR_HIP: return "RSA_ERR_HIP: the HIP runtime reported a launch error";
        default: return "unknown rsa_status";
    }
}

}  // extern "C"
