// rsa_api.cpp -- the C ABI declared in include/rsa.h: argument validation
// (before any HIP call), workspace sizing and dispatch to the kernels.

#include "rsa.h"

#include <hip/hip_runtime_api.h>

#include "rsa_internal.h"

namespace {

constexpr int kMaxL = rsa::kFwdKeyTile * rsa::kFwdMaxTiles;   // longest key range per launch

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// NaN and infinities are recognised by their bits: the library is compiled
// assuming arithmetic never meets a NaN, so a comparison would not reject one.
bool finite_float(float x) {
    uint32_t bits;
    __builtin_memcpy(&bits, &x, sizeof(bits));
    return (bits & 0x7f800000u) != 0x7f800000u;
}

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

// The dropout probability quantised to p8 / 256, p8 = floor(256 p + 1/2);
// false if p is not a number or p8 falls outside [0, 255].
bool dropout_p8(const rsa_dropout* dr, uint32_t* p8) {
    *p8 = 0;
    if (dr == nullptr) return true;
    const float p = dr->p;
    if (!finite_float(p) || !(p >= 0.0f && p < 1.0f)) return false;
    const float q = __builtin_floorf(p * 256.0f + 0.5f);   // exact: p * 256 and the sum are representable
    if (q > 255.0f) return false;
    *p8 = (uint32_t)q;
    return true;
}

template <class Call>
void set_dropout(Call& c, const rsa_dropout* dr, uint32_t p8) {
    c.drop_p8 = p8;
    c.drop_seed = p8 != 0 ? dr->seed : 0;
    c.drop_offset = p8 != 0 ? dr->offset : 0;
}

int check_backward(int B, int H, int L, int d, int N, int dtype) {
    int st = check_sizes(B, H, L, d, N, dtype);
    if (st != RSA_OK) return st;
    if (L > kMaxL) return RSA_ERR_UNSUPPORTED;
    return RSA_OK;
}

rsa::BackwardCall backward_call(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                const float* lse, const uint8_t* mask, int B, int H, int L, int d, int N,
                                int dtype) {
    rsa::BackwardCall c{};
    c.bf16 = dtype == RSA_BF16;
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

// The token-local steps: bf16 only, widths the 128x128 product tiles and
// the 64-wide contraction steps divide, hidden sizes the head split and
// the layer normalisation cover.
int check_linear(int M, int N, int K, int act) {
    if (M <= 0 || N <= 0 || K <= 0) return RSA_ERR_SHAPE;
    if (N % 128 != 0 || K % 64 != 0 || (act != 0 && act != 1)) return RSA_ERR_UNSUPPORTED;
    if ((long long)M > (1ll << 30) || (long long)K > (1ll << 20) || (long long)N > (1ll << 20))
        return RSA_ERR_UNSUPPORTED;
    if ((long long)((M + 127) / 128) * (N / 128) > (1ll << 31) - 1) return RSA_ERR_UNSUPPORTED;   // grid size
    return RSA_OK;
}

int check_heads(int B, int L, int E, int H) {
    if (B <= 0 || L <= 0 || E <= 0 || H <= 0 || E % H != 0) return RSA_ERR_SHAPE;
    const int d = E / H;
    if ((d != 64 && d != 128) || E % 128 != 0) return RSA_ERR_UNSUPPORTED;
    // the head-layout operand is addressed with 32-bit byte offsets
    if ((long long)B * L * E * 2 >= (1ll << 32)) return RSA_ERR_UNSUPPORTED;
    return check_linear(B * L, E, E, 0);
}

int check_layernorm(int rows, int E, float eps) {
    if (rows <= 0 || E <= 0) return RSA_ERR_SHAPE;
    if (E % 8 != 0 || E > 4096 || !finite_float(eps) || !(eps >= 0.0f)) return RSA_ERR_UNSUPPORTED;
    return RSA_OK;
}

size_t layer_workspace(int B, int L, int E, int F) {
    const size_t M = (size_t)B * L;
    return (4 * M * E + M * F) * 2;   // Q, K, V, O, then F1 (A1, h1, A2 reuse Q, K, V)
}

}  // namespace

namespace rsa {

// ---- host-side sizing (no device code) ----

size_t forward_partial_bytes(int B, int H, int Lq, int d, int groups) {
    if (groups <= 1) return 0;
    return (size_t)groups * B * H * Lq * (size_t)(d + 2) * sizeof(float);
}

int forward_rank_groups(int B, int H, int L, int d, int N) {
    // Enough workgroups to cover the 256 CUs about twice, while keeping the
    // partials small next to K and V: at most 8 groups, and each group's key
    // range within the occupancy table.
    const int Lc = L / N;
    const long long qtiles = (long long)B * H * ((Lc + kFwdQueryTile - 1) / kFwdQueryTile);
    int g = 1;
    while (g < 8 && g < N && qtiles * g < 512) g *= 2;
    g = g < N ? g : N;
    while (((long long)((N + g - 1) / g) * Lc + kFwdKeyTile - 1) / kFwdKeyTile > kFwdMaxTiles && g < N) ++g;
    (void)d;
    return g;
}

size_t backward_workspace_bytes(int B, int H, int L, int d) {
    (void)d;
    return 2 * (size_t)B * H * L * sizeof(float);
}

size_t twopass_workspace_bytes(int B, int H, int L) { return (size_t)B * H * L * (size_t)L * sizeof(float); }

int check_backward_call(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, const uint8_t* key_mask, int B, int H, int L, int d, int N, int dtype,
                        int flags, const void* dq, const void* dk, const void* dv) {
    if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv) return RSA_ERR_NULL;
    int st = check_backward(B, H, L, d, N, dtype);
    if (st != RSA_OK) return st;
    if (flags & ~RSA_CAUSAL) return RSA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(key_mask, 16) || !aligned(lse, 4))
        return RSA_ERR_ALIGN;
    return RSA_OK;
}

}  // namespace rsa

extern "C" {

int rsa_forward(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                int B, int H, int L, int d, int N, int dtype,
                void* stream, void* out, float* lse) {
    return rsa_forward_ex(q, k, v, key_mask, B, H, L, d, N, dtype, 0, stream, out, lse);
}

int rsa_forward_ex(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                   int B, int H, int L, int d, int N, int dtype, int flags,
                   void* stream, void* out, float* lse) {
    return rsa_forward_dropout(q, k, v, key_mask, B, H, L, d, N, dtype, flags, nullptr, stream, out, lse);
}

int rsa_forward_dropout(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                        int B, int H, int L, int d, int N, int dtype, int flags, const rsa_dropout* dropout,
                        void* stream, void* out, float* lse) {
    if (!q || !k || !v || !out) return RSA_ERR_NULL;
    uint32_t p8 = 0;
    if (!dropout_p8(dropout, &p8)) return RSA_ERR_UNSUPPORTED;
    int st = check_sizes(B, H, L, d, N, dtype);
    if (st != RSA_OK) return st;
    if (flags & ~RSA_CAUSAL) return RSA_ERR_UNSUPPORTED;
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
    c.causal = (flags & RSA_CAUSAL) != 0;
    set_dropout(c, dropout, p8);
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
    return rsa_forward_rank_ex(q_local, k, v, key_mask, B, H, L, d, N, rank, dtype, 0, workspace, workspace_bytes,
                               stream, out_local, lse_local);
}

int rsa_forward_rank_ex(const void* q_local, const void* k, const void* v, const uint8_t* key_mask,
                        int B, int H, int L, int d, int N, int rank, int dtype, int flags,
                        void* workspace, size_t workspace_bytes,
                        void* stream, void* out_local, float* lse_local) {
    return rsa_forward_rank_dropout(q_local, k, v, key_mask, B, H, L, d, N, rank, dtype, flags, nullptr, workspace,
                                    workspace_bytes, stream, out_local, lse_local);
}

int rsa_forward_rank_dropout(const void* q_local, const void* k, const void* v, const uint8_t* key_mask,
                             int B, int H, int L, int d, int N, int rank, int dtype, int flags,
                             const rsa_dropout* dropout, void* workspace, size_t workspace_bytes,
                             void* stream, void* out_local, float* lse_local) {
    if (!q_local || !k || !v || !out_local) return RSA_ERR_NULL;
    uint32_t p8 = 0;
    if (!dropout_p8(dropout, &p8)) return RSA_ERR_UNSUPPORTED;
    int st = check_sizes(B, H, L, d, N, dtype);
    if (st != RSA_OK) return st;
    if (flags & ~RSA_CAUSAL) return RSA_ERR_UNSUPPORTED;
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
    c.causal = (flags & RSA_CAUSAL) != 0;
    set_dropout(c, dropout, p8);
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
    return rsa_backward_ex(q, k, v, out, dout, lse, key_mask, B, H, L, d, N, dtype, 0, workspace, workspace_bytes,
                           stream, dq, dk, dv);
}

int rsa_backward_ex(const void* q, const void* k, const void* v, const void* out, const void* dout,
                    const float* lse, const uint8_t* key_mask,
                    int B, int H, int L, int d, int N, int dtype, int flags,
                    void* workspace, size_t workspace_bytes,
                    void* stream, void* dq, void* dk, void* dv) {
    return rsa_backward_dropout(q, k, v, out, dout, lse, key_mask, B, H, L, d, N, dtype, flags, nullptr, workspace,
                                workspace_bytes, stream, dq, dk, dv);
}

int rsa_backward_dropout(const void* q, const void* k, const void* v, const void* out, const void* dout,
                         const float* lse, const uint8_t* key_mask,
                         int B, int H, int L, int d, int N, int dtype, int flags, const rsa_dropout* dropout,
                         void* workspace, size_t workspace_bytes,
                         void* stream, void* dq, void* dk, void* dv) {
    int st = rsa::check_backward_call(q, k, v, out, dout, lse, key_mask, B, H, L, d, N, dtype, flags, dq, dk, dv);
    if (st != RSA_OK) return st;
    uint32_t p8 = 0;
    if (!dropout_p8(dropout, &p8)) return RSA_ERR_UNSUPPORTED;
    if (!aligned(workspace, 16)) return RSA_ERR_ALIGN;
    if (!workspace || workspace_bytes < rsa::backward_workspace_bytes(B, H, L, d)) return RSA_ERR_WORKSPACE;
    rsa::BackwardCall c = backward_call(q, k, v, out, dout, lse, key_mask, B, H, L, d, N, dtype);
    c.stats = static_cast<float*>(workspace);
    c.dq = dq;
    c.dk = dk;
    c.dv = dv;
    c.causal = (flags & RSA_CAUSAL) != 0;
    set_dropout(c, dropout, p8);
    return launch_status(rsa::launch_backward(c, rsa::kBwdStageAll, static_cast<hipStream_t>(stream)));
}

int rsa_backward_preprocess(const void* out, const void* dout, const float* lse, int B, int H, int L, int d,
                            int dtype, void* stream, float* rowstats) {
    if (!out || !dout || !lse || !rowstats) return RSA_ERR_NULL;
    int st = check_backward(B, H, L, d, 1, dtype);
    if (st != RSA_OK) return st;
    if (!aligned(out, 16) || !aligned(dout, 16) || !aligned(lse, 4) || !aligned(rowstats, 4)) return RSA_ERR_ALIGN;
    rsa::BackwardCall c = backward_call(nullptr, nullptr, nullptr, out, dout, lse, nullptr, B, H, L, d, 1, dtype);
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
    rsa::BackwardCall c = backward_call(q, k, v, nullptr, dout, nullptr, key_mask, B, H, L, d, N, dtype);
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
    rsa::BackwardCall c = backward_call(q, k, v, nullptr, dout, nullptr, key_mask, B, H, L, d, N, dtype);
    c.stats = const_cast<float*>(rowstats);
    c.dk = dk;
    c.dv = dv;
    return launch_status(rsa::launch_backward(c, rsa::kBwdStageDkDv, static_cast<hipStream_t>(stream)));
}

int rsa_linear(const void* a, const void* w, const float* bias, const void* residual, int M, int N, int K,
               int activation, void* stream, void* out) {
    if (!a || !w || !out) return RSA_ERR_NULL;
    int st = check_linear(M, N, K, activation);
    if (st != RSA_OK) return st;
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(out, 16) || !aligned(bias, 16) || !aligned(residual, 16))
        return RSA_ERR_ALIGN;
    rsa::LinearCall c{};
    c.a = a;
    c.w = w;
    c.bias = bias;
    c.residual = residual;
    c.out0 = out;
    c.M = M;
    c.N = N;
    c.K = K;
    c.act = activation;
    c.layout = rsa::kLinearRows;
    return launch_status(rsa::launch_linear(c, static_cast<hipStream_t>(stream)));
}

int rsa_qkv_projection(const void* x, const void* w_qkv, const float* b_qkv, int B, int L, int E, int H,
                       void* stream, void* q, void* k, void* v) {
    if (!x || !w_qkv || !q || !k || !v) return RSA_ERR_NULL;
    int st = check_heads(B, L, E, H);
    if (st != RSA_OK) return st;
    if (!aligned(x, 16) || !aligned(w_qkv, 16) || !aligned(b_qkv, 16) || !aligned(q, 16) || !aligned(k, 16) ||
        !aligned(v, 16))
        return RSA_ERR_ALIGN;
    rsa::LinearCall c{};
    c.a = x;
    c.w = w_qkv;
    c.bias = b_qkv;
    c.out0 = q;
    c.out1 = k;
    c.out2 = v;
    c.M = B * L;
    c.N = 3 * E;
    c.K = E;
    c.layout = rsa::kLinearQkv;
    c.L = L;
    c.H = H;
    c.d = E / H;
    return launch_status(rsa::launch_linear(c, static_cast<hipStream_t>(stream)));
}

int rsa_output_projection(const void* o, const void* w_o, const float* b_o, const void* residual, int B, int L,
                          int E, int H, void* stream, void* out) {
    if (!o || !w_o || !out) return RSA_ERR_NULL;
    int st = check_heads(B, L, E, H);
    if (st != RSA_OK) return st;
    if (!aligned(o, 16) || !aligned(w_o, 16) || !aligned(b_o, 16) || !aligned(residual, 16) || !aligned(out, 16))
        return RSA_ERR_ALIGN;
    rsa::LinearCall c{};
    c.a = o;
    c.w = w_o;
    c.bias = b_o;
    c.residual = residual;
    c.out0 = out;
    c.M = B * L;
    c.N = E;
    c.K = E;
    c.layout = rsa::kLinearHeadsIn;
    c.L = L;
    c.H = H;
    c.d = E / H;
    return launch_status(rsa::launch_linear(c, static_cast<hipStream_t>(stream)));
}

int rsa_layernorm(const void* x, const float* gamma, const float* beta, int rows, int E, float eps, void* stream,
                  void* y) {
    if (!x || !gamma || !beta || !y) return RSA_ERR_NULL;
    int st = check_layernorm(rows, E, eps);
    if (st != RSA_OK) return st;
    if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(beta, 16) || !aligned(y, 16)) return RSA_ERR_ALIGN;
    return launch_status(rsa::launch_layernorm(x, gamma, beta, rows, E, eps, y, static_cast<hipStream_t>(stream)));
}

size_t rsa_layer_forward_workspace_bytes(int B, int L, int E, int H, int F, int N) {
    if (check_heads(B, L, E, H) != RSA_OK || check_linear(B * L, F, E, 1) != RSA_OK ||
        check_linear(B * L, E, F, 0) != RSA_OK || check_sizes(B, H, L, E / H, N, RSA_BF16) != RSA_OK)
        return 0;
    return layer_workspace(B, L, E, F);
}

int rsa_layer_forward(const void* x, const uint8_t* key_mask, const rsa_layer_weights* w, int B, int L, int E,
                      int H, int F, int N, void* workspace, size_t workspace_bytes, void* stream, void* y) {
    if (!x || !w || !y || !w->w_qkv || !w->w_o || !w->w_ff1 || !w->w_ff2 || !w->ln1_gamma || !w->ln1_beta ||
        !w->ln2_gamma || !w->ln2_beta)
        return RSA_ERR_NULL;
    int st = check_heads(B, L, E, H);
    if (st == RSA_OK) st = check_linear(B * L, F, E, 1);
    if (st == RSA_OK) st = check_linear(B * L, E, F, 0);
    if (st == RSA_OK) st = check_sizes(B, H, L, E / H, N, RSA_BF16);
    if (st == RSA_OK) st = check_layernorm(B * L, E, 1e-12f);
    if (st != RSA_OK) return st;
    if (L > kMaxL) return RSA_ERR_UNSUPPORTED;
    const void* ptrs[] = {x, key_mask, y, workspace, w->w_qkv, w->b_qkv, w->w_o, w->b_o, w->ln1_gamma, w->ln1_beta,
                          w->w_ff1, w->b_ff1, w->w_ff2, w->b_ff2, w->ln2_gamma, w->ln2_beta};
    for (const void* p : ptrs)
        if (!aligned(p, 16)) return RSA_ERR_ALIGN;
    if (!workspace || workspace_bytes < layer_workspace(B, L, E, F)) return RSA_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t me = (size_t)B * L * E;
    uint16_t* ws = static_cast<uint16_t*>(workspace);
    uint16_t *q = ws, *k = ws + me, *v = ws + 2 * me, *o = ws + 3 * me, *f1 = ws + 4 * me;
    uint16_t *a1 = q, *h1 = k, *a2 = v;   // Q, K, V are dead once the attention has run
    const int M = B * L, d = E / H;

    rsa::LinearCall c{};
    c.a = x;
    c.w = w->w_qkv;
    c.bias = w->b_qkv;
    c.out0 = q;
    c.out1 = k;
    c.out2 = v;
    c.M = M;
    c.N = 3 * E;
    c.K = E;
    c.layout = rsa::kLinearQkv;
    c.L = L;
    c.H = H;
    c.d = d;
    hipError_t e = rsa::launch_linear(c, s);
    if (e != hipSuccess) return RSA_ERR_HIP;

    rsa::ForwardCall fc{};
    fc.q = q;
    fc.k = k;
    fc.v = v;
    fc.mask = key_mask;
    fc.out = o;
    fc.B = B;
    fc.H = H;
    fc.L = L;
    fc.d = d;
    fc.N = N;
    fc.Lq = L;
    fc.groups = 1;
    fc.bf16 = true;
    if (rsa::launch_forward(fc, s) != hipSuccess) return RSA_ERR_HIP;

    c = rsa::LinearCall{};
    c.a = o;
    c.w = w->w_o;
    c.bias = w->b_o;
    c.residual = x;
    c.out0 = a1;
    c.M = M;
    c.N = E;
    c.K = E;
    c.layout = rsa::kLinearHeadsIn;
    c.L = L;
    c.H = H;
    c.d = d;
    if (rsa::launch_linear(c, s) != hipSuccess) return RSA_ERR_HIP;
    if (rsa::launch_layernorm(a1, w->ln1_gamma, w->ln1_beta, M, E, 1e-12f, h1, s) != hipSuccess) return RSA_ERR_HIP;

    c = rsa::LinearCall{};
    c.a = h1;
    c.w = w->w_ff1;
    c.bias = w->b_ff1;
    c.out0 = f1;
    c.M = M;
    c.N = F;
    c.K = E;
    c.act = 1;
    c.layout = rsa::kLinearRows;
    if (rsa::launch_linear(c, s) != hipSuccess) return RSA_ERR_HIP;

    c = rsa::LinearCall{};
    c.a = f1;
    c.w = w->w_ff2;
    c.bias = w->b_ff2;
    c.residual = h1;
    c.out0 = a2;
    c.M = M;
    c.N = E;
    c.K = F;
    c.layout = rsa::kLinearRows;
    if (rsa::launch_linear(c, s) != hipSuccess) return RSA_ERR_HIP;
    return launch_status(rsa::launch_layernorm(a2, w->ln2_gamma, w->ln2_beta, M, E, 1e-12f, y, s));
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
        case RSA_ERR_SCRATCH:
            return "RSA_ERR_SCRATCH: rsa_backward_noalloc holds the row statistics of at most 2097152 query rows "
                   "(B * H * L) in its 16 MiB static scratch";
        default: return "unknown rsa_status";
    }
}

}  // extern "C"
