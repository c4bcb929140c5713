// api_host_check.cpp -- the C ABI's host logic (argument validation,
// workspace sizing and carving, dispatch) built without device code and run
// under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py.
//
// The launch functions that rsa_api.cpp calls are replaced here by stubs that
// record each call and check that every pointer the host logic derives from
// a caller's workspace stays inside it. Pointers are fake device addresses:
// no stub ever dereferences one.

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "rsa.h"
#include "rsa_internal.h"

namespace {

struct Range {
    uintptr_t lo = 0, hi = 0;   // [lo, hi) of the current workspace, or empty
};
Range g_ws;
int g_fwd = 0, g_bwd = 0, g_lin = 0, g_ln = 0, g_2p = 0;
rsa::ForwardCall g_last_fwd;
rsa::BackwardCall g_last_bwd;
int g_last_stages = 0;
int g_failures = 0;

#define CHECK(cond)                                                                  \
    do {                                                                             \
        if (!(cond)) {                                                               \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++g_failures;                                                            \
        }                                                                            \
    } while (0)

// p .. p + bytes lies inside the workspace (when p is a workspace pointer)
void check_in_ws(const void* p, size_t bytes) {
    if (g_ws.hi == 0) return;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (a >= g_ws.lo && a < g_ws.hi) CHECK(a + bytes <= g_ws.hi);
}

}  // namespace

namespace rsa {

hipError_t launch_forward(const ForwardCall& c, hipStream_t) {
    ++g_fwd;
    g_last_fwd = c;
    CHECK(c.q && c.k && c.v && c.out);
    CHECK(c.Lq > 0 && c.groups >= 1 && c.L % c.N == 0);
    if (c.groups > 1) check_in_ws(c.part, forward_partial_bytes(c.B, c.H, c.Lq, c.d, c.groups));
    check_in_ws(c.out, (size_t)c.B * c.H * c.Lq * c.d * (c.bf16 ? 2 : 4));
    return hipSuccess;
}

hipError_t launch_forward_twopass(const ForwardCall& c, hipStream_t) {
    ++g_2p;
    check_in_ws(c.part, twopass_workspace_bytes(c.B, c.H, c.L));
    return hipSuccess;
}

hipError_t launch_backward(const BackwardCall& c, int stages, hipStream_t) {
    ++g_bwd;
    g_last_bwd = c;
    g_last_stages = stages;
    check_in_ws(c.stats, backward_workspace_bytes(c.B, c.H, c.L, c.d));
    return hipSuccess;
}

hipError_t launch_linear(const LinearCall& c, hipStream_t) {
    ++g_lin;
    CHECK(c.N % 128 == 0 && c.K % 64 == 0 && c.M > 0);
    check_in_ws(c.a, (size_t)c.M * c.K * 2);
    check_in_ws(c.residual, (size_t)c.M * c.N * 2);
    if (c.layout == kLinearQkv) {
        for (const void* o : {c.out0, c.out1, c.out2}) check_in_ws(o, (size_t)c.M * (c.N / 3) * 2);
    } else {
        check_in_ws(c.out0, (size_t)c.M * c.N * 2);
    }
    return hipSuccess;
}

hipError_t launch_layernorm(const void* x, const float*, const float*, int rows, int E, float, void* y,
                            hipStream_t) {
    ++g_ln;
    check_in_ws(x, (size_t)rows * E * 2);
    check_in_ws(y, (size_t)rows * E * 2);
    return hipSuccess;
}

}  // namespace rsa

namespace {

const uintptr_t P = 0x10000;   // 16-byte aligned fake device address
void* vp(uintptr_t a) { return reinterpret_cast<void*>(a); }
const void* cp(uintptr_t a) { return reinterpret_cast<const void*>(a); }
float* fp(uintptr_t a) { return reinterpret_cast<float*>(a); }
const uint8_t* mp(uintptr_t a) { return reinterpret_cast<const uint8_t*>(a); }

void forward_checks() {
    const int n0 = g_fwd;
    CHECK(rsa_forward(cp(P), cp(P), cp(P), nullptr, 1, 2, 256, 64, 4, RSA_BF16, nullptr, vp(P), nullptr) == RSA_OK);
    CHECK(g_fwd == n0 + 1 && g_last_fwd.groups == 1 && g_last_fwd.Lq == 256 && !g_last_fwd.causal);
    CHECK(rsa_forward(nullptr, cp(P), cp(P), nullptr, 1, 2, 256, 64, 4, RSA_BF16, nullptr, vp(P), nullptr) ==
          RSA_ERR_NULL);
    CHECK(rsa_forward(cp(P), cp(P), cp(P), nullptr, 1, 2, 255, 64, 4, RSA_BF16, nullptr, vp(P), nullptr) ==
          RSA_ERR_SHAPE);
    CHECK(rsa_forward(cp(P), cp(P), cp(P), nullptr, 1, 2, 256, 96, 4, RSA_BF16, nullptr, vp(P), nullptr) ==
          RSA_ERR_UNSUPPORTED);
    CHECK(rsa_forward(cp(P), cp(P), cp(P), mp(P + 1), 1, 2, 256, 64, 4, RSA_BF16, nullptr, vp(P), nullptr) ==
          RSA_ERR_ALIGN);
    CHECK(rsa_forward_ex(cp(P), cp(P), cp(P), nullptr, 1, 2, 256, 64, 4, RSA_F32, RSA_CAUSAL, nullptr, vp(P),
                         fp(P)) == RSA_OK);
    CHECK(g_last_fwd.causal && !g_last_fwd.bf16);
    CHECK(rsa_forward(cp(P), cp(P), cp(P), nullptr, 1 << 15, 1 << 15, 2, 64, 1, RSA_BF16, nullptr, vp(P), nullptr) ==
          RSA_ERR_UNSUPPORTED);   // more rows than the launch grid covers
    CHECK(g_fwd == n0 + 2);
    // dropout: the probability is quantised to p8 / 256 and carried with the seed and offset
    rsa_dropout dr;
    dr.p = 0.1f;
    dr.offset = 9;
    dr.seed = 0x1122334455667788ull;
    CHECK(rsa_forward_dropout(cp(P), cp(P), cp(P), nullptr, 1, 2, 256, 64, 4, RSA_BF16, 0, &dr, nullptr, vp(P),
                              nullptr) == RSA_OK);
    CHECK(g_last_fwd.drop_p8 == 26 && g_last_fwd.drop_offset == 9 && g_last_fwd.drop_seed == dr.seed);
    dr.p = 0.0f;
    CHECK(rsa_forward_dropout(cp(P), cp(P), cp(P), nullptr, 1, 2, 256, 64, 4, RSA_BF16, 0, &dr, nullptr, vp(P),
                              nullptr) == RSA_OK);
    CHECK(g_last_fwd.drop_p8 == 0 && g_last_fwd.drop_seed == 0);
    CHECK(rsa_forward(cp(P), cp(P), cp(P), nullptr, 1, 2, 256, 64, 4, RSA_BF16, nullptr, vp(P), nullptr) == RSA_OK);
    CHECK(g_last_fwd.drop_p8 == 0);
    dr.p = 0.999f;
    CHECK(rsa_forward_dropout(cp(P), cp(P), cp(P), nullptr, 1, 2, 256, 64, 4, RSA_BF16, 0, &dr, nullptr, vp(P),
                              nullptr) == RSA_ERR_UNSUPPORTED);
    dr.p = 1.0f / 512.0f;
    CHECK(rsa_forward_dropout(cp(P), cp(P), cp(P), nullptr, 1, 2, 256, 64, 4, RSA_F32, 0, &dr, nullptr, vp(P),
                              nullptr) == RSA_OK);
    CHECK(g_last_fwd.drop_p8 == 1);
}

void rank_checks() {
    // every rank of the one-rank-share workload, with a workspace of exactly
    // the size the query function returns
    const int B = 1, H = 16, L = 32768, d = 128, N = 64;
    const size_t ws = rsa_forward_rank_workspace_bytes(B, H, L, d, N);
    CHECK(ws > 0);
    const uintptr_t W = 0x40000000;
    g_ws = {W, W + ws};
    for (int rank = 0; rank < N; ++rank) {
        CHECK(rsa_forward_rank(cp(P), cp(P), cp(P), mp(P), B, H, L, d, N, rank, RSA_BF16, vp(W), ws, nullptr,
                               vp(P), fp(P)) == RSA_OK);
        CHECK(g_last_fwd.q_pos0 == rank * (L / N) && g_last_fwd.Lq == L / N && g_last_fwd.groups >= 1);
    }
    CHECK(rsa_forward_rank(cp(P), cp(P), cp(P), mp(P), B, H, L, d, N, N, RSA_BF16, vp(W), ws, nullptr, vp(P),
                           fp(P)) == RSA_ERR_SHAPE);
    CHECK(rsa_forward_rank(cp(P), cp(P), cp(P), mp(P), B, H, L, d, N, 0, RSA_BF16, vp(W), ws - 1, nullptr, vp(P),
                           fp(P)) == RSA_ERR_WORKSPACE);
    g_ws = {};
    // group counts stay within the tile table for every divisor of a long sequence
    for (int n = 1; n <= 4096; n *= 2) {
        const int g = rsa::forward_rank_groups(1, 1, 1 << 20, 64, n);
        CHECK(g >= 1 && g <= n);
        CHECK((long long)((n + g - 1) / g) * ((1 << 20) / n) <= (long long)rsa::kFwdKeyTile * rsa::kFwdMaxTiles);
    }
}

void backward_checks() {
    const int B = 4, H = 12, L = 4096, d = 64, N = 8;
    const size_t ws = rsa_backward_workspace_bytes(B, H, L, d, N, RSA_BF16);
    CHECK(ws == 2ull * B * H * L * 4);
    const uintptr_t W = 0x50000000;
    g_ws = {W, W + ws};
    CHECK(rsa_backward(cp(P), cp(P), cp(P), cp(P), cp(P), fp(P), nullptr, B, H, L, d, N, RSA_BF16, vp(W), ws,
                       nullptr, vp(P), vp(P), vp(P)) == RSA_OK);
    CHECK(g_last_stages == rsa::kBwdStageAll && g_last_bwd.stats == fp(W) && g_last_bwd.bf16);
    CHECK(rsa_backward(cp(P), cp(P), cp(P), cp(P), cp(P), fp(P), nullptr, B, H, L, d, N, RSA_F32, vp(W), ws,
                       nullptr, vp(P), vp(P), vp(P)) == RSA_OK);
    CHECK(!g_last_bwd.bf16 && g_last_bwd.drop_p8 == 0);
    rsa_dropout dr;
    dr.p = 0.5f;
    dr.offset = 3;
    dr.seed = 42;
    CHECK(rsa_backward_dropout(cp(P), cp(P), cp(P), cp(P), cp(P), fp(P), nullptr, B, H, L, d, N, RSA_BF16,
                               RSA_CAUSAL, &dr, vp(W), ws, nullptr, vp(P), vp(P), vp(P)) == RSA_OK);
    CHECK(g_last_bwd.drop_p8 == 128 && g_last_bwd.drop_offset == 3 && g_last_bwd.drop_seed == 42 &&
          g_last_bwd.causal);
    CHECK(rsa_backward(cp(P), cp(P), cp(P), cp(P), cp(P), fp(P), nullptr, B, H, L, d, N, RSA_BF16, vp(W), ws - 4,
                       nullptr, vp(P), vp(P), vp(P)) == RSA_ERR_WORKSPACE);
    CHECK(rsa_backward_ex(cp(P), cp(P), cp(P), cp(P), cp(P), fp(P), nullptr, B, H, L, d, N, RSA_BF16, 8, vp(W), ws,
                          nullptr, vp(P), vp(P), vp(P)) == RSA_ERR_UNSUPPORTED);
    g_ws = {};
    CHECK(rsa_backward_preprocess(cp(P), cp(P), fp(P), B, H, L, d, RSA_BF16, nullptr, fp(P)) == RSA_OK);
    CHECK(g_last_stages == rsa::kBwdStagePre);
    CHECK(rsa_backward_dq(cp(P), cp(P), cp(P), cp(P), fp(P), nullptr, B, H, L, d, N, RSA_BF16, nullptr, vp(P)) ==
          RSA_OK);
    CHECK(g_last_stages == rsa::kBwdStageDq);
    CHECK(rsa_backward_dkdv(cp(P), cp(P), cp(P), cp(P), fp(P), nullptr, B, H, L, d, N, RSA_BF16, nullptr, vp(P),
                            vp(P)) == RSA_OK);
    CHECK(g_last_stages == rsa::kBwdStageDkDv);
    CHECK(rsa_backward_dq(cp(P), cp(P), cp(P), cp(P), nullptr, nullptr, B, H, L, d, N, RSA_BF16, nullptr, vp(P)) ==
          RSA_ERR_NULL);
}

void twopass_checks() {
    const int B = 2, H = 12, L = 8192, d = 64, N = 16;
    const size_t ws = rsa_forward_twopass_workspace_bytes(B, H, L, d, N);
    CHECK(ws == 4ull * B * H * L * L);
    const uintptr_t W = 0x100000000ull;
    g_ws = {W, W + ws};
    CHECK(rsa_forward_twopass(cp(P), cp(P), cp(P), nullptr, B, H, L, d, N, RSA_BF16, vp(W), ws, nullptr, vp(P),
                              fp(P)) == RSA_OK);
    CHECK(rsa_forward_twopass(cp(P), cp(P), cp(P), nullptr, B, H, L, d, N, RSA_F32, vp(W), ws, nullptr, vp(P),
                              fp(P)) == RSA_ERR_UNSUPPORTED);
    g_ws = {};
}

void layer_checks() {
    const int B = 2, L = 256, E = 768, H = 12, F = 3072, N = 4;
    const size_t ws = rsa_layer_forward_workspace_bytes(B, L, E, H, F, N);
    CHECK(ws == (4ull * B * L * E + (size_t)B * L * F) * 2);
    rsa_layer_weights w;
    std::memset(&w, 0, sizeof(w));
    w.w_qkv = cp(P);
    w.w_o = cp(P);
    w.w_ff1 = cp(P);
    w.w_ff2 = cp(P);
    w.ln1_gamma = w.ln1_beta = w.ln2_gamma = w.ln2_beta = fp(P);
    const uintptr_t W = 0x60000000;
    g_ws = {W, W + ws};
    const int l0 = g_lin, n0 = g_ln, f0 = g_fwd;
    CHECK(rsa_layer_forward(cp(P), nullptr, &w, B, L, E, H, F, N, vp(W), ws, nullptr, vp(P)) == RSA_OK);
    CHECK(g_lin == l0 + 4 && g_ln == n0 + 2 && g_fwd == f0 + 1);
    CHECK(rsa_layer_forward(cp(P), nullptr, &w, B, L, E, H, F, N, vp(W), ws - 2, nullptr, vp(P)) ==
          RSA_ERR_WORKSPACE);
    w.w_o = nullptr;
    CHECK(rsa_layer_forward(cp(P), nullptr, &w, B, L, E, H, F, N, vp(W), ws, nullptr, vp(P)) == RSA_ERR_NULL);
    g_ws = {};
    CHECK(rsa_linear(cp(P), cp(P), nullptr, nullptr, 256, 200, 128, 0, nullptr, vp(P)) == RSA_ERR_UNSUPPORTED);
    CHECK(rsa_linear(cp(P), cp(P), fp(P), cp(P), 256, 256, 128, 1, nullptr, vp(P)) == RSA_OK);
    CHECK(rsa_layernorm(cp(P), fp(P), fp(P), 10, 8192, 1e-12f, nullptr, vp(P)) == RSA_ERR_UNSUPPORTED);
    CHECK(rsa_qkv_projection(cp(P), cp(P), nullptr, 2, 64, 768, 7, nullptr, vp(P), vp(P), vp(P)) == RSA_ERR_SHAPE);
    CHECK(rsa_output_projection(cp(P), cp(P), nullptr, nullptr, 2, 64, 1024, 8, nullptr, vp(P)) == RSA_OK);
}

void status_checks() {
    for (int s = -3; s < 12; ++s) {
        const char* t = rsa_status_string(s);
        CHECK(t != nullptr && std::strlen(t) > 0);
    }
}

}  // namespace

int main() {
    forward_checks();
    rank_checks();
    backward_checks();
    twopass_checks();
    layer_checks();
    status_checks();
    if (g_failures) {
        std::fprintf(stderr, "%d host check(s) failed\n", g_failures);
        return 1;
    }
    std::printf("host checks passed: %d forward, %d backward, %d linear, %d norm, %d two-stage launches\n", g_fwd,
                g_bwd, g_lin, g_ln, g_2p);
    return 0;
}
