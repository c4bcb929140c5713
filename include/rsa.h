/*
 * rsa.h -- C ABI of librsa.so, Ring Self-Attention (RSA) on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (review page of "Sequence Parallelism: Making 4D Parallelism
 * Possible", ABSTRACT and proposed-method section): the input sequence is
 * split into N chunks, one per device; to produce the attention output each
 * device's query chunk meets every key chunk and every value chunk, which
 * travel around a ring of devices. The pages give no formula; the library
 * computes plain scaled-dot-product attention,
 *
 *     O = softmax(Q K^T / sqrt(d) + M) V,
 *
 * where M is 0 for valid keys and -inf for padded keys, with the key and
 * value chunks of rank n visited in ring order c = (n - t) mod N for ring
 * step t = 0..N-1. On one GPU the ring is a rotation of chunk pointers inside
 * the kernels; the result does not depend on N beyond rounding.
 *
 * Conventions shared by every entry point
 *   Layout   q, k, v, out, dout, dq, dk, dv: [B, H, L, d] contiguous, row
 *            major, d fastest (a one-rank share uses L/N rows for q and out).
 *            key_mask: [B, L] uint8, nonzero = valid key, the same for every
 *            head and query row; NULL = every key valid.
 *            lse: [B, H, rows] fp32, natural-log sum of exp of the scaled
 *            scores of each query row (-inf for a row with no valid key).
 *   dtype    RSA_F32 (fp32 in, fp32 out) or RSA_BF16 (bf16 in, bf16 out;
 *            products accumulate in fp32).
 *   Sizes    B, H, L, d, N > 0; L % N == 0; d is 64 or 128.
 *   Memory   every pointer except `stream` is device memory owned by the
 *            caller; the library allocates nothing, keeps no pointer after
 *            return and holds no state, so calls are thread-safe.
 *   Stream   work is enqueued on `stream` (a hipStream_t; NULL = default
 *            stream); no entry point synchronises. Device faults surface at
 *            the caller's next synchronisation.
 *   Errors   arguments are validated before any HIP call; a non-zero
 *            rsa_status is returned and nothing is enqueued. RSA_ERR_HIP
 *            reports a failed launch (hipGetLastError). Rows with no valid
 *            key produce zeros (never NaN).
 */
#ifndef RSA_H
#define RSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rsa_status {
    RSA_OK = 0,
    RSA_ERR_NULL = 1,        /* a required pointer is NULL */
    RSA_ERR_SHAPE = 2,       /* a size is <= 0, L % N != 0, or rank outside [0, N) */
    RSA_ERR_UNSUPPORTED = 3, /* d not in {64, 128}, unknown dtype, or a size beyond the kernels' range */
    RSA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
    RSA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the query function returns */
    RSA_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
    RSA_ERR_SCRATCH = 7      /* rsa_backward_noalloc: the sizes need more than its static scratch */
} rsa_status;

typedef enum rsa_dtype { RSA_F32 = 0, RSA_BF16 = 1 } rsa_dtype;

/*
 * Flags of the *_ex entry points. RSA_CAUSAL: the query at sequence position
 * i sees the keys at positions j <= i only (on top of key_mask). The pages
 * describe no causal variant; this is the standard autoregressive mask. In
 * ring order rank n then meets its own chunk first, chunks n-1 .. 0 after it,
 * and the chunks after its own not at all (their tiles are skipped).
 */
#define RSA_CAUSAL 1

/*
 * Full RSA forward: all N ranks' shares at once. Rank n owns query rows
 * [n*L/N, (n+1)*L/N) and visits key/value chunks (n - t) mod N for
 * t = 0..N-1 (ABSTRACT: each chunk on its own device, attention output
 * formed by circulating embeddings in a ring).
 *   q, k, v  [B,H,L,d] of dtype (inputs)
 *   key_mask [B,L] uint8 or NULL
 *   out      [B,H,L,d] of dtype (output)
 *   lse      [B,H,L] fp32 (output) or NULL
 */
int rsa_forward(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                int B, int H, int L, int d, int N, int dtype,
                void* stream, void* out, float* lse);

/* rsa_forward with flags (0 or RSA_CAUSAL; other bits: RSA_ERR_UNSUPPORTED). */
int rsa_forward_ex(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                   int B, int H, int L, int d, int N, int dtype, int flags,
                   void* stream, void* out, float* lse);

/*
 * One rank's share, as one device of the ring computes it (ABSTRACT: no
 * device holds the whole sequence's queries): q_local holds rank `rank`'s
 * L/N query rows, k and v hold all L keys, visited in the ring order of that
 * rank. The ring steps are split into groups processed in parallel (with
 * bf16 and L/N a multiple of 64, group g takes every G-th step, so that
 * padded chunks, met one after another, spread over the groups); each
 * group's unnormalised output and softmax statistics go to `workspace` and
 * are merged exactly (log-sum-exp combination) into out_local. Within a
 * group the steps keep ring order; the grouping changes rounding only.
 *   q_local   [B,H,L/N,d] of dtype (input)
 *   k, v      [B,H,L,d] of dtype (inputs)
 *   workspace device buffer of at least rsa_forward_rank_workspace_bytes()
 *   out_local [B,H,L/N,d] of dtype (output); lse_local [B,H,L/N] fp32 or NULL
 */
int rsa_forward_rank(const void* q_local, const void* k, const void* v, const uint8_t* key_mask,
                     int B, int H, int L, int d, int N, int rank, int dtype,
                     void* workspace, size_t workspace_bytes,
                     void* stream, void* out_local, float* lse_local);

/* rsa_forward_rank with flags (query positions rank * L/N + row). */
int rsa_forward_rank_ex(const void* q_local, const void* k, const void* v, const uint8_t* key_mask,
                        int B, int H, int L, int d, int N, int rank, int dtype, int flags,
                        void* workspace, size_t workspace_bytes,
                        void* stream, void* out_local, float* lse_local);

/* Workspace bytes rsa_forward_rank needs for these sizes (0 if they are invalid). */
size_t rsa_forward_rank_workspace_bytes(int B, int H, int L, int d, int N);

/*
 * The same forward in the pages' own two-stage form (ABSTRACT and
 * proposed-method section: the key chunks circulate first and each rank
 * holds its complete rows of scores; the value chunks circulate second and
 * are weighted by the softmax of those rows). The score rows of every rank,
 * [B,H,L,L] fp32, are written to `workspace`, normalised in place to bf16
 * weights, then multiplied by V. Provided to measure what materialising the
 * rows costs next to rsa_forward, which never holds a row of scores; its
 * result agrees with rsa_forward's within rounding, and does not depend on
 * N (N is validated like rsa_forward's).
 *   q, k, v, key_mask, out, lse  as rsa_forward
 *   workspace  device buffer of at least rsa_forward_twopass_workspace_bytes()
 *              (4 * B * H * L * L bytes); its contents on return are
 *              unspecified
 * Only RSA_BF16, L <= 1048576 and B * H <= 65535 are supported
 * (RSA_ERR_UNSUPPORTED otherwise).
 */
int rsa_forward_twopass(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                        int B, int H, int L, int d, int N, int dtype,
                        void* workspace, size_t workspace_bytes,
                        void* stream, void* out, float* lse);

/* Workspace bytes rsa_forward_twopass needs for these sizes (0 if they are invalid). */
size_t rsa_forward_twopass_workspace_bytes(int B, int H, int L, int d, int N);

/*
 * Backward of the loss <O, dO> (proposed-method section: gradients also pass
 * through the ring): dq, dk, dv for all ranks. `out` and `lse` are the
 * forward's outputs for the same inputs. Rank n's query chunk meets every
 * key chunk in ring order, and the dK/dV contributions of every query chunk
 * are summed at the key chunk they belong to.
 *   q, k, v, out, dout [B,H,L,d] of dtype (inputs); lse [B,H,L] fp32 (input)
 *   workspace          at least rsa_backward_workspace_bytes() (holds the
 *                      row statistics of stage 1 below)
 *   dq, dk, dv         [B,H,L,d] of dtype (outputs)
 * RSA_BF16 (bf16 P and dS operands, fp32 accumulation) and RSA_F32 (every
 * product and element in fp32).
 */
int rsa_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, const uint8_t* key_mask,
                 int B, int H, int L, int d, int N, int dtype,
                 void* workspace, size_t workspace_bytes,
                 void* stream, void* dq, void* dk, void* dv);

/* rsa_backward with flags; out and lse must come from the forward with the
 * same flags. */
int rsa_backward_ex(const void* q, const void* k, const void* v, const void* out, const void* dout,
                    const float* lse, const uint8_t* key_mask,
                    int B, int H, int L, int d, int N, int dtype, int flags,
                    void* workspace, size_t workspace_bytes,
                    void* stream, void* dq, void* dk, void* dv);

/* Workspace bytes rsa_backward needs for these sizes (0 if they are invalid). */
size_t rsa_backward_workspace_bytes(int B, int H, int L, int d, int N, int dtype);

/*
 * ---- Dropout of the attention weights ---------------------------------------
 * The pages do not describe dropout; these entry points add the usual
 * attention dropout to the plain ones. P = softmax(Q K^T / sqrt(d) + M) over
 * the full key length is formed as before (lse unchanged); each weight is
 * then kept with probability 1 - p and scaled by 1 / (1 - p), or dropped:
 * O = (P o Z) V. p is quantised to p8 / 256 with p8 = floor(256 p + 1/2),
 * p8 in [0, 255] (p8 = 0: no dropout; larger p: RSA_ERR_UNSUPPORTED). The
 * keep decision of the weight of query position i and key position j in head
 * b*H + h is byte (j mod 4) of word ((j/8) mod 4) of Philox-4x32-10 (Salmon,
 * Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
 * SC'11) at counter ((j/32)*2 + bit 2 of j, i, b*H + h, offset) and key
 * (seed low 32 bits, seed high 32 bits); kept iff that byte >= p8. The
 * decision depends on positions only, so the result does not depend on N,
 * a rank's share sees the same decisions as the full forward, and the
 * backward, given the same settings, regenerates them.
 */
typedef struct rsa_dropout {
    float p;           /* drop probability */
    uint32_t offset;   /* fourth counter word (e.g. a step number) */
    uint64_t seed;     /* Philox key */
} rsa_dropout;

/* rsa_forward_ex with dropout (dropout NULL or p8 = 0: the plain forward). */
int rsa_forward_dropout(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                        int B, int H, int L, int d, int N, int dtype, int flags, const rsa_dropout* dropout,
                        void* stream, void* out, float* lse);

/* rsa_forward_rank_ex with dropout (query positions rank * L/N + row). */
int rsa_forward_rank_dropout(const void* q_local, const void* k, const void* v, const uint8_t* key_mask,
                             int B, int H, int L, int d, int N, int rank, int dtype, int flags,
                             const rsa_dropout* dropout, void* workspace, size_t workspace_bytes,
                             void* stream, void* out_local, float* lse_local);

/* rsa_backward_ex with dropout: out and lse come from rsa_forward_dropout
 * with the same flags and dropout settings; dV = (P o Z)^T dO,
 * dP = Z o (dO V^T), dS = P o (dP - D) with D = rowsum(dO o out). */
int rsa_backward_dropout(const void* q, const void* k, const void* v, const void* out, const void* dout,
                         const float* lse, const uint8_t* key_mask,
                         int B, int H, int L, int d, int N, int dtype, int flags, const rsa_dropout* dropout,
                         void* workspace, size_t workspace_bytes,
                         void* stream, void* dq, void* dk, void* dv);

/*
 * rsa_backward_ex for callers that cannot allocate device memory where they
 * call it: code under HIP graph capture, serving loops that must not
 * allocate, harnesses that forbid hipMalloc. Same arguments, results and
 * validation as rsa_backward_ex without the workspace: the row statistics go
 * to a static array in device memory of RSA_NOALLOC_SCRATCH_BYTES (16 MiB),
 * which each GPU the library runs on holds until the process ends. Limit:
 * rsa_backward_workspace_bytes() <= RSA_NOALLOC_SCRATCH_BYTES, i.e.
 * B * H * L <= 2097152 query rows; larger sizes return RSA_ERR_SCRATCH
 * before any HIP call. The first call on a device resolves the array's
 * address there (hipGetSymbolAddress; no allocation): make one call before
 * capturing a graph. Every call on one GPU shares the array, so calls that
 * overlap on one GPU (several streams or threads) race; the caller
 * serialises them. The array needs no clearing: the backward's first stage
 * writes every value its later stages read.
 */
#define RSA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int rsa_backward_noalloc(const void* q, const void* k, const void* v, const void* out, const void* dout,
                         const float* lse, const uint8_t* key_mask,
                         int B, int H, int L, int d, int N, int dtype, int flags,
                         void* stream, void* dq, void* dk, void* dv);

/*
 * The three stages rsa_backward runs, for callers that schedule them
 * separately (on several devices dQ stays with its rank while the dK/dV
 * contributions travel the ring back to the key chunk's owner; proposed-
 * method section). Same conventions and validation as rsa_backward. (In
 * rsa_backward with RSA_BF16 the dQ kernel forms stage 1's statistics
 * itself, one launch fewer; they are the same bits.)
 *
 * Stage 1: row statistics of the forward, rowstats fp32 [2][B,H,L]:
 *   rowstats[0][b,h,i] = -sum_x dout[b,h,i,x] * out[b,h,i,x]
 *   rowstats[1][b,h,i] = -lse[b,h,i] * log2(e)   (-inf where lse = -inf)
 */
int rsa_backward_preprocess(const void* out, const void* dout, const float* lse, int B, int H, int L, int d,
                            int dtype, void* stream, float* rowstats);

/* Stage 2: dq from q, k, v, dout and stage 1's rowstats (rank n's query
 * chunk meets the key chunks in ring order). */
int rsa_backward_dq(const void* q, const void* k, const void* v, const void* dout, const float* rowstats,
                    const uint8_t* key_mask, int B, int H, int L, int d, int N, int dtype,
                    void* stream, void* dq);

/* Stage 3: dk and dv (key chunk c meets query chunk (c + t) mod N at ring
 * step t; its contributions are summed in that order). */
int rsa_backward_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* rowstats,
                      const uint8_t* key_mask, int B, int H, int L, int d, int N, int dtype,
                      void* stream, void* dk, void* dv);

/*
 * ---- The sequence-parallel layer around RSA -------------------------------
 * Review page, ABSTRACT: RSA sits inside a Transformer whose sequence is split
 * into chunks, one per device; every other step of the layer acts on one
 * token at a time and so runs on a chunk with no exchange. The tensor-
 * parallelism page ("一文捋順千億模型訓練技術", section 二, 1D tensor
 * parallelism, parts (2) and (3)) describes those steps: two fully connected
 * layers with GeLU between them, and attention heads that are independent.
 * Residual sums and post-normalisation follow BERT's encoder layer (the
 * pages' workloads are BERT-shaped; the pages do not print the layer).
 *
 * Conventions of these entry points: matrices and activations are bf16,
 * biases, gamma and beta fp32; products accumulate in fp32 and each result
 * is rounded once to bf16 (nearest even). A weight matrix w [N,K] maps K
 * inputs to N outputs (out = in w^T), the layout of a PyTorch Linear weight.
 * Widths: N % 128 == 0 and K % 64 == 0 for products (RSA_ERR_UNSUPPORTED
 * otherwise); the hidden size E = H*d with d in {64, 128} and E % 128 == 0.
 * Pointers are device memory owned by the caller, 16-byte aligned (NULL
 * allowed where stated); validation, streams and errors as above.
 */

/*
 * out[M,N] = act(a[M,K] w[N,K]^T + bias[N]) + residual[M,N]
 *   activation  0: none, 1: GeLU in its erf form, z Phi(z) (not the tanh approximation;
 *               erfc to 1.2e-7 relative), applied before the residual
 *   bias, residual  may be NULL
 */
int rsa_linear(const void* a, const void* w, const float* bias, const void* residual, int M, int N, int K,
               int activation, void* stream, void* out);

/*
 * Q, K, V [B,H,L,d] from x [B,L,E]: t = x w_qkv^T + b_qkv, w_qkv [3E,E];
 * columns [0,E) of t give Q, [E,2E) K, [2E,3E) V, and head h takes columns
 * h*d .. h*d+d-1 of each (the head split is fused into the product's store).
 * b_qkv [3E] may be NULL.
 */
int rsa_qkv_projection(const void* x, const void* w_qkv, const float* b_qkv, int B, int L, int E, int H,
                       void* stream, void* q, void* k, void* v);

/*
 * out[B,L,E] = merge(o) w_o^T + b_o + residual, where merge reads the
 * attention output o [B,H,L,d] as [B,L,H*d] (fused into the product's
 * operand load). b_o and residual may be NULL.
 */
int rsa_output_projection(const void* o, const void* w_o, const float* b_o, const void* residual, int B, int L,
                          int E, int H, void* stream, void* out);

/*
 * y = (x - mean) / sqrt(var + eps) * gamma + beta over each row of x
 * [rows, E] (var the population variance, statistics in fp32);
 * E % 8 == 0 and E <= 4096.
 */
int rsa_layernorm(const void* x, const float* gamma, const float* beta, int rows, int E, float eps, void* stream,
                  void* y);

/* The layer's weights (device pointers): matrices bf16, vectors fp32. */
typedef struct rsa_layer_weights {
    const void* w_qkv;          /* [3E, E] */
    const float* b_qkv;         /* [3E] or NULL */
    const void* w_o;            /* [E, E] */
    const float* b_o;           /* [E] or NULL */
    const float* ln1_gamma;     /* [E] */
    const float* ln1_beta;      /* [E] */
    const void* w_ff1;          /* [F, E] */
    const float* b_ff1;         /* [F] or NULL */
    const void* w_ff2;          /* [E, F] */
    const float* b_ff2;         /* [E] or NULL */
    const float* ln2_gamma;     /* [E] */
    const float* ln2_beta;      /* [E] */
} rsa_layer_weights;

/*
 * One encoder layer over the whole sequence (every chunk), RSA as its
 * attention:
 *   Q,K,V = split(x w_qkv^T + b_qkv);  O = RSA(Q, K, V, key_mask, N)
 *   A1 = merge(O) w_o^T + b_o + x;     h1 = LayerNorm(A1; ln1)
 *   F1 = GeLU(h1 w_ff1^T + b_ff1);     A2 = F1 w_ff2^T + b_ff2 + h1
 *   y  = LayerNorm(A2; ln2)            (eps = 1e-12)
 *   x, y       [B,L,E] bf16; key_mask as rsa_forward; F % 128 == 0
 *   workspace  at least rsa_layer_forward_workspace_bytes() (intermediates)
 */
int rsa_layer_forward(const void* x, const uint8_t* key_mask, const rsa_layer_weights* w, int B, int L, int E,
                      int H, int F, int N, void* workspace, size_t workspace_bytes, void* stream, void* y);

/* Workspace bytes rsa_layer_forward needs (0 if the sizes are invalid). */
size_t rsa_layer_forward_workspace_bytes(int B, int L, int E, int H, int F, int N);

/* A static, human-readable name for a status code. */
const char* rsa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* RSA_H */
