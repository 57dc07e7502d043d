/*
 * vpce.h -- C ABI of libvpce: the vocabulary projection fused with
 * cross-entropy, computed tile by tile over R vocabulary shards with an online
 * log-sum-exp, on one AMD MI355X (gfx950).
 *
 * Operation ("Flattening Every Memory Peak in Long-Context Mixture-of-Experts
 * Training", section 3.2 "Ring-DTP", Figure 3): a rank holds a local batch of
 * N tokens with hidden states H [N x d] and targets y [N], and the vocabulary
 * projection W [V x d] split into R contiguous shards. Every batch meets every
 * shard once; each meeting forms a strip of logits Z = H W_r^T, folds it into a
 * per-token running (max, sum-exp, target-logit) state and releases it. After
 * all shards the exact negative log-likelihood of each token is known. The
 * backward pass replays the shards, recomputes the logits from the saved
 * per-token normaliser, and produces dH and dW. The N x V logit tensor is
 * never stored: the device working set is fixed by tile and chunk sizes and
 * does not depend on V.
 *
 * Conventions shared by every call:
 *  - H, W, labels, loss, lse, dloss, dH, dW and workspace are DEVICE pointers
 *    owned by the caller. H is row-major [N x d], W row-major [V x d]; both are
 *    bfloat16 (VPCE_BF16) or float32 (VPCE_F32). labels are int64 [N].
 *  - Shard r of R covers vocabulary rows [v0_r, v1_r): contiguous intervals,
 *    the first (V mod R) shards one row longer than the others.
 *  - A token whose label equals ignore_index contributes nothing to the loss or
 *    to any gradient. loss is the mean of the per-token losses over the other
 *    tokens; if there are none, loss = 0 and dH = dW = 0.
 *  - A label outside [0, V) that is not ignore_index is a caller error that is
 *    reported in the data, not by the status: that token's loss is NaN, so the
 *    mean is NaN. Kernels never trap.
 *  - The library allocates no device memory and never synchronises the host:
 *    all work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *    Argument errors are detected on the host and returned BEFORE anything is
 *    enqueued. A failed kernel launch returns VPCE_ERR_HIP.
 *  - Functions are reentrant; the library keeps no state between calls.
 *    Concurrent calls must use distinct workspaces.
 *  - Requirements: 0 <= N <= 2000000, 1 <= d <= 2000000, V >= 1,
 *    1 <= R <= V, V < 2^31, d a multiple of 8 (VPCE_BF16) or 4 (VPCE_F32),
 *    H and W 16-byte aligned,
 *    every other pointer 4-byte aligned (labels 8, workspace 256).
 */
#ifndef VPCE_H
#define VPCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VPCE_BF16 = 0, /* bfloat16 H and W, fp32 accumulation */
  VPCE_F32 = 1   /* float32 H and W, fp32 accumulation */
} vpce_dtype_t;

typedef enum {
  VPCE_OK = 0,
  VPCE_ERR_NULL = 1,        /* a required pointer is NULL */
  VPCE_ERR_SHAPE = 2,       /* N or d out of range, V < 1, R < 1, R > V,
                               V >= 2^31, or d not a multiple of 8 (bf16)
                               / 4 (f32) */
  VPCE_ERR_UNSUPPORTED = 3, /* unknown dtype */
  VPCE_ERR_ALIGN = 4,       /* a pointer is not aligned as required */
  VPCE_ERR_WORKSPACE = 5,   /* workspace_bytes < vpce_workspace_bytes(...) */
  VPCE_ERR_HIP = 6          /* a kernel launch failed */
} vpce_status_t;

/*
 * Bytes of device workspace that vpce_forward and vpce_backward need for this
 * shape. Pure host function (no GPU call). The result does not depend on V:
 * the forward keeps per-token partial states for R shards times a fixed number
 * of vocabulary splits, the backward a fixed-width chunk of recomputed
 * logit gradients. Returns 0 for arguments vpce_forward would reject.
 */
size_t vpce_workspace_bytes(int64_t N, int64_t d, int64_t V, int32_t R,
                            int32_t dtype);

/*
 * Forward (section 3.2: per-shard strip, online log-sum-exp fold, target logit
 * from the owning shard, exact NLL after the last shard).
 *   H        [N x d]  dtype       hidden states of the local batch
 *   W        [V x d]  dtype       vocabulary projection (all R shards)
 *   labels   [N]      int64       targets; ignore_index marks skipped tokens
 *   loss     [1]      float32     out: mean NLL over non-ignored tokens
 *   lse      [N]      float32     out: log-sum-exp of every token's logits
 *                                 (ignored tokens included); this is the
 *                                 normaliser the backward pass needs
 *   workspace, workspace_bytes    scratch of at least vpce_workspace_bytes()
 *   stream                        hipStream_t to enqueue on
 * Returns VPCE_OK or an error status (nothing enqueued on argument errors).
 */
int32_t vpce_forward(const void* H, const void* W, const int64_t* labels,
                     int64_t N, int64_t d, int64_t V, int32_t R,
                     int64_t ignore_index, int32_t dtype, float* loss,
                     float* lse, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * Backward (section 3.2: the same rounds replayed, each logit strip recomputed
 * and turned into G = softmax - onehot from the saved normaliser; the local
 * batch's gradient accumulates over the rounds, each shard's gradient lands in
 * that shard's rows).
 *   H, W, labels, N, d, V, R, ignore_index, dtype: as in vpce_forward.
 *   lse      [N]      float32     the normaliser written by vpce_forward
 *   dloss    [1]      float32     upstream gradient of the mean loss, read on
 *                                 the device (NULL means 1.0)
 *   dH       [N x d]  float32     out, overwritten: dloss/n_valid * G W
 *   dW       [V x d]  float32     out, overwritten: dloss/n_valid * G^T H
 * with G_ij = valid_i * (exp(z_ij - lse_i) - [j == y_i]). The token count
 * n_valid is recounted from labels. Rows of dH for ignored tokens are exactly
 * zero. Results are bitwise reproducible for a fixed shape (no atomics).
 */
int32_t vpce_backward(const void* H, const void* W, const int64_t* labels,
                      const float* lse, const float* dloss, int64_t N,
                      int64_t d, int64_t V, int32_t R, int64_t ignore_index,
                      int32_t dtype, float* dH, float* dW, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* vpce_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* VPCE_H */
