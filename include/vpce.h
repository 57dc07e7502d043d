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
 *  - Functions are reentrant; the library keeps no state between calls
 *    (except the device address of the static scratch of
 *    vpce_forward_noalloc, see there). Concurrent calls must use distinct
 *    workspaces.
 *  - Requirements: 0 <= N <= 2000000, 1 <= d <= 1000000, V >= 1,
 *    1 <= R <= V, V < 2^31, d a multiple of 8 (VPCE_BF16) or 4 (VPCE_F32),
 *    H, W, dH and dW 16-byte aligned (a shard's rows of W or dW then are
 *    too), every other pointer 4-byte aligned (labels 8, workspace 256).
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
  VPCE_ERR_WORKSPACE = 5,   /* workspace too small for the call (see the
                               workspace notes of each call), or a budget
                               that cannot hold the operation */
  VPCE_ERR_HIP = 6,         /* a kernel launch failed (or, for
                               vpce_forward_noalloc, the device address of its
                               scratch could not be obtained) */
  VPCE_ERR_SCRATCH = 7      /* vpce_forward_noalloc: the shape needs more
                               than VPCE_NOALLOC_SCRATCH_BYTES */
} vpce_status_t;

/*
 * Bytes of device workspace that one buffer serving both vpce_forward and
 * vpce_backward needs for this shape at the widest backward chunk (8192
 * vocabulary columns). Pure host function (no GPU call). The result does not
 * depend on V: the forward keeps per-token partial states for R shards times
 * a fixed number of vocabulary splits, the backward a fixed-width chunk of
 * recomputed logit gradients. Returns 0 for arguments vpce_forward would
 * reject. Sizing helper of this library: the memory it sizes stands in for
 * the per-round logit strip of section 3.2 (see vpce_workspace_bytes_chunk),
 * but no passage defines the call itself.
 */
size_t vpce_workspace_bytes(int64_t N, int64_t d, int64_t V, int32_t R,
                            int32_t dtype);

/*
 * As vpce_workspace_bytes, for a backward chunk of chunk_cols vocabulary
 * columns (a multiple of 256 in [256, 8192]; 0 is returned otherwise). The
 * backward chunk is the memory that stands in for the logit strip of section
 * 3.2: the backward's workspace is its gradient chunk G [N x C] (bf16 for
 * bf16 inputs, fp32 for fp32), one N x C strip. Narrower chunks cost more
 * passes of the fp32 dH read-modify-write.
 */
size_t vpce_workspace_bytes_chunk(int64_t N, int64_t d, int64_t V, int32_t R,
                                  int32_t dtype, int64_t chunk_cols);

/*
 * Byte-budget planner (section 3.2: the strip size is chosen so that it fits
 * the device; section 4: a configuration's per-device bytes are fixed by the
 * launch configuration and can be checked before launch). Pure host function.
 *   budget_bytes     device bytes available to one forward + backward: the
 *                    caller's buffers (H, W, labels, lse, loss, dH, dW) plus
 *                    one shared workspace
 *   chunk_cols       out: the widest backward chunk that fits
 *   workspace_bytes  out: vpce_workspace_bytes_chunk(..., *chunk_cols)
 *   peak_bytes       out: exact device bytes live during the backward, the
 *                    step's peak: the caller's buffers plus the workspace
 *                    (each buffer at its exact size; an allocator that rounds
 *                    sizes up adds its own rounding)
 * R is the ring degree fixed by the parallel layout and is not chosen here:
 * with the strip never formed, R changes only the forward's per-token partial
 * states. Returns VPCE_OK, an argument error as vpce_forward would, or
 * VPCE_ERR_WORKSPACE if even a 256-column chunk does not fit (outputs are
 * then left untouched).
 */
int32_t vpce_plan(int64_t N, int64_t d, int64_t V, int32_t R, int32_t dtype,
                  size_t budget_bytes, int64_t* chunk_cols,
                  size_t* workspace_bytes, size_t* peak_bytes);

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
 *   workspace, workspace_bytes    scratch; the forward uses only its part,
 *                                 which any buffer of at least
 *                                 vpce_workspace_bytes_chunk(..., 256) holds
 *   stream                        hipStream_t to enqueue on
 * Returns VPCE_OK or an error status (nothing enqueued on argument errors).
 * Results are bitwise reproducible for a fixed shape on one device model: the
 * number of vocabulary splits per shard follows the device's compute-unit
 * count, and it sets the order in which the fp32 partial states are merged.
 */
int32_t vpce_forward(const void* H, const void* W, const int64_t* labels,
                     int64_t N, int64_t d, int64_t V, int32_t R,
                     int64_t ignore_index, int32_t dtype, float* loss,
                     float* lse, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * ---- Allocation-free forward ----------------------------------------------
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. The same
 * computation and kernels as vpce_forward (bitwise the same loss and lse),
 * with the forward's scratch (per-token partial states of every shard and
 * vocabulary split, target logits, per-block loss sums) taken from a static
 * device array of VPCE_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on, from the first call on that GPU until the process ends. The
 * call allocates and frees nothing (no hipMalloc, no hipFree); the caller
 * still provides H, W, labels, loss and lse.
 *
 * Scratch needed: vpce_forward_noalloc_bytes(N, d, V, R, dtype), about
 * (8 R S + 4) N bytes with S = max(1, ceil(512 / (ceil(N / 256) R))) vocabulary
 * splits per shard (at most 16); larger shapes return VPCE_ERR_SCRATCH
 * before anything is enqueued. Nothing in the scratch needs clearing between
 * calls: every call writes all it reads.
 *
 * All calls on one GPU share that GPU's scratch: calls that may overlap in
 * time on one GPU (different streams, or different host threads without
 * ordering) race and give undefined results. Serialise them, e.g. on one
 * stream. The first call on each GPU looks up the array's device address
 * (hipGetSymbolAddress, with that GPU current) and keeps it; that lookup is
 * the library's only state between calls.
 */
#define VPCE_NOALLOC_SCRATCH_BYTES (64u << 20)

int32_t vpce_forward_noalloc(const void* H, const void* W,
                             const int64_t* labels, int64_t N, int64_t d,
                             int64_t V, int32_t R, int64_t ignore_index,
                             int32_t dtype, float* loss, float* lse,
                             void* stream);

/* Scratch bytes vpce_forward_noalloc needs for this shape (0 for arguments
   vpce_forward would reject). Pure host function. */
size_t vpce_forward_noalloc_bytes(int64_t N, int64_t d, int64_t V, int32_t R,
                                  int32_t dtype);

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
 *   workspace, workspace_bytes    scratch: the backward runs with the widest
 *                                 chunk whose backward part fits (at least
 *                                 the 256-column one, else
 *                                 VPCE_ERR_WORKSPACE)
 * with G_ij = valid_i * (exp(z_ij - lse_i) - [j == y_i]). The token count
 * n_valid is recounted from labels. Rows of dH for ignored tokens are exactly
 * zero. Results are bitwise reproducible for a fixed shape, lse and
 * workspace size (no atomics; the tile shapes chosen from the device's
 * compute-unit count change no summation order); the chunk width changes only
 * the fp32 summation order of dH.
 */
int32_t vpce_backward(const void* H, const void* W, const int64_t* labels,
                      const float* lse, const float* dloss, int64_t N,
                      int64_t d, int64_t V, int32_t R, int64_t ignore_index,
                      int32_t dtype, float* dH, float* dW, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * ---- Timed variants ---------------------------------------------------------
 *
 * vpce_forward_traced and vpce_backward_traced do exactly the work of
 * vpce_forward and vpce_backward (same arguments, same results) and also
 * record timing events around their kernel launches, so that a caller can
 * measure each kernel's duration with hipEventElapsedTime on the stream the
 * kernels run on. Builder utility for measurement; no passage of the paper
 * defines it.
 *   events        2 * max_launches hipEvent_t handles created by the caller
 *                 (with timing enabled); events[2i] is recorded on `stream`
 *                 right before the i-th launch and events[2i + 1] right after
 *   max_launches  how many launches to bracket (0 is allowed: nothing is
 *                 recorded)
 *   kinds         out [max_launches]: vpce_kernel_kind_t of each bracketed
 *                 launch
 *   n_launches    out: the number of kernels the call launched (may exceed
 *                 max_launches; the later ones are not bracketed)
 * Argument errors are returned before anything is enqueued, as for the
 * untimed calls (a NULL event among the first 2 * max_launches is
 * VPCE_ERR_NULL). If an event cannot be recorded, VPCE_ERR_HIP is returned.
 */
typedef enum {
  VPCE_KERNEL_FORWARD_TILE = 1, /* logit tiles + online log-sum-exp */
  VPCE_KERNEL_MERGE = 2,        /* fold of shard/split partials, token NLL */
  VPCE_KERNEL_RECOMPUTE = 3,    /* backward: logit recompute, G chunk */
  VPCE_KERNEL_PRODUCTS = 4,     /* backward: a chunk's dW rows = G^T H and
                                   dH += G W_chunk, one launch */
  VPCE_KERNEL_OTHER = 7         /* fills, loss mean, gradient scale */
} vpce_kernel_kind_t;

int32_t vpce_forward_traced(const void* H, const void* W,
                            const int64_t* labels, int64_t N, int64_t d,
                            int64_t V, int32_t R, int64_t ignore_index,
                            int32_t dtype, float* loss, float* lse,
                            void* workspace, size_t workspace_bytes,
                            void* stream, void* const* events,
                            int32_t max_launches, int32_t* kinds,
                            int32_t* n_launches);

int32_t vpce_backward_traced(const void* H, const void* W,
                             const int64_t* labels, const float* lse,
                             const float* dloss, int64_t N, int64_t d,
                             int64_t V, int32_t R, int64_t ignore_index,
                             int32_t dtype, float* dH, float* dW,
                             void* workspace, size_t workspace_bytes,
                             void* stream, void* const* events,
                             int32_t max_launches, int32_t* kinds,
                             int32_t* n_launches);

/*
 * ---- Shard-level calls: one batch meets one vocabulary shard --------------
 *
 * Ring-DTP moves either the activations or the weight shard around the ring
 * (section 3.2 and Figure 9 of the paper above); the gradient of the moving
 * tensor travels with it. vpce_forward / vpce_backward run the move-weights
 * order for one rank on one device. The calls below are the per-hop steps of
 * either order: a batch (H, labels) carries a running per-token state from
 * shard to shard, then its lse, then its dH, while each shard keeps its dW.
 *
 * The running state of a batch is 3 x N floats, [m | s | t], base 2:
 *   m_i = log2(e) * max over the logits z_ij seen so far (-inf before any),
 *   s_i = sum over those logits of 2^(log2(e) * z_ij - m_i)   (0 before any),
 *   t_i = the target logit z_{i,y_i} once its shard has been folded (NaN
 *         before, and for ignored or out-of-range labels).
 * After every shard has been folded, lse_i = ln 2 * (m_i + log2 s_i). The fold
 * order changes results only through fp32 rounding.
 *
 * The loss over several batches is a mean over all their tokens: each
 * finished batch adds (sum of its token losses, its valid-token count) to a
 * running fp64 pair `totals` (a ring of devices all-reduces that pair), and
 * the backward of every batch scales G by dloss / totals[1].
 *
 * Workspace: any buffer of at least vpce_workspace_bytes(N, d, V, 1, dtype)
 * bytes serves every shard-level call for that batch (the backward fits its
 * chunk to the buffer as vpce_backward does).
 */

/* Which tensor a ring of R ranks sends per hop. */
typedef enum {
  VPCE_RING_MOVE_WEIGHTS = 0,     /* shards travel, batches stay */
  VPCE_RING_MOVE_ACTIVATIONS = 1  /* batches travel, shards stay */
} vpce_ring_mode_t;

/*
 * The cheaper direction for a ring of R ranks with N tokens each (section
 * 3.2: the bytes sent per hop are N*d*b if activations move and (V/R)*d*b if
 * weights move; weights move exactly when the shard is the smaller, i.e. when
 * the widest shard ceil(V/R) has fewer rows than the batch has tokens). Pure
 * host function. Writes the mode and both per-hop payloads in bytes.
 */
int32_t vpce_ring_mode(int64_t N, int64_t d, int64_t V, int32_t R,
                       int32_t dtype, int32_t* mode, size_t* activation_bytes,
                       size_t* weight_bytes);

/* state [3 x N] = [-inf | 0 | NaN]: the empty running state of a batch. */
int32_t vpce_state_init(float* state, int64_t N, void* stream);

/*
 * Fold one shard into a batch's running state.
 *   H        [N x d]        dtype   the batch's hidden states
 *   W_shard  [v_count x d]  dtype   rows v_begin .. v_begin + v_count - 1 of W
 *   labels   [N]            int64   the batch's targets, vocabulary indices in
 *                                   [0, V) (or ignore_index)
 *   V                               size of the whole vocabulary
 *   state    [3 x N]        float32 in/out, as defined above
 * Requires 0 <= v_begin, 1 <= v_count, v_begin + v_count <= V, and the
 * conventions of vpce_forward for everything else.
 */
int32_t vpce_shard_fold(const void* H, const void* W_shard,
                        const int64_t* labels, int64_t N, int64_t d, int64_t V,
                        int64_t v_begin, int64_t v_count,
                        int64_t ignore_index, int32_t dtype, float* state,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Close a batch whose state has seen every shard: write lse [N] (for every
 * token), add (sum of its valid tokens' losses lse_i - t_i, its valid-token
 * count) to totals [2] (fp64, in/out, the caller zeroes it before the first
 * batch), and, when loss is not NULL, write the mean over everything in
 * totals so far (0 if no valid token). A valid token with an out-of-range
 * label has t = NaN, so the loss is NaN, as in vpce_forward.
 */
int32_t vpce_state_finish(const float* state, const int64_t* labels,
                          int64_t N, int64_t ignore_index, float* lse,
                          double* totals, float* loss, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Backward of one (batch, shard) meeting: recompute the shard's logits from
 * the batch's lse, G = (dloss / totals[1]) * valid * (softmax - onehot), and
 * ACCUMULATE dH += G W_shard and dW_shard += G^T H (both fp32; the caller
 * zeroes them before the first meeting). dloss [1] on the device, NULL = 1.
 * Same arguments and requirements as vpce_shard_fold otherwise.
 */
int32_t vpce_shard_backward(const void* H, const void* W_shard,
                            const int64_t* labels, const float* lse,
                            const double* totals, const float* dloss,
                            int64_t N, int64_t d, int64_t V, int64_t v_begin,
                            int64_t v_count, int64_t ignore_index,
                            int32_t dtype, float* dH, float* dW_shard,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/* Static, NUL-terminated description of a status code. Library utility;
   no passage of the paper defines it. */
const char* vpce_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* VPCE_H */
