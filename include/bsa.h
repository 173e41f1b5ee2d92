/*
 * bsa.h -- C ABI of libbsa.so: 3D Block Sparse Attention (BSA) on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation is the one described in "LongCat-Video Technical Report"
 * (paper-graph-ui deep dive), section "Block Sparse Attention":
 *   1. the latent grid T x H x W is cut into blocks of ct x ch x cw tokens
 *      ("3D block partitioning"; the default chunk shape [4, 4, 8] comes from
 *      the zhaifeiyue notes, section 3, "3D Block Sparse Attention");
 *   2. Q and K are mean-pooled per block ("Pooled block similarity
 *      computation");
 *   3. S_pool = Q_pool K_pool^T / sqrt(d) is scored per (batch, head) and each
 *      query block keeps its top-k key blocks, or, in CDF mode, the smallest
 *      set of most probable key blocks whose softmax mass reaches p, clamped
 *      to [k_min, k_max] ("Block selection via pooled attention scores";
 *      Top-r and CDF-p modes under "Implementation details and design
 *      trade-offs");
 *   4. attention runs only over the kept key blocks ("Sparse attention
 *      computation": non-selected keys are excluded from the softmax).
 * Block-causal attention follows section "Block Attention with KV-Cache for
 * Efficient Multi-Task Inference", "Attention structure": the first
 * cond_frames latent frames are condition tokens that attend only to
 * condition tokens; the other (noisy) tokens attend to all tokens.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors. q, k, v, o are bfloat16 [batch, heads, S, head_dim], contiguous,
 *   S = T*H*W tokens in latent order s = (t*H + h)*W + w. Pointers are device
 *   pointers, 16-byte aligned. head_dim must be 128.
 * Blocks. nT = ceil(T/ct), nH = ceil(H/ch), nW = ceil(W/cw) (section "Block
 *   Sparse Attention", "3D block partitioning"); block id
 *   i = (bt*nH + bh)*nW + bw; a query block holds ct*ch*cw = 64 or 128 slots.
 *   Where a chunk does not divide the grid, the last block along that axis is
 *   partial: it holds only the tokens of its box inside the grid, is pooled
 *   over those tokens, and a query block that selects it attends to those
 *   tokens only. Key blocks are numbered the same way with the key chunk
 *   (ctk, chk, cwk) when one is given (Nk of them), else they are the query
 *   blocks (Nk = Nb).
 * Ownership. The caller owns every buffer. The library never allocates,
 *   frees, or synchronises; all work is enqueued on `stream` (a hipStream_t;
 *   NULL is the default stream). Workspace contents do not carry over from
 *   one call to the next. Outputs must not alias inputs.
 * Errors. Arguments are checked on the host before anything is launched; a
 *   bad call returns a negative status and launches nothing.
 *   bsa_last_error() gives a message for the last failure on this thread.
 *   A launch failure reported by the HIP runtime returns BSA_ERR_LAUNCH.
 * Empty problems. batch == 0 or heads == 0 is valid: nothing is launched and
 *   pointers may be NULL.
 * Concurrency. Calls are asynchronous and stream-ordered. Two calls may not
 *   share a workspace unless they are ordered on one stream.
 * Determinism. Identical inputs give bit-identical idx, cnt and o.
 */
#ifndef BSA_H_
#define BSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bsa_status {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARG = -1, /* a pointer, size or parameter is out of range */
  BSA_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels implement */
  BSA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  BSA_ERR_LAUNCH = -4       /* the HIP runtime rejected a kernel launch */
} bsa_status;

/* Selection modes (Top-r and CDF-p modes of the deep dive's
 * "Implementation details and design trade-offs"). */
enum { BSA_TOPK = 0, BSA_CDF = 1 };

/* Problem shape: latent grid, heads, chunk shape, block-causal split. */
typedef struct bsa_problem {
  int32_t batch;       /* >= 0 */
  int32_t heads;       /* >= 0 */
  int32_t head_dim;    /* must be 128 */
  int32_t T, H, W;     /* latent grid, each > 0; T*H*W < 2^24 */
  int32_t ct, ch, cw;  /* query chunk shape; ct*ch*cw must be 64 or 128 */
  int32_t cond_frames; /* 0: no block-causal mask; else a multiple of ct (and of
                          ctk), < T */
  float scale;         /* softmax scale; <= 0 selects 1/sqrt(head_dim) */
  int32_t ctk, chk, cwk; /* key chunk shape; all 0: the same as the query chunk.
                            Otherwise ctk*chk*cwk must be 64, 128, 256, 512 or
                            1024 ("Implementation details
                            and design trade-offs": query blocks of 64-128 and
                            key blocks of 64-1024 tokens). Key-block ids in idx
                            then refer to these blocks. */
} bsa_problem;

/* Block-selection rule. */
typedef struct bsa_select_params {
  int32_t mode;  /* BSA_TOPK or BSA_CDF */
  int32_t k;     /* top-k: key blocks per query block, >= 1; clamped per row
                    to the number of key blocks that row may see */
  float cdf_p;   /* CDF: 0 < p <= 1 */
  int32_t k_min; /* CDF: lower clamp on the count, >= 1 */
  int32_t k_max; /* CDF: upper clamp on the count, >= k_min */
} bsa_select_params;

/* Row length of the idx array written by bsa_select: k (top-k) or k_max
 * (CDF), the most key blocks one query block can keep under the rule
 * ("Top-r" and "CDF-p" modes, deep dive "Implementation details and design
 * trade-offs"). `problem` may be NULL; when given it is validated too.
 * Returns -1 on an invalid problem or parameters. */
int32_t bsa_index_stride(const bsa_problem* problem, const bsa_select_params* params);

/* Bytes of device workspace one BSA step needs when bsa_select and
 * bsa_attention share a single buffer (the larger of the two sizes below;
 * the calls are ordered on one stream, so the buffer can be reused).
 * Returns 0 on invalid arguments. */
size_t bsa_workspace_bytes(const bsa_problem* problem, const bsa_select_params* params);

/* Bytes of device workspace bsa_select needs: pooled Q (512 bytes per query
 * block) and pooled K (512 bytes per key block), fp32, per (batch, head),
 * each part rounded up to 256 bytes. The pooled scores never leave the chip.
 * Returns 0 on invalid arguments. */
size_t bsa_select_workspace_bytes(const bsa_problem* problem,
                                  const bsa_select_params* params);

/* Bytes of device workspace bsa_attention and dense_attention need. The
 * current kernels need none (0); the workspace arguments are kept so that a
 * kernel that needs scratch can be added without changing the ABI. Returns 0
 * on invalid arguments too. */
size_t bsa_attention_workspace_bytes(const bsa_problem* problem);

/* Block selection: pooling, pooled scores, softmax and top-k / CDF selection
 * with the block-causal restriction (steps 1-3 above).
 *   q, k     bf16 [batch, heads, S, 128], read only.
 *   idx      int32 [batch, heads, Nb, stride] out: kept key-block ids
 *            (0 .. Nk-1) of each query block in ascending order, then -1 up
 *            to stride.
 *   cnt      int32 [batch, heads, Nb] out: number of kept key blocks.
 *   Ties between equal pooled scores keep the lower key-block id. A
 *   condition query block only considers condition key blocks.
 * Limits: Nk <= 32768 key blocks per (batch, head) (BSA_ERR_UNSUPPORTED). */
bsa_status bsa_select(const bsa_problem* problem, const bsa_select_params* params,
                      const void* q, const void* k, int32_t* idx, int32_t* cnt,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Sparse attention over the kept key blocks (step 4 above): for every query
 * block, softmax(Q K_sel^T * scale) V_sel over the tokens of its kept key
 * blocks, written in latent order.
 *   idx, cnt   as written by bsa_select (any ascending or unordered list of
 *              key-block ids is accepted); ids outside [0, Nk) are skipped
 *              and cnt is clamped to [0, idx_stride]. A query block with no
 *              key blocks gets zeros. Key blocks of 64 tokens are taken two
 *              at a time (the last one of an odd count alone).
 *   o          bf16 [batch, heads, S, 128] out.
 * The softmax is computed in fp32 from bf16 products accumulated in fp32;
 * the probabilities are rounded to bf16 before multiplying V. */
bsa_status bsa_attention(const bsa_problem* problem, const void* q, const void* k,
                         const void* v, const int32_t* idx, const int32_t* cnt,
                         int32_t idx_stride, void* o, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Dense softmax attention over every key the query may see (all keys, or
 * condition keys only for condition queries when cond_frames > 0): the
 * baseline that BSA is measured against. The pages' baseline is dense
 * FlashAttention-3 on one H800 (the charles2530 write-up, section "高效推理：
 * C2F 与 BSA", speed table; deep dive, "Block Sparse Attention": BSA keeps
 * under 10 % of the dense attention compute). Here it runs on the same tile
 * engine as bsa_attention, with every allowed key block taken in order, so
 * the speedup measures the sparsity, not a different kernel. The key chunk
 * plays no part. Arguments as for bsa_attention. */
bsa_status dense_attention(const bsa_problem* problem, const void* q, const void* k,
                           const void* v, void* o, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Training forward: bsa_attention that also writes each query's softmax
 * log-normaliser, which bsa_attention_bwd needs to recompute probabilities
 * (the operator has a forward and a backward pass: deep dive, section "Block
 * Sparse Attention", "Implementation details and design trade-offs").
 *   lse   float32 [batch, heads, S] out, latent order, 4-byte aligned:
 *         natural log of sum_j exp(scale q.k_j) over the query's kept keys,
 *         with the sum taken over the same bf16-rounded probabilities the
 *         forward multiplies V with; -inf for a query block with no key block.
 * Everything else (arguments, checks, o) as for bsa_attention; o is
 * bit-identical to bsa_attention's. */
bsa_status bsa_attention_lse(const bsa_problem* problem, const void* q, const void* k,
                             const void* v, const int32_t* idx, const int32_t* cnt,
                             int32_t idx_stride, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Bytes of device workspace bsa_attention_bwd needs: 1 KB of per-query
 * statistics per query block and a bit mask of Nk x Nb bits per (batch,
 * head), each part rounded up to 256 bytes. Returns 0 on invalid arguments. */
size_t bsa_attention_bwd_workspace_bytes(const bsa_problem* problem);

/* Backward of bsa_attention with the key-block selection held fixed (the
 * selection is discrete and carries no gradient; the training use of the
 * selection is in the deep dive's "Block selection via pooled attention
 * scores", the backward pass in "Implementation details and design
 * trade-offs"). Computes the gradients of L = sum(dout * o) with respect to
 * q, k and v, where for query block i with kept keys K_J, values V_J:
 *   P = softmax(scale Q_i K_J^T),  D = rowsum(dout_i * o_i),
 *   dS = P * (dout_i V_J^T - D),
 *   dq_i = scale dS K_J,  dk_J += scale dS^T Q_i,  dv_J += P^T dout_i.
 *   q, k, v       the forward's inputs.
 *   o, lse        as written by bsa_attention_lse for the same q, k, v, idx, cnt.
 *   dout          bf16 [batch, heads, S, 128]: dL/do.
 *   idx, cnt      the forward's key-block lists. The valid ids of a row must
 *                 be distinct (bsa_select's are); ids outside [0, Nk) are
 *                 skipped and cnt is clamped to [0, idx_stride], as in the
 *                 forward.
 *   dq, dk, dv    bf16 [batch, heads, S, 128] out, every element written
 *                 (zero for query blocks with no key block and for keys no
 *                 query block kept). They must not overlap the inputs or
 *                 each other.
 * P is recomputed in fp32 from lse; the products run in bf16 with fp32
 * accumulation (P and dS are rounded to bf16 as MFMA operands). No
 * floating-point atomics: results are bit-identical from run to run.
 * Limits: Nb, Nk <= 4096 blocks per (batch, head) (BSA_ERR_UNSUPPORTED
 * otherwise). Every chunk shape of the forward is supported: query blocks of
 * 64 or 128 tokens, key blocks of 64 to 1024 tokens, partial blocks. */
bsa_status bsa_attention_bwd(const bsa_problem* problem, const void* q, const void* k,
                             const void* v, const void* o, const void* dout, const float* lse,
                             const int32_t* idx, const int32_t* cnt, int32_t idx_stride, void* dq,
                             void* dk, void* dv, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Condition-KV cache for multi-step inference. Condition frames are fixed
 * over all denoising steps, so their keys and values are computed once and
 * cached, and X_cond (condition queries over condition keys) does not change;
 * each later step recomputes only X_noisy = Attention(Q_noisy, [K_cond,
 * K_noisy], [V_cond, V_noisy]) (deep dive, section "Block Attention with
 * KV-Cache for Efficient Multi-Task Inference", "Why this is efficient").
 * The three calls below serve those steps: the caller keeps K_cond/V_cond in
 * the leading (condition) rows of k and v, writes each step's noisy rows
 * after them, and calls bsa_select_noisy + bsa_attention_noisy, which read
 * and write noisy query rows only.
 *
 * Bytes of the pooled condition-key cache: 4*128 per condition key block per
 * (batch, head) (0 when cond_frames is 0 or on invalid arguments). */
size_t bsa_cond_cache_bytes(const bsa_problem* problem);

/* Pools the condition key blocks of k into `cache` (fp32 [batch, heads,
 * condition key blocks, 128]); once per sequence, when K_cond is known. The
 * values equal the condition rows bsa_select pools for itself. */
bsa_status bsa_pool_cond_keys(const bsa_problem* problem, const void* k, float* cache,
                              size_t cache_bytes, void* stream);

/* bsa_select for the noisy query blocks only: idx and cnt rows of condition
 * query blocks are not written. Pooled keys of the condition key blocks come
 * from `cache` (bsa_pool_cond_keys); those of the noisy key blocks and the
 * pooled noisy queries are computed from k and q. Noisy rows are
 * bit-identical to bsa_select's for the same q and k. Workspace as for
 * bsa_select. With cond_frames = 0 it is bsa_select (cache may be NULL). */
bsa_status bsa_select_noisy(const bsa_problem* problem, const bsa_select_params* params,
                            const void* q, const void* k, const float* cache, size_t cache_bytes,
                            int32_t* idx, int32_t* cnt, void* workspace, size_t workspace_bytes,
                            void* stream);

/* bsa_attention for the noisy query blocks only: o rows of condition tokens
 * are not written (they keep the X_cond of an earlier step). Noisy rows are
 * bit-identical to bsa_attention's. */
bsa_status bsa_attention_noisy(const bsa_problem* problem, const void* q, const void* k,
                               const void* v, const int32_t* idx, const int32_t* cnt,
                               int32_t idx_stride, void* o, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Allocation-free selection, for callers that cannot allocate device memory
 * around the call: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation. Same arguments, checks and results as
 * bsa_select (idx and cnt are bit-identical), with the workspace taken from a
 * static device array inside the library instead of the caller's buffer.
 *   Limit. The array holds bsa_select_noalloc_max_workspace_bytes() bytes
 *          (64 MiB); a problem whose bsa_select_workspace_bytes() exceeds it
 *          is rejected with BSA_ERR_WORKSPACE before anything is launched.
 *   Memory. Each GPU the library runs on holds its own copy of the array
 *          until the process ends; its address is looked up once per device,
 *          on that device's first call. The call allocates and frees nothing.
 *   Concurrency. Every call on one GPU shares that GPU's array, which keeps
 *          the last call's contents (no byte of it is read before the same
 *          call writes it): calls that overlap on one GPU, on different
 *          streams or threads, race and must not be issued. */
size_t bsa_select_noalloc_max_workspace_bytes(void);
bsa_status bsa_select_noalloc(const bsa_problem* problem, const bsa_select_params* params,
                              const void* q, const void* k, int32_t* idx, int32_t* cnt,
                              void* stream);

/* Static description of a status code. */
const char* bsa_status_string(int32_t status);

/* Message for the last non-OK status returned on the calling thread ("" if
 * none). The pointer stays valid until the next call on that thread. */
const char* bsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H_ */
