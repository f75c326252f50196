/*
 * dflash.h — C ABI of the MI355X (gfx950) DFlash block-diffusion draft pass.
 *
 * DFlash ("DFlash: Block Diffusion for Flash Speculative Decoding",
 * arXiv 2602.06036) drafts a whole block of tokens in one forward pass of a
 * small block-diffusion drafter.  Hidden features from several layers of the
 * frozen target model are fused and injected as key/value entries into every
 * draft layer's KV cache (paper Fig. 2, "DFlash Inference Design"; atlas
 * summary, "Approach").  The target verifies the block in parallel and the
 * matched prefix is accepted; the reported metric is the acceptance length
 * tau at temperature 0 (atlas summary, "Key results", "Experimental setup").
 *
 * The three calls follow that statement of the problem:
 *   dflash_fuse_ctx     fuse target features of newly verified positions and
 *                       append them as injected K/V to every layer's cache;
 *   dflash_draft_block  one pass over (anchor, mask, ..., mask) for every
 *                       sequence, ending in an LM-head argmax per mask row;
 *   dflash_accept_len   greedy verification: matched-prefix length and the
 *                       next anchor.
 *
 * Conventions
 *   - Every device pointer is owned by the caller (e.g. allocated through
 *     PyTorch).  The library never allocates, frees or retains device memory;
 *     the host descriptors it creates (dflash_model, dflash_ctx) hold only
 *     pointers into caller memory and host-side metadata.  The one exception
 *     is the fixed-size static scratch of dflash_step_noalloc, a device array
 *     in the library's code object that the runtime places on each GPU the
 *     library runs on.
 *   - Calls are stream-ordered and asynchronous: they enqueue kernels on the
 *     given stream and return.  Only dflash_ctx_create waits for its own
 *     stream (it uploads a host-computed RoPE table).
 *   - Validation happens before any launch: on error nothing is enqueued and
 *     no context length changes.  Errors are negative dflash_status codes; the
 *     detail is in dflash_last_error() (thread-local).  No C++ exception
 *     crosses this interface.  A failed kernel launch returns DFLASH_EHIP.
 *   - A context is used by one stream at a time; different contexts may be
 *     used concurrently with different workspaces.
 *
 * Numerics: weights are bf16; activations, the residual stream, the injected
 * K/V cache, softmax probabilities and logits carry fp32-quality values (each
 * stored as an unevaluated pair of bf16 numbers hi + lo where it feeds a
 * matrix-core product); all products accumulate in fp32.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP stream handle (hipStream_t); NULL means the default stream. */
typedef void* dflash_stream;

typedef enum {
  DFLASH_OK = 0,
  DFLASH_EINVAL = -1,      /* null pointer or invalid argument value          */
  DFLASH_ESHAPE = -2,      /* shapes inconsistent with the model / context    */
  DFLASH_ECAPACITY = -3,   /* appending would exceed a sequence's capacity    */
  DFLASH_EWORKSPACE = -4,  /* workspace smaller than dflash_workspace_bytes() */
  DFLASH_EALIGN = -5,      /* a pointer is not 16-byte (buffers: 256-byte) aligned */
  DFLASH_EHIP = -6,        /* the HIP runtime reported an error               */
  DFLASH_EUNSUPPORTED = -7 /* valid but outside what the kernels implement    */
} dflash_status;

/* Drafter hyper-parameters.  Supported: head_dim 64 or 128; hidden,
 * intermediate, n_q_heads*head_dim and n_target_layers*hidden multiples of
 * 256; n_q_heads a multiple of n_kv_heads with at most 8 query heads per kv
 * head; hidden at most 16384; vocab a multiple of 64; 2 <= max_block <= 32.
 * mask_token_id is an ordinary embedding row. */
typedef struct {
  int32_t n_layers;
  int32_t hidden;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t intermediate;
  int32_t vocab;
  int32_t n_target_layers;
  int32_t mask_token_id;
  int32_t max_block;
  float rms_eps;      /* RMSNorm epsilon, inside the square root */
  double rope_theta;  /* rotate-half RoPE base */
} dflash_config;

typedef struct dflash_model dflash_model;
typedef struct dflash_ctx dflash_ctx;

/* Number of weight pointers dflash_model_create expects: 3 + 9 * n_layers. */
int32_t dflash_weight_count(const dflash_config* cfg);

/* Describe a drafter whose bf16 weights already sit in device memory.
 * weights[] order: w_fc [H][L_t*H], embed [V][H] (also the LM head),
 * final_norm [H]; then for each layer l: attn_norm [H], wq [n_q*d][H],
 * wk [n_kv*d][H], wv [n_kv*d][H], wo [H][n_q*d], mlp_norm [H],
 * wgate [I][H], wup [I][H], wdown [H][I].  Matrices are row-major
 * [out][in] (the nn.Linear layout); every pointer 16-byte aligned.
 * The pointers must stay valid for the model's lifetime. */
int dflash_model_create(const dflash_config* cfg, const void* const* weights, dflash_model** out);
void dflash_model_destroy(dflash_model* model);

/* Bytes of the packed weight copy dflash_model_pack writes (0 if model is
 * NULL): the fusion map, the LM head and every layer's q|k|v, O, gate|up and
 * down matrices, each padded to 256 bytes (3.34 GB for the 5-layer,
 * hidden-4096 drafter). */
size_t dflash_model_pack_bytes(const dflash_model* model);

/* Optional speed-up for few-row calls (decode steps of one or two
 * sequences).  Writes, on `stream`, a copy of the weights listed above into
 * dev_buf (caller-owned device memory, 256-byte aligned, at least
 * dflash_model_pack_bytes bytes) in the order the few-row GEMM streams them:
 * for each GEMM's output rows, in the row order its kernel maps them
 * (q|k|v stacked; gate and up rows interleaved eight and eight), column
 * tile t (16 rows) and k-step s (32 columns) form one contiguous 1 KB block
 * in MFMA lane order, so each wave load reads 1 KB contiguous; the blocks go
 * tile-major (fusion map, O, down) or k-major, all tiles of one k-step side
 * by side (LM head, q|k|v, gate|up).  This is a
 * layout change only: results are bitwise identical with and without it.
 * The model then reads the copy for calls of at most 32 GEMM rows; the
 * original weights stay in use for everything else and must stay valid.
 * dev_buf must stay valid and unmodified while the model uses it, which
 * includes passes already enqueued when the model is switched back or
 * repacked; calls on other streams must first wait for `stream`.  dev_buf = NULL switches the
 * model back to the original weights.  Errors: DFLASH_EINVAL (model NULL),
 * DFLASH_EALIGN, DFLASH_EWORKSPACE (bytes too small), DFLASH_EHIP (launch
 * failure; the model keeps its previous weights).  Not thread-safe against
 * concurrent calls that use the same model. */
int dflash_model_pack(dflash_model* model, void* dev_buf, size_t bytes, dflash_stream stream);

/* Device bytes needed for a context of n_seqs sequences holding up to
 * capacity[b] verified positions each (host array).  Per layer and kv head
 * the cache is a run of 64-slot tiles, each one contiguous block of four
 * planes: K hi and K lo as [slot][d], V hi and V lo transposed as [d][slot]
 * (bf16 pairs carrying fp32 values, 8 bytes per cached element pair).  Each
 * sequence owns whole tiles covering its capacity plus a headroom of
 * max_block slots that dflash_draft_block writes its block K/V into.  An fp32
 * RoPE cos/sin table computed in fp64 on the host precedes the cache.
 * Returns 0 if the arguments are invalid. */
size_t dflash_ctx_bytes(const dflash_config* cfg, int32_t n_seqs, const int64_t* capacity);

/* Lay a context over caller memory dev_buf (256-byte aligned, >= bytes from
 * dflash_ctx_bytes).  Zero-fills the K/V region and uploads the RoPE table on
 * `stream`, then waits for that stream.  All sequences start empty.
 * 1 <= n_seqs <= 128. */
int dflash_ctx_create(const dflash_model* model, void* dev_buf, size_t bytes, int32_t n_seqs,
                      const int64_t* capacity, dflash_stream stream, dflash_ctx** out);
void dflash_ctx_destroy(dflash_ctx* ctx);

/* Current number of verified positions of sequence `seq` (host metadata). */
int64_t dflash_ctx_length(const dflash_ctx* ctx, int32_t seq);

/* Forget positions >= new_len of sequence `seq` (host metadata only; the
 * stale cache entries are overwritten by later appends). */
int dflash_ctx_truncate(dflash_ctx* ctx, int32_t seq, int64_t new_len);

/* Workspace bytes for dflash_draft_block over all sequences of a context
 * with n_seqs sequences at block size `block`, and for dflash_fuse_ctx calls
 * appending up to max_new_tokens positions in total.  With n_seqs = n the
 * same size serves dflash_draft_anchored over up to n blocks. */
size_t dflash_workspace_bytes(const dflash_model* model, int32_t n_seqs, int32_t block,
                              int64_t max_new_tokens);

/* Append n_new[b] newly verified positions to each sequence (DFlash paper
 * Fig. 2: fused target features are injected into every draft layer's KV
 * cache).  features: device bf16 [sum_b n_new[b]][n_target_layers*hidden],
 * sequences packed in order, each row the selected target layers
 * concatenated.  For every row: h = W_fc f (fp32 accumulate), then for each
 * layer K = RoPE(W_k h, p) and V = W_v h are written at position
 * p = length(b) + t.  n_new is a host array [n_seqs]; entries may be 0.
 * Lengths advance on the host when the call is enqueued.
 * Errors: DFLASH_ECAPACITY if length(b) + n_new[b] > capacity[b]. */
int dflash_fuse_ctx(const dflash_model* model, dflash_ctx* ctx, const void* features,
                    const int32_t* n_new, void* ws, size_t ws_bytes, dflash_stream stream);

/* One block-diffusion draft pass for every sequence of the context (forum
 * post, section 1: a candidate block in a single forward pass; atlas summary,
 * "Approach").  Sequence b's block is the token anchors[b] followed by
 * block-1 mask tokens at positions length(b) .. length(b)+block-1; each layer
 * attends over [injected context K/V | block K/V] with no mask.  Row i >= 1
 * predicts the token at its own position: draft[b][i-1] is the lowest index
 * of the largest logit.
 *   anchors: device int32 [n_seqs];   draft: device int32 [n_seqs][block-1]
 *   logits:  NULL, or device fp32 [n_seqs][block-1][vocab] (written if given)
 * The block's K/V are written into the context's headroom slots (positions
 * >= length), which does not change any length.  2 <= block <= max_block.
 * Token ids are not range-checked on the host (they live in device memory):
 * an anchor (or, in the calls that take them, a block token) outside
 * [0, vocab) is clamped to 0 or vocab - 1 before its embedding row is read,
 * so it can never read outside the embedding; pass valid ids. */
int dflash_draft_block(const dflash_model* model, const dflash_ctx* ctx, const int32_t* anchors,
                       int32_t block, int32_t* draft, float* logits, void* ws, size_t ws_bytes,
                       dflash_stream stream);

/* Sampling parameters of sampled drafts and of their verification.  The
 * random numbers are a pure function of (seed, purpose, block index b,
 * position i, vocabulary index v): word i mod 4 of Philox4x64-10 (Salmon et
 * al., SC'11) at counter (v, i div 4, b, 0) and key (seed, purpose), its top
 * 53 bits mapped to (0, 1).  Use a fresh seed for every drafted block. */
typedef struct {
  double temperature; /* > 0 (at most 1e6); temperature 0 is dflash_draft_block */
  uint64_t seed;
} dflash_sampling;

/* dflash_draft_block with sampled drafts: position i of block b takes the
 * token with the largest logit / T + G, G = -log(-log(U)) its Gumbel number
 * (purpose 1), i.e. a sample from softmax(logits / T).  The pages evaluate
 * greedy drafts only (atlas summary, "Key results": temperature 0); this is
 * the sampled counterpart that lossless verification needs.  logits (NULL or
 * as for dflash_draft_block) receives the raw logits, the q that
 * dflash_verify_sample takes.  Other arguments and errors as for
 * dflash_draft_block, plus DFLASH_EINVAL for a NULL or out-of-range
 * `sampling`. */
int dflash_draft_sample(const dflash_model* model, const dflash_ctx* ctx, const int32_t* anchors, int32_t block,
                        const dflash_sampling* sampling, int32_t* draft, float* logits, void* ws, size_t ws_bytes,
                        dflash_stream stream);

/* Lossless verification of sampled blocks (the paper, Introduction:
 * speculative decoding verifies the drafts with the target and is lossless;
 * the rule is standard speculative sampling).  For each sequence b, in
 * position order i = 1..block-1, draft x is kept when
 * U(seed, 2, b, i, 0) * q_i(x) < p_i(x), with q_i = softmax(draft_logits / T)
 * and p_i = softmax(target_logits / T); at the first position where it is
 * not, next_token[b] is the largest log(max(0, p_i - q_i)) + G (purpose 3)
 * and accept[b] = i - 1; when every draft is kept, next_token[b] is the
 * largest target_logits[block-1] / T + G at position block (purpose 3) and
 * accept[b] = block - 1.  Arithmetic is fp64.  2 <= block <= 1024 and
 * 1 <= vocab <= 262144.
 *   draft          device int32 [n_seqs][block-1] (clamped into [0, vocab))
 *   draft_logits   device fp32 [n_seqs][block-1][vocab]
 *   target_logits  device fp32 [n_seqs][block][vocab]; row i-1 is the
 *                  target's distribution for position i
 *   accept, next_token  device int32 [n_seqs]
 *   ws             device scratch, 16-byte aligned, of
 *                  dflash_verify_workspace_bytes(n_seqs, block, vocab) bytes
 *                  (0 for bad sizes)
 * Errors: DFLASH_EINVAL (NULL pointer, bad sizes or sampling),
 * DFLASH_EALIGN, DFLASH_EWORKSPACE, DFLASH_EHIP. */
size_t dflash_verify_workspace_bytes(int32_t n_seqs, int32_t block, int32_t vocab);
int dflash_verify_sample(const int32_t* draft, const float* draft_logits, const float* target_logits, int32_t n_seqs,
                         int32_t block, int32_t vocab, const dflash_sampling* sampling, int32_t* accept,
                         int32_t* next_token, void* ws, size_t ws_bytes, dflash_stream stream);

/* Several denoising passes over the block (forum post, section 1: a draft's
 * efficiency is block size over diffusion steps times the acceptance rate;
 * DFlash uses one step).  The pages do not state how a later step re-masks;
 * this takes the plainest reading: pass 1 reads init_tokens (device int32
 * [n_seqs][block-1] for positions 1..block-1, or NULL for mask tokens) and
 * every later pass feeds the previous pass's drafts in their place.  draft
 * and logits (NULL or as for dflash_draft_block) hold the last pass's result;
 * init_tokens may alias draft.  n_steps = 1 with init_tokens = NULL is
 * dflash_draft_block.  1 <= n_steps <= 64; other arguments as for
 * dflash_draft_block. */
int dflash_draft_refine(const dflash_model* model, const dflash_ctx* ctx, const int32_t* anchors,
                        const int32_t* init_tokens, int32_t block, int32_t n_steps, int32_t* draft, float* logits,
                        void* ws, size_t ws_bytes, dflash_stream stream);

/* Draft many blocks anchored at given positions of shared contexts: the
 * forward of the paper's training attention (Fig. 4: the target's context
 * features condition the drafter, and masked blocks start at randomly
 * sampled clean anchor tokens; atlas summary "Approach": random anchor-token
 * block sampling).  Block j sits at positions anchor_pos[j] ..
 * anchor_pos[j] + block - 1 of sequence block_seq[j]; its queries see that
 * sequence's injected context keys at positions < anchor_pos[j] and the
 * block's own keys, bidirectionally, and nothing of any other block; so a
 * block at anchor_pos[j] = length drafts exactly as dflash_draft_block would.
 *   n_blocks      1 .. 128
 *   block_seq     host int32 [n_blocks], each in [0, n_seqs of ctx)
 *   anchor_pos    host int64 [n_blocks], each in [0, length of its sequence]
 *   anchors       device int32 [n_blocks]: the token at each anchor position
 *   block_tokens  device int32 [n_blocks][block-1] for positions 1..block-1,
 *                 or NULL for mask tokens
 *   draft, logits device [n_blocks][block-1] (logits: [..][vocab] or NULL)
 * The context is only read: blocks may overlap one another and the context.
 * The workspace must hold dflash_workspace_bytes(model, n_blocks, block, 0)
 * bytes.  Errors as for dflash_draft_block, plus DFLASH_EINVAL for a block
 * index or anchor position out of range. */
int dflash_draft_anchored(const dflash_model* model, const dflash_ctx* ctx, int32_t n_blocks,
                          const int32_t* block_seq, const int64_t* anchor_pos, const int32_t* anchors,
                          const int32_t* block_tokens, int32_t block, int32_t* draft, float* logits, void* ws,
                          size_t ws_bytes, dflash_stream stream);

/* One steady-state decode iteration in a single call: append n_new[b]
 * verified positions to each sequence (as dflash_fuse_ctx) and then draft a
 * block at the new lengths (as dflash_draft_block).  When the block rows and
 * the appended rows together number at most 32, the appended positions ride
 * as extra rows of every layer's q|k|v projection, which reads the W_k and
 * W_v the separate context projection would read again, and the K/V
 * projection pass of dflash_fuse_ctx disappears (the DFlash paper's Fig. 2
 * cache receives the same values up to float32 summation order).  Otherwise
 * the two calls run one after the other.  Arguments as for the two calls;
 * the workspace must hold dflash_workspace_bytes(model, n_seqs, block,
 * sum n_new).  Lengths advance only if every launch was enqueued. */
int dflash_step(const dflash_model* model, dflash_ctx* ctx, const void* features, const int32_t* n_new,
                const int32_t* anchors, int32_t block, int32_t* draft, float* logits, void* ws, size_t ws_bytes,
                dflash_stream stream);

/* Bytes of the library-held device scratch of dflash_step_noalloc (per GPU). */
#define DFLASH_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)

/* dflash_step for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  It
 * takes no workspace argument: its kernels use a scratch array of
 * DFLASH_NOALLOC_SCRATCH_BYTES (48 MiB) that the library holds in device
 * memory, one copy per GPU it runs on, kept until the process ends.  The call
 * itself allocates nothing (no hipMalloc, no allocating library routine);
 * its first call on a device looks up that device's copy.  The caller still
 * passes every input and output as for dflash_step, and the results are the
 * same.  Enough for decode-sized steps: one or two sequences at block 16, or
 * one at block 32, of the 5-layer hidden-4096 drafter.
 *   - Larger steps (dflash_workspace_bytes(model, n_seqs, block, sum n_new)
 *     above the limit) are rejected with DFLASH_EWORKSPACE before any work is
 *     enqueued.
 *   - `stream` must belong to the current device (DFLASH_EINVAL otherwise).
 *   - Every call on one GPU shares that GPU's scratch and leaves its contents
 *     behind; no kernel reads a scratch byte its own call has not written.
 *     Calls that overlap on one GPU (different streams or host threads) race
 *     on it: serialise them.
 * Other errors as for dflash_step. */
int dflash_step_noalloc(const dflash_model* model, dflash_ctx* ctx, const void* features, const int32_t* n_new,
                        const int32_t* anchors, int32_t block, int32_t* draft, float* logits, dflash_stream stream);

/* dflash_step with sampled drafts (as dflash_draft_sample). */
int dflash_step_sample(const dflash_model* model, dflash_ctx* ctx, const void* features, const int32_t* n_new,
                       const int32_t* anchors, int32_t block, const dflash_sampling* sampling, int32_t* draft,
                       float* logits, void* ws, size_t ws_bytes, dflash_stream stream);

/* Greedy verification (atlas summary, "Key results": temperature 0; metric:
 * acceptance length tau).  draft: device int32 [n_seqs][block-1] for block
 * positions 1..block-1; target: device int32 [n_seqs][block], the target's
 * tokens for positions 1..block (the last is the bonus token).
 * accept[b] = number of leading positions where draft == target (0..block-1),
 * next_anchor[b] = target[b][accept[b]] (skipped when NULL); tau = accept + 1.
 * n_seqs >= 0, 2 <= block <= 4096. */
int dflash_accept_len(const int32_t* draft, const int32_t* target, int32_t n_seqs, int32_t block,
                      int32_t* accept, int32_t* next_anchor, dflash_stream stream);

/* Stages of the draft pass that a measurement probe can bracket. */
typedef enum {
  DFLASH_STAGE_NONE = 0,
  DFLASH_STAGE_LM_HEAD = 1,    /* final-norm output x shared embedding, with the argmax partials */
  DFLASH_STAGE_GATE_UP = 2,    /* gate|up projection with the SwiGLU product (once per layer) */
  DFLASH_STAGE_DOWN = 3,       /* down projection + residual (once per layer) */
  DFLASH_STAGE_QKV = 4,        /* q|k|v projection with RoPE and the block K/V write (once per layer) */
  DFLASH_STAGE_OPROJ = 5,      /* output projection + residual (once per layer) */
  DFLASH_STAGE_ATTENTION = 6,  /* split-key attention and its merge (once per layer) */
  DFLASH_STAGE_FUSION = 7,     /* feature fusion GEMM of dflash_fuse_ctx (once per row chunk) */
  DFLASH_STAGE_KV_PROJ = 8,    /* context K/V projection of dflash_fuse_ctx (per layer and chunk) */
  DFLASH_STAGE_COUNT = 9
} dflash_stage;

/* Measurement probe (instrumentation, not part of the method).  After
 * dflash_probe_arm, every launch of `stage` made by dflash_draft_block or
 * dflash_fuse_ctx with this model is bracketed by a pair of HIP events
 * recorded on the call's stream, for up to max_launches launches (later ones
 * are counted as missed and not timed).  The events are created here (host
 * API objects, no device memory).  dflash_probe_read waits for the recorded
 * events, returns the summed duration in milliseconds and the number of timed
 * launches, then disarms the probe and releases its events.  Arming an armed
 * probe discards the earlier recording.  One probe per model; not for use
 * from several host threads at once.  Errors: DFLASH_EINVAL for a bad stage
 * or count, DFLASH_EHIP if event creation or timing fails. */
int dflash_probe_arm(dflash_model* model, int stage, int32_t max_launches);
int dflash_probe_read(dflash_model* model, double* total_ms, int32_t* launches, int32_t* missed);

const char* dflash_status_str(int status);
const char* dflash_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
