/*
 * bpt.h -- C ABI of the MI355X (gfx950) Blockwise Parallel Transformer layer.
 *
 * One pre-norm transformer layer computed the blockwise way described in
 * "Blockwise Parallel Transformer for Long Context Large Models" (§3.2 the
 * two nested loops, §3.4 the online softmax, Algorithm 1 and the memory
 * analysis): for every query block, key/value blocks stream through an online
 * softmax (running max and sum, no s x s score matrix); the attention outputs
 * of all query blocks are written to the saved buffer, the output projection
 * and residual run over the whole sequence (a position-wise product), and
 * Norm2 and the position-wise FFN run over groups of whole query blocks (at
 * most 8192 rows and at most half the sequence; one block if larger), so
 * neither the s x s scores nor an s x ffn_dim FFN intermediate is ever
 * materialised. The backward recomputes what it needs ("recomputation is
 * also done blockwise", same page, memory analysis) and rebuilds attention
 * scores from the saved output and per-row log-sum-exp ("Training memory:
 * model states, activations and checkpointing", §3, what changes the count:
 * FlashAttention keeps O and one fp32 log-sum-exp per row and head). An
 * optional head-chunk loop runs a subset of heads at a time ("Untied Ulysses:
 * Memory-Efficient Context Parallelism via Headwise Chunking", §3.2 and §3.4).
 *
 *   h1 = x + Attn(Norm1(x)) W_o + b_o,   y = h1 + FFN(Norm2(h1))
 *
 * Conventions
 *   - Every pointer argument of the compute entry points is a DEVICE pointer
 *     (gfx950 global memory) owned by the caller; descriptors and weight /
 *     gradient tables themselves are host structs read during the call.
 *   - Row-major, contiguous. y = x W, so a weight is [in, out].
 *   - The library never allocates device memory: the caller passes the saved
 *     buffer and a workspace whose sizes the *_size functions return.
 *   - Work is enqueued asynchronously on the caller's HIP stream; the call
 *     does not synchronise. Inputs are never modified.
 *   - All validation happens before the first launch; on a non-zero status
 *     nothing has been written. A launch failure returns BPT_EHIP (message in
 *     bpt_last_error()).
 *   - Thread-safe: no mutable global state besides a thread-local message and
 *     the opt-in kernel-timing totals (mutex-guarded, see bpt_timing_enable).
 */
#ifndef BPT_H_
#define BPT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BPT_ABI_VERSION 2

typedef enum {
  BPT_OK = 0,
  BPT_EINVAL = 1,       /* bad shape, block size, pointer or alignment        */
  BPT_EWORKSPACE = 2,   /* ws_bytes below bpt_layer_workspace_size()          */
  BPT_EUNSUPPORTED = 3, /* valid but not built (e.g. head_dim outside 32/64/128) */
  BPT_EHIP = 4          /* a HIP launch failed                               */
} bpt_status;

/* Storage type of x, y, dx, weights and the saved buffer. BPT_BF16 stores
 * bfloat16 and accumulates every product, softmax statistic and norm statistic
 * in fp32; BPT_F32 stores and computes in fp32. */
typedef enum { BPT_F32 = 0, BPT_BF16 = 1 } bpt_dtype;

/* LayerNorm: (v - mean) / sqrt(biased var + eps) * g + b.
 * RMSNorm:   v / sqrt(mean(v^2) + eps) * g. */
typedef enum { BPT_LAYERNORM = 0, BPT_RMSNORM = 1 } bpt_norm;

/* FFN(z) = act(z W_1 + b_1) W_2 + b_2 with act = ReLU or exact-erf GeLU, or
 * SwiGLU: (silu(z W_1 + b_1) * (z W_3)) W_2 + b_2 (W_1 = gate, W_3 = up). */
typedef enum { BPT_RELU = 0, BPT_GELU_ERF = 1, BPT_SWIGLU = 2 } bpt_ffn;

typedef struct {
  int32_t abi_version; /* = BPT_ABI_VERSION */
  int32_t dtype;       /* bpt_dtype */
  int32_t norm;        /* bpt_norm */
  int32_t ffn;         /* bpt_ffn */
  int32_t causal;      /* 1: key j visible to query i iff j <= i */
  int32_t use_rope;    /* 1: rotate pairs (2i, 2i+1) of Q and K by p * rope_base^(-2i/d) */
  int64_t batch;       /* independent sequences */
  int64_t seq_len;     /* s; multiple of 16 */
  int64_t hidden;      /* h = n_heads * head_dim; multiple of 64 */
  int64_t n_heads;     /* query heads H */
  int64_t n_kv_heads;  /* KV heads; divides H; query head q uses KV head q / (H / n_kv_heads) */
  int64_t head_dim;    /* d in {32, 64, 128} */
  int64_t ffn_dim;     /* f; multiple of 64 */
  int64_t q_block;     /* c_q: rows per BPT query block; divides s, multiple of 8. Norm2 and the
                          FFN run on groups of whole query blocks (see the file comment). */
  int64_t kv_block;    /* c_kv: key/value block of the online softmax; divides s. Results do not
                          depend on it; the kernel streams K/V through LDS in 64-row tiles. */
  int64_t head_chunk;  /* U: query heads per stage; divides H and is a multiple of H / n_kv_heads */
  double rope_base;    /* e.g. 500000.0 */
  float norm_eps;      /* e.g. 1e-5 */
  int32_t window;      /* causal sliding window W >= 1 (key j visible to query i iff
                          i - W < j <= i; requires causal = 1), or 0 for none. A positional
                          bias of -inf outside the window ("Blockwise Parallel Transformer...",
                          §3.4: the bias generated from query and key block positions); key
                          blocks wholly outside every row's window are skipped. */
  float dropout_p;     /* dropout on the attention probabilities, in [0, 1): element (query i,
                          key j) of global query head h in sequence b is dropped iff byte
                          j % 4 of word i % 4 of Philox4x32-10(counter (i/4, j/4, h, b), key
                          (seed low, seed high)) is below t = round(256 dropout_p); kept ones
                          are scaled by 256 / (256 - t). The masks are regenerated in the
                          backward, never stored ("Training memory...", §3: FlashAttention
                          regenerates the dropout mask from the random-number state). 0 (or
                          t = 0): no dropout. */
  int32_t reserved;
  uint64_t seed;       /* dropout seed */
} bpt_layer_desc;

/* Layer weights, storage dtype. w_qkv is [h, (H + 2 n_kv_heads) d] packed Q | K | V, head k in
 * columns [k d, (k+1) d) of its part; w_o [H d, h]; w_1 [h, f]; w_2 [f, h]; w_3 [h, f] (SwiGLU
 * only). Biases and norm shifts may be NULL (treated as zero); n1_b / n2_b must be NULL for
 * RMSNorm. n1_g and n2_g are required. */
typedef struct {
  const void *w_qkv, *b_qkv, *w_o, *b_o, *w_1, *b_1, *w_2, *b_2, *w_3;
  const void *n1_g, *n1_b, *n2_g, *n2_b;
} bpt_layer_weights;

/* Parameter gradients, fp32, same shapes as the weights. A NULL entry is not
 * computed. accumulate = 0 overwrites, 1 adds to the existing contents. */
typedef struct {
  float *dw_qkv, *db_qkv, *dw_o, *db_o, *dw_1, *db_1, *dw_2, *db_2, *dw_3;
  float *dn1_g, *dn1_b, *dn2_g, *dn2_b;
  int32_t accumulate;
  int32_t reserved;
} bpt_layer_grads;

/* Host-only check of a descriptor (no device work): the shape rules above, the block sizes
 * dividing s ("Blockwise Parallel Transformer...", §3.4, the sequence split into blocks),
 * head_chunk holding whole GQA groups ("Untied Ulysses...", §3.4, each stage projects the KV
 * heads its query heads use) and the built combinations (head_dim 32/64/128; fp32 only up to
 * head_dim 64; hidden up to 16384). Returns BPT_OK, BPT_EINVAL or BPT_EUNSUPPORTED and
 * leaves a message in bpt_last_error(). */
bpt_status bpt_layer_validate(const bpt_layer_desc* desc);

/* Bytes of the forward->backward state: the attention output O [b, s, H d] in the storage
 * dtype plus one fp32 base-2 log-sum-exp per (batch, head, row) ("Training memory...", §3:
 * the FlashAttention saved set, O plus one fp32 statistic per row and head; "Blockwise
 * Parallel Transformer...", §3.4 memory analysis: about 2bsh per layer). Linear in s.
 * Returns 0 for an invalid descriptor. */
size_t bpt_layer_saved_size(const bpt_layer_desc* desc);

/* Workspace bytes for the forward (backward = 0) or the backward (backward = 1). Affine in s
 * with no s * ffn_dim term ("Blockwise Parallel Transformer...", §3.2: the FFN intermediate
 * exists for one query block at a time; here for one group of whole query blocks of at most
 * min(8192, s / 2) rows, or one block if larger). Returns 0 for an invalid descriptor. */
size_t bpt_layer_workspace_size(const bpt_layer_desc* desc, int32_t backward);

/* Forward of the layer ("Blockwise Parallel Transformer...", §3.2 and Algorithm 1: blockwise
 * attention with the online softmax of §3.4, then the FFN per query block, with residuals;
 * pre-norm placement as in "Training memory...", §5 code). x, y: [b, s, h] in the storage
 * dtype, device memory, 16-byte aligned. saved: bpt_layer_saved_size bytes (16-byte aligned),
 * written here and read by the backward. ws: workspace of at least
 * bpt_layer_workspace_size(desc, 0) bytes, 256-byte aligned; contents undefined on return.
 * stream: a hipStream_t (NULL = the default stream). Inputs are not modified. Returns
 * BPT_EINVAL / BPT_EWORKSPACE / BPT_EUNSUPPORTED before any launch, BPT_EHIP if a launch
 * fails (then y and saved are undefined). */
bpt_status bpt_layer_forward(const bpt_layer_desc* desc, const void* x,
                             const bpt_layer_weights* w, void* y, void* saved, void* ws,
                             size_t ws_bytes, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same computation, arguments (minus the
 * workspace) and results as bpt_layer_forward. Its workspace is a static
 * device array of bpt_layer_noalloc_scratch_bytes() bytes (64 MiB) inside the
 * library, one per GPU, held until the process ends; it calls no hipMalloc,
 * hipFree or other allocating routine. A layer whose forward workspace
 * (bpt_layer_workspace_size(desc, 0)) exceeds it returns BPT_EWORKSPACE
 * before any launch. Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (other streams, other host threads) race and must
 * be serialised by the caller. The array keeps the last call's contents; the
 * forward writes every scratch element before reading it. */
bpt_status bpt_layer_forward_noalloc(const bpt_layer_desc* desc, const void* x,
                                     const bpt_layer_weights* w, void* y, void* saved,
                                     void* stream);

/* Size in bytes of the static scratch of bpt_layer_forward_noalloc. */
size_t bpt_layer_noalloc_scratch_bytes(void);

/* Recompute-based backward ("Blockwise Parallel Transformer...", §3.4 memory analysis: the
 * backward recomputes blockwise; "Training memory...", §2 per-operation gradient rules and §3
 * FlashAttention backward from O and the log-sum-exp). x: the forward's input; saved: the
 * forward's saved buffer (unchanged); dy: cotangent of y [b, s, h]; dx: [b, s, h] (storage
 * dtype) written; grads: fp32 parameter gradients (summed over the batch), 4-byte aligned,
 * overwritten or accumulated per grads->accumulate. ws: at least
 * bpt_layer_workspace_size(desc, 1) bytes, 256-byte aligned. Same error behaviour as the
 * forward; on BPT_EHIP dx and the gradients are undefined. */
bpt_status bpt_layer_backward(const bpt_layer_desc* desc, const void* x,
                              const bpt_layer_weights* w, const void* saved, const void* dy,
                              void* dx, const bpt_layer_grads* grads, void* ws, size_t ws_bytes,
                              void* stream);

/* Static description of a status code (never NULL). */
const char* bpt_status_string(bpt_status status);

/* ---- Stack of layers with activation checkpointing ----
 * "Training memory...", §3 (full checkpointing; checkpoint every k layers, peak
 * M(k) = (L/k) c + k A): n_layers layers of one shape, each with its own weights, applied in
 * sequence. With checkpoint_every = k >= 1 the forward keeps only the input of every k-th
 * layer (c = one activation [b, s, h]); the backward rebuilds one segment of k layers at a time
 * from its checkpoint (one extra forward per layer), keeping that segment's layer inputs and
 * saved states (A per layer), then runs its layers' backward in reverse. k = 0 keeps every
 * layer's input and saved state from the forward (no recompute). Results do not depend on k. */
typedef struct {
  bpt_layer_desc layer;     /* shape and options of every layer */
  int64_t n_layers;         /* L >= 1 */
  int64_t checkpoint_every; /* k in 0..L (see above) */
} bpt_stack_desc;

bpt_status bpt_stack_validate(const bpt_stack_desc* desc);

/* Bytes kept from the forward for the backward: k >= 1: (ceil(L / k) - 1) activations (the
 * first segment's checkpoint is x itself); k = 0: L - 1 activations and L layer saved buffers
 * (each rounded up to 256 bytes). */
size_t bpt_stack_saved_size(const bpt_stack_desc* desc);

/* Forward: two activations plus (k >= 1) one layer saved buffer plus the layer's forward
 * workspace. Backward: (k >= 1) k - 1 activations, k layer saved buffers and one activation of
 * the rebuilt segment, two gradient activations, and the layer's workspace. */
size_t bpt_stack_workspace_size(const bpt_stack_desc* desc, int32_t backward);

/* x, y: [b, s, h]; w: array of n_layers weight tables (layer 0 first); saved and ws 256-byte
 * aligned. Otherwise as bpt_layer_forward. */
bpt_status bpt_stack_forward(const bpt_stack_desc* desc, const void* x,
                             const bpt_layer_weights* w, void* y, void* saved, void* ws,
                             size_t ws_bytes, void* stream);

/* grads: array of n_layers gradient tables (each with its own accumulate flag). x, w and
 * saved as given to / written by the forward; dy: cotangent of y; dx written. */
bpt_status bpt_stack_backward(const bpt_stack_desc* desc, const void* x,
                              const bpt_layer_weights* w, const void* saved, const void* dy,
                              void* dx, const bpt_layer_grads* grads, void* ws, size_t ws_bytes,
                              void* stream);

/* ---- Blockwise LM head with cross-entropy loss ----
 * "Blockwise Parallel Transformer for Long Context Large Models", §3.4 (handling of the
 * cross-entropy loss: blockwise evaluation never holds all positions' logits) and "Training
 * memory...", §3 (the logits, 4sbV bytes in fp32): for each row i of z [rows, hidden],
 *   logits_i = z_i W_head,  loss_i = logsumexp(logits_i) - logits_i[t_i],
 * with the log-sum-exp in fp32; a target outside [0, vocab) marks an ignored row (loss 0, no
 * gradient). Rows run in chunks of chunk_rows: the forward reduces each chunk's logits inside
 * the GEMM's epilogue to per-row log-sum-exp partials (nothing of size rows x vocab is
 * written); the backward recomputes a chunk's logits and holds only that chunk's
 * dlogits = g_i (softmax_i - onehot(t_i)) [chunk_rows, vocab] before dz = dlogits W_head^T
 * and dW_head += z^T dlogits. */
typedef struct {
  int32_t abi_version; /* = BPT_ABI_VERSION */
  int32_t dtype;       /* bpt_dtype of z, w_head and dz (losses, dloss, dw_head: fp32) */
  int64_t rows;        /* positions (batch x sequence) */
  int64_t hidden;      /* h, multiple of 64 */
  int64_t vocab;       /* V, multiple of 64 (pad the vocabulary) */
  int64_t chunk_rows;  /* rows per chunk, multiple of 64; chunk_rows x vocab < 2^31 */
} bpt_lm_head_desc;

/* Host-only check of an LM-head descriptor (the rules above). */
bpt_status bpt_lm_head_validate(const bpt_lm_head_desc* desc);

/* Bytes of the forward->backward state: one fp32 (base-2) log-sum-exp per row. */
size_t bpt_lm_head_saved_size(const bpt_lm_head_desc* desc);

/* Workspace bytes: forward (backward = 0) chunk_rows x (vocab / 32) (max, sum) pairs plus
 * chunk_rows floats; backward (1) chunk_rows x vocab dlogits in the storage dtype; the fused
 * call (2) both, plus chunk_rows x vocab fp32 logits and chunk_rows floats. Independent of
 * rows. Returns 0 for an invalid descriptor or another value of `backward`. */
size_t bpt_lm_head_workspace_size(const bpt_lm_head_desc* desc, int32_t backward);

/* Forward. z: [rows, hidden] (16-byte aligned); w_head: [hidden, vocab] (16-byte aligned);
 * targets: int32 [rows]; loss: fp32 [rows] written (the per-row loss; sum or average it as
 * needed); saved: bpt_lm_head_saved_size bytes written; ws: workspace (256-byte aligned). All
 * device pointers, asynchronous on `stream`. Same error behaviour as bpt_layer_forward. */
bpt_status bpt_lm_head_forward(const bpt_lm_head_desc* desc, const void* z, const void* w_head,
                               const int32_t* targets, float* loss, void* saved, void* ws,
                               size_t ws_bytes, void* stream);

/* Backward from dloss: fp32 [rows], the cotangent of each row's loss (e.g. 1 / number of
 * counted rows for a mean). dz: [rows, hidden] in the storage dtype, overwritten; dw_head:
 * fp32 [hidden, vocab], overwritten (accumulate = 0) or added to (1); either may be NULL (not
 * computed), not both. saved: the forward's saved buffer. */
bpt_status bpt_lm_head_backward(const bpt_lm_head_desc* desc, const void* z, const void* w_head,
                                const int32_t* targets, const void* saved, const float* dloss,
                                void* dz, float* dw_head, int32_t accumulate, void* ws,
                                size_t ws_bytes, void* stream);

/* Forward and backward in one call, for callers that know each row's loss cotangent before
 * the forward (training with a fixed reduction, e.g. dloss = 1 / number of counted rows).
 * Same computation as bpt_lm_head_forward followed by bpt_lm_head_backward with that dloss
 * ("Blockwise Parallel Transformer...", §3.4, handling of the cross-entropy loss): per chunk,
 * the logits GEMM keeps the chunk's fp32 logits in the workspace next to the log-sum-exp
 * partials, and the chunk's dlogits are formed from them, so the logits are computed once
 * instead of twice; still nothing of size rows x vocab exists at once. Outputs: loss as the
 * forward; saved (may be NULL) the forward's saved state; dz, dw_head and accumulate as the
 * backward (either may be NULL, not both). ws: bpt_lm_head_workspace_size(desc, 2) bytes.
 * Results equal the two calls' bit for bit. Same error behaviour as the other calls. */
bpt_status bpt_lm_head_forward_backward(const bpt_lm_head_desc* desc, const void* z,
                                        const void* w_head, const int32_t* targets,
                                        const float* dloss, float* loss, void* saved, void* dz,
                                        float* dw_head, int32_t accumulate, void* ws,
                                        size_t ws_bytes, void* stream);

/* ---- Kernel timing (instrumentation for benchmarks and profiling) ----
 * When a class is enabled, every launch of that kernel class is bracketed by
 * HIP events recorded on the same stream; bpt_timing_read() waits for the
 * recorded events and returns, per class, the summed event-to-event duration
 * in milliseconds and the number of launches since the last reset. The state
 * is process-wide (shared by all threads and devices); calls that overlap
 * while timing is enabled are attributed to whichever class they launch. */
typedef enum {
  BPT_KERNEL_ATTN_FWD = 0,     /* blockwise attention forward                     */
  BPT_KERNEL_ATTN_BWD_DKDV = 1, /* attention backward, dK and dV pass             */
  BPT_KERNEL_ATTN_BWD_DQ = 2,  /* attention backward, dQ pass                     */
  BPT_KERNEL_GEMM = 3,         /* projections and FFN GEMMs with fused epilogues  */
  BPT_KERNEL_ROWWISE = 4,      /* norms, reductions, RoPE table, fills, D = rowsum */
  BPT_KERNEL_LM_HEAD = 5,      /* GEMMs of the LM head (logits, dz, dW_head)      */
  BPT_KERNEL_CLASSES = 6
} bpt_kernel_class;

/* Enable timing for the classes whose bit (1 << class) is set; 0 disables. */
bpt_status bpt_timing_enable(uint32_t class_mask);

/* total_ms[BPT_KERNEL_CLASSES] and launches[BPT_KERNEL_CLASSES] (host arrays,
 * either may be NULL); reset = 1 clears the totals. Returns BPT_EHIP if an
 * event query fails. */
bpt_status bpt_timing_read(double* total_ms, int64_t* launches, int32_t reset);

/* ---- Measurement helper ----
 * Dense bf16 MFMA throughput the current device sustains, in TFLOP/s: runs
 * (synchronously, on `stream`) a kernel of independent 32x32x16 bf16 MFMA
 * chains on every CU, two waves per SIMD, and times it with HIP events. Used
 * to report utilisation against a practical peak next to the datasheet one.
 * Allocates no device memory; BPT_EHIP if the launch or timing fails. */
bpt_status bpt_mfma_peak_probe(double* tflops, void* stream);

/* Message of the last failing call on this host thread ("" if none). */
const char* bpt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BPT_H_ */
