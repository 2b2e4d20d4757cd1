/*
 * upipe.h — C ABI of the headwise-chunked attention library for MI355X (gfx950).
 *
 * The operation: one GPU's share of a transformer attention layer under
 * head-split context parallelism — the full sequence of N tokens and a subset
 * of heads (n_q_heads query heads, n_kv_heads key/value heads). The heads are
 * processed one small chunk of `chunk_heads` query heads at a time inside one
 * caller-sized workspace that every chunk reuses: project the chunk's Q (and
 * the K/V of its key/value group), run causal attention over the whole
 * sequence, fold the chunk's share of the output projection into y, then move
 * to the next chunk. This is the scheme the talk "Road to 5 Million Tokens:
 * Breaking Barriers in Long Context Training" calls Untied Ulysses / UPipe
 * (memeeeeeex.com article "500 万トークンへの道 — Max Ryabinin (Together AI) の
 * Untied Ulysses", section "Untied Ulysses (UPipe) — head 単位のチャンク化";
 * liquidgold.cc notes, section "Primary Contribution"). The pages give no
 * formulas; the math is the textbook layer
 *
 *   q_h = rope(norm_q(x Wq_h^T)), k_g = rope(norm_k(x Wk_g^T)), v_g = x Wv_g^T
 *   O_h = softmax(q_h k_g^T / sqrt(head_dim) + causal mask) v_g,  g = h / (Hq/Hkv)
 *   y   = sum_h O_h Wo_h^T
 *
 * with rotate-half RoPE (pairs (i, i + d/2), angle p * theta^(-2i/d) at token
 * index p, formed in fp64), optional per-head RMSNorm of q and k over head_dim
 * before RoPE, and key j visible to query i iff j <= i.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    never allocates or frees device memory and keeps no state between calls
 *    (apart from the opt-in kernel timing declared at the end).
 *  - Layouts are row-major and contiguous, nn.Linear style [out][in]:
 *      x, y, dy, dx  [N][D]               io dtype
 *      wq            [Hq*d][D]            head h = rows h*d .. h*d+d-1
 *      wk, wv        [Hkv*d][D]
 *      wo            [D][Hq*d]            head h = columns h*d .. h*d+d-1
 *      q_norm_w, k_norm_w  [d] io dtype, or both NULL (no q/k norm)
 *      lse           [Hq][N] fp32, natural log of the softmax denominators
 *      dwq, dwk, dwv, dwo  fp32, same shapes as the weights
 *      dq_norm_w, dk_norm_w  [d] fp32 (required iff the norm weights are given)
 *  - io dtype is UPIPE_F32 (float) or UPIPE_BF16 (bfloat16); accumulation is
 *    always fp32.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    and the call returns without synchronising; outputs are valid once the
 *    stream reaches that point. The workspace must not be touched by other
 *    work until then. Calls with distinct workspaces and outputs may run
 *    concurrently.
 *  - Every output is overwritten, never accumulated into.
 *  - Errors: a negative return code. Arguments are validated on the host
 *    before anything is enqueued; on a validation error nothing is launched
 *    and no output is touched. A failed kernel launch returns UPIPE_ERR_HIP
 *    (outputs are then unspecified).
 *
 * Supported shapes: N >= 1; D a positive multiple of 128; head_dim 64 or 128;
 * n_q_heads a multiple of n_kv_heads; chunk_heads divides n_q_heads and
 * either divides or is a multiple of the group size G = n_q_heads/n_kv_heads.
 * Tensors must be 16-byte aligned, the workspace 256-byte aligned.
 */
#ifndef UPIPE_H_
#define UPIPE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { UPIPE_F32 = 0, UPIPE_BF16 = 1 } upipe_dtype_t;

enum {
  UPIPE_OK = 0,
  UPIPE_ERR_INVALID_ARG = -1, /* a null pointer, a non-positive size, bad head counts */
  UPIPE_ERR_UNSUPPORTED = -2, /* head_dim not 64/128, D not a multiple of 128, bad chunking */
  UPIPE_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than upipe_attn_workspace_bytes */
  UPIPE_ERR_ALIGNMENT = -4,   /* a tensor not 16-B aligned or the workspace not 256-B aligned */
  UPIPE_ERR_HIP = -5,         /* a HIP launch failed */
  UPIPE_ERR_SCRATCH = -6      /* upipe_attn_fwd_noalloc: needs more than its built-in scratch */
};

/*
 * Bytes of workspace that upipe_attn_fwd (backward = 0) or upipe_attn_bwd
 * (backward = 1) needs for these sizes. Pure host arithmetic, no HIP call.
 * Returns 0 when the arguments would be rejected by the entry point.
 * The per-chunk part grows with chunk_heads, not with n_q_heads: this is the
 * one small buffer that every chunk reuses, the method's memory saving
 * (memeeeeeex.com article, section "Untied Ulysses (UPipe) — head 単位の
 * チャンク化": the next chunk reuses the previous chunk's buffer;
 * liquidgold.cc notes, "Primary Contribution").
 */
size_t upipe_attn_workspace_bytes(int64_t n_tokens, int64_t d_model, int n_q_heads,
                                  int n_kv_heads, int head_dim, int chunk_heads,
                                  int qk_norm, upipe_dtype_t dtype, int backward);

/*
 * Chunk-size chooser: the largest chunk_heads whose workspace fits in
 * budget_bytes. A larger chunk holds more heads at once, so it needs more
 * memory and runs a little faster (the trade-off reported in the talk's
 * results: memeeeeeex.com article, section "結果と教訓"; liquidgold.cc notes,
 * results part); the largest chunk that fits is therefore the pick.
 * Candidates are exactly the chunk sizes the entry points accept for these
 * sizes (divisors of n_q_heads that divide or are multiples of
 * G = n_q_heads/n_kv_heads). The size compared with the budget is the
 * backward's workspace when backward != 0 (it is the larger of the two),
 * else the forward's. Pure host arithmetic, no HIP call.
 *   ws_bytes: if non-NULL, receives upipe_attn_workspace_bytes of the choice
 * Returns the chosen chunk_heads (>= 1); UPIPE_ERR_WORKSPACE when not even
 * chunk_heads = 1 fits; or the error code the entry points give for these
 * sizes (UPIPE_ERR_INVALID_ARG, UPIPE_ERR_UNSUPPORTED). *ws_bytes is left
 * untouched on error.
 */
int upipe_choose_chunk_heads(int64_t n_tokens, int64_t d_model, int n_q_heads, int n_kv_heads,
                             int head_dim, int qk_norm, upipe_dtype_t dtype, int backward,
                             size_t budget_bytes, size_t* ws_bytes);

/*
 * Forward pass: y = attention layer(x) over the share, and lse for backward.
 * Chunks of chunk_heads query heads run in order; each projects its Q (the
 * first chunk of a kv group also projects that group's K and V), runs causal
 * GQA flash attention, and adds O_c Wo_c^T into y (the first chunk writes y).
 * This is the chunk loop of the memeeeeeex.com article, section "Untied
 * Ulysses (UPipe) — head 単位のチャンク化" (per chunk: recompute the heads,
 * compute attention, store the partial result, move on), and of the
 * liquidgold.cc notes, "Primary Contribution" (heads processed in chunks so
 * that only one chunk's intermediates exist at a time).
 *   x [N][D], wq [Hq*d][D], wk/wv [Hkv*d][D], wo [D][Hq*d]  (io dtype, in)
 *   q_norm_w, k_norm_w [d] or both NULL; norm_eps their epsilon
 *   y [N][D] io dtype (out), lse [Hq][N] fp32 (out)
 *   workspace: >= upipe_attn_workspace_bytes(..., backward = 0) bytes
 */
int upipe_attn_fwd(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int n_q_heads,
                   int n_kv_heads, int head_dim, double rope_theta, int chunk_heads,
                   const void* x, const void* wq, const void* wk, const void* wv,
                   const void* wo, const void* q_norm_w, const void* k_norm_w,
                   float norm_eps, void* y, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * Backward pass for upstream gradient dy, given the lse that upipe_attn_fwd
 * returned for the same inputs. Nothing else is kept from the forward:
 * per chunk the projections and the attention output O are recomputed (O from
 * the saved lse), then the attention backward and the projection gradients
 * run, chunk by chunk, in the same reused workspace. The same chunk loop as
 * the forward (memeeeeeex.com article, section "Untied Ulysses (UPipe) — head
 * 単位のチャンク化", whose chunks are "recomputed"; liquidgold.cc notes,
 * "Primary Contribution"), with the talk's activation checkpointing applied
 * inside the op ("Road to 5 Million Tokens", transcript, checkpointing part).
 *   dy [N][D] io dtype (in), lse [Hq][N] fp32 (in)
 *   dx [N][D] io dtype (out)
 *   dwq, dwk, dwv, dwo fp32 (out), shapes of wq, wk, wv, wo
 *   dq_norm_w, dk_norm_w [d] fp32 (out) iff q_norm_w/k_norm_w are given, else NULL
 *   workspace: >= upipe_attn_workspace_bytes(..., backward = 1) bytes
 */
int upipe_attn_bwd(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int n_q_heads,
                   int n_kv_heads, int head_dim, double rope_theta, int chunk_heads,
                   const void* x, const void* wq, const void* wk, const void* wv,
                   const void* wo, const void* q_norm_w, const void* k_norm_w,
                   float norm_eps, const void* dy, const float* lse, void* dx,
                   float* dwq, float* dwk, float* dwv, float* dwo, float* dq_norm_w,
                   float* dk_norm_w, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * upipe_attn_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results as upipe_attn_fwd, without the
 * workspace: the chunk buffers live in a scratch array of
 * UPIPE_NOALLOC_SCRATCH_BYTES that the library holds in each GPU's memory
 * (a static device array, allocated with the library's code when it loads
 * on that GPU and kept until the process ends). The call allocates nothing.
 * Limit: upipe_attn_workspace_bytes(..., backward = 0) of the arguments must
 * not exceed UPIPE_NOALLOC_SCRATCH_BYTES (bf16, head_dim 128, chunk_heads 1:
 * about 65000 tokens), else UPIPE_ERR_SCRATCH and nothing is launched.
 * Every call on a GPU uses that GPU's one scratch array: calls that overlap
 * in time on one GPU (other streams, other threads) race and must not be
 * issued; calls in stream order are safe. The forward writes every scratch
 * byte it reads in the same call, so nothing needs clearing between calls.
 * The scratch used is the current device's (hipGetDevice), which must be the
 * device of the tensors and the stream. The first call on a device looks up
 * that device's scratch address (UPIPE_ERR_HIP if the lookup fails).
 */
#define UPIPE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int upipe_attn_fwd_noalloc(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int n_q_heads,
                           int n_kv_heads, int head_dim, double rope_theta, int chunk_heads,
                           const void* x, const void* wq, const void* wk, const void* wv,
                           const void* wo, const void* q_norm_w, const void* k_norm_w,
                           float norm_eps, void* y, float* lse, void* stream);

/*
 * upipe_attn_bwd with bitwise reproducible results: the same arguments,
 * workspace and outputs, and gradients that are identical from run to run
 * and across streams (for a fixed device and library build). Every sum that
 * upipe_attn_bwd spreads over workgroups with fp32 atomic adds is taken in a
 * fixed order instead: the token-split weight-gradient products store their
 * partial tiles in free workspace and add them split by split, and the key
 * blocks of the attention backward are never split over workgroups by head.
 * The results agree with upipe_attn_bwd's to rounding; short sequences run
 * slower (fewer workgroups per key block), long ones at about the same speed.
 * The pages define no such mode; it is the reproducibility a training run
 * needs to compare runs bit for bit.
 */
int upipe_attn_bwd_deterministic(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int n_q_heads,
                                 int n_kv_heads, int head_dim, double rope_theta, int chunk_heads,
                                 const void* x, const void* wq, const void* wk, const void* wv,
                                 const void* wo, const void* q_norm_w, const void* k_norm_w,
                                 float norm_eps, const void* dy, const float* lse, void* dx,
                                 float* dwq, float* dwk, float* dwv, float* dwo, float* dq_norm_w,
                                 float* dk_norm_w, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Sequence-tiled gated-SiLU MLP, the component next to the attention op in
 * the talk's memory stack: the element-wise parts of the model (the MLP and
 * the loss) are tiled along the sequence, so that no intermediate is as long
 * as the whole sequence ("Road to 5 Million Tokens", talk transcript, the
 * part after CPU offloading, on Arctic sequence length training;
 * liquidgold.cc notes, "Progression of Techniques", item 6). The models the
 * talk trains (Llama 3, Qwen3) use the bias-free gated SiLU MLP:
 *
 *   y = (silu(x Wg^T) * (x Wu^T)) Wd^T,   silu(z) = z / (1 + e^-z)
 *
 * computed tile_tokens rows at a time through one reused workspace whose
 * size grows with tile_tokens, not with N. The backward recomputes each
 * tile's activations from x (activation checkpointing) and adds the tile's
 * share of every weight gradient.
 *   x, y, dy, dx  [N][D] io dtype
 *   w_gate, w_up  [F][D] io dtype (nn.Linear [out][in]); w_down [D][F]
 *   dw_gate, dw_up [F][D], dw_down [D][F] fp32 (out, overwritten)
 * Supported: N >= 1; D and F positive multiples of 128; tile_tokens a
 * positive multiple of 128 (a tile larger than N is one tile). Pointers,
 * streams, validation and error codes follow the conventions above; the
 * workspace must hold upipe_mlp_workspace_bytes(..., backward) bytes.
 */
size_t upipe_mlp_workspace_bytes(int64_t n_tokens, int64_t d_model, int64_t d_ff,
                                 int64_t tile_tokens, upipe_dtype_t dtype, int backward);

int upipe_mlp_fwd(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int64_t d_ff,
                  int64_t tile_tokens, const void* x, const void* w_gate, const void* w_up,
                  const void* w_down, void* y, void* workspace, size_t workspace_bytes,
                  void* stream);

int upipe_mlp_bwd(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int64_t d_ff,
                  int64_t tile_tokens, const void* x, const void* w_gate, const void* w_up,
                  const void* w_down, const void* dy, void* dx, float* dw_gate, float* dw_up,
                  float* dw_down, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sequence-tiled cross-entropy loss of the LM head, the other element-wise
 * part that the talk's memory stack tiles along the sequence (same passages
 * as the MLP above): the [N][V] logits never exist; tile_tokens rows of them
 * at a time are consumed by the GEMM's epilogue.
 *
 *   z = h W^T,  lse_i = log sum_v exp z[i, v],  loss_i = lse_i - z[i, t_i]
 *   backward, for per-token upstream gradients g_i:
 *   dz = (softmax(z) - onehot(t)) g,  dh = dz W,  dW = dz^T h
 *
 *   h, dh [N][D] io dtype; W [V][D] io dtype (nn.Linear [out][in]);
 *   targets [N] int32, each in [0, V) (a target outside that range makes its
 *   loss NaN in the forward and contributes no onehot in the backward);
 *   loss, lse, g [N] fp32 (lse is written by the forward and read by the
 *   backward); dW [V][D] fp32 (out, overwritten).
 * Supported: N >= 1; D and V positive multiples of 128; tile_tokens a
 * positive multiple of 128. Pointers, streams, validation and error codes as
 * above; the workspace must hold upipe_loss_workspace_bytes(...) bytes.
 */
size_t upipe_loss_workspace_bytes(int64_t n_tokens, int64_t d_model, int64_t vocab,
                                  int64_t tile_tokens, upipe_dtype_t dtype, int backward);

int upipe_loss_fwd(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int64_t vocab,
                   int64_t tile_tokens, const void* h, const void* w, const int32_t* targets,
                   float* loss, float* lse, void* workspace, size_t workspace_bytes, void* stream);

int upipe_loss_bwd(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int64_t vocab,
                   int64_t tile_tokens, const void* h, const void* w, const int32_t* targets,
                   const float* lse, const float* g, void* dh, float* dw, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * One pre-norm transformer block (Llama style, no biases) around the
 * attention op and the tiled MLP above, trained with activation
 * checkpointing: the talk recomputes each block's activations from its input
 * in the backward pass and keeps (or offloads to the CPU) only the block
 * inputs ("Road to 5 Million Tokens", talk transcript, the memory-
 * optimization progression; liquidgold.cc notes, "Progression of
 * Techniques", items 4 and 5). The pages do not write the block out; this is
 * the plainest reading for the Llama models they train:
 *   a = rmsnorm(x; attn_norm)      h = x + attention(a)
 *   b = rmsnorm(h; mlp_norm)       y = h + mlp(b)
 *   rmsnorm(u; g) = g * u / sqrt(mean over d_model of u^2 + norm_eps)
 * with attention as upipe_attn_fwd (chunk_heads query heads at a time, q/k
 * norm optional) and mlp as upipe_mlp_fwd (tile_tokens rows at a time).
 * The residual stream h is rounded to the io dtype before its norm, as a
 * stored activation would be. The MLP half runs tile by tile: per tile, the
 * residual add, the norm, the MLP and the second residual add (fused into the
 * MLP's last product); no [N][d_ff] buffer exists.
 *
 * Backward, from the block input alone (h_mid and lse NULL): the norm of x
 * and the attention forward are recomputed (the talk's checkpointing), then
 * per tile the MLP half's backward, then the attention backward (which
 * recomputes O from the lse, as upipe_attn_bwd does) and the first norm's
 * backward. With h_mid and lse from the forward, the attention forward is
 * not rerun. Every gradient is overwritten.
 *
 *   x, y, dy, dx, h_mid [N][D] io dtype; lse [Hq][N] fp32
 *   weights: attn_norm, mlp_norm [D]; wq, wk, wv, wo, q_norm, k_norm as in
 *   upipe_attn_fwd; w_gate, w_up, w_down as in upipe_mlp_fwd (io dtype)
 *   grads: the same shapes in fp32 (q_norm, k_norm iff those weights are given)
 * Supported: the attention op's and the MLP's shapes, and d_model <= 8192.
 * Pointers, streams, validation and error codes follow the conventions
 * above; the workspace must hold upipe_block_workspace_bytes(...) bytes.
 */
typedef struct {
  int64_t n_tokens, d_model, d_ff, tile_tokens;
  int n_q_heads, n_kv_heads, head_dim, chunk_heads;
  double rope_theta;
  float norm_eps;    /* the block's two norms over d_model */
  float qk_norm_eps; /* the per-head q/k norm (when its weights are given) */
} upipe_block_shape_t;

typedef struct {
  const void* attn_norm;
  const void *wq, *wk, *wv, *wo;
  const void *q_norm, *k_norm; /* both NULL: no q/k norm */
  const void* mlp_norm;
  const void *w_gate, *w_up, *w_down;
} upipe_block_weights_t;

typedef struct {
  float* attn_norm;
  float *wq, *wk, *wv, *wo;
  float *q_norm, *k_norm;
  float* mlp_norm;
  float *w_gate, *w_up, *w_down;
} upipe_block_grads_t;

/* Workspace bytes for upipe_block_fwd (backward = 0) or upipe_block_bwd
 * (backward = 1); 0 when the entry point would reject the arguments. */
size_t upipe_block_workspace_bytes(const upipe_block_shape_t* shape, int qk_norm, upipe_dtype_t dtype,
                                   int backward);

/* Forward: y (out). h_mid (out, may be NULL) = the residual stream after
 * the attention; lse (out, may be NULL) = the attention's log-sum-exps. */
int upipe_block_fwd(upipe_dtype_t dtype, const upipe_block_shape_t* shape, const void* x,
                    const upipe_block_weights_t* w, void* y, void* h_mid, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Backward for upstream gradient dy: dx and every weight gradient (out).
 * h_mid and lse: both NULL (recompute from x) or both as the forward wrote
 * them for the same inputs. */
int upipe_block_bwd(upipe_dtype_t dtype, const upipe_block_shape_t* shape, const void* x,
                    const upipe_block_weights_t* w, const void* h_mid, const float* lse,
                    const void* dy, void* dx, const upipe_block_grads_t* grads, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * A stack of n_layers blocks of one shape (each with its own weights), with
 * the block inputs offloaded to host memory between the passes: the talk
 * keeps each transformer block's input off the GPU after the forward and
 * prefetches it back for the backward ("Road to 5 Million Tokens", talk
 * transcript, the part on CPU offloading; liquidgold.cc notes, "Progression
 * of Techniques", item 5). The GPU holds two activation and two gradient
 * buffers and one block workspace, whatever n_layers is.
 *
 * Forward: block l's input is copied to host_inputs[l] on copy_stream while
 * block l runs on stream; block l + 1, which reuses that input's buffer,
 * waits for the copy. y = the last block's output.
 * Backward: block l's input is copied back into a device buffer on
 * copy_stream while the blocks above it run their backward (two layers
 * ahead); block l runs upipe_block_bwd from its input alone (checkpointing)
 * and passes its dx down. dx = the first block's input gradient.
 *
 *   weights, grads: host arrays of n_layers structs (device pointers inside)
 *   x, y, dy, dx [N][D] io dtype (device)
 *   host_inputs [n_layers][N][D] io dtype, written by the forward and read by
 *   the backward. Host memory from hipHostMalloc (pinned) lets the copies run
 *   beside the compute; any memory HIP can copy gives the same results.
 *   copy_stream: a second stream for the copies (NULL: stream itself, no
 *   overlap). Both calls order the copies against stream with events: every
 *   output, host_inputs included, is complete once stream reaches the end of
 *   the call's work.
 * Every layer's weights (and gradients) are checked before anything is
 * enqueued; all layers must agree on having q/k norm.
 */
size_t upipe_stack_workspace_bytes(const upipe_block_shape_t* shape, int qk_norm, upipe_dtype_t dtype);

int upipe_stack_fwd(upipe_dtype_t dtype, const upipe_block_shape_t* shape, int n_layers,
                    const upipe_block_weights_t* weights, const void* x, void* y, void* host_inputs,
                    void* workspace, size_t workspace_bytes, void* stream, void* copy_stream);

int upipe_stack_bwd(upipe_dtype_t dtype, const upipe_block_shape_t* shape, int n_layers,
                    const upipe_block_weights_t* weights, const void* host_inputs, const void* dy, void* dx,
                    const upipe_block_grads_t* grads, void* workspace, size_t workspace_bytes, void* stream,
                    void* copy_stream);

/*
 * Optional per-kernel timing (for benchmarks and profilers; off by default).
 * While enabled, every kernel the library enqueues is bracketed by two
 * hipEvents on the caller's stream, and its algorithmic work (flops of the
 * exact math it implements: 2*M*N*K for a GEMM, 4*d per visible (query, key)
 * pair per head for attention forward, 8*d for the dK/dV kernel and 6*d for
 * the dQ kernel of the attention backward) is noted.
 * upipe_profile_stop waits for the recorded events, writes per-kind totals
 * (milliseconds, launch counts, flops) into arrays of n_kinds entries, and
 * turns timing off. Process-wide state: do not profile concurrent calls from
 * several threads. Returns UPIPE_OK or UPIPE_ERR_HIP.
 */
enum {
  UPIPE_KERNEL_PROJECTION = 0,      /* Q/K/V and dO projection GEMMs (+ norm/RoPE epilogue) */
  UPIPE_KERNEL_OUT_GEMM = 1,        /* y (+)= O Wo^T and dx (+)= dq Wq style GEMMs */
  UPIPE_KERNEL_ATTN_FWD = 2,        /* causal attention forward (online softmax) */
  UPIPE_KERNEL_ATTN_RECOMPUTE = 3,  /* backward's forward recompute from the saved LSE */
  UPIPE_KERNEL_ATTN_BWD_DKDV = 4,   /* attention backward, key-stationary: dK, dV (8*d per pair) */
  UPIPE_KERNEL_ATTN_BWD_DQ = 5,     /* attention backward, query-stationary: dQ (6*d per pair) */
  UPIPE_KERNEL_WGRAD = 6,           /* split-K weight-gradient GEMMs */
  UPIPE_KERNEL_OTHER = 7,           /* RoPE/RMSNorm backward, transposes, fills */
  UPIPE_KERNEL_MLP_GEMM = 8,        /* MLP products of x, a and dy (gated-SiLU epilogues) and dx */
  UPIPE_KERNEL_MLP_WGRAD = 9,       /* MLP weight-gradient GEMMs */
  UPIPE_KERNEL_LOSS_GEMM = 10,      /* LM-head logits (loss epilogues), their reduction, dh */
  UPIPE_KERNEL_LOSS_WGRAD = 11,     /* LM-head weight-gradient GEMMs */
  UPIPE_KERNEL_BLOCK_NORM = 12,     /* the block's row RMSNorms (forward, backward) */
  UPIPE_KERNEL_KINDS = 13
};
int upipe_profile_start(void);
int upipe_profile_stop(double* total_ms, int64_t* launches, double* flops, int n_kinds);

/* Static text for an error code. */
const char* upipe_strerror(int code);

/*
 * Dense bf16 MFMA peak of a device from its properties: compute units x
 * maximum engine clock x 4096 flop per clock per compute unit (CDNA4's dense
 * bf16 rate per CU). Used by benchmarks to state the peak they divide by.
 *   device: HIP device ordinal; compute_units, clock_khz: may be NULL
 * Returns UPIPE_OK, or UPIPE_ERR_HIP when the device cannot be queried
 * (outputs untouched).
 */
int upipe_device_peak(int device, double* bf16_dense_tflops, int* compute_units, int* clock_khz);

/* Library version as major*10000 + minor*100 + patch. */
int upipe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* UPIPE_H_ */
