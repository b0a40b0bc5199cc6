/*
 * lf.h - C ABI of the MI355X (gfx950) Longformer band + global attention library.
 *
 * Source of the operations: the page "FasterTransformer Longformer 推理加速实践：
 * PyTorch 集成、输入约束与端到端性能解析" (cited as [FT-LF]), sections
 * "使用前提：四条硬性约束" (four hard constraints) and "Longformer Encoder 计算流程"
 * (encoder computation flow: input list, preprocessing list, per-layer steps 1-6).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are device pointers to caller-owned, contiguous buffers, unless a
 *    comment says otherwise.  The library keeps no reference after a call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *    call only enqueues work on `stream` and returns without waiting, except
 *    lf_check_masks, which synchronises.  Keep buffers alive until the stream has
 *    passed the call.  Outputs must not alias inputs.
 *  - dtype: one of lf_dtype.  Activations, masks and outputs share it.
 *  - head_dim is fixed at 64 ([FT-LF] hard constraint 2); it is not a parameter.
 *  - q, k, v, kg, vg, out are [B, H, S, 64] row-major; qg is [B, H, G, 64];
 *    local_mask, global_mask and local_bias are [B, S]; global_idx is int32 [B, S];
 *    global_count is int32 [B].
 *  - Masks ([FT-LF] input list): local_mask 1.0 = token attends, 0.0 = padding;
 *    global_mask 0.0 = global token, -10000.0 = ordinary token.
 *  - Shape rules are checked on the host before anything is enqueued: B, H, S >= 1;
 *    W even and >= 2; S % W == 0 and S >= 2W ([FT-LF] hard constraint 1);
 *    0 <= G <= W ([FT-LF] hard constraint 3, in the inclusive form the page says
 *    the code checks); B*H*S <= 2^31 - 1; S < 2^24 for fp16 / bf16; pointers
 *    non-NULL (qg may be NULL when G == 0).  On a violation nothing is enqueued, outputs are untouched, the call
 *    returns LF_ERR_INVALID_ARGUMENT and lf_last_error() names the rule.
 *  - Data-dependent preconditions are NOT checked on the fast path (the result is
 *    unspecified when they are violated): global tokens sit contiguously at the
 *    head of each sequence ([FT-LF] hard constraint 4); at most G of them per
 *    sequence; masks hold only the values above.  lf_check_masks verifies them,
 *    and setting the environment variable LF_DEBUG_CHECK=1 makes lf_attn_forward
 *    call it first.
 *  - Work split (fp16 / bf16): when the band tiles (B * H * ceil(S / 256) workgroups)
 *    plus B * H leave none of the device's CUs short, the global rows of each (b, h)
 *    run in a workgroup of their own; otherwise they are split over the band tiles'
 *    workgroups and merged by the last one.  The two differ only in rounding order.
 *    LF_ATTN_NO_GWG=1 (read on every call) selects the second on every grid.
 *    On the split path, sequences of 8192 tokens and more run 128-row workgroups,
 *    two per CU, with the splits of alternate dispatch generations before or after
 *    the band work; shorter ones run 256-row workgroups, one per CU.  The outputs
 *    agree to rounding order; LF_ATTN_WAVES=4 or 8 (read on every call) forces the
 *    128-row (4 waves) or the 256-row (8 waves) workgroups.  In the 256-row
 *    workgroups with at most 32 global tokens (and W >= 160), four more
 *    waves compute the tile's key split of the global rows, its merge and the last
 *    tile's combine while the band waves run the band loop, and the band waves take
 *    the global keys inside their first and last band steps (blocks there that lie
 *    outside every row's window) rather than in a step of their own;
 *    LF_ATTN_NO_HELP=1 (read on every call) leaves the split to the band waves,
 *    after their loop.  Local and global rows agree to rounding order either way.
 *  - Return value: an lf_status.  LF_ERR_HIP means a HIP call failed while
 *    enqueuing; lf_last_error() (thread-local) holds the message.
 */
#ifndef LF_H
#define LF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LF_F32 = 0, LF_F16 = 1, LF_BF16 = 2 } lf_dtype;

typedef enum {
  LF_OK = 0,
  LF_ERR_INVALID_ARGUMENT = 1,
  LF_ERR_UNSUPPORTED = 2,
  LF_ERR_HIP = 3,
  LF_ERR_PRECONDITION = 4
} lf_status;

/*
 * Global-token index extraction ([FT-LF] computation flow, preprocessing item 1).
 * For each batch row b, position s is flagged iff global_mask[b,s] == 0.0.
 * global_idx[b,:] receives a stable partition of 0..S-1: the flagged positions in
 * ascending order, then the other positions in descending order (the layout of a
 * flagged device partition).  global_count[b] receives the number of flagged
 * positions.  Integer results; bit-exact.
 */
int lf_init_global_idx(int dtype, const void* global_mask, int B, int S,
                       int32_t* global_idx, int32_t* global_count, void* stream);

/*
 * Local-mask shift ([FT-LF] computation flow, preprocessing item 2):
 * local_bias = fma(local_mask, 10000, -10000) evaluated in fp32 and stored in
 * `dtype` with round-to-nearest-even (1 -> 0, 0 -> -10000; bf16 stores -9984).
 * local_mask and local_bias are [B, S]; any B*S >= 1 is accepted.
 */
int lf_mask_shift(int dtype, const void* local_mask, int B, int S, void* local_bias,
                  void* stream);

/*
 * Band + global attention ([FT-LF] computation flow, per-layer steps 3 and 4).
 * With scale c = 1/8 (= 1/sqrt(64)), n_b = number of global tokens of sequence b
 * (positions 0..n_b-1 under the head-of-sequence precondition) and live keys
 * those with local_mask == 1:
 *   - a row with local_mask 0 is written as +0.0;
 *   - a global row s = r (r < n_b) is softmax_j(c <qg[r], kg[j]>) . vg[j] over
 *     every live key j of the sequence;
 *   - any other row s is softmax over the live keys j with |j - s| <= W/2,
 *     j >= n_b, plus the live global keys j < n_b, of c <q[s], k[j]>, weighting
 *     v[j].  Global keys are therefore counted once.
 * A padded key (local_mask 0) is excluded from every row.  The page adds the shifted
 * mask (-10000) to its scores; exp(x - 10000) is exactly 0 in fp32 for any score a
 * row with one live key can reach, so excluding the key gives the same result, and the
 * kernels exclude it (-inf) instead of adding the bias.
 * fp16 / bf16: one launch on MFMA with fp32 accumulation, reading both masks itself.
 * fp32: the index extraction and mask shift, then the vector-ALU kernel; when the
 * global rows' keys are split (G > 0, sequences of more than one 256-row tile), a
 * third launch combines their per-split partial states.
 * Scratch, per (device, stream), never waiting for the host: the split tickets of the
 * global-row merge sit in a slot of a static device array (64 slots per device, one per
 * stream that calls; zero-filled on the stream when the slot is handed out, left zero
 * by every call); the global-row partials (and fp32's preprocessed masks) sit in a
 * device buffer kept for the stream, allocated and, when a larger shape needs more,
 * replaced with hipMallocAsync / hipFreeAsync on `stream` (stream-ordered: no host
 * sync).  lf_release_stream_scratch frees that buffer.  Calls on one stream share its
 * scratch (they run in order); calls on different streams do not.  While `stream` is
 * being captured into a graph, a call uses neither: it allocates and frees its own
 * scratch and tickets on the stream (capture-safe).
 */
int lf_attn_forward(int dtype, const void* q, const void* k, const void* v,
                    const void* qg, const void* kg, const void* vg,
                    const void* local_mask, const void* global_mask,
                    int B, int H, int S, int W, int G, void* out, void* stream);

/*
 * lf_attn_forward for callers that cannot allocate device memory: code under stream
 * capture, tight serving loops, harnesses that forbid allocation.  Same arguments,
 * computation, work split and results (bit for bit) as lf_attn_forward.  It calls no
 * allocator: its split tickets and global-row partials (fp32: and the preprocessed masks)
 * live in one static device array per device, 32 MiB, held until the process ends
 * (lf_attn_forward_noalloc_max_scratch() bytes of it for partials, the rest for 16384
 * tickets).  The array's device address is looked up once per device (on the first
 * call there, which also zero-fills the tickets with a kernel on `stream`); every call
 * leaves the tickets zero.  Every call on a device shares that device's array, which
 * keeps the last call's contents: calls that overlap in time on one device (on
 * different streams or threads) race and must not be made.  A shape whose scratch
 * exceeds the array (partials of B*H*n_split*G*272 bytes, n_split <= 32), or with
 * B*H > 16384 and G > 0, returns LF_ERR_UNSUPPORTED with nothing enqueued.
 */
size_t lf_attn_forward_noalloc_max_scratch(void);
int lf_attn_forward_noalloc(int dtype, const void* q, const void* k, const void* v,
                            const void* qg, const void* kg, const void* vg,
                            const void* local_mask, const void* global_mask,
                            int B, int H, int S, int W, int G, void* out, void* stream);

/*
 * Frees the scratch buffer lf_attn_forward / lf_attn_forward_any_globals keep for
 * `stream` on the current device (stream-ordered: hipFreeAsync on `stream`, after the
 * calls already enqueued there).  The next call on the stream allocates a new one.
 */
int lf_release_stream_scratch(void* stream);

/*
 * Band + global attention with the global tokens at any positions (the global
 * attention pattern of the Longformer model itself, which the [FT-LF] page names as
 * the case its head-of-sequence constraint excludes, section "使用前提：四条硬性约束").
 * Same arguments, layouts, precision and errors as lf_attn_forward, with positions
 * P_b = the flagged positions of batch row b in ascending order (flag: global_mask
 * == 0.0), n_b = |P_b| <= G:
 *   - a row with local_mask 0 is written as +0.0;
 *   - the global row s = P_b[r] is softmax_j(c <qg[r], kg[j]>) . vg[j] over every
 *     live key j (qg row r belongs to the r-th global position);
 *   - any other row s is softmax over the live keys j with |j - s| <= W/2 and j not
 *     in P_b, plus the live keys of P_b, of c <q[s], k[j]>, weighting v[j].
 * With leading global tokens this equals lf_attn_forward.  Two launches on `stream`:
 * the index extraction (as lf_init_global_idx) into library-owned device memory,
 * then the attention, which gathers the global keys through that index.  The index
 * sits in the stream's scratch buffer, beside the partials (same scratch rules as
 * lf_attn_forward).  Data-dependent preconditions (masks
 * 0/1 and 0/-10000, n_b <= G) are checked only by lf_check_masks or under
 * LF_DEBUG_CHECK=1, which here skips the head-of-sequence test.
 */
int lf_attn_forward_any_globals(int dtype, const void* q, const void* k, const void* v,
                                const void* qg, const void* kg, const void* vg,
                                const void* local_mask, const void* global_mask,
                                int B, int H, int S, int W, int G, void* out, void* stream);

/* Bytes of workspace lf_attn_forward_pre needs for this shape (0 on bad arguments). */
size_t lf_attn_workspace_bytes(int dtype, int B, int H, int S, int W, int G);

/*
 * Same computation as lf_attn_forward on already-preprocessed masks: global_idx /
 * global_count from lf_init_global_idx and local_bias from lf_mask_shift.  It
 * allocates nothing and is one kernel launch (fp32 with split global-row keys: two,
 * the second combining the splits).  `workspace` (device, 256-byte
 * aligned, ws_bytes >= lf_attn_workspace_bytes) starts with B*H int32 split
 * tickets followed by the partial results of the global rows.  The tickets must be
 * zero before the first call that uses the workspace (zero-fill it once after
 * allocating it); every call leaves them zero again, the rest of the workspace may
 * hold anything.  Calls that share a workspace must not overlap in time.
 */
int lf_attn_forward_pre(int dtype, const void* q, const void* k, const void* v,
                        const void* qg, const void* kg, const void* vg,
                        const int32_t* global_idx, const int32_t* global_count,
                        const void* local_bias, int B, int H, int S, int W, int G,
                        void* out, void* workspace, size_t ws_bytes, void* stream);

/*
 * Synchronous check of the data-dependent preconditions: every local_mask value is
 * 0 or 1; every global_mask value is 0 or -10000 (as stored in `dtype`); the
 * global tokens of each sequence are positions 0..n_b-1 with n_b <= G.  Returns
 * LF_OK or LF_ERR_PRECONDITION (lf_last_error() names the first violation).
 */
int lf_check_masks(int dtype, const void* local_mask, const void* global_mask, int B,
                   int S, int G, void* stream);

/*
 * Weights of one encoder layer ([FT-LF] computation flow, per-layer steps 1-6).
 * All are device pointers in the layer dtype.  Matrices are [out, in] row-major
 * (y = x W^T + b).  w_proj is [5*hidden, hidden]: row blocks Q | K | V |
 * global-K | global-V, and inside each block head h owns rows 64h .. 64h+63.
 */
typedef struct {
  const void* w_proj; const void* b_proj;   /* [5D, D], [5D] */
  const void* w_qg;   const void* b_qg;     /* [D, D],  [D]  global query */
  const void* w_o;    const void* b_o;      /* [D, D],  [D]  attention output */
  const void* ln1_g;  const void* ln1_b;    /* [D] */
  const void* w_ffn1; const void* b_ffn1;   /* [F, D],  [F] */
  const void* w_ffn2; const void* b_ffn2;   /* [D, F],  [D] */
  const void* ln2_g;  const void* ln2_b;    /* [D] */
} lf_layer_weights;

/* Workspace bytes lf_encoder_layer needs (0 on bad arguments). */
size_t lf_encoder_layer_workspace_bytes(int dtype, int B, int S, int hidden, int H, int ffn,
                                        int W, int G);

/*
 * One post-LayerNorm Longformer encoder layer ([FT-LF] computation flow, per-layer
 * steps 1-6):
 *   [q|k|v|kg|vg] = x W_proj^T + b_proj, split into heads; qg = x[:, :G] W_qg^T + b_qg;
 *   a  = band + global attention (as lf_attn_forward, scale attn_scale), heads joined;
 *   h1 = LayerNorm(x + a W_o^T + b_o; ln1)    (biased variance, eps ln_eps)
 *   y  = LayerNorm(h1 + GELU(h1 W_1^T + b_1) W_2^T + b_2; ln2)
 *        (erf GELU; erf evaluated within 1.5e-7 absolute)
 * x, y: [B, S, hidden] in `dtype` (LF_F16, LF_BF16 or LF_F32; fp32 runs its GEMMs on
 * fp32 MFMA and its attention on the vector ALUs from masks preprocessed inside the
 * call).  Shape rules: the attention rules of lf_attn_forward, plus hidden == 64*H,
 * hidden and ffn multiples of 128, hidden one of 256, 512, 768, 1024, 2048, 4096
 * (LayerNorm row widths), B*S*ffn*sizeof(dtype) < 2^31.  w_qg / b_qg may be
 * NULL when G == 0.  `workspace` (device, 256-byte aligned, ws_bytes >=
 * lf_encoder_layer_workspace_bytes) holds every intermediate: attention tickets
 * first, then q, k, v, kg, vg, qg, the attention output, the fp32 pre-LayerNorm
 * rows, h1 in fp32 and in `dtype`, the FFN intermediate, and the fp32 partial sums of
 * the GEMMs whose grids are split over K (those with few output tiles).  Its first bytes (the
 * tickets) must be zero before the first call that uses it (zero-fill it once after
 * allocating); every call leaves them zero.  The residual stream (x + projection,
 * h1) is kept in fp32; GEMM inputs are rounded to `dtype`.  Calls sharing a
 * workspace must not overlap in time.  Enqueues 7 launches on `stream` (the
 * global-query projection rides in the packed projection's launch), 8 when the masks
 * are preprocessed inside the call (fp32), no sync.  The result does not depend on
 * how a GEMM is split over K: partial sums are added in a fixed order.
 * Weight layout: [out, in] (y = x W^T), so that both MFMA operands of every GEMM are
 * contiguous along the reduction dimension; a caller holding [in, out] weights (the
 * layout the page's plugin produces by transposing the model's weights) transposes
 * them once at load time.
 */
int lf_encoder_layer(int dtype, const lf_layer_weights* w, const void* x,
                     const void* local_mask, const void* global_mask, int B, int S,
                     int hidden, int H, int ffn, int W, int G, float attn_scale,
                     float ln_eps, void* y, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes lf_ffn_block needs (0 on bad arguments). */
size_t lf_ffn_block_workspace_bytes(int dtype, int M, int D, int F, int fused);

/*
 * The FFN block of a layer ([FT-LF] computation flow, per-layer step 6), on its own:
 *   y = LayerNorm(resid + GELU(h W_1^T + b_1) W_2^T + b_2; ln_g, ln_b)
 * over M rows (biased variance, eps ln_eps; erf GELU evaluated within 1.5e-7).
 * h: [M, D] in `dtype` (the GEMM input); resid: [M, D] fp32 (the residual stream);
 * w1: [F, D], w2: [D, F], b1: [F], b2, ln_g, ln_b: [D], all in `dtype`; y: [M, D] in
 * `dtype`.  Device pointers; nothing is written but y and the workspace.
 *   fused = 0: two GEMMs, as lf_encoder_layer runs them (the GELU output goes
 *     through memory in `dtype`, [M, F]); 2 or 3 launches.
 *   fused = 1: one kernel forms GELU(h W_1^T + b_1) chunk by chunk on chip (rounded
 *     to `dtype`, as the two-GEMM path stores it) and multiplies it into W_2 at once,
 *     the operator fusion of the page "300%加速！PaddleNLP FastFFN如何让大模型训练"飞"起来"
 *     (section "技术原理深入解析", item 1); then the LayerNorm kernel sums its fp32
 *     partials (one per F slice when M is small) with b_2 and resid.  fp16 / bf16,
 *     D in {256, 512, 768, 1024}; else LF_ERR_UNSUPPORTED.  2 launches.
 * Shape rules: D and F multiples of 128, D a LayerNorm width (256, 512, 768, 1024,
 * 2048, 4096), M*F*sizeof(dtype) < 2^31.  `workspace`: device, 256-byte aligned,
 * ws_bytes >= lf_ffn_block_workspace_bytes (no zeroing needed).  The two modes agree
 * to rounding (their partial sums are grouped differently); each is deterministic.
 * Enqueued on `stream`, no sync.
 */
int lf_ffn_block(int dtype, const void* h, const float* resid, const void* w1, const void* b1,
                 const void* w2, const void* b2, const void* ln_g, const void* ln_b, int M,
                 int D, int F, float ln_eps, int fused, void* y, void* workspace,
                 size_t ws_bytes, void* stream);

/* Workspace bytes lf_encoder_forward needs (0 on bad arguments). */
size_t lf_encoder_forward_workspace_bytes(int dtype, int B, int S, int hidden, int H, int ffn,
                                          int W, int G);

/*
 * A stack of n_layers encoder layers ([FT-LF] computation flow: the preprocessing
 * list runs once — global-token index extraction and the local-mask shift — then the
 * per-layer steps 1-6 run for every layer).  w points to n_layers weight sets, layer
 * l using w[l]; each layer is lf_encoder_layer's computation, with the attention
 * reading the preprocessed masks.  x is never written; the layer outputs alternate
 * between y and an activation buffer in the workspace so that the last layer writes
 * y.  Same shape rules, dtype, precision and workspace convention as
 * lf_encoder_layer (ws_bytes >= lf_encoder_forward_workspace_bytes; its first bytes
 * zero before the first use, left zero).  Enqueues 1 + 7 * n_layers launches.
 */
int lf_encoder_forward(int dtype, const lf_layer_weights* w, int n_layers, const void* x,
                       const void* local_mask, const void* global_mask, int B, int S,
                       int hidden, int H, int ffn, int W, int G, float attn_scale,
                       float ln_eps, void* y, void* workspace, size_t ws_bytes, void* stream);

/*
 * lf_encoder_layer / lf_encoder_forward with the global tokens at any positions (the
 * Longformer model's own global pattern, which the [FT-LF] page's head-of-sequence
 * constraint excludes, section "使用前提：四条硬性约束").  Same arguments, shape
 * rules, dtypes, workspace sizes (lf_encoder_layer_workspace_bytes /
 * lf_encoder_forward_workspace_bytes) and conventions.  With P_b the flagged
 * positions of batch row b in ascending order (global_mask == 0.0), n_b = |P_b| <= G:
 * qg row r of batch row b is projected from x[b, P_b[r]] (rows from n_b on from the
 * other positions of the global-index partition; the attention never reads them),
 * and the attention is lf_attn_forward_any_globals'.  With leading global tokens the
 * result equals lf_encoder_layer / lf_encoder_forward.  The layer call runs the
 * global-index partition itself first (8 launches); the stack runs it once.
 */
int lf_encoder_layer_any_globals(int dtype, const lf_layer_weights* w, const void* x,
                                 const void* local_mask, const void* global_mask, int B, int S,
                                 int hidden, int H, int ffn, int W, int G, float attn_scale,
                                 float ln_eps, void* y, void* workspace, size_t ws_bytes,
                                 void* stream);
int lf_encoder_forward_any_globals(int dtype, const lf_layer_weights* w, int n_layers,
                                   const void* x, const void* local_mask, const void* global_mask,
                                   int B, int S, int hidden, int H, int ffn, int W, int G,
                                   float attn_scale, float ln_eps, void* y, void* workspace,
                                   size_t ws_bytes, void* stream);

/*
 * Measurement hook.  After lf_kernel_timing_start(capacity), each of the next
 * `capacity` lf_attn_forward / lf_attn_forward_pre calls made on this thread
 * records a HIP event pair on its own stream immediately around its main
 * attention kernel (the band + global-row launch).  lf_kernel_timing_stop waits
 * for the recorded events, returns the number of timed launches and their summed
 * duration in milliseconds, releases the events and ends the recording.
 * capacity must be in 1 .. 1000000.
 */
int lf_kernel_timing_start(int capacity);
int lf_kernel_timing_stop(int* launches, double* total_ms);

/* Static text for a status code. */
const char* lf_status_string(int status);

/* Message of the last failed call on this thread ("" if none). */
const char* lf_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LF_H */
