/*
 * h3k — forward pass of the AdaLN-modulated DiT block on MI355X (gfx950).
 *
 * Sources (cited by page title and section; the pages print no formula, so
 * the definitions below are the readings this library implements):
 *   [H3-review]  "Redis 之父下场手写推理引擎：antirez 用约 24000 行原生代码驯服视频生成模型"
 *                (text-matrix.pages.dev): knob list (--layers 50/45/40), speed/quality
 *                section (int8 MLP, then int8 QKV projection; hard constraints are
 *                validated and rejected, unsupported entries are removed rather than
 *                left to produce bad output).
 *   [H3-memory]  "37GiB模型如何装进统一内存 h3.c 零拷贝权重与激活内存别名技巧详解"
 *                (m.nxbn.cn): technique 2 (block order QKV -> attention -> MLP,
 *                50 blocks per denoising step, one QKV buffer re-used for the attention
 *                input and the normalised MLP input, the attention output buffer re-used
 *                for the MLP output, byte-identical results), technique 3 (AdaLN is
 *                precomputed; int8 weights let the caller drop the BF16 originals).
 *   [ctypes]     "h3.c ComfyUI plugin" article (m.xxqk.cn), sections 3.1, 4.2, 5.2:
 *                integer status codes, explicit argument types, an explicit context
 *                instead of globals, and nothing returned that the caller must free.
 *
 * The block (one token row t, hidden size D, H heads of size d, MLP width F):
 *   mod  = W_ada c + b_ada, six D-chunks: shift_a, scale_a, gate_a, shift_m, scale_m, gate_m
 *   h    = LN(x) (1 + scale_a) + shift_a            LN: no affine, biased variance, eps
 *   q|k|v = h W_qkv^T + b_qkv                        W_qkv rows ordered [Q | K | V]
 *   o    = per head softmax(q k^T / sqrt(d)) v       full attention over all N tokens
 *   x1   = x + gate_a * (o W_out^T + b_out)
 *   h2   = LN(x1) (1 + scale_m) + shift_m
 *   u    = GELU_tanh(h2 W_up^T + b_up)
 *   y    = x1 + gate_m * (u W_down^T + b_down)
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers (HBM) unless marked "host".  The caller owns
 *     all memory; the library never allocates or frees device memory and never
 *     synchronises the stream (only h3k_profiler_read waits, on its own events).
 *   - Work is enqueued on `stream` and is asynchronous.
 *   - Every argument is validated before the first launch.  On any error nothing
 *     is enqueued, outputs are untouched, and h3k_last_error() explains.
 *   - Tensors are dense and row-major; base pointers 16-byte aligned, the
 *     workspace 256-byte aligned.  Weight matrices use the [out, in] layout.
 *   - bf16 is the IEEE-style bfloat16 bit pattern (uint16), int8 is int8_t.
 *   - The library keeps no mutable global state apart from a thread-local error
 *     message, so calls on different streams may run concurrently as long as
 *     they do not share output or workspace memory.
 */
#ifndef H3K_H
#define H3K_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ([ctypes] 3.1: integer status returns) ------------------ */
typedef int32_t h3k_status;
#define H3K_OK               0
#define H3K_ERR_NULL         1  /* a required pointer is NULL                         */
#define H3K_ERR_SHAPE        2  /* a size is out of range or inconsistent (D != H*d) */
#define H3K_ERR_DTYPE        3  /* unknown dtype code                                 */
#define H3K_ERR_ALIGN        4  /* pointer not 16-byte (workspace: 256-byte) aligned  */
#define H3K_ERR_WORKSPACE    5  /* workspace smaller than h3k_dit_workspace_size      */
#define H3K_ERR_OVERLAP      6  /* output memory overlaps an input or the workspace  */
#define H3K_ERR_UNSUPPORTED  7  /* valid but not implemented (e.g. head_dim 96)       */
#define H3K_ERR_HIP          8  /* no device, or a HIP launch failed                  */

/* ---- element types ---------------------------------------------------------- */
typedef int32_t h3k_dtype;
#define H3K_F32   0
#define H3K_BF16  1
#define H3K_INT8  2

/* Block configuration (host struct, passed by pointer).
 * Supported: head_dim in {64, 128}; hidden = n_heads * head_dim <= 8192;
 * mlp_hidden a multiple of 64; cond_dim a multiple of 8 and <= 16384;
 * n_tokens >= 1.  act_dtype F32 or BF16.  weight_dtype equal to act_dtype, or
 * INT8 with BF16 activations (per-output-channel scales, see h3k_quantize_weights_int8).
 * alias_activations: 1 lets the lifetime planner overlap intermediate buffers in
 * the workspace ([H3-memory] technique 2), 0 gives each its own region; the
 * output is bit-identical either way.  The environment variable
 * H3K_DISABLE_ACTIVATION_ALIAS=1 forces 0, as a diagnostic switch.
 * int8_fc2_rows: 1 runs the MLP-down projection (FC2) with int8 activations as
 * well ([H3-review] speed/quality section, the row-quantised FC2: one activation
 * scale per token row): u is quantised per row by the rule of
 * h3k_quantize_weights_int8, and FC2 is the int8 x int8 product with int32
 * accumulation, scaled by the row and channel scales (h3k_linear_int8).
 * Needs weight_dtype INT8, act_dtype BF16 and mlp_hidden a multiple of 128 and
 * <= 2^17 (so that the int32 sum of int8 products cannot overflow);
 * 0 leaves FC2 as for the other projections.
 * int8_mlp_group: 0 gives every INT8 matrix per-row scales; G in {32, 64, 128}
 * quantises the two MLP matrices in groups of G input channels instead
 * ([H3-review] speed/quality section: the default MLP engine is int8 with group
 * quantisation; the page gives no group size): s_up is then [F, D/G] and
 * s_down [D, F/G] (h3k_quantize_weights_int8_groups), the QKV and output
 * projections keep per-row scales.  Needs weight_dtype INT8, act_dtype BF16,
 * hidden and mlp_hidden multiples of G, and int8_fc2_rows = 0.
 * rope_frames, rope_height, rope_width: 0, 0, 0 leaves attention without
 * positional terms (every workload of the pages' benchmark); a grid T x H x W
 * with T*H*W = n_tokens (tokens laid out frame, row, column) rotates q and k
 * after their bias by the 3D RoPE of h3k_rope_3d, fused into the QKV
 * projection's epilogue ([H3-review], note on native-256 RoPE).  Needs BF16
 * activations and n_tokens <= 2^24.  rope_half_spatial = 1 halves the spatial coordinates (the
 * page's rule for native-256 generation on 256 square canvases).
 * token_reduction_first, token_reduction_last: for h3k_dit_stack_forward, a
 * layer range [first, last) run on merged tokens ([H3-review] knob list: video
 * tokens paired two by two along rows to shorten the sequence in the middle
 * layers): before block `first` tokens 2m and 2m+1 become their mean
 * (h3k_token_merge; row neighbours when rows have an even length, 54 for the
 * 864x480 latent), the blocks of the range run on n_tokens/2 tokens, and after
 * block last-1 each token gets its own state from before the merge plus the
 * change the range made to its pair (h3k_token_unmerge).  0, 0 (or any empty
 * range) runs every block on all tokens.  Needs an even n_tokens and no RoPE;
 * the workspace then also holds the merged stream. */
typedef struct h3k_dit_config {
  int32_t n_tokens;
  int32_t hidden;
  int32_t n_heads;
  int32_t head_dim;
  int32_t mlp_hidden;
  int32_t cond_dim;
  float   ln_eps;            /* 1e-6 in every workload */
  h3k_dtype act_dtype;
  h3k_dtype weight_dtype;
  int32_t alias_activations;
  int32_t int8_fc2_rows;
  int32_t int8_mlp_group;
  int32_t rope_frames;
  int32_t rope_height;
  int32_t rope_width;
  int32_t rope_half_spatial;
  int32_t token_reduction_first;
  int32_t token_reduction_last;
} h3k_dit_config;

/* Weights of one block; all device pointers.
 * w_ada [6D, C] and b_ada [6D] in act_dtype.  Projection matrices
 * w_qkv [3D, D], w_out [D, D], w_up [F, D], w_down [D, F] in weight_dtype;
 * with INT8 weights, s_* are the fp32 per-row scales ([rows]), otherwise NULL;
 * with int8_mlp_group = G, s_up and s_down hold one scale per group instead
 * ([F, D/G] and [D, F/G], row-major).
 * Biases b_qkv [3D], b_out [D], b_up [F], b_down [D] in act_dtype; any bias may be
 * NULL, meaning zero. */
typedef struct h3k_dit_block_weights {
  const void *w_ada, *b_ada;
  const void *w_qkv, *b_qkv; const float *s_qkv;
  const void *w_out, *b_out; const float *s_out;
  const void *w_up,  *b_up;  const float *s_up;
  const void *w_down, *b_down; const float *s_down;
} h3k_dit_block_weights;

/* Optional per-kernel GPU-event timer (an explicit context, [ctypes] 4.2).
 * Created and destroyed by the caller; records one hipEvent per launched
 * kernel when attached to a forward call through h3k_dit_stats.profiler. */
typedef struct h3k_profiler h3k_profiler;

/* Kernel kinds reported by the profiler, in block order. */
#define H3K_K_ADALN      0  /* AdaLN modulation GEMV                     */
#define H3K_K_LN_MOD     1  /* LayerNorm + AdaLN modulation (both calls) */
#define H3K_K_QKV        2  /* QKV projection GEMM                       */
#define H3K_K_ATTENTION  3  /* flash attention                           */
#define H3K_K_OUT        4  /* out-projection GEMM + gated residual      */
#define H3K_K_UP         5  /* MLP up GEMM + GELU                        */
#define H3K_K_DOWN       6  /* MLP down GEMM + gated residual            */
#define H3K_K_ACT_QUANT  7  /* row quantiser of u (int8_fc2_rows only)   */
#define H3K_K_TOKEN_MERGE   8  /* token reduction: merge (once per stack) */
#define H3K_K_TOKEN_UNMERGE 9  /* token reduction: restore (once per stack) */
#define H3K_K_COUNT      10

/* Statistics of a forward call (host struct).  `profiler` is an input
 * (optional); the rest are outputs ([H3-memory], "verify it yourself": the
 * engine's --profile reports peak live tensor storage and dispatch counts). */
typedef struct h3k_dit_stats {
  uint64_t workspace_bytes;     /* out: bytes the plan uses                         */
  uint64_t peak_live_bytes;     /* out: largest sum of simultaneously live buffers  */
  uint64_t unaliased_bytes;     /* out: workspace the same call needs without aliasing */
  int32_t  dispatches;          /* out: kernels enqueued by the call                */
  int32_t  alias_activations;   /* out: aliasing actually used (after the env switch) */
  int32_t  tail_splits;         /* out: kernels whose partial last wave was split (GEMM
                                   tiles along k, attention workgroups along the keys);
                                   each enqueued one more kernel, counted in dispatches */
  int32_t  _reserved;
  h3k_profiler* profiler;       /* in: NULL, or a profiler that records every launch */
} h3k_dit_stats;

/* Workspace layout of one block (host struct), for inspection and tests.
 * Index with H3K_T_*.  Offsets are byte offsets into the workspace.
 * The QKV region holds Q and K as one row-major [N, 2D] matrix, followed at
 * qkv_vt_offset by V transposed, [D, vt_pitch] (vt_pitch = N rounded up to 8),
 * so that the attention kernel reads V along the key axis.  After the tensors
 * (part_offset) lies the scratch of split tails: when a bf16 out-projection
 * or MLP GEMM's last wave of 256x256 output tiles would leave at least half
 * of the GPU's compute units idle, each of those tiles is split along k into
 * up to 8 workgroups whose fp32 partial tiles a second kernel sums in a fixed
 * order; likewise the attention's last round of workgroups (head_dim 128) is
 * split along the keys and combined by a second kernel (sized for 256 CUs;
 * H3K_DISABLE_TAIL_SPLIT=1 turns both off).
 * With INT8 weights the staging buffer follows (wstage_offset): each int8
 * projection weight is widened to bf16 there (times its group scales, if
 * any) right before its GEMM, which then runs as a bf16 GEMM with the
 * per-channel scale in its epilogue; the resident weights stay int8
 * (H3K_DISABLE_WEIGHT_STAGING=1 widens inside the GEMM instead, same bits).
 * With token reduction the merged stream comes last. */
#define H3K_T_MOD  0   /* fp32 [6D]   */
#define H3K_T_H    1   /* [N, D]      */
#define H3K_T_QKV  2   /* [N, 2D] + [D, vt_pitch] */
#define H3K_T_O    3   /* [N, D]      */
#define H3K_T_X1   4   /* [N, D]      */
#define H3K_T_H2   5   /* [N, D]      */
#define H3K_T_U    6   /* [N, F]      */
#define H3K_T_UQ   7   /* int8 [N, F] (int8_fc2_rows only, else 0 bytes) */
#define H3K_T_US   8   /* fp32 [N]    (int8_fc2_rows only, else 0 bytes) */
#define H3K_T_COUNT 9
typedef struct h3k_dit_plan_info {
  uint64_t offset[H3K_T_COUNT];
  uint64_t bytes[H3K_T_COUNT];
  int32_t  first_step[H3K_T_COUNT];  /* kernel step that writes it (0..8; step 7 quantises u) */
  int32_t  last_step[H3K_T_COUNT];   /* last kernel step that reads it    */
  uint64_t qkv_vt_offset;            /* byte offset of V^T inside the workspace */
  int64_t  vt_pitch;                 /* elements per V^T row */
  uint64_t workspace_bytes;
  uint64_t peak_live_bytes;
  uint64_t unaliased_bytes;
  int32_t  alias_activations;
  int32_t  _reserved;
  uint64_t part_offset;              /* scratch of split tails: byte offset ...            */
  uint64_t part_bytes;               /* ... and size (0 when no kernel can split)          */
  uint64_t wstage_offset;            /* int8 weights: bf16 staging buffer, byte offset ...  */
  uint64_t wstage_bytes;             /* ... and size (0 unless INT8 weights)               */
} h3k_dit_plan_info;

/* Message for the last non-OK status returned on this thread (never NULL). */
const char* h3k_last_error(void);

/* Bytes of workspace a block or stack forward needs with this config (host out).
 * Stacks of any length re-use the one-block workspace (blocks run in sequence). */
h3k_status h3k_dit_workspace_size(const h3k_dit_config* cfg, int32_t n_blocks, uint64_t* bytes_out);

/* The lifetime plan used by the forward calls (host out).  Pure host code. */
h3k_status h3k_dit_plan(const h3k_dit_config* cfg, h3k_dit_plan_info* info_out);

/* One block: out[N, D] = block(x[N, D], c[C]).  x, c, out in act_dtype.
 * `out` must not overlap x, c, any weight or the workspace.
 * stats (host, nullable).  Follows the block order of [H3-memory] technique 2. */
h3k_status h3k_dit_block_forward(const h3k_dit_config* cfg, const h3k_dit_block_weights* weights,
                                 const void* x, const void* c, void* out,
                                 void* workspace, uint64_t workspace_bytes,
                                 hipStream_t stream, h3k_dit_stats* stats);

/* n_blocks blocks in sequence with a shared c: x_{l+1} = block_l(x_l, c);
 * out = x_{n_blocks}.  `blocks` is a HOST array of n_blocks weight structs.
 * Running the first L of a longer stack gives exactly the state after L blocks
 * of it ([H3-review] knob list: --layers 50 / 45 / 40).  Intermediate states
 * live in `out`, so the caller needs no extra buffer. */
h3k_status h3k_dit_stack_forward(const h3k_dit_config* cfg, const h3k_dit_block_weights* blocks,
                                 int32_t n_blocks, const void* x, const void* c, void* out,
                                 void* workspace, uint64_t workspace_bytes,
                                 hipStream_t stream, h3k_dit_stats* stats);

/* One block without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and result as h3k_dit_block_forward
 * (byte-identical output), but the block's intermediates live in a static
 * device array of the library of H3K_NOALLOC_SCRATCH_BYTES (128 MiB): each GPU
 * the library runs on holds its own copy until the process ends.  A config
 * whose workspace (h3k_dit_workspace_size) exceeds it is rejected with
 * H3K_ERR_WORKSPACE before anything is enqueued.  The call allocates nothing;
 * its first call on a device looks up the array's device address there.
 * All calls on one GPU share the array, so calls that overlap in time on one
 * GPU (e.g. on two streams) race on it; serialise them. */
#define H3K_NOALLOC_SCRATCH_BYTES (128ull << 20)
h3k_status h3k_dit_block_forward_noalloc(const h3k_dit_config* cfg, const h3k_dit_block_weights* weights,
                                         const void* x, const void* c, void* out,
                                         hipStream_t stream, h3k_dit_stats* stats);

/* Per-output-channel symmetric int8 quantisation of w [rows, cols] (F32 or BF16);
 * with int8_fc2_rows the forward calls apply the same rule to the rows of u:
 *   scales[o] = max_k |w[o,k]| / 127   (one fp32 division, correctly rounded)
 *   q[o,k]    = clamp(rint(w[o,k] / scales[o]), -127, 127)  (ties to even)
 * A zero row gives scale 0 and q 0.  Bit-exact with any IEEE fp32 implementation
 * of the same two divisions.  Once the stream has passed this call the caller
 * may free w ([H3-memory] technique 3; [H3-review] speed/quality section).
 * rows <= 2^31-1, cols <= 2^20; q [rows, cols] int8, scales [rows] fp32. */
h3k_status h3k_quantize_weights_int8(const void* w, h3k_dtype w_dtype, int64_t rows, int64_t cols,
                                     int8_t* q, float* scales, hipStream_t stream);

/* Group-wise symmetric int8 quantisation of w [rows, cols] (F32 or BF16): each
 * row's columns are cut into blocks of `group` (32, 64 or 128; cols a multiple
 * of it), and every block gets its own scale by the rule above:
 *   scales[o, g] = max_{k in block g} |w[o,k]| / 127
 *   q[o,k]       = clamp(rint(w[o,k] / scales[o, k / group]), -127, 127)
 * A zero block gives scale 0 and q 0.  Bit-exact like h3k_quantize_weights_int8
 * ([H3-review] speed/quality section: the group-quantised int8 MLP; the group
 * size is the caller's choice).  q [rows, cols] int8, scales [rows, cols/group]
 * fp32, row-major; cols <= 2^20. */
h3k_status h3k_quantize_weights_int8_groups(const void* w, h3k_dtype w_dtype, int64_t rows, int64_t cols,
                                            int32_t group, int8_t* q, float* scales, hipStream_t stream);

/* ---- building blocks of the block forward, exposed for testing and timing --- */

/* mod[rows] (fp32) = W[rows, cols] c[cols] + b[rows] (b nullable), W, b, c in dtype.
 * The AdaLN modulation precompute of [H3-memory] technique 3 (rows = 6D). */
h3k_status h3k_adaln_modulation(h3k_dtype dtype, int32_t rows, int32_t cols, const void* w,
                                const void* b, const void* c, float* mod, hipStream_t stream);

/* out[n, D] = LN(x[n, D]) * (1 + scale[D]) + shift[D]; x, out in dtype with row
 * pitches ldx, ldo (elements); shift, scale fp32.  Rows independent.
 * The modulated LayerNorm ahead of the QKV projection and of the MLP. */
h3k_status h3k_ln_modulate(h3k_dtype dtype, int32_t n, int32_t D, float eps,
                           const void* x, int64_t ldx, const float* shift, const float* scale,
                           void* out, int64_t ldo, hipStream_t stream);

/* Epilogues of h3k_linear. z = x W^T (times the per-row weight scale for INT8) + bias. */
#define H3K_EPI_BIAS            0  /* y = z                          */
#define H3K_EPI_GELU            1  /* y = GELU_tanh(z)               */
#define H3K_EPI_GATED_RESIDUAL  2  /* y = residual + gate * z        */

/* y = epilogue(x[m, k] W[n, k]^T ...).  x, bias, residual, y in act_dtype; W in
 * weight_dtype (== act_dtype, or INT8 with BF16 act, w_scale [n] fp32);
 * gate [n] fp32.  Output columns j < split_col go to y[i*ldy + j]; columns
 * j >= split_col go transposed to yt[(j - split_col)*ldyt + i] (pass
 * split_col = n when nothing is transposed).  The transposed part supports
 * only H3K_EPI_BIAS.  k must be a multiple of 64 (BF16) or 16 (F32).
 * Row pitches ldx, ldw, ldr, ldy, ldyt in elements; y must not overlap x or W. */
h3k_status h3k_linear(h3k_dtype act_dtype, h3k_dtype weight_dtype, int64_t m, int64_t n, int64_t k,
                      const void* x, int64_t ldx, const void* w, int64_t ldw, const float* w_scale,
                      const void* bias, int32_t epilogue, const void* residual, int64_t ldr,
                      const float* gate, void* y, int64_t ldy, void* yt, int64_t ldyt,
                      int64_t split_col, hipStream_t stream);

/* Both operands int8 (the row-quantised FC2 of [H3-review]'s speed/quality section):
 *   z[i, j] = x_scale[i] * w_scale[j] * sum_k xq[i, k] wq[j, k]   (int32 sum, exact;
 *             converted to fp32 once, then the two scale products in fp32)
 *   y = epilogue(z + bias) as for h3k_linear (H3K_EPI_*), row-major only.
 * xq [m, ldx] and wq [n, ldw] int8 with x_scale [m], w_scale [n] fp32 (e.g. from
 * h3k_quantize_weights_int8 on the activations and on the weights); bias [n],
 * residual [m, ldr] and y [m, ldy] BF16; gate [n] fp32.  k a multiple of 128 and
 * k <= 2^17 (the int32 sum cannot overflow), ldx and ldw multiples of 16,
 * n a multiple of 8.  y must not overlap the inputs. */
h3k_status h3k_linear_int8(int64_t m, int64_t n, int64_t k, const int8_t* xq, int64_t ldx, const float* x_scale,
                           const int8_t* wq, int64_t ldw, const float* w_scale, const void* bias,
                           int32_t epilogue, const void* residual, int64_t ldr, const float* gate,
                           void* y, int64_t ldy, hipStream_t stream);

/* Group-wise int8 weights with BF16 activations (the group-quantised int8 MLP of
 * [H3-review]'s speed/quality section):
 *   z[i, j] = sum_k x[i, k] * bf16(wq[j, k] * w_scale[j, k / group])
 *   y = epilogue(z + bias) as for h3k_linear (H3K_EPI_*), row-major only.
 * Each weight is dequantised in fp32 and rounded to bf16 once, on its way to
 * the bf16 matrix cores; the sum is fp32.  x [m, ldx], bias [n], residual
 * [m, ldr] and y [m, ldy] BF16; wq [n, ldw] int8 with w_scale [n, k/group] fp32
 * (e.g. from h3k_quantize_weights_int8_groups); gate [n] fp32.  group in
 * {32, 64, 128}; k a multiple of 64 and of group; n a multiple of 8; ldx a
 * multiple of 8 and ldw of 16.  y must not overlap the inputs. */
h3k_status h3k_linear_int8_groups(int64_t m, int64_t n, int64_t k, int32_t group, const void* x, int64_t ldx,
                                  const int8_t* wq, int64_t ldw, const float* w_scale, const void* bias,
                                  int32_t epilogue, const void* residual, int64_t ldr, const float* gate, void* y,
                                  int64_t ldy, hipStream_t stream);

/* Token reduction ([H3-review] knob list): xm[m] = (x[2m] + x[2m+1]) / 2 for
 * m < n_tokens/2, in fp32, rounded once to dtype.  x [n_tokens, ldx], xm
 * [n_tokens/2, ldxm] in dtype (F32 or BF16); n_tokens even; D, ldx and ldxm
 * multiples of 8.  xm must not overlap x. */
h3k_status h3k_token_merge(h3k_dtype dtype, int64_t n_tokens, int64_t D, const void* x, int64_t ldx, void* xm,
                           int64_t ldxm, hipStream_t stream);

/* The restore after the reduced layers:
 *   out[2m+j] = entry[2m+j] + (xm[m] - merge(entry)[m]),  j = 0, 1,
 * with merge(entry) recomputed exactly as h3k_token_merge rounds it, so an xm
 * equal to h3k_token_merge(entry) gives back entry bit for bit.  entry, out
 * [n_tokens, ld] and xm [n_tokens/2, ldxm] in dtype; out may be entry itself
 * (with ldo == ld_entry) but must not otherwise overlap the inputs. */
h3k_status h3k_token_unmerge(h3k_dtype dtype, int64_t n_tokens, int64_t D, const void* entry, int64_t ld_entry,
                             const void* xm, int64_t ldxm, void* out, int64_t ldo, hipStream_t stream);

/* 3D rotary position embedding, in place, of x [n_tokens, ldx] BF16 whose first
 * `cols` columns are heads of head_dim (e.g. the q and k columns of a QKV
 * output).  Row n is the token at (t, h, w) = (n / (H W), (n / W) % H, n % W) of
 * the grid frames x height x width; half_spatial = 1 halves h and w ([H3-review],
 * note on native-256 RoPE: spatial coordinates halved on 256 square canvases).
 * Each head is cut into a time, a height and a width slice of d/4, 3d/8, 3d/8
 * dimensions, and the pair (2i, 2i+1) of the slice of axis a turns by
 * pos_a * 10000^(-2i / d_a):  (x, y) -> (x cos - y sin, x sin + y cos).
 * head_dim a multiple of 16 (<= 256), cols a multiple of head_dim, ldx >= cols
 * and a multiple of 4, frames * height * width = n_tokens <= 2^24
 * (H3K_ERR_UNSUPPORTED beyond). */
h3k_status h3k_rope_3d(int64_t n_tokens, int64_t cols, int32_t head_dim, int32_t frames, int32_t height,
                       int32_t width, int32_t half_spatial, void* x, int64_t ldx, hipStream_t stream);

/* o[n, H*d] = per head softmax(q k^T / sqrt(d)) v, non-causal, no positional
 * terms; q [n, ldq], k [n, ldk] row-major (head j = columns j*d..j*d+d-1), v given
 * transposed as vt [H*d, ldvt] with ldvt >= n rounded up to 8.  dtype F32 or BF16;
 * d in {64, 128}.  Full self-attention over all tokens ([H3-memory] technique 2).
 * q_prescaled = 1 (BF16 only): q is given already multiplied by log2(e)/sqrt(d),
 * the layout the block's QKV projection writes (its epilogue folds the softmax
 * scale of the base-2 exponentials into q, with the one rounding it makes
 * anyway); the result is the same softmax.  0: q as above. */
h3k_status h3k_attention(h3k_dtype dtype, int32_t n, int32_t n_heads, int32_t head_dim,
                         const void* q, int64_t ldq, const void* k, int64_t ldk,
                         const void* vt, int64_t ldvt, void* o, int64_t ldo, int32_t q_prescaled,
                         hipStream_t stream);

/* ---- profiler ------------------------------------------------------------- */
/* capacity: max kernel launches recorded between resets (events are created here). */
h3k_status h3k_profiler_create(int32_t capacity, h3k_profiler** out /* host */);
h3k_status h3k_profiler_destroy(h3k_profiler* p);
h3k_status h3k_profiler_reset(h3k_profiler* p);
/* Waits for the recorded events, then reports the summed GPU time (ms) and the
 * launch count of one kernel kind since the last reset (host outs).  Returns
 * H3K_ERR_SHAPE if more launches were made than the capacity. */
h3k_status h3k_profiler_read(h3k_profiler* p, int32_t kernel_kind, double* total_ms, int32_t* launches);

/* ---- device ------------------------------------------------------------- */
/* The GPU a measurement ran on ([H3-memory], "verify it yourself": figures are
 * taken on the machine at hand), from the HIP device properties of `device`,
 * so that a harness can derive a peak rate from the compute units and the
 * clock and set it beside the published one (host struct). */
typedef struct h3k_device_info {
  int32_t  compute_units;      /* CUs                                       */
  int32_t  peak_clock_khz;     /* peak shader clock                         */
  int32_t  lds_bytes_per_cu;   /* LDS a workgroup can use                   */
  int32_t  wavefront_size;     /* lanes per wave                            */
  uint64_t hbm_bytes;          /* device memory                             */
  char     arch[64];           /* architecture name, NUL-terminated         */
} h3k_device_info;
/* Fills *out for device `device` (0 .. count-1).  H3K_ERR_NULL for a NULL out,
 * H3K_ERR_HIP if the runtime has no such device (out untouched).  Enqueues nothing. */
h3k_status h3k_get_device_info(int32_t device, h3k_device_info* out /* host */);

#ifdef __cplusplus
}
#endif
#endif /* H3K_H */
