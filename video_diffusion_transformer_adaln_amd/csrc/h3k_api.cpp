// C-ABI of the h3k library: argument validation, the activation lifetime
// planner, the launch sequence of one block and of a stack of blocks, and a
// hipEvent-based per-kernel profiler.  Host code only; all device work is in
// the .hip kernel files.
//
// Conventions (h3.c ComfyUI-plugin article, sections 3.1 / 4.2 / 5.2): integer
// status codes, no hidden global state (only a thread-local error message),
// an explicit profiler context, nothing returned that the caller must free.
// Invalid or unsupported arguments are rejected before any launch (h3-metal
// review, hard-constraint and unsupported-entry paragraphs).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "api_internal.hpp"
#include "h3k.h"
#include "kernels.hpp"

using namespace h3k;

namespace {

thread_local std::string g_err = "no error";

h3k_status fail(h3k_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define H3K_TRY(expr)                    \
  do {                                   \
    const h3k_status _s = (expr);        \
    if (_s != H3K_OK) return _s;         \
  } while (0)

constexpr uint64_t kAlign = 256;
constexpr int64_t kMaxOffset = (int64_t(1) << 31) - 1;   // 32-bit buffer offsets in the kernels
constexpr int64_t kMaxRopeTokens = int64_t(1) << 24;       // token coordinates through an exact fp32 quotient
constexpr int64_t kMaxInt8K = int64_t(1) << 17;           // int8 x int8 k-sums stay below 2^31 in int32

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }
int64_t esize(h3k_dtype d) { return d == H3K_F32 ? 4 : d == H3K_BF16 ? 2 : 1; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  uintptr_t lo = 0, hi = 0;   // [lo, hi)
  const char* name = "";
};
Range rng(const void* p, int64_t bytes, const char* name) {
  Range r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + (bytes > 0 ? (uintptr_t)bytes : 0);
  r.name = name;
  return r;
}
bool overlaps(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }
// bytes spanned by a [rows, cols] matrix with row pitch ld
int64_t span(int64_t rows, int64_t cols, int64_t ld, int64_t es) {
  return rows <= 0 ? 0 : ((rows - 1) * ld + cols) * es;
}

h3k_status check_device() {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(H3K_ERR_HIP, "no usable HIP device: %s", hipGetErrorString(e));
  return H3K_OK;
}

h3k_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(H3K_ERR_HIP, "launch of %s failed: %s", what, hipGetErrorString(e));
  return H3K_OK;
}

// ---------------------------------------------------------------- config
h3k_status validate_config(const h3k_dit_config* c) {
  if (!c) return fail(H3K_ERR_NULL, "config is NULL");
  if (c->act_dtype != H3K_F32 && c->act_dtype != H3K_BF16)
    return c->act_dtype == H3K_INT8 ? fail(H3K_ERR_UNSUPPORTED, "int8 activations are not supported")
                                    : fail(H3K_ERR_DTYPE, "unknown act_dtype %d", c->act_dtype);
  if (c->weight_dtype != H3K_F32 && c->weight_dtype != H3K_BF16 && c->weight_dtype != H3K_INT8)
    return fail(H3K_ERR_DTYPE, "unknown weight_dtype %d", c->weight_dtype);
  if (c->weight_dtype != c->act_dtype && !(c->weight_dtype == H3K_INT8 && c->act_dtype == H3K_BF16))
    return fail(H3K_ERR_UNSUPPORTED, "weight_dtype must equal act_dtype, or be INT8 with BF16 activations");
  if (c->n_tokens < 1 || c->hidden < 1 || c->n_heads < 1 || c->head_dim < 1 || c->mlp_hidden < 1 || c->cond_dim < 1)
    return fail(H3K_ERR_SHAPE, "all sizes must be >= 1 (N=%d D=%d H=%d d=%d F=%d C=%d)", c->n_tokens, c->hidden,
                c->n_heads, c->head_dim, c->mlp_hidden, c->cond_dim);
  if ((int64_t)c->n_heads * c->head_dim != c->hidden)
    return fail(H3K_ERR_SHAPE, "hidden %d != n_heads %d * head_dim %d", c->hidden, c->n_heads, c->head_dim);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(H3K_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", c->head_dim);
  if (c->hidden > 8192) return fail(H3K_ERR_UNSUPPORTED, "hidden %d > 8192", c->hidden);
  if (c->mlp_hidden % 64 != 0) return fail(H3K_ERR_UNSUPPORTED, "mlp_hidden %d not a multiple of 64", c->mlp_hidden);
  if (c->cond_dim % 8 != 0 || c->cond_dim > 8192)
    return fail(H3K_ERR_UNSUPPORTED, "cond_dim %d must be a multiple of 8 and <= 8192", c->cond_dim);
  if (!(c->ln_eps > 0.0f) || !(c->ln_eps < 1.0f)) return fail(H3K_ERR_SHAPE, "ln_eps must be in (0, 1)");
  if (c->int8_fc2_rows != 0 && c->int8_fc2_rows != 1) return fail(H3K_ERR_SHAPE, "int8_fc2_rows must be 0 or 1");
  if (c->int8_fc2_rows &&
      (c->weight_dtype != H3K_INT8 || c->act_dtype != H3K_BF16 || c->mlp_hidden % 128 != 0))
    return fail(H3K_ERR_UNSUPPORTED, "int8_fc2_rows needs INT8 weights, BF16 activations and mlp_hidden a multiple of 128");
  if (c->int8_fc2_rows && c->mlp_hidden > kMaxInt8K)   // |sum| <= k * 127^2 must fit the int32 accumulator
    return fail(H3K_ERR_UNSUPPORTED, "int8_fc2_rows needs mlp_hidden <= 2^17 (int32 accumulation), got %d",
                c->mlp_hidden);
  const int g = c->int8_mlp_group;
  if (g != 0 && g != 32 && g != 64 && g != 128) return fail(H3K_ERR_SHAPE, "int8_mlp_group must be 0, 32, 64 or 128");
  if (g && (c->weight_dtype != H3K_INT8 || c->act_dtype != H3K_BF16))
    return fail(H3K_ERR_UNSUPPORTED, "int8_mlp_group needs INT8 weights and BF16 activations");
  if (g && (c->hidden % g || c->mlp_hidden % g))
    return fail(H3K_ERR_SHAPE, "hidden and mlp_hidden must be multiples of int8_mlp_group %d", g);
  if (g && c->int8_fc2_rows)
    return fail(H3K_ERR_UNSUPPORTED, "int8_mlp_group and int8_fc2_rows cannot be combined (FC2 needs channel scales)");
  const bool rope = c->rope_frames || c->rope_height || c->rope_width;
  if (c->rope_half_spatial != 0 && c->rope_half_spatial != 1) return fail(H3K_ERR_SHAPE, "rope_half_spatial must be 0 or 1");
  if (rope) {
    if (c->rope_frames < 1 || c->rope_height < 1 || c->rope_width < 1 ||
        (int64_t)c->rope_frames * c->rope_height * c->rope_width != c->n_tokens)
      return fail(H3K_ERR_SHAPE, "RoPE grid %d x %d x %d does not hold the %d tokens", c->rope_frames, c->rope_height,
                  c->rope_width, c->n_tokens);
    if (c->act_dtype != H3K_BF16) return fail(H3K_ERR_UNSUPPORTED, "RoPE needs BF16 activations");
    if (c->n_tokens > kMaxRopeTokens) return fail(H3K_ERR_UNSUPPORTED, "RoPE supports at most 2^24 tokens");
  } else if (c->rope_half_spatial) {
    return fail(H3K_ERR_SHAPE, "rope_half_spatial without a RoPE grid");
  }
  const int tf = c->token_reduction_first, tl = c->token_reduction_last;
  if (tf < 0 || tl < 0 || (tl != 0 && tl < tf))
    return fail(H3K_ERR_SHAPE, "token reduction range [%d, %d) is not a layer range", tf, tl);
  if (tl > tf) {
    if (c->n_tokens % 2) return fail(H3K_ERR_SHAPE, "token reduction needs an even token count (got %d)", c->n_tokens);
    if (rope) return fail(H3K_ERR_UNSUPPORTED, "token reduction and RoPE cannot be combined");
  }
  const int64_t eb = esize(c->act_dtype);
  const int64_t rows = (int64_t)c->n_tokens + 256;
  const int64_t widest = std::max<int64_t>(2 * (int64_t)c->hidden, c->mlp_hidden);
  if (rows * widest * eb > kMaxOffset || ((int64_t)c->mlp_hidden + 256) * c->hidden * eb > kMaxOffset ||
      (3 * (int64_t)c->hidden + 256) * c->hidden * eb > kMaxOffset)
    return fail(H3K_ERR_UNSUPPORTED, "an operand exceeds 2 GiB (32-bit offsets in the kernels)");
  return H3K_OK;
}

bool alias_enabled(const h3k_dit_config* c) {
  const char* env = std::getenv("H3K_DISABLE_ACTIVATION_ALIAS");
  if (env && std::strcmp(env, "1") == 0) return false;
  return c->alias_activations != 0;
}

// ---------------------------------------------------------------- planner
// Kernel steps of one block: 0 AdaLN, 1 LN, 2 QKV, 3 attention, 4 out-proj,
// 5 LN, 6 MLP up, 7 row quantiser of u (int8_fc2_rows only), 8 MLP down.  A tensor is live from the step that writes it
// to the last step that reads it.  With aliasing, each tensor is placed
// first-fit (lowest 256-aligned offset) among the already placed tensors
// whose live ranges intersect its own, in a fixed order; without aliasing,
// each gets its own region.  The plan depends only on the config, so it is
// deterministic, and no kernel reads workspace bytes it did not write first.
// Token reduction keeps the merged stream ([N/2, D] in act_dtype) after the
// block's tensors, at workspace_bytes - reduction_bytes.
uint64_t reduction_bytes(const h3k_dit_config* c) {
  if (c->token_reduction_last <= c->token_reduction_first) return 0;
  return align_up((uint64_t)(c->n_tokens / 2) * c->hidden * esize(c->act_dtype), kAlign);
}

// Scratch for the partial results of split tails, by the launchers' rules at
// the 256 compute units of MI355X (on another CU count the launchers cap
// their split ways by this size): the fp32 partial tiles of k-split tail
// tiles of the bf16 out-projection, MLP up and MLP down GEMMs
// (tail_split_ways), and the partial results of the key-split last round of
// the bf16 attention (attn_split_ways).  The steps never overlap, so one
// region serves all.  With token reduction the reduced blocks use the same
// region, so it covers both token counts.  Placed after the block's tensors
// (before the merged stream).
constexpr int64_t kPlanCus = 256;
uint64_t split_bytes_for(const h3k_dit_config* c, int64_t N) {
  const int64_t D = c->hidden, F = c->mlp_hidden, H = c->n_heads;
  int64_t need = 0;
  if (c->weight_dtype == H3K_BF16 || c->weight_dtype == H3K_INT8) {   // bf16 or staged int8 weights
    const int64_t tm = (N + 255) / 256;
    const int64_t nk[3][2] = {{D, D}, {F, D}, {D, F}};   // (n, k) of out, up, down
    for (int i = 0; i < 3; ++i) {
      if (i == 2 && c->int8_fc2_rows) continue;            // int8 x int8: not split
      const int64_t tiles = tm * ((nk[i][0] + 255) / 256);
      const int S = tail_split_ways(tiles, nk[i][1] / 64, kPlanCus, kPlanCus);
      if (S) need = std::max(need, (tiles % kPlanCus) * S * kPartTileBytes);
    }
  }
  if (c->head_dim == 128) {
    int S = 0;
    const int nw = attn_shape128(N, H, kPlanCus, INT64_MAX / 4, &S);
    const int64_t slots = kPlanCus * (nw == 4 ? 2 : 1);
    const int64_t blocks = (N + nw * 32 - 1) / (nw * 32) * H;
    if (S) need = std::max(need, (blocks % slots) * S * attn_unit_bytes(nw));
  }
  return (uint64_t)need;
}
uint64_t split_bytes(const h3k_dit_config* c) {
  if (c->act_dtype != H3K_BF16) return 0;
  uint64_t b = split_bytes_for(c, c->n_tokens);
  if (c->token_reduction_last > c->token_reduction_first) b = std::max(b, split_bytes_for(c, c->n_tokens / 2));
  return align_up(b, kAlign);
}
constexpr int kSplitSteps[4] = {3, 4, 6, 8};   // attention, out, up and down

// Staging buffer of the int8-weight projections (bf16 activations): each
// int8 weight matrix is widened to bf16 there right before its GEMM, which
// then runs as a bf16 GEMM with the channel scale in its epilogue.  Sized for
// the largest of the block's projection weights (the int8 x int8 FC2 reads
// its int8 weights directly).  Placed after the k-split scratch.
uint64_t stage_bytes(const h3k_dit_config* c) {
  if (c->weight_dtype != H3K_INT8 || c->act_dtype != H3K_BF16) return 0;
  const uint64_t D = c->hidden, F = c->mlp_hidden;
  return align_up(std::max(3 * D * D, D * F) * 2, kAlign);
}
constexpr int kGemmSteps[4] = {2, 4, 6, 8};  // QKV, out, up, down

void make_plan(const h3k_dit_config* c, bool alias, h3k_dit_plan_info* P) {
  std::memset(P, 0, sizeof(*P));
  const uint64_t N = c->n_tokens, D = c->hidden, F = c->mlp_hidden, eb = esize(c->act_dtype);
  const uint64_t vt_pitch = align_up(N, 8);
  const uint64_t qk_bytes = align_up(N * 2 * D * eb, kAlign);
  uint64_t bytes[H3K_T_COUNT];
  bytes[H3K_T_MOD] = 6 * D * 4;
  bytes[H3K_T_H] = N * D * eb;
  bytes[H3K_T_QKV] = qk_bytes + D * vt_pitch * eb;
  bytes[H3K_T_O] = N * D * eb;
  bytes[H3K_T_X1] = N * D * eb;
  bytes[H3K_T_H2] = N * D * eb;
  bytes[H3K_T_U] = N * F * eb;
  const bool q8 = c->int8_fc2_rows != 0;
  bytes[H3K_T_UQ] = q8 ? N * F : 0;
  bytes[H3K_T_US] = q8 ? N * 4 : 0;
  const int first[H3K_T_COUNT] = {0, 1, 2, 3, 4, 5, 6, 7, 7};
  const int last[H3K_T_COUNT] = {8, 2, 3, 4, 8, 6, q8 ? 7 : 8, 8, 8};
  uint64_t off[H3K_T_COUNT];
  uint64_t unaliased = 0;
  for (int t = 0; t < H3K_T_COUNT; ++t) unaliased += align_up(bytes[t], kAlign);
  if (!alias) {
    uint64_t cur = 0;
    for (int t = 0; t < H3K_T_COUNT; ++t) { off[t] = cur; cur += align_up(bytes[t], kAlign); }
  } else {
    for (int t = 0; t < H3K_T_COUNT; ++t) {
      std::vector<std::pair<uint64_t, uint64_t>> busy;   // [lo, hi) of conflicting placed tensors
      for (int u = 0; u < t; ++u)
        if (first[u] <= last[t] && first[t] <= last[u]) busy.push_back({off[u], off[u] + align_up(bytes[u], kAlign)});
      std::sort(busy.begin(), busy.end());
      uint64_t cand = 0;
      const uint64_t need = align_up(bytes[t], kAlign);
      for (const auto& b : busy) {
        if (cand + need <= b.first) break;
        cand = std::max(cand, b.second);
      }
      off[t] = cand;
    }
  }
  const uint64_t sp = split_bytes(c), st = stage_bytes(c);
  uint64_t ws = 0, peak = 0;
  for (int t = 0; t < H3K_T_COUNT; ++t) ws = std::max(ws, off[t] + align_up(bytes[t], kAlign));
  for (int s = 0; s <= 8; ++s) {
    uint64_t live = 0;
    for (int t = 0; t < H3K_T_COUNT; ++t)
      if (first[t] <= s && s <= last[t]) live += align_up(bytes[t], kAlign);
    for (int k : kSplitSteps)
      if (s == k) live += sp;
    for (int k : kGemmSteps)
      if (s == k) live += st;
    peak = std::max(peak, live);
  }
  for (int t = 0; t < H3K_T_COUNT; ++t) {
    P->offset[t] = off[t];
    P->bytes[t] = bytes[t];
    P->first_step[t] = first[t];
    P->last_step[t] = last[t];
  }
  P->qkv_vt_offset = off[H3K_T_QKV] + qk_bytes;
  P->vt_pitch = (int64_t)vt_pitch;
  const uint64_t red = reduction_bytes(c);
  P->part_offset = ws;
  P->part_bytes = sp;
  P->wstage_offset = ws + sp;
  P->wstage_bytes = st;
  P->workspace_bytes = ws + sp + st + red;
  P->peak_live_bytes = peak + red;
  P->unaliased_bytes = unaliased + sp + st + red;
  P->alias_activations = alias ? 1 : 0;
}

}  // namespace

// ---------------------------------------------------------------- profiler
struct h3k_profiler {
  int capacity = 0;
  std::vector<hipEvent_t> events;
  int n_events = 0;
  struct Interval { int before, after, kind; };
  std::vector<Interval> intervals;
  bool overflow = false;
};

namespace {

// Records a start event; each `done(kind)` records the event that closes the
// interval of the kernel just enqueued.
struct Recorder {
  h3k_profiler* p;
  hipStream_t s;
  int prev = -1;
  bool on = false;
  Recorder(h3k_profiler* prof, hipStream_t stream) : p(prof), s(stream) {
    if (p && p->n_events < (int)p->events.size()) {
      prev = p->n_events++;
      on = hipEventRecord(p->events[prev], s) == hipSuccess;
    } else if (p) {
      p->overflow = true;
    }
  }
  void done(int kind) {
    if (!on) return;
    if (p->n_events >= (int)p->events.size()) { p->overflow = true; on = false; return; }
    const int e = p->n_events++;
    if (hipEventRecord(p->events[e], s) != hipSuccess) { on = false; return; }
    p->intervals.push_back({prev, e, kind});
    prev = e;
  }
};

h3k_status validate_weights(const h3k_dit_config* c, const h3k_dit_block_weights* w, int idx) {
  if (!w) return fail(H3K_ERR_NULL, "weights of block %d are NULL", idx);
  const void* req[] = {w->w_ada, w->w_qkv, w->w_out, w->w_up, w->w_down};
  const char* names[] = {"w_ada", "w_qkv", "w_out", "w_up", "w_down"};
  for (int i = 0; i < 5; ++i)
    if (!req[i]) return fail(H3K_ERR_NULL, "block %d: %s is NULL", idx, names[i]);
  const bool w8 = c->weight_dtype == H3K_INT8;
  const float* sc[] = {w->s_qkv, w->s_out, w->s_up, w->s_down};
  for (int i = 0; i < 4; ++i) {
    if (w8 && !sc[i]) return fail(H3K_ERR_NULL, "block %d: int8 weights need scale %s", idx, names[i + 1]);
    if (sc[i] && !aligned(sc[i], 16)) return fail(H3K_ERR_ALIGN, "block %d: scales of %s not 16-byte aligned", idx, names[i + 1]);
  }
  const void* all[] = {w->w_ada, w->b_ada, w->w_qkv, w->b_qkv, w->w_out, w->b_out, w->w_up, w->b_up, w->w_down, w->b_down};
  for (const void* p : all)
    if (p && !aligned(p, 16)) return fail(H3K_ERR_ALIGN, "block %d: a weight or bias pointer is not 16-byte aligned", idx);
  return H3K_OK;
}

void weight_ranges(const h3k_dit_config* c, const h3k_dit_block_weights* w, std::vector<Range>& out) {
  const int64_t D = c->hidden, F = c->mlp_hidden, C = c->cond_dim;
  const int64_t ea = esize(c->act_dtype), ew = esize(c->weight_dtype);
  out.push_back(rng(w->w_ada, 6 * D * C * ea, "w_ada"));
  out.push_back(rng(w->b_ada, 6 * D * ea, "b_ada"));
  out.push_back(rng(w->w_qkv, 3 * D * D * ew, "w_qkv"));
  out.push_back(rng(w->b_qkv, 3 * D * ea, "b_qkv"));
  out.push_back(rng(w->s_qkv, 3 * D * 4, "s_qkv"));
  out.push_back(rng(w->w_out, D * D * ew, "w_out"));
  out.push_back(rng(w->b_out, D * ea, "b_out"));
  out.push_back(rng(w->s_out, D * 4, "s_out"));
  out.push_back(rng(w->w_up, F * D * ew, "w_up"));
  out.push_back(rng(w->b_up, F * ea, "b_up"));
  const int64_t g = c->int8_mlp_group;
  out.push_back(rng(w->s_up, F * (g ? D / g : 1) * 4, "s_up"));
  out.push_back(rng(w->w_down, D * F * ew, "w_down"));
  out.push_back(rng(w->b_down, D * ea, "b_down"));
  out.push_back(rng(w->s_down, D * (g ? F / g : 1) * 4, "s_down"));
}

h3k_status validate_forward(const h3k_dit_config* c, const h3k_dit_block_weights* blocks, int32_t n_blocks,
                            const void* x, const void* cond, void* out, void* ws, uint64_t ws_bytes,
                            h3k_dit_plan_info* plan) {
  H3K_TRY(validate_config(c));
  if (!blocks) return fail(H3K_ERR_NULL, "weights array is NULL");
  if (n_blocks < 1) return fail(H3K_ERR_SHAPE, "n_blocks %d < 1", n_blocks);
  if (!x || !cond || !out || !ws) return fail(H3K_ERR_NULL, "x, c, out and workspace must be non-NULL");
  if (!aligned(x, 16) || !aligned(cond, 16) || !aligned(out, 16))
    return fail(H3K_ERR_ALIGN, "x, c and out must be 16-byte aligned");
  if (!aligned(ws, kAlign)) return fail(H3K_ERR_ALIGN, "workspace must be 256-byte aligned");
  for (int i = 0; i < n_blocks; ++i) H3K_TRY(validate_weights(c, &blocks[i], i));
  make_plan(c, alias_enabled(c), plan);
  if (ws_bytes < plan->workspace_bytes)
    return fail(H3K_ERR_WORKSPACE, "workspace %llu bytes < %llu required", (unsigned long long)ws_bytes,
                (unsigned long long)plan->workspace_bytes);
  const int64_t ea = esize(c->act_dtype);
  const int64_t act = (int64_t)c->n_tokens * c->hidden * ea;
  const Range ro = rng(out, act, "out");
  std::vector<Range> ins = {rng(x, act, "x"), rng(cond, (int64_t)c->cond_dim * ea, "c"),
                            rng(ws, (int64_t)plan->workspace_bytes, "workspace")};
  for (int i = 0; i < n_blocks; ++i) weight_ranges(c, &blocks[i], ins);
  for (const Range& r : ins)
    if (overlaps(ro, r)) return fail(H3K_ERR_OVERLAP, "out overlaps %s", r.name);
  const Range rw = rng(ws, (int64_t)plan->workspace_bytes, "workspace");
  for (size_t i = 0; i < ins.size(); ++i)
    if (std::strcmp(ins[i].name, "workspace") != 0 && overlaps(rw, ins[i]))
      return fail(H3K_ERR_OVERLAP, "workspace overlaps %s", ins[i].name);
  return H3K_OK;
}

// Enqueue the eight kernels of one block (nine with int8_fc2_rows).  x may
// equal out (stack in place: x is last read by the out-projection, out is
// first written by MLP down).
// `part`/`part_bytes`: the scratch of split tails (see split_bytes); null / 0:
// no split.  `kernels` counts the kernels enqueued, `splits` the kernels
// (GEMMs, attention) whose last wave was split.
h3k_status run_block(const h3k_dit_config* c, const h3k_dit_plan_info* P, const h3k_dit_block_weights* w,
                     const void* x, const void* cond, void* out, char* ws, float* part, uint64_t part_bytes,
                     void* wstage, uint64_t wstage_bytes, hipStream_t s, Recorder& rec, int& kernels, int& splits) {
  // one GEMM: its kernels (one, or two when its tail tiles are split; one more
  // when int8 weights are widened into the staging buffer first) counted
  auto gemm = [&](LinearArgs& L, const char* what, bool may_split) -> h3k_status {
    if (may_split) { L.part = part; L.part_bytes = (int64_t)part_bytes; }
    if (L.weight == kINT8 && L.act == kBF16) { L.wstage = wstage; L.wstage_bytes = (int64_t)wstage_bytes; }
    int nk = 0;
    H3K_TRY(launched(launch_linear(L, s, &nk), what));
    kernels += nk;
    splits += nk - 1 - (L.wstage != nullptr && L.wstage_bytes >= L.n * L.k * 2);
    return H3K_OK;
  };
  const DType act = (DType)c->act_dtype;
  const DType wt = (DType)c->weight_dtype;
  const int N = c->n_tokens, D = c->hidden, F = c->mlp_hidden;
  const int64_t eb = esize(c->act_dtype);
  float* mod = reinterpret_cast<float*>(ws + P->offset[H3K_T_MOD]);
  char* h = ws + P->offset[H3K_T_H];
  char* qkv = ws + P->offset[H3K_T_QKV];
  char* vt = ws + P->qkv_vt_offset;
  char* o = ws + P->offset[H3K_T_O];
  char* x1 = ws + P->offset[H3K_T_X1];
  char* h2 = ws + P->offset[H3K_T_H2];
  char* u = ws + P->offset[H3K_T_U];
  const float *shift_a = mod, *scale_a = mod + D, *gate_a = mod + 2 * D;
  const float *shift_m = mod + 3 * D, *scale_m = mod + 4 * D, *gate_m = mod + 5 * D;

  H3K_TRY(launched(launch_adaln_gemv(act, 6 * D, c->cond_dim, w->w_ada, w->b_ada, cond, mod, s), "AdaLN GEMV"));
  rec.done(H3K_K_ADALN);
  H3K_TRY(launched(launch_ln_modulate(act, N, D, c->ln_eps, x, D, shift_a, scale_a, h, D, s), "LayerNorm 1"));
  rec.done(H3K_K_LN_MOD);
  kernels += 2;

  LinearArgs L{};
  L.act = act; L.weight = wt;
  L.m = N; L.n = 3 * D; L.k = D;
  L.x = h; L.ldx = D; L.w = w->w_qkv; L.ldw = D; L.w_scale = w->s_qkv; L.bias = w->b_qkv;
  L.epi = kEpiBias; L.y = qkv; L.ldy = 2 * D; L.yt = vt; L.ldyt = P->vt_pitch; L.split_col = 2 * D;
  if (c->rope_frames) {                        // q and k (the row-major part) rotated after the bias
    L.epi = kEpiBiasRope;
    L.rope_hd = c->head_dim; L.rope_h = c->rope_height; L.rope_w = c->rope_width;
    L.rope_spatial = c->rope_half_spatial ? 0.5f : 1.0f;
  }
  // bf16: q is stored times log2(e)/sqrt(d), the softmax scale in the base-2
  // exponent the attention kernel takes, so its scores need no rescaling
  const bool q_pre = act == kBF16;
  if (q_pre) {
    L.scale_cols = D;
    L.col_scale = 1.4426950408889634f / std::sqrt((float)c->head_dim);
  }
  H3K_TRY(gemm(L, "QKV projection", false));
  rec.done(H3K_K_QKV);

  AttentionArgs A{};
  A.dt = act; A.n = N; A.n_heads = c->n_heads; A.head_dim = c->head_dim;
  A.q = qkv; A.ldq = 2 * D; A.k = qkv + D * eb; A.ldk = 2 * D; A.vt = vt; A.ldvt = P->vt_pitch;
  A.o = o; A.ldo = D; A.q_prescaled = q_pre;
  A.part = part;
  A.part_bytes = (int64_t)part_bytes;
  {
    int nk = 0;
    H3K_TRY(launched(launch_attention(A, s, &nk), "attention"));
    kernels += nk;
    splits += nk - 1;
  }
  rec.done(H3K_K_ATTENTION);

  L = LinearArgs{};
  L.act = act; L.weight = wt;
  L.m = N; L.n = D; L.k = D;
  L.x = o; L.ldx = D; L.w = w->w_out; L.ldw = D; L.w_scale = w->s_out; L.bias = w->b_out;
  L.epi = kEpiGatedResidual; L.residual = x; L.ldr = D; L.gate = gate_a;
  L.y = x1; L.ldy = D; L.split_col = D;
  H3K_TRY(gemm(L, "out projection", true));
  rec.done(H3K_K_OUT);

  H3K_TRY(launched(launch_ln_modulate(act, N, D, c->ln_eps, x1, D, shift_m, scale_m, h2, D, s), "LayerNorm 2"));
  rec.done(H3K_K_LN_MOD);
  ++kernels;

  L = LinearArgs{};
  L.act = act; L.weight = wt;
  L.m = N; L.n = F; L.k = D;
  L.x = h2; L.ldx = D; L.w = w->w_up; L.ldw = D; L.w_scale = w->s_up; L.bias = w->b_up;
  L.group = c->int8_mlp_group;
  L.epi = kEpiGelu; L.y = u; L.ldy = F; L.split_col = F;
  H3K_TRY(gemm(L, "MLP up", true));
  rec.done(H3K_K_UP);

  L = LinearArgs{};
  L.act = act; L.weight = wt;
  L.m = N; L.n = D; L.k = F;
  L.x = u; L.ldx = F; L.w = w->w_down; L.ldw = F; L.w_scale = w->s_down; L.bias = w->b_down;
  L.group = c->int8_mlp_group;
  if (c->int8_fc2_rows) {
    int8_t* uq = reinterpret_cast<int8_t*>(ws + P->offset[H3K_T_UQ]);
    float* us = reinterpret_cast<float*>(ws + P->offset[H3K_T_US]);
    H3K_TRY(launched(launch_quantize_int8(act, u, N, F, uq, us, s), "row quantiser of u"));
    rec.done(H3K_K_ACT_QUANT);
    ++kernels;
    L.act = kINT8; L.x = uq; L.x_scale = us;
  }
  L.epi = kEpiGatedResidual; L.residual = x1; L.ldr = D; L.gate = gate_m;
  L.y = out; L.ldy = D; L.split_col = D;
  H3K_TRY(gemm(L, "MLP down", true));
  rec.done(H3K_K_DOWN);
  return H3K_OK;
}

h3k_status forward(const h3k_dit_config* cfg, const h3k_dit_block_weights* blocks, int32_t n_blocks, const void* x,
                   const void* c, void* out, void* workspace, uint64_t workspace_bytes, hipStream_t stream,
                   h3k_dit_stats* stats) {
  h3k_dit_plan_info plan;
  H3K_TRY(validate_forward(cfg, blocks, n_blocks, x, c, out, workspace, workspace_bytes, &plan));
  if (cfg->token_reduction_last > cfg->token_reduction_first && cfg->token_reduction_last > n_blocks)
    return fail(H3K_ERR_SHAPE, "token reduction range [%d, %d) beyond the %d blocks", cfg->token_reduction_first,
                cfg->token_reduction_last, n_blocks);
  H3K_TRY(check_device());
  const int tf = cfg->token_reduction_first, tl = cfg->token_reduction_last;
  const bool reduce = tl > tf;
  Recorder rec(stats ? stats->profiler : nullptr, stream);
  char* ws = static_cast<char*>(workspace);
  // the reduced layers run on the merged stream, in place, with the plan of a
  // config of N/2 tokens (it fits in the full plan's part of the workspace)
  h3k_dit_config half = *cfg;
  half.n_tokens = cfg->n_tokens / 2;
  half.token_reduction_first = half.token_reduction_last = 0;
  h3k_dit_plan_info plan_half;
  void* xm = nullptr;
  if (reduce) {
    make_plan(&half, plan.alias_activations != 0, &plan_half);
    xm = ws + plan.workspace_bytes - reduction_bytes(cfg);
  }
  const DType act = (DType)cfg->act_dtype;
  const int64_t N = cfg->n_tokens, D = cfg->hidden;
  // the k-split scratch of the full plan serves the reduced blocks too
  float* part = reinterpret_cast<float*>(ws + plan.part_offset);
  const char* nosplit = std::getenv("H3K_DISABLE_TAIL_SPLIT");
  const uint64_t part_bytes = (nosplit && std::strcmp(nosplit, "1") == 0) ? 0 : plan.part_bytes;
  void* wstage = ws + plan.wstage_offset;
  const char* nostage = std::getenv("H3K_DISABLE_WEIGHT_STAGING");
  const uint64_t wstage_bytes = (nostage && std::strcmp(nostage, "1") == 0) ? 0 : plan.wstage_bytes;
  int kernels = 0, splits = 0;
  for (int l = 0; l < n_blocks; ++l) {
    const void* src = l == 0 ? x : out;
    if (reduce && l == tf) {
      H3K_TRY(launched(launch_token_merge(act, N, D, src, D, xm, D, stream), "token merge"));
      rec.done(H3K_K_TOKEN_MERGE);
      ++kernels;
    }
    if (reduce && l >= tf && l < tl)
      H3K_TRY(run_block(&half, &plan_half, &blocks[l], xm, c, xm, ws, part, part_bytes, wstage, wstage_bytes, stream,
                        rec, kernels, splits));
    else
      H3K_TRY(run_block(cfg, &plan, &blocks[l], src, c, out, ws, part, part_bytes, wstage, wstage_bytes, stream, rec,
                        kernels, splits));
    if (reduce && l == tl - 1) {                // entry state: x if the range starts at block 0, else out
      H3K_TRY(launched(launch_token_unmerge(act, N, D, tf == 0 ? x : out, D, xm, D, out, D, stream),
                       "token unmerge"));
      rec.done(H3K_K_TOKEN_UNMERGE);
      ++kernels;
    }
  }
  if (stats) {
    stats->workspace_bytes = plan.workspace_bytes;
    stats->peak_live_bytes = plan.peak_live_bytes;
    stats->unaliased_bytes = plan.unaliased_bytes;
    stats->dispatches = kernels;
    stats->tail_splits = splits;
    stats->alias_activations = plan.alias_activations;
  }
  return H3K_OK;
}

}  // namespace

namespace h3k {

h3k_status api_fail(h3k_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

h3k_status api_forward(const h3k_dit_config* cfg, const h3k_dit_block_weights* blocks, int32_t n_blocks,
                       const void* x, const void* c, void* out, void* workspace, uint64_t workspace_bytes,
                       hipStream_t stream, h3k_dit_stats* stats) {
  return forward(cfg, blocks, n_blocks, x, c, out, workspace, workspace_bytes, stream, stats);
}

}  // namespace h3k

// ======================================================================== C ABI
extern "C" {

const char* h3k_last_error(void) { return g_err.c_str(); }

h3k_status h3k_dit_workspace_size(const h3k_dit_config* cfg, int32_t n_blocks, uint64_t* bytes_out) {
  H3K_TRY(validate_config(cfg));
  if (n_blocks < 1) return fail(H3K_ERR_SHAPE, "n_blocks %d < 1", n_blocks);
  if (!bytes_out) return fail(H3K_ERR_NULL, "bytes_out is NULL");
  h3k_dit_plan_info p;
  make_plan(cfg, alias_enabled(cfg), &p);
  *bytes_out = p.workspace_bytes;
  return H3K_OK;
}

h3k_status h3k_dit_plan(const h3k_dit_config* cfg, h3k_dit_plan_info* info_out) {
  H3K_TRY(validate_config(cfg));
  if (!info_out) return fail(H3K_ERR_NULL, "info_out is NULL");
  make_plan(cfg, alias_enabled(cfg), info_out);
  return H3K_OK;
}

h3k_status h3k_dit_block_forward(const h3k_dit_config* cfg, const h3k_dit_block_weights* weights, const void* x,
                                 const void* c, void* out, void* workspace, uint64_t workspace_bytes,
                                 hipStream_t stream, h3k_dit_stats* stats) {
  return forward(cfg, weights, 1, x, c, out, workspace, workspace_bytes, stream, stats);
}

h3k_status h3k_dit_stack_forward(const h3k_dit_config* cfg, const h3k_dit_block_weights* blocks, int32_t n_blocks,
                                 const void* x, const void* c, void* out, void* workspace, uint64_t workspace_bytes,
                                 hipStream_t stream, h3k_dit_stats* stats) {
  return forward(cfg, blocks, n_blocks, x, c, out, workspace, workspace_bytes, stream, stats);
}

h3k_status h3k_quantize_weights_int8(const void* w, h3k_dtype w_dtype, int64_t rows, int64_t cols, int8_t* q,
                                     float* scales, hipStream_t stream) {
  if (w_dtype != H3K_F32 && w_dtype != H3K_BF16)
    return fail(w_dtype == H3K_INT8 ? H3K_ERR_UNSUPPORTED : H3K_ERR_DTYPE, "w_dtype must be F32 or BF16");
  if (rows < 0 || cols < 1 || rows > 0x7fffffff || cols > (1 << 20))
    return fail(H3K_ERR_SHAPE, "rows %lld / cols %lld out of range", (long long)rows, (long long)cols);
  if (!w || !q || !scales) return fail(H3K_ERR_NULL, "w, q and scales must be non-NULL");
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(scales, 16))
    return fail(H3K_ERR_ALIGN, "w, q and scales must be 16-byte aligned");
  const Range rw = rng(w, rows * cols * esize(w_dtype), "w"), rq = rng(q, rows * cols, "q"),
              rs = rng(scales, rows * 4, "scales");
  if (overlaps(rq, rw) || overlaps(rs, rw) || overlaps(rq, rs))
    return fail(H3K_ERR_OVERLAP, "q, scales and w must not overlap");
  if (rows == 0) return H3K_OK;
  H3K_TRY(check_device());
  return launched(launch_quantize_int8((DType)w_dtype, w, rows, cols, q, scales, stream), "int8 quantiser");
}

h3k_status h3k_quantize_weights_int8_groups(const void* w, h3k_dtype w_dtype, int64_t rows, int64_t cols,
                                            int32_t group, int8_t* q, float* scales, hipStream_t stream) {
  if (w_dtype != H3K_F32 && w_dtype != H3K_BF16)
    return fail(w_dtype == H3K_INT8 ? H3K_ERR_UNSUPPORTED : H3K_ERR_DTYPE, "w_dtype must be F32 or BF16");
  if (group != 32 && group != 64 && group != 128) return fail(H3K_ERR_SHAPE, "group must be 32, 64 or 128 (got %d)", group);
  if (rows < 0 || cols < group || cols % group || rows > 0x7fffffff || cols > (1 << 20))
    return fail(H3K_ERR_SHAPE, "rows %lld / cols %lld out of range (cols a multiple of the group)", (long long)rows,
                (long long)cols);
  if (!w || !q || !scales) return fail(H3K_ERR_NULL, "w, q and scales must be non-NULL");
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(scales, 16))
    return fail(H3K_ERR_ALIGN, "w, q and scales must be 16-byte aligned");
  const Range rw = rng(w, rows * cols * esize(w_dtype), "w"), rq = rng(q, rows * cols, "q"),
              rs = rng(scales, rows * (cols / group) * 4, "scales");
  if (overlaps(rq, rw) || overlaps(rs, rw) || overlaps(rq, rs))
    return fail(H3K_ERR_OVERLAP, "q, scales and w must not overlap");
  if (rows == 0) return H3K_OK;
  H3K_TRY(check_device());
  return launched(launch_quantize_int8_groups((DType)w_dtype, w, rows, cols, group, q, scales, stream),
                  "int8 group quantiser");
}

h3k_status h3k_adaln_modulation(h3k_dtype dtype, int32_t rows, int32_t cols, const void* w, const void* b,
                                const void* c, float* mod, hipStream_t stream) {
  if (dtype != H3K_F32 && dtype != H3K_BF16) return fail(H3K_ERR_DTYPE, "dtype must be F32 or BF16");
  if (rows < 1 || cols < 8 || cols % 8 != 0 || cols > 8192)
    return fail(H3K_ERR_SHAPE, "rows >= 1, cols a multiple of 8 in [8, 8192] (got %d, %d)", rows, cols);
  if (!w || !c || !mod) return fail(H3K_ERR_NULL, "w, c and mod must be non-NULL");
  if (!aligned(w, 16) || !aligned(c, 16) || (b && !aligned(b, 16)) || !aligned(mod, 16))
    return fail(H3K_ERR_ALIGN, "pointers must be 16-byte aligned");
  const int64_t e = esize(dtype);
  const Range rm = rng(mod, (int64_t)rows * 4, "mod");
  if (overlaps(rm, rng(w, (int64_t)rows * cols * e, "w")) || overlaps(rm, rng(c, cols * e, "c")) ||
      overlaps(rm, rng(b, b ? rows * e : 0, "b")))
    return fail(H3K_ERR_OVERLAP, "mod overlaps an input");
  H3K_TRY(check_device());
  return launched(launch_adaln_gemv((DType)dtype, rows, cols, w, b, c, mod, stream), "AdaLN GEMV");
}

h3k_status h3k_ln_modulate(h3k_dtype dtype, int32_t n, int32_t D, float eps, const void* x, int64_t ldx,
                           const float* shift, const float* scale, void* out, int64_t ldo, hipStream_t stream) {
  if (dtype != H3K_F32 && dtype != H3K_BF16) return fail(H3K_ERR_DTYPE, "dtype must be F32 or BF16");
  const int vec = dtype == H3K_F32 ? 4 : 8;
  if (n < 0 || D < vec || D % vec != 0 || D > 8192 || ldx < D || ldo < D || ldx % vec || ldo % vec)
    return fail(H3K_ERR_SHAPE, "bad sizes n=%d D=%d ldx=%lld ldo=%lld", n, D, (long long)ldx, (long long)ldo);
  if (!(eps > 0.0f)) return fail(H3K_ERR_SHAPE, "eps must be > 0");
  if (!x || !shift || !scale || !out) return fail(H3K_ERR_NULL, "x, shift, scale and out must be non-NULL");
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(shift, 4) || !aligned(scale, 4))
    return fail(H3K_ERR_ALIGN, "x and out must be 16-byte aligned");
  const int64_t e = esize(dtype);
  const Range ro = rng(out, span(n, D, ldo, e), "out");
  if (overlaps(ro, rng(x, span(n, D, ldx, e), "x")) && out != x)
    return fail(H3K_ERR_OVERLAP, "out partially overlaps x");
  if (overlaps(ro, rng(shift, D * 4, "shift")) || overlaps(ro, rng(scale, D * 4, "scale")))
    return fail(H3K_ERR_OVERLAP, "out overlaps shift/scale");
  if (n == 0) return H3K_OK;
  H3K_TRY(check_device());
  return launched(launch_ln_modulate((DType)dtype, n, D, eps, x, ldx, shift, scale, out, ldo, stream),
                  "LayerNorm+modulation");
}

h3k_status h3k_linear(h3k_dtype act_dtype, h3k_dtype weight_dtype, int64_t m, int64_t n, int64_t k, const void* x,
                      int64_t ldx, const void* w, int64_t ldw, const float* w_scale, const void* bias,
                      int32_t epilogue, const void* residual, int64_t ldr, const float* gate, void* y, int64_t ldy,
                      void* yt, int64_t ldyt, int64_t split_col, hipStream_t stream) {
  if (act_dtype != H3K_F32 && act_dtype != H3K_BF16) return fail(H3K_ERR_DTYPE, "act_dtype must be F32 or BF16");
  if (weight_dtype != act_dtype && !(weight_dtype == H3K_INT8 && act_dtype == H3K_BF16))
    return fail(H3K_ERR_UNSUPPORTED, "weight_dtype must equal act_dtype, or be INT8 with BF16 activations");
  if (epilogue < H3K_EPI_BIAS || epilogue > H3K_EPI_GATED_RESIDUAL) return fail(H3K_ERR_SHAPE, "bad epilogue %d", epilogue);
  const int kq = act_dtype == H3K_F32 ? 16 : 64;
  if (m < 0 || n < 8 || n % 8 || k < kq || k % kq)
    return fail(H3K_ERR_SHAPE, "need m >= 0, n a multiple of 8, k a multiple of %d (m=%lld n=%lld k=%lld)", kq,
                (long long)m, (long long)n, (long long)k);
  if (split_col < 0 || split_col > n || split_col % 8)
    return fail(H3K_ERR_SHAPE, "split_col must be a multiple of 8 in [0, n]");
  if (ldx < k || ldw < k || ldx % 8 || ldw % (16 / esize(weight_dtype)) ||
      (split_col > 0 && (ldy < split_col || ldy % 8)))
    return fail(H3K_ERR_SHAPE, "bad row pitches");
  if (!x || !w || (split_col > 0 && !y)) return fail(H3K_ERR_NULL, "x, w and y must be non-NULL");
  if (weight_dtype == H3K_INT8 && !w_scale) return fail(H3K_ERR_NULL, "INT8 weights need w_scale");
  if (epilogue == H3K_EPI_GATED_RESIDUAL && (!residual || !gate || ldr < split_col || ldr % 8))
    return fail(H3K_ERR_NULL, "gated residual needs residual (ldr >= split_col, multiple of 8) and gate");
  if (split_col < n) {
    if (!yt || ldyt < m || ldyt % 8) return fail(H3K_ERR_SHAPE, "transposed part needs yt with ldyt >= m, multiple of 8");
    if (epilogue != H3K_EPI_BIAS) return fail(H3K_ERR_UNSUPPORTED, "transposed output supports only H3K_EPI_BIAS");
  }
  const void* al[] = {x, w, bias, residual, y, yt};
  for (const void* p : al)
    if (p && !aligned(p, 16)) return fail(H3K_ERR_ALIGN, "pointers must be 16-byte aligned");
  if ((w_scale && !aligned(w_scale, 16)) || (gate && !aligned(gate, 16)))
    return fail(H3K_ERR_ALIGN, "w_scale and gate must be 16-byte aligned");
  const int64_t ea = esize(act_dtype), ew = esize(weight_dtype);
  if ((m + 256) * ldx * ea > kMaxOffset || (n + 256) * ldw * ew > kMaxOffset)
    return fail(H3K_ERR_UNSUPPORTED, "operand exceeds 2 GiB (32-bit offsets)");
  const Range rx = rng(x, span(m, k, ldx, ea), "x"), rw = rng(w, span(n, k, ldw, ew), "w");
  const Range ry = rng(y, span(m, split_col, ldy, ea), "y"), ryt = rng(yt, span(n - split_col, m, ldyt, ea), "yt");
  if (overlaps(ry, rx) || overlaps(ry, rw) || overlaps(ryt, rx) || overlaps(ryt, rw) || overlaps(ry, ryt))
    return fail(H3K_ERR_OVERLAP, "outputs overlap inputs");
  if (residual && residual != y && overlaps(ry, rng(residual, span(m, split_col, ldr, ea), "residual")))
    return fail(H3K_ERR_OVERLAP, "y partially overlaps residual");
  if (m == 0) return H3K_OK;
  H3K_TRY(check_device());
  LinearArgs L{};
  L.act = (DType)act_dtype; L.weight = (DType)weight_dtype;
  L.m = m; L.n = n; L.k = k;
  L.x = x; L.ldx = ldx; L.w = w; L.ldw = ldw; L.w_scale = w_scale; L.bias = bias;
  L.epi = (Epilogue)epilogue; L.residual = residual; L.ldr = ldr; L.gate = gate;
  L.y = y; L.ldy = ldy; L.yt = yt; L.ldyt = ldyt; L.split_col = split_col;
  return launched(launch_linear(L, stream), "linear");
}

h3k_status h3k_linear_int8(int64_t m, int64_t n, int64_t k, const int8_t* xq, int64_t ldx, const float* x_scale,
                           const int8_t* wq, int64_t ldw, const float* w_scale, const void* bias, int32_t epilogue,
                           const void* residual, int64_t ldr, const float* gate, void* y, int64_t ldy,
                           hipStream_t stream) {
  if (epilogue < H3K_EPI_BIAS || epilogue > H3K_EPI_GATED_RESIDUAL) return fail(H3K_ERR_SHAPE, "bad epilogue %d", epilogue);
  if (m < 0 || n < 8 || n % 8 || k < 128 || k % 128 || k > kMaxInt8K)
    return fail(H3K_ERR_SHAPE, "need m >= 0, n a multiple of 8, k a multiple of 128 and <= 2^17 (m=%lld n=%lld k=%lld)",
                (long long)m, (long long)n, (long long)k);
  if (ldx < k || ldw < k || ldx % 16 || ldw % 16 || ldy < n || ldy % 8)
    return fail(H3K_ERR_SHAPE, "bad row pitches");
  if (!xq || !x_scale || !wq || !w_scale || !y) return fail(H3K_ERR_NULL, "xq, x_scale, wq, w_scale and y must be non-NULL");
  if (epilogue == H3K_EPI_GATED_RESIDUAL && (!residual || !gate || ldr < n || ldr % 8))
    return fail(H3K_ERR_NULL, "gated residual needs residual (ldr >= n, multiple of 8) and gate");
  const void* al[] = {xq, wq, bias, residual, y, x_scale, w_scale, gate};
  for (const void* p : al)
    if (p && !aligned(p, 16)) return fail(H3K_ERR_ALIGN, "pointers must be 16-byte aligned");
  if ((m + 256) * ldx > kMaxOffset || (n + 256) * ldw > kMaxOffset)
    return fail(H3K_ERR_UNSUPPORTED, "operand exceeds 2 GiB (32-bit offsets)");
  const Range rx = rng(xq, span(m, k, ldx, 1), "xq"), rw = rng(wq, span(n, k, ldw, 1), "wq");
  const Range rxs = rng(x_scale, m * 4, "x_scale"), rws = rng(w_scale, n * 4, "w_scale");
  const Range ry = rng(y, span(m, n, ldy, 2), "y");
  if (overlaps(ry, rx) || overlaps(ry, rw) || overlaps(ry, rxs) || overlaps(ry, rws))
    return fail(H3K_ERR_OVERLAP, "y overlaps an input");
  if (residual && residual != y && overlaps(ry, rng(residual, span(m, n, ldr, 2), "residual")))
    return fail(H3K_ERR_OVERLAP, "y partially overlaps residual");
  if (m == 0) return H3K_OK;
  H3K_TRY(check_device());
  LinearArgs L{};
  L.act = kINT8; L.weight = kINT8;
  L.m = m; L.n = n; L.k = k;
  L.x = xq; L.ldx = ldx; L.x_scale = x_scale; L.w = wq; L.ldw = ldw; L.w_scale = w_scale; L.bias = bias;
  L.epi = (Epilogue)epilogue; L.residual = residual; L.ldr = ldr; L.gate = gate;
  L.y = y; L.ldy = ldy; L.split_col = n;
  return launched(launch_linear(L, stream), "int8 linear");
}

h3k_status h3k_linear_int8_groups(int64_t m, int64_t n, int64_t k, int32_t group, const void* x, int64_t ldx,
                                  const int8_t* wq, int64_t ldw, const float* w_scale, const void* bias,
                                  int32_t epilogue, const void* residual, int64_t ldr, const float* gate, void* y,
                                  int64_t ldy, hipStream_t stream) {
  if (epilogue < H3K_EPI_BIAS || epilogue > H3K_EPI_GATED_RESIDUAL) return fail(H3K_ERR_SHAPE, "bad epilogue %d", epilogue);
  if (group != 32 && group != 64 && group != 128) return fail(H3K_ERR_SHAPE, "group must be 32, 64 or 128 (got %d)", group);
  if (m < 0 || n < 8 || n % 8 || k < 64 || k % 64 || k % group)
    return fail(H3K_ERR_SHAPE, "need m >= 0, n a multiple of 8, k a multiple of 64 and of the group (m=%lld n=%lld k=%lld)",
                (long long)m, (long long)n, (long long)k);
  if (ldx < k || ldw < k || ldx % 8 || ldw % 16 || ldy < n || ldy % 8) return fail(H3K_ERR_SHAPE, "bad row pitches");
  if (!x || !wq || !w_scale || !y) return fail(H3K_ERR_NULL, "x, wq, w_scale and y must be non-NULL");
  if (epilogue == H3K_EPI_GATED_RESIDUAL && (!residual || !gate || ldr < n || ldr % 8))
    return fail(H3K_ERR_NULL, "gated residual needs residual (ldr >= n, multiple of 8) and gate");
  const void* al[] = {x, wq, bias, residual, y, w_scale, gate};
  for (const void* p : al)
    if (p && !aligned(p, 16)) return fail(H3K_ERR_ALIGN, "pointers must be 16-byte aligned");
  if ((m + 256) * ldx * 2 > kMaxOffset || (n + 256) * ldw > kMaxOffset || (n + 256) * (k / group) * 4 > kMaxOffset)
    return fail(H3K_ERR_UNSUPPORTED, "operand exceeds 2 GiB (32-bit offsets)");
  const Range rx = rng(x, span(m, k, ldx, 2), "x"), rw = rng(wq, span(n, k, ldw, 1), "wq");
  const Range rs = rng(w_scale, n * (k / group) * 4, "w_scale"), ry = rng(y, span(m, n, ldy, 2), "y");
  if (overlaps(ry, rx) || overlaps(ry, rw) || overlaps(ry, rs)) return fail(H3K_ERR_OVERLAP, "y overlaps an input");
  if (residual && residual != y && overlaps(ry, rng(residual, span(m, n, ldr, 2), "residual")))
    return fail(H3K_ERR_OVERLAP, "y partially overlaps residual");
  if (m == 0) return H3K_OK;
  H3K_TRY(check_device());
  LinearArgs L{};
  L.act = kBF16; L.weight = kINT8; L.group = group;
  L.m = m; L.n = n; L.k = k;
  L.x = x; L.ldx = ldx; L.w = wq; L.ldw = ldw; L.w_scale = w_scale; L.bias = bias;
  L.epi = (Epilogue)epilogue; L.residual = residual; L.ldr = ldr; L.gate = gate;
  L.y = y; L.ldy = ldy; L.split_col = n;
  return launched(launch_linear(L, stream), "int8 group linear");
}

h3k_status h3k_token_merge(h3k_dtype dtype, int64_t n_tokens, int64_t D, const void* x, int64_t ldx, void* xm,
                           int64_t ldxm, hipStream_t stream) {
  if (dtype != H3K_F32 && dtype != H3K_BF16) return fail(H3K_ERR_DTYPE, "dtype must be F32 or BF16");
  if (n_tokens < 0 || n_tokens % 2 || n_tokens > 0x7fffffff || D < 8 || D % 8 || ldx < D || ldxm < D || ldx % 8 ||
      ldxm % 8)
    return fail(H3K_ERR_SHAPE, "need an even token count, D and the pitches multiples of 8");
  if (!x || !xm) return fail(H3K_ERR_NULL, "x and xm must be non-NULL");
  if (!aligned(x, 16) || !aligned(xm, 16)) return fail(H3K_ERR_ALIGN, "x and xm must be 16-byte aligned");
  const int64_t e = esize(dtype);
  if (overlaps(rng(xm, span(n_tokens / 2, D, ldxm, e), "xm"), rng(x, span(n_tokens, D, ldx, e), "x")))
    return fail(H3K_ERR_OVERLAP, "xm overlaps x");
  if (n_tokens == 0) return H3K_OK;
  H3K_TRY(check_device());
  return launched(launch_token_merge((DType)dtype, n_tokens, D, x, ldx, xm, ldxm, stream), "token merge");
}

h3k_status h3k_token_unmerge(h3k_dtype dtype, int64_t n_tokens, int64_t D, const void* entry, int64_t ld_entry,
                             const void* xm, int64_t ldxm, void* out, int64_t ldo, hipStream_t stream) {
  if (dtype != H3K_F32 && dtype != H3K_BF16) return fail(H3K_ERR_DTYPE, "dtype must be F32 or BF16");
  if (n_tokens < 0 || n_tokens % 2 || n_tokens > 0x7fffffff || D < 8 || D % 8 || ld_entry < D || ldxm < D || ldo < D ||
      ld_entry % 8 || ldxm % 8 || ldo % 8)
    return fail(H3K_ERR_SHAPE, "need an even token count, D and the pitches multiples of 8");
  if (!entry || !xm || !out) return fail(H3K_ERR_NULL, "entry, xm and out must be non-NULL");
  if (!aligned(entry, 16) || !aligned(xm, 16) || !aligned(out, 16))
    return fail(H3K_ERR_ALIGN, "entry, xm and out must be 16-byte aligned");
  const int64_t e = esize(dtype);
  const Range ro = rng(out, span(n_tokens, D, ldo, e), "out");
  if (overlaps(ro, rng(xm, span(n_tokens / 2, D, ldxm, e), "xm")))
    return fail(H3K_ERR_OVERLAP, "out overlaps xm");
  if (out != entry && overlaps(ro, rng(entry, span(n_tokens, D, ld_entry, e), "entry")))
    return fail(H3K_ERR_OVERLAP, "out partially overlaps entry (it may only be entry itself)");
  if (out == entry && ldo != ld_entry) return fail(H3K_ERR_SHAPE, "in place needs ldo == ld_entry");
  if (n_tokens == 0) return H3K_OK;
  H3K_TRY(check_device());
  return launched(launch_token_unmerge((DType)dtype, n_tokens, D, entry, ld_entry, xm, ldxm, out, ldo, stream),
                  "token unmerge");
}

h3k_status h3k_rope_3d(int64_t n_tokens, int64_t cols, int32_t head_dim, int32_t frames, int32_t height,
                       int32_t width, int32_t half_spatial, void* x, int64_t ldx, hipStream_t stream) {
  if (head_dim < 16 || head_dim % 16 || head_dim > 256) return fail(H3K_ERR_SHAPE, "head_dim must be a multiple of 16 in [16, 256]");
  if (n_tokens < 0 || n_tokens > 0x7fffffff || cols < head_dim || cols % head_dim || ldx < cols || ldx % 4)
    return fail(H3K_ERR_SHAPE, "need cols a multiple of head_dim and ldx >= cols, a multiple of 4");
  if (frames < 1 || height < 1 || width < 1 || (int64_t)frames * height * width != n_tokens)
    return fail(H3K_ERR_SHAPE, "grid %d x %d x %d does not hold the %lld tokens", frames, height, width,
                (long long)n_tokens);
  if (n_tokens > kMaxRopeTokens) return fail(H3K_ERR_UNSUPPORTED, "RoPE supports at most 2^24 tokens");
  if (half_spatial != 0 && half_spatial != 1) return fail(H3K_ERR_SHAPE, "half_spatial must be 0 or 1");
  if (!x) return fail(H3K_ERR_NULL, "x must be non-NULL");
  if (!aligned(x, 16)) return fail(H3K_ERR_ALIGN, "x must be 16-byte aligned");
  if (n_tokens == 0) return H3K_OK;
  H3K_TRY(check_device());
  return launched(launch_rope(n_tokens, cols, head_dim, height, width, half_spatial ? 0.5f : 1.0f, x, ldx, stream),
                  "RoPE");
}

h3k_status h3k_attention(h3k_dtype dtype, int32_t n, int32_t n_heads, int32_t head_dim, const void* q, int64_t ldq,
                         const void* k, int64_t ldk, const void* vt, int64_t ldvt, void* o, int64_t ldo,
                         int32_t q_prescaled, hipStream_t stream) {
  if (dtype != H3K_F32 && dtype != H3K_BF16) return fail(H3K_ERR_DTYPE, "dtype must be F32 or BF16");
  if (q_prescaled != 0 && q_prescaled != 1) return fail(H3K_ERR_SHAPE, "q_prescaled must be 0 or 1");
  if (q_prescaled && dtype != H3K_BF16) return fail(H3K_ERR_UNSUPPORTED, "q_prescaled needs BF16");
  if (head_dim != 64 && head_dim != 128) return fail(H3K_ERR_UNSUPPORTED, "head_dim %d not supported", head_dim);
  const int64_t D = (int64_t)n_heads * head_dim;
  if (n < 0 || n_heads < 1 || ldq < D || ldk < D || ldo < D || ldq % 8 || ldk % 8 || ldo % 8 || ldvt < ((n + 7) / 8) * 8 ||
      ldvt % 8)
    return fail(H3K_ERR_SHAPE, "bad sizes or pitches (ldvt must be >= n rounded up to 8)");
  if (!q || !k || !vt || !o) return fail(H3K_ERR_NULL, "q, k, vt and o must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(vt, 16) || !aligned(o, 16))
    return fail(H3K_ERR_ALIGN, "pointers must be 16-byte aligned");
  const int64_t e = esize(dtype);
  if (((int64_t)n + 256) * std::max(ldq, ldk) * e > kMaxOffset || D * ldvt * e > kMaxOffset)
    return fail(H3K_ERR_UNSUPPORTED, "operand exceeds 2 GiB");
  const Range ro = rng(o, span(n, D, ldo, e), "o");
  if (overlaps(ro, rng(q, span(n, D, ldq, e), "q")) || overlaps(ro, rng(k, span(n, D, ldk, e), "k")) ||
      overlaps(ro, rng(vt, span(D, n, ldvt, e), "vt")))
    return fail(H3K_ERR_OVERLAP, "o overlaps an input");
  if (n == 0) return H3K_OK;
  H3K_TRY(check_device());
  AttentionArgs A{};
  A.dt = (DType)dtype; A.n = n; A.n_heads = n_heads; A.head_dim = head_dim;
  A.q = q; A.ldq = ldq; A.k = k; A.ldk = ldk; A.vt = vt; A.ldvt = ldvt; A.o = o; A.ldo = ldo;
  A.q_prescaled = q_prescaled != 0;
  return launched(launch_attention(A, stream), "attention");
}

h3k_status h3k_profiler_create(int32_t capacity, h3k_profiler** out) {
  if (!out) return fail(H3K_ERR_NULL, "out is NULL");
  if (capacity < 1 || capacity > (1 << 20)) return fail(H3K_ERR_SHAPE, "capacity out of range");
  H3K_TRY(check_device());
  h3k_profiler* p = new h3k_profiler();
  p->capacity = capacity;
  // one start event per call plus one per kernel: at most 2 per launch
  p->events.resize(2 * (size_t)capacity);
  for (size_t i = 0; i < p->events.size(); ++i) {
    if (hipEventCreate(&p->events[i]) != hipSuccess) {
      for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(p->events[j]);
      delete p;
      return fail(H3K_ERR_HIP, "hipEventCreate failed");
    }
  }
  *out = p;
  return H3K_OK;
}

h3k_status h3k_profiler_destroy(h3k_profiler* p) {
  if (!p) return fail(H3K_ERR_NULL, "profiler is NULL");
  for (hipEvent_t e : p->events) (void)hipEventDestroy(e);
  delete p;
  return H3K_OK;
}

h3k_status h3k_profiler_reset(h3k_profiler* p) {
  if (!p) return fail(H3K_ERR_NULL, "profiler is NULL");
  p->n_events = 0;
  p->intervals.clear();
  p->overflow = false;
  return H3K_OK;
}

h3k_status h3k_profiler_read(h3k_profiler* p, int32_t kind, double* total_ms, int32_t* launches) {
  if (!p || !total_ms || !launches) return fail(H3K_ERR_NULL, "NULL argument");
  if (kind < 0 || kind >= H3K_K_COUNT) return fail(H3K_ERR_SHAPE, "kernel kind %d out of range", kind);
  if (p->overflow) return fail(H3K_ERR_SHAPE, "profiler capacity exceeded; reset it or create a larger one");
  double sum = 0.0;
  int cnt = 0;
  for (const auto& iv : p->intervals) {
    if (iv.kind != kind) continue;
    if (hipEventSynchronize(p->events[iv.after]) != hipSuccess) return fail(H3K_ERR_HIP, "hipEventSynchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p->events[iv.before], p->events[iv.after]) != hipSuccess)
      return fail(H3K_ERR_HIP, "hipEventElapsedTime failed");
    sum += ms;
    ++cnt;
  }
  *total_ms = sum;
  *launches = cnt;
  return H3K_OK;
}

h3k_status h3k_get_device_info(int32_t device, h3k_device_info* out) {
  if (!out) return fail(H3K_ERR_NULL, "out is NULL");
  int count = 0;
  const hipError_t ec = hipGetDeviceCount(&count);
  if (ec != hipSuccess) return fail(H3K_ERR_HIP, "no usable HIP device: %s", hipGetErrorString(ec));
  if (device < 0 || device >= count) return fail(H3K_ERR_HIP, "device %d: the runtime sees %d devices", device, count);
  hipDeviceProp_t pr;
  const hipError_t ep = hipGetDeviceProperties(&pr, device);
  if (ep != hipSuccess) return fail(H3K_ERR_HIP, "hipGetDeviceProperties(%d) failed: %s", device, hipGetErrorString(ep));
  h3k_device_info d;
  std::memset(&d, 0, sizeof(d));
  d.compute_units = pr.multiProcessorCount;
  d.peak_clock_khz = pr.clockRate;
  d.lds_bytes_per_cu = (int32_t)pr.maxSharedMemoryPerMultiProcessor;
  d.wavefront_size = pr.warpSize;
  d.hbm_bytes = (uint64_t)pr.totalGlobalMem;
  std::snprintf(d.arch, sizeof(d.arch), "%s", pr.gcnArchName);
  *out = d;
  return H3K_OK;
}

}  // extern "C"
