// Drives the C ABI of h3k_api.cpp, linked with launch_stubs.cpp, under
// AddressSanitizer and UBSan on the CPU: valid calls on exactly sized host
// buffers (each its own allocation, so that any access a launcher stand-in
// makes outside them is reported), invalid calls that must be rejected, the
// lifetime planner over a range of shapes, and the event profiler.
// Prints "host sanitize OK" and exits 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "h3k.h"

extern "C" int64_t h3k_stub_launches();

namespace {

int g_fail = 0;
#define CHECK(cond)                                                                     \
  do {                                                                                  \
    if (!(cond)) {                                                                      \
      std::fprintf(stderr, "%s:%d: CHECK failed: %s (%s)\n", __FILE__, __LINE__, #cond, \
                   h3k_last_error());                                                   \
      ++g_fail;                                                                         \
    }                                                                                   \
  } while (0)

// one exactly sized, 256-byte aligned allocation per buffer
struct Pool {
  std::vector<void*> ptrs;
  void* get(size_t bytes) {
    if (bytes == 0) return nullptr;
    void* p = nullptr;
    if (posix_memalign(&p, 256, bytes) != 0) std::abort();
    std::memset(p, 0, bytes);
    ptrs.push_back(p);
    return p;
  }
  ~Pool() {
    for (void* p : ptrs) std::free(p);
  }
};

int64_t esz(h3k_dtype d) { return d == H3K_F32 ? 4 : d == H3K_BF16 ? 2 : 1; }

h3k_dit_config make_cfg(int n, int heads, int hd, int F, int C, h3k_dtype act, h3k_dtype wt, int alias) {
  h3k_dit_config c;
  std::memset(&c, 0, sizeof(c));
  c.n_tokens = n;
  c.hidden = heads * hd;
  c.n_heads = heads;
  c.head_dim = hd;
  c.mlp_hidden = F;
  c.cond_dim = C;
  c.ln_eps = 1e-6f;
  c.act_dtype = act;
  c.weight_dtype = wt;
  c.alias_activations = alias;
  return c;
}

h3k_dit_block_weights make_weights(Pool& pool, const h3k_dit_config& c) {
  const int64_t D = c.hidden, F = c.mlp_hidden, C = c.cond_dim;
  const int64_t ea = esz(c.act_dtype), ew = esz(c.weight_dtype);
  const bool w8 = c.weight_dtype == H3K_INT8;
  const int64_t g = c.int8_mlp_group;
  h3k_dit_block_weights w;
  w.w_ada = pool.get(6 * D * C * ea);
  w.b_ada = pool.get(6 * D * ea);
  w.w_qkv = pool.get(3 * D * D * ew);
  w.b_qkv = pool.get(3 * D * ea);
  w.s_qkv = w8 ? static_cast<float*>(pool.get(3 * D * 4)) : nullptr;
  w.w_out = pool.get(D * D * ew);
  w.b_out = pool.get(D * ea);
  w.s_out = w8 ? static_cast<float*>(pool.get(D * 4)) : nullptr;
  w.w_up = pool.get(F * D * ew);
  w.b_up = pool.get(F * ea);
  w.s_up = w8 ? static_cast<float*>(pool.get(F * (g ? D / g : 1) * 4)) : nullptr;
  w.w_down = pool.get(D * F * ew);
  w.b_down = pool.get(D * ea);
  w.s_down = w8 ? static_cast<float*>(pool.get(D * (g ? F / g : 1) * 4)) : nullptr;
  return w;
}

// one block and a short stack on exactly sized buffers; the planner's
// invariants on the way
void run_config(const char* name, h3k_dit_config c, int n_blocks) {
  Pool pool;
  h3k_dit_plan_info info;
  CHECK(h3k_dit_plan(&c, &info) == H3K_OK);
  for (int t = 0; t < H3K_T_COUNT; ++t)
    CHECK(info.offset[t] % 256 == 0 && info.offset[t] + info.bytes[t] <= info.part_offset &&
          info.part_offset + info.part_bytes <= info.workspace_bytes);
  for (int s = 0; s <= 8; ++s)
    for (int a = 0; a < H3K_T_COUNT; ++a)
      for (int b = a + 1; b < H3K_T_COUNT; ++b) {
        const bool live = info.first_step[a] <= s && s <= info.last_step[a] && info.first_step[b] <= s &&
                          s <= info.last_step[b] && info.bytes[a] && info.bytes[b];
        if (live)
          CHECK(info.offset[a] + info.bytes[a] <= info.offset[b] || info.offset[b] + info.bytes[b] <= info.offset[a]);
      }
  uint64_t ws_bytes = 0;
  CHECK(h3k_dit_workspace_size(&c, n_blocks, &ws_bytes) == H3K_OK);
  const int64_t act = (int64_t)c.n_tokens * c.hidden * esz(c.act_dtype);
  void* x = pool.get(act);
  void* cond = pool.get((size_t)c.cond_dim * esz(c.act_dtype));
  void* out = pool.get(act);
  void* ws = pool.get(ws_bytes);
  std::vector<h3k_dit_block_weights> blocks;
  for (int l = 0; l < n_blocks; ++l) blocks.push_back(make_weights(pool, c));
  h3k_dit_stats st;
  std::memset(&st, 0, sizeof(st));
  const int64_t before = h3k_stub_launches();
  if (c.token_reduction_last <= c.token_reduction_first) {
    CHECK(h3k_dit_block_forward(&c, &blocks[0], x, cond, out, ws, ws_bytes, nullptr, &st) == H3K_OK);
    // int8 weights: each projection with bf16 activations widens its weights first
    const int staged = c.weight_dtype == H3K_INT8 ? (c.int8_fc2_rows ? 3 : 4) : 0;
    CHECK((staged == 0) == (info.wstage_bytes == 0));
    CHECK(st.dispatches == (c.int8_fc2_rows ? 9 : 8) + st.tail_splits + staged);
    CHECK(st.tail_splits >= 0 && st.tail_splits <= 4);
    CHECK(h3k_stub_launches() - before == st.dispatches);
    CHECK(st.workspace_bytes == ws_bytes);
  }
  const int64_t before_stack = h3k_stub_launches();
  CHECK(h3k_dit_stack_forward(&c, blocks.data(), n_blocks, x, cond, out, ws, ws_bytes, nullptr, &st) == H3K_OK);
  CHECK(h3k_stub_launches() - before_stack == st.dispatches);
  CHECK(info.part_offset + info.part_bytes <= ws_bytes);
  // rejected before any launch: short workspace, out inside the workspace, misaligned x
  const int64_t mark = h3k_stub_launches();
  CHECK(h3k_dit_stack_forward(&c, blocks.data(), n_blocks, x, cond, out, ws, ws_bytes - 1, nullptr, nullptr) ==
        H3K_ERR_WORKSPACE);
  CHECK(h3k_dit_stack_forward(&c, blocks.data(), n_blocks, x, cond, ws, ws, ws_bytes, nullptr, nullptr) ==
        H3K_ERR_OVERLAP);
  CHECK(h3k_dit_stack_forward(&c, blocks.data(), n_blocks, static_cast<char*>(x) + 4, cond, out, ws, ws_bytes,
                              nullptr, nullptr) == H3K_ERR_ALIGN);
  CHECK(h3k_stub_launches() == mark);
  std::printf("  %s: workspace %llu bytes, %d blocks\n", name, (unsigned long long)ws_bytes, n_blocks);
}

void kernel_entry_points() {
  Pool pool;
  // linear with a transposed part, gated residual, int8 x int8, group-wise int8
  const int64_t m = 300, n = 320, k = 128;
  void* x = pool.get(m * k * 2);
  void* w = pool.get(n * k * 2);
  void* y = pool.get(m * 256 * 2);
  void* yt = pool.get((n - 256) * 304 * 2);
  CHECK(h3k_linear(H3K_BF16, H3K_BF16, m, n, k, x, k, w, k, nullptr, nullptr, H3K_EPI_BIAS, nullptr, 0, nullptr, y,
                   256, yt, 304, 256, nullptr) == H3K_OK);
  void* r = pool.get(m * n * 2);
  float* gate = static_cast<float*>(pool.get(n * 4));
  void* y2 = pool.get(m * n * 2);
  CHECK(h3k_linear(H3K_BF16, H3K_BF16, m, n, k, x, k, w, k, nullptr, nullptr, H3K_EPI_GATED_RESIDUAL, r, n, gate, y2,
                   n, nullptr, 0, n, nullptr) == H3K_OK);
  int8_t* xq = static_cast<int8_t*>(pool.get(m * k));
  float* xs = static_cast<float*>(pool.get(m * 4));
  int8_t* wq = static_cast<int8_t*>(pool.get(n * k));
  float* ws = static_cast<float*>(pool.get(n * 4));
  CHECK(h3k_linear_int8(m, n, k, xq, k, xs, wq, k, ws, nullptr, H3K_EPI_GELU, nullptr, 0, nullptr, y2, n, nullptr) ==
        H3K_OK);
  float* wsg = static_cast<float*>(pool.get(n * (k / 64) * 4));
  CHECK(h3k_linear_int8_groups(m, n, k, 64, x, k, wq, k, wsg, nullptr, H3K_EPI_BIAS, nullptr, 0, nullptr, y2, n,
                               nullptr) == H3K_OK);
  // quantisers
  void* w32 = pool.get(n * k * 4);
  CHECK(h3k_quantize_weights_int8(w32, H3K_F32, n, k, wq, ws, nullptr) == H3K_OK);
  CHECK(h3k_quantize_weights_int8_groups(w32, H3K_F32, n, k, 64, wq, wsg, nullptr) == H3K_OK);
  // attention, both q layouts; the V^T pitch rounded up to 8
  const int na = 37, H = 2, d = 128, Da = H * d, ldvt = 40;
  void* q = pool.get(na * Da * 2);
  void* kk = pool.get(na * Da * 2);
  void* vt = pool.get(Da * ldvt * 2);
  void* o = pool.get(na * Da * 2);
  CHECK(h3k_attention(H3K_BF16, na, H, d, q, Da, kk, Da, vt, ldvt, o, Da, 0, nullptr) == H3K_OK);
  CHECK(h3k_attention(H3K_BF16, na, H, d, q, Da, kk, Da, vt, ldvt, o, Da, 1, nullptr) == H3K_OK);
  CHECK(h3k_attention(H3K_BF16, na, H, d, q, Da, kk, Da, vt, 32, o, Da, 0, nullptr) == H3K_ERR_SHAPE);
  // LayerNorm + modulation, AdaLN GEMV, RoPE, token merge / restore
  float* shift = static_cast<float*>(pool.get(Da * 4));
  float* scale = static_cast<float*>(pool.get(Da * 4));
  CHECK(h3k_ln_modulate(H3K_BF16, na, Da, 1e-6f, q, Da, shift, scale, o, Da, nullptr) == H3K_OK);
  void* wa = pool.get(6 * Da * 64 * 2);
  void* cv = pool.get(64 * 2);
  float* mod = static_cast<float*>(pool.get(6 * Da * 4));
  CHECK(h3k_adaln_modulation(H3K_BF16, 6 * Da, 64, wa, nullptr, cv, mod, nullptr) == H3K_OK);
  void* xr = pool.get(24 * 128 * 2);
  CHECK(h3k_rope_3d(24, 128, 64, 2, 3, 4, 1, xr, 128, nullptr) == H3K_OK);
  void* xm = pool.get(12 * 128 * 2);
  CHECK(h3k_token_merge(H3K_BF16, 24, 128, xr, 128, xm, 128, nullptr) == H3K_OK);
  CHECK(h3k_token_unmerge(H3K_BF16, 24, 128, xr, 128, xm, 128, xr, 128, nullptr) == H3K_OK);
}

void profiler() {
  Pool pool;
  h3k_dit_config c = make_cfg(40, 2, 64, 128, 64, H3K_BF16, H3K_BF16, 1);
  uint64_t ws_bytes = 0;
  CHECK(h3k_dit_workspace_size(&c, 1, &ws_bytes) == H3K_OK);
  const int64_t act = 40 * 128 * 2;
  void* x = pool.get(act);
  void* cond = pool.get(64 * 2);
  void* out = pool.get(act);
  void* ws = pool.get(ws_bytes);
  h3k_dit_block_weights w = make_weights(pool, c);
  h3k_profiler* p = nullptr;
  CHECK(h3k_profiler_create(4, &p) == H3K_OK);
  h3k_dit_stats st;
  std::memset(&st, 0, sizeof(st));
  st.profiler = p;
  CHECK(h3k_dit_block_forward(&c, &w, x, cond, out, ws, ws_bytes, nullptr, &st) == H3K_OK);
  double ms = 0;
  int32_t launches = 0;
  CHECK(h3k_profiler_read(p, H3K_K_ADALN, &ms, &launches) == H3K_ERR_SHAPE);   // 8 launches > capacity 4
  CHECK(h3k_profiler_reset(p) == H3K_OK);
  CHECK(h3k_profiler_destroy(p) == H3K_OK);
  CHECK(h3k_profiler_create(16, &p) == H3K_OK);
  st.profiler = p;
  CHECK(h3k_dit_block_forward(&c, &w, x, cond, out, ws, ws_bytes, nullptr, &st) == H3K_OK);
  CHECK(h3k_profiler_read(p, H3K_K_LN_MOD, &ms, &launches) == H3K_OK);
  CHECK(launches == 2 && ms == 2.0);
  CHECK(h3k_profiler_read(p, H3K_K_COUNT, &ms, &launches) == H3K_ERR_SHAPE);
  CHECK(h3k_profiler_destroy(p) == H3K_OK);
}

void device_info() {
  CHECK(h3k_get_device_info(0, nullptr) == H3K_ERR_NULL);
  h3k_device_info d;
  std::memset(&d, 0x5A, sizeof(d));
  CHECK(h3k_get_device_info(1, &d) == H3K_ERR_HIP);
  CHECK(h3k_get_device_info(-1, &d) == H3K_ERR_HIP);
  CHECK(d.compute_units == 0x5A5A5A5A);   // untouched on error
  CHECK(h3k_get_device_info(0, &d) == H3K_OK);
  CHECK(d.compute_units == 256 && d.peak_clock_khz == 2400000 && d.lds_bytes_per_cu == 160 * 1024);
  CHECK(d.wavefront_size == 64 && d.hbm_bytes == (uint64_t(288) << 30));
  CHECK(std::strcmp(d.arch, "gfx950:sramecc+:xnack-") == 0);
}

}  // namespace

int main(int argc, char** argv) {
  const bool full = argc > 1 && std::strcmp(argv[1], "full") == 0;
  std::printf("block and stack forward on exact host buffers:\n");
  run_config("fp32 512 tokens, 4x64 heads", make_cfg(512, 4, 64, 1024, 256, H3K_F32, H3K_F32, 1), 2);
  for (int alias = 0; alias <= 1; ++alias) {
    run_config(alias ? "bf16 37 tokens, alias on" : "bf16 37 tokens, alias off",
               make_cfg(37, 2, 128, 384, 64, H3K_BF16, H3K_BF16, alias), 3);
  }
  h3k_dit_config c8 = make_cfg(333, 2, 128, 640, 256, H3K_BF16, H3K_INT8, 1);
  run_config("int8 weights", c8, 2);
  c8.int8_fc2_rows = 1;
  run_config("int8 weights, row-quantised FC2", c8, 2);
  c8.int8_fc2_rows = 0;
  c8.int8_mlp_group = 64;
  run_config("int8 weights, group-wise MLP", c8, 2);
  h3k_dit_config cr = make_cfg(333, 2, 128, 640, 256, H3K_BF16, H3K_BF16, 1);
  cr.rope_frames = 3; cr.rope_height = 3; cr.rope_width = 37; cr.rope_half_spatial = 1;
  run_config("3D RoPE", cr, 2);
  h3k_dit_config ct = make_cfg(334, 2, 128, 640, 256, H3K_BF16, H3K_BF16, 1);
  ct.token_reduction_first = 1; ct.token_reduction_last = 3;
  run_config("token reduction 1..2", ct, 4);
  run_config("bf16 6144 tokens, 24x128 heads", make_cfg(6144, 24, 128, 12288, 3072, H3K_BF16, H3K_BF16, 1), 1);
  if (full) {
    run_config("bf16 22680 tokens, 40x128 heads", make_cfg(22680, 40, 128, 13824, 5120, H3K_BF16, H3K_BF16, 1), 1);
    h3k_dit_config c4 = make_cfg(22680, 40, 128, 13824, 5120, H3K_BF16, H3K_INT8, 0);
    c4.int8_fc2_rows = 1;
    run_config("int8 22680 tokens, row-quantised FC2, alias off", c4, 1);
  }
  kernel_entry_points();
  profiler();
  device_info();
  if (g_fail) {
    std::printf("host sanitize FAILED: %d checks\n", g_fail);
    return 1;
  }
  std::printf("host sanitize OK (%lld launches)\n", (long long)h3k_stub_launches());
  return 0;
}
