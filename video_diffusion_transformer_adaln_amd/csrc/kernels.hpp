// Host-side launchers of the gfx950 kernels.  Each launcher assumes its
// arguments were validated by the C-ABI layer (h3k_api.cpp) and only
// enqueues work on `stream`; it returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3k {

enum DType : int32_t { kF32 = 0, kBF16 = 1, kINT8 = 2 };
enum Epilogue : int32_t { kEpiBias = 0, kEpiGelu = 1, kEpiGatedResidual = 2, kEpiBiasRope = 3 };

// mod[rows] = W[rows, cols] c + b   (fp32 out)
hipError_t launch_adaln_gemv(DType dt, int rows, int cols, const void* w, const void* b,
                             const void* c, float* mod, hipStream_t stream);

// out = LN(x) * (1 + scale) + shift, row-wise
hipError_t launch_ln_modulate(DType dt, int n, int D, float eps, const void* x, int64_t ldx,
                              const float* shift, const float* scale, void* out, int64_t ldo,
                              hipStream_t stream);

struct LinearArgs {
  DType act, weight;
  int64_t m, n, k;
  const void* x; int64_t ldx;
  const void* w; int64_t ldw;
  const float* w_scale;
  const void* bias;
  Epilogue epi;
  const void* residual; int64_t ldr;
  const float* gate;
  void* y; int64_t ldy;
  void* yt; int64_t ldyt;
  int64_t split_col;
  const float* x_scale;   // per-row activation scales (act = kINT8 only)
  int group;              // int8 weights: 0 = w_scale per row [n]; else w_scale [n, k / group]
  int rope_hd, rope_h, rope_w;   // kEpiBiasRope: head size and grid H, W (rows are tokens)
  float rope_spatial;            // 1, or 0.5 to halve the spatial coordinates
  int64_t scale_cols;            // bf16 row-major output: columns < scale_cols are multiplied by
  float col_scale;               // col_scale after the bias (and rotation), before the rounding
  float* part;                   // bf16 x bf16, row-major output: scratch for k-split tail tiles
  int64_t part_bytes;            // (fp32 partial tiles); null / 0: no split
  void* wstage;                  // int8 weights, bf16 activations: n * k bf16 to widen the weights
  int64_t wstage_bytes;          // into before a bf16 GEMM; null / too small: widened in the GEMM
};
// Enqueues the GEMM (and, when its tail tiles are split along k, the kernel
// that sums their partial tiles and applies the epilogue); *kernels (if not
// null) receives the number of kernels enqueued.
hipError_t launch_linear(const LinearArgs& a, hipStream_t stream, int* kernels = nullptr);

// Tail split of the 256x256-tile bf16 GEMM (one workgroup per compute unit):
// with `tiles` tiles on `cus` CUs, the last tiles % cus tiles form a partial
// last wave.  When that wave would leave at least half the CUs idle, each of
// its tiles is split along k into S workgroups (S <= 8, at least 4 k-tiles
// of 64 each, tail * S <= min(cus, cap_tiles)), whose fp32 partial tiles a
// second kernel sums in a fixed order.  The split must shed at least 2048 of
// k per tail workgroup, (1 - 1/S) k >= 2048: measured on MI355X, writing and
// re-reading up to 64 MiB of partial tiles and the second launch cost about
// 30 us, what a 256x256 tile's MFMAs take for about 1000 of k.  Returns S, or
// 0 for no split.
constexpr int64_t kPartTileBytes = 256 * 256 * 4;
inline int tail_split_ways(int64_t tiles, int64_t kt, int64_t cus, int64_t cap_tiles) {
  if (tiles < 1 || cus < 1) return 0;
  const int64_t tail = tiles % cus;
  if (tail == 0 || 2 * tail > cus) return 0;
  int64_t s = kt / 4 < 8 ? kt / 4 : 8;
  const int64_t room = (cap_tiles < cus ? cap_tiles : cus) / tail;
  if (room < s) s = room;
  if (s < 2 || (s - 1) * kt < 32 * s) return 0;   // (1 - 1/S) * 64 kt >= 2048
  return (int)s;
}

struct AttentionArgs {
  DType dt;
  int n, n_heads, head_dim;
  const void* q; int64_t ldq;
  const void* k; int64_t ldk;
  const void* vt; int64_t ldvt;
  void* o; int64_t ldo;
  bool q_prescaled;       // bf16: q already multiplied by log2(e) / sqrt(head_dim)
  float* part;            // bf16, head_dim 128: scratch for key-split tail blocks
  int64_t part_bytes;     // (unnormalised partial results); null / 0: no split
};
// *kernels (if not null): kernels enqueued (two when the tail blocks are split along the keys)
hipError_t launch_attention(const AttentionArgs& a, hipStream_t stream, int* kernels = nullptr);

// Workgroup shape of the bf16 attention for head_dim 128: 4 waves (128
// queries, two workgroups per CU) for sequences of at most 8192 tokens with
// fewer than 1024 workgroups of 8 waves, else 8 waves (256 queries, one per CU).
inline int attn_waves128(int64_t n, int64_t heads) {
  const int64_t wg8 = (n + 255) / 256 * heads;
  return (wg8 < 4 * 256 && n <= 8192) ? 4 : 8;
}
// Bytes of one key-split partial result: the workgroup's queries' unnormalised
// O (fp32, head_dim 128) plus their running reference and row sum.
inline int64_t attn_unit_bytes(int nw) { return (int64_t)nw * 32 * (128 + 2) * 4; }
// Key split of the attention's last round (bf16, head_dim 128): `blocks`
// workgroups, `slots` resident at once, T key tiles of 32.  When the last
// round would leave at least half the slots idle, each of its workgroups is
// split into S key ranges (S <= 8, at least 8 tiles each, tail * S <=
// min(slots, cap_units)) whose partial results a second kernel combines; the
// split must shed at least 2048 keys per workgroup, (1 - 1/S) 32 T >= 2048.
// Returns S, or 0 for no split.
inline int attn_split_ways(int64_t blocks, int64_t T, int64_t slots, int64_t cap_units) {
  if (blocks < 1 || slots < 1) return 0;
  const int64_t tail = blocks % slots;
  if (tail == 0 || 2 * tail > slots) return 0;
  int64_t s = T / 8 < 8 ? T / 8 : 8;
  const int64_t room = (cap_units < slots ? cap_units : slots) / tail;
  if (room < s) s = room;
  if (s < 2 || (s - 1) * T < 64 * s) return 0;
  return (int)s;
}
// Workgroup shape (returned: 4 or 8 waves) and key split (*split, 0 for none)
// of the bf16 attention for head_dim 128 on `cus` compute units with
// `cap_bytes` of scratch for partial results (0: no split).  Where 8-wave
// workgroups can split their last round, they are taken even for short
// sequences: measured on MI355X at 6144 tokens x 24 heads, 8 waves with the
// split 400 us, 4 waves with it 415 us, 4 waves without 430 us.
inline int attn_shape128(int64_t n, int64_t heads, int64_t cus, int64_t cap_bytes, int* split) {
  const int64_t T = (n + 31) / 32;
  int nw = attn_waves128(n, heads), s = 0;
  if (cus > 0 && cap_bytes > 0) {
    const int s8 = attn_split_ways((n + 255) / 256 * heads, T, cus, cap_bytes / attn_unit_bytes(8));
    if (s8) {
      nw = 8;
      s = s8;
    } else if (nw == 4) {
      s = attn_split_ways((n + 127) / 128 * heads, T, 2 * cus, cap_bytes / attn_unit_bytes(4));
    }
  }
  *split = s;
  return nw;
}

// token reduction: xm[m] = (x[2m] + x[2m+1]) / 2 for m < n/2 (D a multiple of 8)
hipError_t launch_token_merge(DType dt, int64_t n, int64_t D, const void* x, int64_t ldx, void* xm, int64_t ldm,
                              hipStream_t stream);
// out[2m+j] = entry[2m+j] + xm[m] - merge(entry)[m]; out may alias entry
hipError_t launch_token_unmerge(DType dt, int64_t n, int64_t D, const void* entry, int64_t lde, const void* xm,
                                int64_t ldm, void* out, int64_t ldo, hipStream_t stream);

// in place: x[n, cols] (bf16, row pitch ldx), heads of head_dim consecutive
// columns, rotated by the 3D RoPE of each row's token over the (T, H, W) grid
hipError_t launch_rope(int64_t n, int64_t cols, int head_dim, int height, int width, float spatial, void* x,
                       int64_t ldx, hipStream_t stream);

hipError_t launch_quantize_int8(DType dt, const void* w, int64_t rows, int64_t cols, int8_t* q,
                                float* scales, hipStream_t stream);
// group in {32, 64, 128}, cols a multiple of it; scales [rows, cols / group]
hipError_t launch_quantize_int8_groups(DType dt, const void* w, int64_t rows, int64_t cols, int group, int8_t* q,
                                       float* scales, hipStream_t stream);

}  // namespace h3k
