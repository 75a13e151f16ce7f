// Device-side helpers shared by the gfx950 kernels: vector types, bf16
// conversion, wave reductions, the LDS chunk swizzle and the XCD-aware
// workgroup remap.
#pragma once
#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace h3k {

constexpr int kWave = 64;
// MI355X (gfx950) has 8 accelerator complex dies; consecutive workgroup ids
// are dispatched round-robin over them, and each has its own L2.
constexpr int kXcds = 8;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Position of 16-byte chunk `c` of LDS row `r` for rows of 8 chunks
// (128 bytes): XOR with a row hash so that 8 (32-bank view) or 16 (64-bank
// view) consecutive rows reading the same logical chunk hit distinct banks.
__device__ __forceinline__ int swz8(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }
// Same for rows of 16 chunks (256 bytes).
__device__ __forceinline__ int swz16(int r, int c) { return c ^ (r & 15); }

// 16-byte direct-to-LDS buffer load: lane l's 16 bytes land at lds_dst + 16 l.
// (A plain device function: host compilation never instantiates its body.)
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, char* lds_dst, uint32_t voff, uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, soff, 0, 0);
}
// Workgroup barrier without a memory fence (__syncthreads would also wait
// for every outstanding load, including direct-to-LDS loads meant to stay in
// flight); the empty asm statements keep the compiler from moving memory
// accesses across it.  Callers wait for what must be visible first.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// s_waitcnt vmcnt(N), expcnt and lgkmcnt left at their maxima (vmcnt is 6
// bits: bits 3:0 and 15:14 of the immediate)
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// s_waitcnt lgkmcnt(0): this wave's LDS reads and writes have completed
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// 3D rotary position embedding over a (T, H, W) latent grid, tokens laid out
// frame, row, column ([H3-review], note on native-256 RoPE, which halves the
// spatial coordinates on 256 square canvases: spatial = 0.5, else 1).  A
// head's d dimensions are cut into a time, a height and a width slice of
// d/4, 3d/8, 3d/8; the pair (2i, 2i+1) of the slice of axis a turns by
// pos_a * 10000^(-2i / d_a).
struct RopeGeom {
  int head_dim;          // 0: no rotation
  int height, width;     // the grid's H and W (T = tokens / (H W))
  float spatial;         // 1 or 0.5
};
// cos and sin of the angle pos * 10000^(-2i/da) of rotation pair i of an
// axis slice of width da.  10000^(-2i/da) = 2^(-2i log2(10000) / da); the
// angle in turns, reduced to [0, 1) exactly (fract), for v_sin_f32 /
// v_cos_f32, which take turns.  Positions are grid coordinates (< 2^16), so
// the angle's fp32 error stays far below bf16 resolution.
__device__ __forceinline__ void rope_cs(float pos, int i, int da, float& cs, float& sn) {
  const float theta = __builtin_amdgcn_exp2f(-2.0f * 13.287712379549449f * (float)i / (float)da);
  const float turns = pos * theta * 0.15915494309189535f;
  const float fr = turns - floorf(turns);
  sn = __builtin_amdgcn_sinf(fr);
  cs = __builtin_amdgcn_cosf(fr);
}
__device__ __forceinline__ void rope_apply(float& x, float& y, float cs, float sn) {
  const float nx = x * cs - y * sn;
  y = x * sn + y * cs;
  x = nx;
}
// Exact a / b for 0 <= a < 2^24, b > 0 through one fp32 multiply and one
// correction step (the float quotient is off by at most one), instead of
// the integer division sequence.
__device__ __forceinline__ int div_small(int a, int b) {
  int q = (int)((float)a * __builtin_amdgcn_rcpf((float)b));
  const int r = a - q * b;
  q += (r >= b) - (r < 0);
  return q;
}
// Grid coordinates of token `tok` (frame-major, then rows, then columns).
__device__ __forceinline__ void rope_coords(int tok, const RopeGeom& g, int& t, int& h, int& w) {
  const int hw = g.height * g.width;
  t = div_small(tok, hw);
  const int r = tok - t * hw;
  h = div_small(r, g.width);
  w = r - h * g.width;
}
// Rotate the pair (x, y) at even dimension j (0 <= j < head_dim) of a head of
// token `tok`.
__device__ __forceinline__ void rope_rotate(float& x, float& y, int tok, int j, const RopeGeom& g) {
  const int d = g.head_dim, dt = d / 4, dh = (d - dt) / 2;
  int t, h, w;
  rope_coords(tok, g, t, h, w);
  float pos;
  int i, da;
  if (j < dt) { pos = (float)t; i = j >> 1; da = dt; }
  else if (j < dt + dh) { pos = (float)h * g.spatial; i = (j - dt) >> 1; da = dh; }
  else { pos = (float)w * g.spatial; i = (j - dt - dh) >> 1; da = d - dt - dh; }
  float cs, sn;
  rope_cs(pos, i, da, cs, sn);
  rope_apply(x, y, cs, sn);
}
// The same rotation from a table of (cos, sin) per axis position and pair:
// frames x d/8 pairs, then height x 3d/16, then width x 3d/16 (rope_table_entry
// fills entry e), so a tile's epilogue takes no transcendental per element.
__device__ __forceinline__ int rope_table_size(const RopeGeom& g, int frames) {
  const int d = g.head_dim, dt = d / 4, dh = (d - dt) / 2, dw = d - dt - dh;
  return frames * (dt / 2) + g.height * (dh / 2) + g.width * (dw / 2);
}
__device__ __forceinline__ float2 rope_table_entry(int e, const RopeGeom& g, int frames) {
  const int d = g.head_dim, dt = d / 4, dh = (d - dt) / 2, dw = d - dt - dh;
  const int nt = dt / 2, nh = dh / 2, nw = dw / 2;
  float pos;
  int i, da;
  if (e < frames * nt) { pos = (float)(e / nt); i = e % nt; da = dt; }
  else if ((e -= frames * nt) < g.height * nh) { pos = (float)(e / nh) * g.spatial; i = e % nh; da = dh; }
  else { e -= g.height * nh; pos = (float)(e / nw) * g.spatial; i = e % nw; da = dw; }
  float2 r;
  rope_cs(pos, i, da, r.x, r.y);
  return r;
}
__device__ __forceinline__ void rope_rotate_table(float& x, float& y, int tok, int j, const RopeGeom& g, int frames,
                                                  const float2* tab) {
  const int d = g.head_dim, dt = d / 4, dh = (d - dt) / 2, dw = d - dt - dh;
  int t, h, w;
  rope_coords(tok, g, t, h, w);
  int e;
  if (j < dt) e = t * (dt / 2) + (j >> 1);
  else if (j < dt + dh) e = frames * (dt / 2) + h * (dh / 2) + ((j - dt) >> 1);
  else e = frames * (dt / 2) + g.height * (dh / 2) + w * (dw / 2) + ((j - dt - dh) >> 1);
  const float2 cs = tab[e];
  rope_apply(x, y, cs.x, cs.y);
}

// Remap a linear workgroup id so that each XCD receives one contiguous range
// of logical tiles (neighbouring tiles then share that XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int q = nblocks / kXcds, r = nblocks % kXcds;
  const int xcd = bid % kXcds, local = bid / kXcds;
  return (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// GELU, tanh form.  Uses the identity 0.5 (1 + tanh(y)) = 1 / (1 + exp(-2y)),
// so gelu(z) = z / (1 + exp(-2y)) with y = sqrt(2/pi) (z + 0.044715 z^3).
// The exponent -2 y log2(e) is folded to z (c1 + c2 z^2), c1 = -2 sqrt(2/pi)
// log2(e), c2 = 0.044715 c1 (one multiply, one fma, one multiply), then
// v_exp_f32 (exp2) and the reciprocal through v_rcp_f32; within 1e-6
// relative of the exact function.  For z -> -inf the exponential overflows
// to +inf and the result is -0.
__device__ __forceinline__ float gelu_tanh(float z) {
  const float c1 = -2.3022082f;                   // -2 sqrt(2/pi) log2(e)
  const float c2 = -0.10294324f;                  // 0.044715 c1
  const float e = __builtin_amdgcn_exp2f(z * fmaf(z * z, c2, c1));
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// Compute units of the current device (host; one runtime query per device and
// thread), 0 if the runtime cannot tell.
inline int device_compute_units() {
  constexpr int kMaxDev = 64;
  thread_local int cached[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  if (!cached[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = v;
  }
  return cached[dev];
}

}  // namespace h3k
