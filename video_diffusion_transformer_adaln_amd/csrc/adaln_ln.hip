// AdaLN modulation GEMV and the fused LayerNorm + AdaLN modulation kernel.
//
// Both are bound by HBM bandwidth: the GEMV streams the [6D, C] AdaLN matrix
// once (the modulation precompute of the h3.c memory-techniques page,
// technique 3), and the LayerNorm reads one activation row and writes one.
#include "common.hpp"
#include "kernels.hpp"

namespace h3k {

// ---------------------------------------------------------------------------
// mod[row] = sum_k W[row, k] c[k] + b[row].  One wave per GEMV_ROWS output
// rows, 16-byte loads along k (the rows' loads of several iterations in
// flight per lane: one row per wave left the HBM stream latency-bound at
// ~3.7 TB/s).  c is read straight from global memory (it is small and stays
// in the L1/L2 caches), so a workgroup starts streaming W at once; W is read
// with nontemporal loads (read once: 50 -> 47 us for 30720 x 5120 bf16).
// The sum order is fixed by (lane, iteration), so results are deterministic.
constexpr int GEMV_ROWS = 4;
template <typename T>
__global__ __launch_bounds__(256) void adaln_gemv_kernel(const T* __restrict__ w, const T* __restrict__ b,
                                                         const T* __restrict__ c, float* __restrict__ mod,
                                                         int rows, int cols) {
  constexpr int RW = GEMV_ROWS;
  const int lane = threadIdx.x % kWave;
  const int row0 = (blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave) * RW;
  if (row0 >= rows) return;
  constexpr int V = 16 / sizeof(T);
  const T* wr[RW];
  float acc[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    wr[r] = w + (int64_t)min(row0 + r, rows - 1) * cols;
    acc[r] = 0.f;
  }
#pragma unroll 8
  for (int k0 = lane * V; k0 < cols; k0 += kWave * V) {
    u32x4 raw[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) raw[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wr[r] + k0));
    const u32x4 craw = *reinterpret_cast<const u32x4*>(c + k0);
    const T* ce = reinterpret_cast<const T*>(&craw);
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const T* e = reinterpret_cast<const T*>(&raw[r]);
#pragma unroll
      for (int j = 0; j < V; ++j) acc[r] += to_f32(e[j]) * to_f32(ce[j]);
    }
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const float a = wave_sum(acc[r]);
    if (lane == 0 && row0 + r < rows) mod[row0 + r] = a + (b ? to_f32(b[row0 + r]) : 0.f);
  }
}

hipError_t launch_adaln_gemv(DType dt, int rows, int cols, const void* w, const void* b, const void* c,
                             float* mod, hipStream_t stream) {
  const dim3 block(256), grid((rows + 4 * GEMV_ROWS - 1) / (4 * GEMV_ROWS));
  if (dt == kBF16)
    adaln_gemv_kernel<bf16><<<grid, block, 0, stream>>>((const bf16*)w, (const bf16*)b, (const bf16*)c, mod, rows,
                                                        cols);
  else
    adaln_gemv_kernel<float><<<grid, block, 0, stream>>>((const float*)w, (const float*)b, (const float*)c, mod,
                                                         rows, cols);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// out = LN(x) (1 + scale) + shift.  One wave per row (two rows per wave, for
// fewer shift/scale reads, measured 7 % slower: half the waves fit); the row is
// held in registers (MAXC 16-byte chunks per lane, in its storage type,
// widened to fp32 in each pass, which keeps the register count and so the
// number of rows in flight per CU up), so mean and the biased variance are
// two exact passes over registers, each closed by a wave reduction.  Rows
// are read and the results written with nontemporal accesses (each byte is
// touched once; measured on MI355X, 101 -> 90 us a call at D = 5120 with the
// register change below).
template <int MAXC> constexpr int ln_rows() { return 1; }   // rows per wave
template <typename T, int MAXC>
__global__ __launch_bounds__(256) void ln_modulate_kernel(const T* __restrict__ x, int64_t ldx,
                                                          const float* __restrict__ shift,
                                                          const float* __restrict__ scale, T* __restrict__ out,
                                                          int64_t ldo, int n, int D, float eps) {
  constexpr int V = 16 / sizeof(T);
  constexpr int R = ln_rows<MAXC>();
  const int lane = threadIdx.x % kWave;
  const int row0 = (blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave) * R;
  if (row0 >= n) return;
  const int chunks = D / V;
  u32x4 raw[R][MAXC];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const T* xr = x + (int64_t)min(row0 + r, n - 1) * ldx;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int ch = lane + i * kWave;
      raw[r][i] = ch < chunks ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + ch * V))
                              : u32x4{0, 0, 0, 0};
    }
  }
  // element j of chunk i, widened to fp32.  For bf16 the widening (a shift or
  // a mask of the 32-bit word) is an opaque instruction, so each pass redoes
  // it instead of keeping a widened copy of the row live: 120 -> 90 registers
  // for D = 5120, five waves per SIMD instead of four.
  auto elem = [&](int r, int i, int j) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t w = raw[r][i][j >> 1];
      float v;
      if (j & 1) asm volatile("v_and_b32 %0, 0xffff0000, %1" : "=v"(v) : "v"(w));
      else asm volatile("v_lshlrev_b32 %0, 16, %1" : "=v"(v) : "v"(w));
      return v;
    } else {
      return to_f32(reinterpret_cast<const T*>(&raw[r][i])[j]);
    }
  };
  float mean[R], rstd[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int ch = lane + i * kWave;
      if (ch < chunks) {
#pragma unroll
        for (int j = 0; j < V; ++j) s += elem(r, i, j);
      }
    }
    mean[r] = wave_sum(s) / (float)D;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int ch = lane + i * kWave;
      if (ch < chunks) {
#pragma unroll
        for (int j = 0; j < V; ++j) { const float dlt = elem(r, i, j) - mean[r]; ss += dlt * dlt; }
      }
    }
    rstd[r] = 1.0f / sqrtf(wave_sum(ss) / (float)D + eps);
  }
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int ch = lane + i * kWave;
    if (ch < chunks) {
      const int c0 = ch * V;
      float sc[V], sh[V];
#pragma unroll
      for (int j = 0; j < V; ++j) { sc[j] = 1.0f + scale[c0 + j]; sh[j] = shift[c0 + j]; }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (row0 + r >= n) break;
        u32x4 res;
        T* e = reinterpret_cast<T*>(&res);
#pragma unroll
        for (int j = 0; j < V; ++j) e[j] = from_f32<T>((elem(r, i, j) - mean[r]) * rstd[r] * sc[j] + sh[j]);
        __builtin_nontemporal_store(res, reinterpret_cast<u32x4*>(out + (int64_t)(row0 + r) * ldo + c0));
      }
    }
  }
}

template <typename T, int MAXC>
static void ln_launch(int n, int D, float eps, const void* x, int64_t ldx, const float* shift,
                      const float* scale, void* out, int64_t ldo, hipStream_t stream) {
  const int rows_per_block = 4 * ln_rows<MAXC>();
  ln_modulate_kernel<T, MAXC><<<dim3((n + rows_per_block - 1) / rows_per_block), dim3(256), 0, stream>>>(
      (const T*)x, ldx, shift, scale, (T*)out, ldo, n, D, eps);
}

template <typename T>
static void ln_dispatch(int n, int D, float eps, const void* x, int64_t ldx, const float* shift,
                        const float* scale, void* out, int64_t ldo, hipStream_t stream) {
  constexpr int V = 16 / sizeof(T);
  const int per_lane = (D / V + kWave - 1) / kWave;
  if (per_lane <= 2)       ln_launch<T, 2>(n, D, eps, x, ldx, shift, scale, out, ldo, stream);
  else if (per_lane <= 4)  ln_launch<T, 4>(n, D, eps, x, ldx, shift, scale, out, ldo, stream);
  else if (per_lane <= 6)  ln_launch<T, 6>(n, D, eps, x, ldx, shift, scale, out, ldo, stream);
  else if (per_lane <= 8)  ln_launch<T, 8>(n, D, eps, x, ldx, shift, scale, out, ldo, stream);
  else if (per_lane <= 10) ln_launch<T, 10>(n, D, eps, x, ldx, shift, scale, out, ldo, stream);
  else if (per_lane <= 12) ln_launch<T, 12>(n, D, eps, x, ldx, shift, scale, out, ldo, stream);
  else if (per_lane <= 16) ln_launch<T, 16>(n, D, eps, x, ldx, shift, scale, out, ldo, stream);
  else                     ln_launch<T, 32>(n, D, eps, x, ldx, shift, scale, out, ldo, stream);
}

hipError_t launch_ln_modulate(DType dt, int n, int D, float eps, const void* x, int64_t ldx,
                              const float* shift, const float* scale, void* out, int64_t ldo,
                              hipStream_t stream) {
  if (dt == kBF16) ln_dispatch<bf16>(n, D, eps, x, ldx, shift, scale, out, ldo, stream);
  else ln_dispatch<float>(n, D, eps, x, ldx, shift, scale, out, ldo, stream);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// In-place 3D RoPE of a bf16 matrix (rows = tokens): one thread per 4
// consecutive columns (two rotation pairs), 8-byte loads and stores.
__global__ __launch_bounds__(256) void rope_kernel(bf16* __restrict__ x, int64_t ldx, int64_t n, int64_t quads,
                                                   RopeGeom g) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n * quads) return;
  const int64_t row = idx / quads;
  const int c = (int)(idx - row * quads) * 4;
  bf16* px = x + row * ldx + c;
  u32x2 raw = *reinterpret_cast<const u32x2*>(px);
  bf16* e = reinterpret_cast<bf16*>(&raw);
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = static_cast<float>(e[i]);
  const int j = c % g.head_dim;
  rope_rotate(v[0], v[1], (int)row, j, g);
  rope_rotate(v[2], v[3], (int)row, j + 2, g);
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = static_cast<bf16>(v[i]);
  *reinterpret_cast<u32x2*>(px) = raw;
}

hipError_t launch_rope(int64_t n, int64_t cols, int head_dim, int height, int width, float spatial, void* x,
                       int64_t ldx, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t quads = cols / 4;
  const int64_t blocks = (n * quads + 255) / 256;
  rope_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>((bf16*)x, ldx, n, quads,
                                                                 RopeGeom{head_dim, height, width, spatial});
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-row symmetric int8 quantiser: s = max|w| / 127, q = clamp(rint(w/s)).
// One wave per row, four rows per workgroup.  Each lane handles groups of 8
// consecutive elements (one 16-byte load for bf16, two for fp32; one 8-byte
// store of 8 int8): pass 1 takes the absmax (exact, order-independent), pass 2
// re-reads the row (mostly from L2) and does one correctly rounded fp32
// division per element and round-half-to-even.  Rows whose length is not a
// multiple of 8 (or not 16-byte aligned as a result) take a per-element path.
// The vector paths divide through the reciprocal with an exact fallback
// (quant8), which gives the same bits as the division.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
  static __device__ __forceinline__ void load(const bf16* p, float (&v)[8]) {
    const u32x4 r = *reinterpret_cast<const u32x4*>(p);
    const bf16* e = reinterpret_cast<const bf16*>(&r);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = static_cast<float>(e[i]);
  }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float (&v)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
};

__device__ __forceinline__ int quant1(float v, float s) {
  if (s == 0.f) return 0;
  return (int)fminf(127.f, fmaxf(-127.f, rintf(v / s)));
}

// The same value through the reciprocal, with a rounding test in the manner
// of Ziv (exact result from a fast approximation unless it lies near a
// rounding boundary): y = v * r with r = v_rcp_f32(s) (within 1 ulp of 1/s)
// is within 2^-15 of v / s, and the correctly rounded quotient fl(v / s)
// within 2^-18 of it, since |v / s| <= 127 (1 + 2^-23) < 128.  When y lies
// more than 2^-12 from every k + 1/2, rint(y) = rint(fl(v / s)); otherwise
// (or when y is not finite, e.g. for a subnormal s) it returns false and the
// caller takes quant1's correctly rounded division.  For s > 0 only.
__device__ __forceinline__ bool quant_fast(float v, float r, int& q) {
  const float y = v * r;
  const float f = y - floorf(y);
  if (!(fabsf(f - 0.5f) > 0x1p-12f)) return false;
  q = (int)fminf(127.f, fmaxf(-127.f, rintf(y)));
  return true;
}
// eight values of one scale: the fast path, then the exact division for any
// value the rounding test sends back (rare: about 2^-11 of them)
__device__ __forceinline__ void quant8(const float (&v)[8], float s, uint32_t& lo, uint32_t& hi) {
  int q[8];
  bool ok = s > 0.f;
  const float r = __builtin_amdgcn_rcpf(s);
#pragma unroll
  for (int i = 0; i < 8; ++i) ok = quant_fast(v[i], r, q[i]) && ok;
  if (!ok) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = quant1(v[i], s);
  }
  lo = hi = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t b = (uint32_t)(q[i] & 0xff);
    if (i < 4) lo |= b << (8 * i);
    else hi |= b << (8 * (i - 4));
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void quantize_int8_kernel(const T* __restrict__ w, int64_t rows, int64_t cols,
                                                            int8_t* __restrict__ q, float* __restrict__ scales) {
  const int lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const T* wr = w + row * cols;
  int8_t* qr = q + row * cols;
  if constexpr (!VEC) {
    float mx = 0.f;
    for (int64_t k = lane; k < cols; k += kWave) mx = fmaxf(mx, fabsf(to_f32(wr[k])));
    mx = wave_max(mx);
    const float s = mx / 127.0f;
    if (lane == 0) scales[row] = s;
    for (int64_t k = lane; k < cols; k += kWave) qr[k] = (int8_t)quant1(to_f32(wr[k]), s);
    return;
  }
  const int64_t groups = cols / 8;
  float mx = 0.f;
#pragma unroll 4
  for (int64_t g = lane; g < groups; g += kWave) {
    float v[8];
    Vec8<T>::load(wr + g * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(v[i]));
  }
  mx = wave_max(mx);
  const float s = mx / 127.0f;
  if (lane == 0) scales[row] = s;
#pragma unroll 4
  for (int64_t g = lane; g < groups; g += kWave) {
    float v[8];
    Vec8<T>::load(wr + g * 8, v);
    uint32_t lo, hi;
    quant8(v, s, lo, hi);
    *reinterpret_cast<u32x2*>(qr + g * 8) = u32x2{lo, hi};
  }
}

// Group-wise variant: every block of G consecutive weights of a row (G in
// {32, 64, 128}, cols a multiple of G) gets its own scale, s = max|w| / 127
// over the block, and q = clamp(rint(w / s)) as above.  One wave per row;
// lane l holds the 8 consecutive values of chunk (it*64 + l), so a group is
// G/8 adjacent lanes and its maximum is a butterfly over those lanes.  The
// values stay in registers: one pass over the row.
template <typename T, int G>
__global__ __launch_bounds__(256) void quantize_int8_groups_kernel(const T* __restrict__ w, int64_t rows,
                                                                   int64_t cols, int8_t* __restrict__ q,
                                                                   float* __restrict__ scales) {
  constexpr int LG = G / 8;                    // lanes per group
  const int lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const T* wr = w + row * cols;
  int8_t* qr = q + row * cols;
  float* sr = scales + row * (cols / G);
  const int64_t chunks = cols / 8;             // a multiple of LG
  for (int64_t c0 = 0; c0 < chunks; c0 += kWave) {
    const int64_t c = c0 + lane;
    if (c >= chunks) break;                    // whole groups drop out together
    float v[8];
    Vec8<T>::load(wr + c * 8, v);
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(v[i]));
#pragma unroll
    for (int off = LG / 2; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
    const float sc = mx / 127.0f;
    if (lane % LG == 0) sr[c / LG] = sc;
    uint32_t lo, hi;
    quant8(v, sc, lo, hi);
    *reinterpret_cast<u32x2*>(qr + c * 8) = u32x2{lo, hi};
  }
}

template <typename T>
static void launch_groups(const T* w, int64_t rows, int64_t cols, int group, int8_t* q, float* scales,
                          hipStream_t stream) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (group == 32) quantize_int8_groups_kernel<T, 32><<<grid, dim3(256), 0, stream>>>(w, rows, cols, q, scales);
  else if (group == 64) quantize_int8_groups_kernel<T, 64><<<grid, dim3(256), 0, stream>>>(w, rows, cols, q, scales);
  else quantize_int8_groups_kernel<T, 128><<<grid, dim3(256), 0, stream>>>(w, rows, cols, q, scales);
}

hipError_t launch_quantize_int8_groups(DType dt, const void* w, int64_t rows, int64_t cols, int group, int8_t* q,
                                       float* scales, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (dt == kBF16) launch_groups((const bf16*)w, rows, cols, group, q, scales, stream);
  else launch_groups((const float*)w, rows, cols, group, q, scales, stream);
  return hipGetLastError();
}

// One-pass variants: the row stays in registers between the absmax and the
// quantisation, so it is read from memory once (the two-pass kernel's second
// read of a 27 KB row of u misses the L2 once many rows are in flight).  A
// row of up to 64 MAXC chunks of 8 values takes one wave (WAVES = 1, four
// rows per workgroup); longer rows take the four waves of a workgroup
// (WAVES = 4, their maxima met in LDS), so that each lane holds at most 16
// chunks and enough rows stay in flight per CU.  The row is read and the
// codes written with nontemporal accesses (each byte once; the u rows of
// 22680 x 13824 bf16 180 -> 168 us on MI355X).
template <typename T, int MAXC, int WAVES>
__global__ __launch_bounds__(256) void quantize_int8_rows_kernel(const T* __restrict__ w, int64_t rows,
                                                                 int64_t cols, int8_t* __restrict__ q,
                                                                 float* __restrict__ scales) {
  constexpr int W = 16 / sizeof(T);            // 16-byte words per 8 values
  constexpr int LANES = WAVES * kWave;         // lanes per row
  __shared__ float wmax[4];
  const int lane = threadIdx.x % LANES;
  const int64_t row = (int64_t)blockIdx.x * (256 / LANES) + threadIdx.x / LANES;
  if (WAVES == 1 && row >= rows) return;       // (a 4-wave workgroup is one whole row)
  const T* wr = w + row * cols;
  int8_t* qr = q + row * cols;
  const int groups = (int)(cols / 8);
  u32x4 raw[MAXC][8 / W];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int g = lane + i * LANES;
#pragma unroll
    for (int h = 0; h < 8 / W; ++h)
      raw[i][h] = g < groups ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wr + g * 8 + h * W))
                             : u32x4{0, 0, 0, 0};
  }
  auto vals = [&](int i, float (&v)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = to_f32(reinterpret_cast<const T*>(&raw[i][j / W])[j % W]);
  };
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    float v[8];
    vals(i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(v[j]));
  }
  mx = wave_max(mx);
  if constexpr (WAVES > 1) {
    if (threadIdx.x % kWave == 0) wmax[threadIdx.x / kWave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  }
  const float s = mx / 127.0f;
  if (lane == 0) scales[row] = s;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int g = lane + i * LANES;
    if (g < groups) {
      float v[8];
      vals(i, v);
      uint32_t lo, hi;
      quant8(v, s, lo, hi);
      __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(qr + (int64_t)g * 8));
    }
  }
}

template <typename T>
static bool launch_rows_one_pass(const T* w, int64_t rows, int64_t cols, int8_t* q, float* scales,
                                 hipStream_t stream) {
  if (cols % 8) return false;
  const int64_t per_wave = (cols / 8 + kWave - 1) / kWave, per_wg = (cols / 8 + 255) / 256;
  const dim3 g1((unsigned)((rows + 3) / 4)), g4((unsigned)rows);
  if (per_wave <= 4) quantize_int8_rows_kernel<T, 4, 1><<<g1, dim3(256), 0, stream>>>(w, rows, cols, q, scales);
  else if (per_wave <= 8) quantize_int8_rows_kernel<T, 8, 1><<<g1, dim3(256), 0, stream>>>(w, rows, cols, q, scales);
  else if (per_wave <= 16) quantize_int8_rows_kernel<T, 16, 1><<<g1, dim3(256), 0, stream>>>(w, rows, cols, q, scales);
  else if (per_wg <= 8) quantize_int8_rows_kernel<T, 8, 4><<<g4, dim3(256), 0, stream>>>(w, rows, cols, q, scales);
  else if (per_wg <= 16) quantize_int8_rows_kernel<T, 16, 4><<<g4, dim3(256), 0, stream>>>(w, rows, cols, q, scales);
  else return false;
  return true;
}

hipError_t launch_quantize_int8(DType dt, const void* w, int64_t rows, int64_t cols, int8_t* q, float* scales,
                                hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4));
  const bool vec = cols % 8 == 0;   // row starts then stay 16-byte aligned (w and q are)
  if (dt == kBF16) {
    if (launch_rows_one_pass((const bf16*)w, rows, cols, q, scales, stream)) return hipGetLastError();
    if (vec) quantize_int8_kernel<bf16, true><<<grid, dim3(256), 0, stream>>>((const bf16*)w, rows, cols, q, scales);
    else quantize_int8_kernel<bf16, false><<<grid, dim3(256), 0, stream>>>((const bf16*)w, rows, cols, q, scales);
  } else {
    if (launch_rows_one_pass((const float*)w, rows, cols, q, scales, stream)) return hipGetLastError();
    if (vec) quantize_int8_kernel<float, true><<<grid, dim3(256), 0, stream>>>((const float*)w, rows, cols, q, scales);
    else quantize_int8_kernel<float, false><<<grid, dim3(256), 0, stream>>>((const float*)w, rows, cols, q, scales);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Token reduction ([H3-review] knob list: video tokens paired two by two along
// rows in the middle layers).  merge: xm[m] = (x[2m] + x[2m+1]) / 2, exact in
// fp32 for bf16 inputs, one rounding at the store.  unmerge: out[2m+j] =
// entry[2m+j] + (xm[m] - merge(entry)[m]), where merge(entry) is recomputed
// with the very same operations, so its rounded value equals what the merge
// stored and unchanged reduced layers give back `entry` bit for bit.  One
// thread per 8 columns of a token pair; out may alias entry (each thread
// reads its own pair before writing it).
template <typename T> struct Vec8Store;
template <> struct Vec8Store<bf16> {
  static __device__ __forceinline__ void store(bf16* p, const float (&v)[8]) {
    u32x4 r;
    bf16* e = reinterpret_cast<bf16*>(&r);
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = static_cast<bf16>(v[i]);
    *reinterpret_cast<u32x4*>(p) = r;
  }
};
template <> struct Vec8Store<float> {
  static __device__ __forceinline__ void store(float* p, const float (&v)[8]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
};
template <typename T> __device__ __forceinline__ float round_to(float v) { return static_cast<float>(static_cast<T>(v)); }

template <typename T>
__global__ __launch_bounds__(256) void token_merge_kernel(const T* __restrict__ x, int64_t ldx, T* __restrict__ xm,
                                                          int64_t ldm, int64_t pairs, int64_t oct) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= pairs * oct) return;
  const int64_t m = idx / oct;
  const int64_t c = (idx - m * oct) * 8;
  float a[8], b[8], r[8];
  Vec8<T>::load(x + (2 * m) * ldx + c, a);
  Vec8<T>::load(x + (2 * m + 1) * ldx + c, b);
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (a[i] + b[i]) * 0.5f;
  Vec8Store<T>::store(xm + m * ldm + c, r);
}

template <typename T>
__global__ __launch_bounds__(256) void token_unmerge_kernel(const T* entry, int64_t lde, const T* __restrict__ xm,
                                                            int64_t ldm, T* out, int64_t ldo, int64_t pairs,
                                                            int64_t oct) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= pairs * oct) return;
  const int64_t m = idx / oct;
  const int64_t c = (idx - m * oct) * 8;
  float a[8], b[8], y[8];
  Vec8<T>::load(entry + (2 * m) * lde + c, a);
  Vec8<T>::load(entry + (2 * m + 1) * lde + c, b);
  Vec8<T>::load(xm + m * ldm + c, y);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float d = y[i] - round_to<T>((a[i] + b[i]) * 0.5f);
    a[i] += d;
    b[i] += d;
  }
  Vec8Store<T>::store(out + (2 * m) * ldo + c, a);
  Vec8Store<T>::store(out + (2 * m + 1) * ldo + c, b);
}

hipError_t launch_token_merge(DType dt, int64_t n, int64_t D, const void* x, int64_t ldx, void* xm, int64_t ldm,
                              hipStream_t stream) {
  const int64_t pairs = n / 2, oct = D / 8;
  if (pairs == 0) return hipSuccess;
  const dim3 grid((unsigned)((pairs * oct + 255) / 256));
  if (dt == kBF16)
    token_merge_kernel<bf16><<<grid, dim3(256), 0, stream>>>((const bf16*)x, ldx, (bf16*)xm, ldm, pairs, oct);
  else
    token_merge_kernel<float><<<grid, dim3(256), 0, stream>>>((const float*)x, ldx, (float*)xm, ldm, pairs, oct);
  return hipGetLastError();
}

hipError_t launch_token_unmerge(DType dt, int64_t n, int64_t D, const void* entry, int64_t lde, const void* xm,
                                int64_t ldm, void* out, int64_t ldo, hipStream_t stream) {
  const int64_t pairs = n / 2, oct = D / 8;
  if (pairs == 0) return hipSuccess;
  const dim3 grid((unsigned)((pairs * oct + 255) / 256));
  if (dt == kBF16)
    token_unmerge_kernel<bf16><<<grid, dim3(256), 0, stream>>>((const bf16*)entry, lde, (const bf16*)xm, ldm,
                                                               (bf16*)out, ldo, pairs, oct);
  else
    token_unmerge_kernel<float><<<grid, dim3(256), 0, stream>>>((const float*)entry, lde, (const float*)xm, ldm,
                                                                (float*)out, ldo, pairs, oct);
  return hipGetLastError();
}

}  // namespace h3k
