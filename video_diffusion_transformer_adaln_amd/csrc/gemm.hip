// Projection GEMMs of the DiT block: y = epilogue(x W^T), with x the
// activations [m, k] and W the weight [n, k] (both k-contiguous).
//
//  * bf16 path: 256x256x64 workgroup tile, 8 waves (two per SIMD, so one
//    wave's waits overlap the other's MFMAs), each wave a 64x128 sub-tile of
//    v_mfma_f32_16x16x32_bf16 (fp32 accumulators in VGPRs).  Measured on
//    MI355X, streams of the 16x16x32 form hold a 10-14 % higher clock under
//    the power limit than the 32x32x16 form for the same work.  Operands go
//    global -> LDS by direct-to-LDS loads (buffer_load ... lds) into a ring
//    of five 32 KiB operand slots (all 160 KiB of gfx950's LDS), so the
//    activation tile of k-tile t+2 and the weight tile of t+1 are in flight
//    while t is multiplied.  Each load instruction moves 8 whole 128-byte
//    rows: measured on MI355X, half-line (64-byte) row pieces halve the
//    vector-memory return rate, and one k-tile of loads in flight per
//    workgroup cannot cover the loaded L2/Infinity-Cache latency.
//  * int8-weight path (W8A16), same ring: the activation tiles arrive by
//    direct-to-LDS loads, the weight tile is read as int8 (half the bytes)
//    into registers a step before it is widened to bf16 exactly and stored
//    into its slot, one step before it is multiplied on the bf16 MFMA.  The
//    per-output-channel scale is applied to the fp32 accumulator in the
//    epilogue (it factors out of the k-sum); group-wise scales are applied
//    while widening (each 16-weight chunk lies in one group).
//  * int8 x int8 path (row-quantised activations and int8 weights), same
//    ring and fragment reads: a k-tile row is 128 int8 values, and
//    v_mfma_i32_16x16x64_i8 takes a 16-byte chunk per lane like the bf16
//    MFMA (int32 accumulators, exact).  Measured on MI355X, 5 % faster than
//    the 32x32x32 form with the same results.
//  * int8 weights with a staging buffer (inside the block): the weight is
//    widened to bf16 by dequant_int8_kernel first, then the bf16 ring kernel
//    runs with the channel scale in its epilogue (template value SC): the same
//    bits as the W8A16 ring kernel, at the bf16 kernel's speed.
//  * tail split (with a caller scratch, bf16 operands, row-major output): when
//    the last wave of tiles would leave at least half the CUs idle, its tiles
//    are split along k; gemm_tail_kernel sums the fp32 partial tiles in a
//    fixed order and applies the epilogue (tail_split_ways gives S).
//  * fp32 path: a plain LDS-tiled SIMT kernel for the small fp32 workload.
//
// Epilogues (fused, fp32 math, one rounding at the store): bias; bias + GELU
// (tanh form); gated residual r + g * z.  Columns at or beyond split_col are
// written transposed (V^T for the attention kernel).
//
// Output layout trick: the MFMA accumulator holds 4 consecutive rows of its
// A operand per lane, so the operand whose index is contiguous in the output
// is fed as A: weights for the row-major output (4 consecutive features per
// lane), activations for the transposed output (4 consecutive tokens).
#include "common.hpp"
#include "kernels.hpp"

namespace h3k {

struct GemmParams {
  const void* x; int64_t ldx;
  const float* x_scale;   // int8 activations: per-row scales
  const void* w; int64_t ldw;
  const float* w_scale;   // int8 weights: [n] per channel, or [n, k / group] per group
  int group_shift;        // log2 of the group size (group-wise int8 weights)
  RopeGeom rope;          // kEpiBiasRope: rotation of the row-major columns
  const bf16* bias;
  const bf16* residual; int64_t ldr;
  const float* gate;
  bf16* y; int64_t ldy;
  bf16* yt; int64_t ldyt;
  int64_t split_col;
  int64_t scale_cols;     // columns < scale_cols are multiplied by col_scale after the bias
  float col_scale;
  int m, n, k;
  int tiles_m, tiles_n;
  // Tail split (bf16 x bf16, row-major output): tiles full_tiles .. of the
  // tile order below are each split along k into tail_split workgroups that
  // store fp32 partial tiles to part; gemm_tail_kernel finishes them.
  int full_tiles, tail_split;
  float* part;
};

constexpr int BM = 256, BN = 256;


// Signed byte B of v as fp32 (one v_cvt_f32_i32 with a sign-extended SDWA
// byte select).
template <int B> __device__ __forceinline__ float sbyte_f32(uint32_t v) {
  float r;
  if constexpr (B == 0)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(v));
  else if constexpr (B == 1)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(v));
  else if constexpr (B == 2)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(v));
  else
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(v));
  return r;
}
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {static_cast<bf16>(a), static_cast<bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
// 8 int8 -> 8 bf16, exact (|q| <= 127 fits bf16's 8-bit significand): each
// byte converted to fp32 and rounded to bf16 (no rounding occurs), 1.5
// vector instructions per value.  With SCALED, bf16(q * s): the product is
// rounded once to fp32 (q has 8 significant bits, so q * s is exact unless s
// is subnormal) and then to bf16.
template <bool SCALED>
__device__ __forceinline__ u32x4 i8x8_to_bf16(const u32x2& q, float s) {
  auto f = [&](float v) { return SCALED ? v * s : v; };
  u32x4 o;
  o[0] = pack_bf16(f(sbyte_f32<0>(q[0])), f(sbyte_f32<1>(q[0])));
  o[1] = pack_bf16(f(sbyte_f32<2>(q[0])), f(sbyte_f32<3>(q[0])));
  o[2] = pack_bf16(f(sbyte_f32<0>(q[1])), f(sbyte_f32<1>(q[1])));
  o[3] = pack_bf16(f(sbyte_f32<2>(q[1])), f(sbyte_f32<3>(q[1])));
  return o;
}

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zero, which masks the ragged edges of the token and feature axes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Accumulator quads.  A wave's 64x128 sub-tile of 16x16 MFMA tiles leaves
// each lane 32 quads: four consecutive A-rows (features of the row-major
// output, tokens of the transposed one) at one B-row.  Quad q (0..7) of
// 32-row B block jb is acc[I][2 jb + h] (I = q/2, h = q%2), at A-row
// a_row0 + ai and B-row b_row0 + 32 jb + br with ai = 16 I + 4 (lane/16),
// br = 16 h + lane%16.
__device__ __forceinline__ void quad(const f32x4 (&acc)[4][8], int jb, int q, int lane, float (&v)[4], int& ai,
                                     int& br) {
  const int I = q >> 1, h = q & 1;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = acc[I][2 * jb + h][e];
  ai = 16 * I + 4 * (lane >> 4);
  br = 16 * h + (lane & 15);
}

// Epilogue math, fp32, one bf16 rounding at the store.
// Row-major output, first step: features f..f+3 of token t, channel scale and
// bias, then the column scale (the attention scale folded into q; f..f+3 lie
// on one side of scale_cols, a multiple of 8).  Channel scale and bias are
// one explicit fma (a v * s + b the compiler would be free to fuse or not,
// which would let kernels with the same arithmetic round differently).
__device__ __forceinline__ float scale_add(float v, float s, float b, bool has_bias) {
  return has_bias ? __builtin_fmaf(v, s, b) : v * s;
}
template <bool W8>
__device__ __forceinline__ void scale_bias4(const GemmParams& p, float (&v)[4], int f) {
  const float cs = (int64_t)f < p.scale_cols ? p.col_scale : 1.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float b = p.bias ? static_cast<float>(p.bias[f + e]) : 0.0f;
    if constexpr (W8) v[e] = scale_add(v[e], p.w_scale[f + e], b, p.bias != nullptr);
    else if (p.bias) v[e] += b;
    v[e] *= cs;
  }
}
// The ring kernel's epilogue takes a lane's bias and channel-scale values from
// registers, read together once per tile (EpiConsts): read per quad, each
// read and its wait in turn, they cost about as much as the tile's stores
// (measured on MI355X: 8-12 % of a projection GEMM with k = 5120).
// Row-major output: feature feat0 + a_row0 + 16 I + 4 (lane/16) + e at
// [4 I + e], and cs[I] its column scale; transposed output: feature feat0 +
// b_row0 + 32 jb + 16 h + lane%16 at [2 jb + h].  s holds the channel scales
// where they apply (zero otherwise).  Without a bias, b holds -0: x + (-0) = x and
// fma(x, s, -0) = x s for every x, so the bias is added unconditionally.
struct EpiConsts {
  float b[16];
  float s[16];
  float cs[4];
};
template <bool SCALE>
__device__ __forceinline__ void load_epi_consts(const GemmParams& p, int feat0, int a_row0, int b_row0, bool trans,
                                                int lane, EpiConsts& c) {
  // buffer reads: a null bias (or no scales) reads as zero, and so do
  // features >= n, which are never stored
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.bias, p.bias ? (uint32_t)p.n * 2u : 0u);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.w_scale, SCALE ? (uint32_t)p.n * 4u : 0u);
  const uint32_t sign = p.bias ? 0u : 0x80000000u;
  auto lo = [sign](uint32_t w) { return __builtin_bit_cast(float, (w << 16) | sign); };
  auto hi = [sign](uint32_t w) { return __builtin_bit_cast(float, (w & 0xffff0000u) | sign); };
  // Both branches read into locals first and then write every member in the
  // same order, so that the compiler can merge the two sets of writes
  // element by element (a mismatched order makes it index the struct, which
  // then lives in scratch memory).
  float b[16], sc[16], cs[4];
  if (!trans) {
    u32x2 bw[4];
    u32x4 sw[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const uint32_t f = (uint32_t)(feat0 + a_row0 + 16 * I + 4 * (lane >> 4));
      bw[I] = __builtin_amdgcn_raw_buffer_load_b64(rb, f * 2u, 0, 0);
      if constexpr (SCALE) sw[I] = __builtin_amdgcn_raw_buffer_load_b128(rs, f * 4u, 0, 0);
      cs[I] = (int64_t)f < p.scale_cols ? p.col_scale : 1.0f;
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const uint32_t w0 = bw[I][0], w1 = bw[I][1];
      b[4 * I + 0] = lo(w0);
      b[4 * I + 1] = hi(w0);
      b[4 * I + 2] = lo(w1);
      b[4 * I + 3] = hi(w1);
      // each element copied out before the cast: this compiler reads a
      // bit-cast vector element such as v[e] at element 0's address
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = SCALE ? (uint32_t)sw[I][e] : 0u;
        sc[4 * I + e] = __builtin_bit_cast(float, w);
      }
    }
  } else {
    uint32_t bw[8], sw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t f = (uint32_t)(feat0 + b_row0 + 32 * (i >> 1) + 16 * (i & 1) + (lane & 15));
      bw[i] = __builtin_amdgcn_raw_buffer_load_b16(rb, f * 2u, 0, 0);
      sw[i] = SCALE ? __builtin_amdgcn_raw_buffer_load_b32(rs, f * 4u, 0, 0) : 0u;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      b[i] = i < 8 ? lo(bw[i & 7]) : 0.0f;
      sc[i] = i < 8 ? __builtin_bit_cast(float, sw[i & 7]) : 0.0f;
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) cs[I] = 1.0f;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    c.b[i] = b[i];
    c.s[i] = sc[i];
  }
#pragma unroll
  for (int I = 0; I < 4; ++I) c.cs[I] = cs[I];
}
// scale_bias4 with the values of quad row I from EpiConsts (the same
// arithmetic); with PRE false they are read from memory instead
template <bool W8, bool PRE>
__device__ __forceinline__ void scale_bias4c(const GemmParams& p, float (&v)[4], int f, const EpiConsts& ec, int I) {
  if constexpr (!PRE) {
    scale_bias4<W8>(p, v, f);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = (W8 ? __builtin_fmaf(v[e], ec.s[4 * I + e], ec.b[4 * I + e]) : v[e] + ec.b[4 * I + e]) * ec.cs[I];
  }
}
// bias and channel scale of transposed-output feature f (EpiConsts index i)
template <bool W8, bool PRE>
__device__ __forceinline__ void bias_scale1(const GemmParams& p, int f, const EpiConsts& ec, int i, float& bb,
                                            float& sc) {
  if constexpr (PRE) {
    bb = ec.b[i];
    sc = W8 ? ec.s[i] : 1.0f;
  } else {
    bb = p.bias ? static_cast<float>(p.bias[f]) : -0.0f;   // as in EpiConsts
    sc = W8 ? p.w_scale[f] : 1.0f;
  }
}
// Second step: the activation, rotation or gated residual (r + g z as one
// explicit fma, for the reason given at scale_add).
template <int EPI>
__device__ __forceinline__ void epilogue4(const GemmParams& p, float (&v)[4], int t, int f,
                                          const float2* rope_tab = nullptr) {
  if constexpr (EPI == kEpiGelu) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = gelu_tanh(v[e]);
  }
  if constexpr (EPI == kEpiBiasRope) {   // features f..f+3 are the pairs (j, j+1), (j+2, j+3) of a head
    const int j = f % p.rope.head_dim;
    if (rope_tab) {
      const int frames = p.m / (p.rope.height * p.rope.width);
      rope_rotate_table(v[0], v[1], t, j, p.rope, frames, rope_tab);
      rope_rotate_table(v[2], v[3], t, j + 2, p.rope, frames, rope_tab);
    } else {
      rope_rotate(v[0], v[1], t, j, p.rope);
      rope_rotate(v[2], v[3], t, j + 2, p.rope);
    }
  }
  if constexpr (EPI == kEpiGatedResidual) {
    const u32x2 rr = *reinterpret_cast<const u32x2*>(p.residual + (int64_t)t * p.ldr + f);
    const bf16* re = reinterpret_cast<const bf16*>(&rr);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(p.gate[f + e], v[e], static_cast<float>(re[e]));
  }
}
__device__ __forceinline__ u32x2 pack4(const float (&v)[4]) {
  u32x2 out;
  bf16* oe = reinterpret_cast<bf16*>(&out);
#pragma unroll
  for (int e = 0; e < 4; ++e) oe[e] = static_cast<bf16>(v[e]);
  return out;
}

// Fused epilogue of one wave's 64x128 accumulator sub-tile, stored straight
// from the accumulator layout (8-byte pieces, 32 rows per instruction); used
// for the tile that straddles split_col.
template <int EPI, bool W8, bool PRE, typename AccT>
__device__ __forceinline__ void store_tile(const GemmParams& p, const AccT& acc, int a_row0, int b_row0, int tok0,
                                           int feat0, bool trans, int lane, const EpiConsts& ec) {
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float v[4];
      int ai, br;
      quad(acc, jb, q, lane, v, ai, br);
      if (!trans) {
        const int f = feat0 + a_row0 + ai;
        const int t = tok0 + b_row0 + jb * 32 + br;
        if (t >= p.m || f >= p.n) continue;
        scale_bias4c<W8, PRE>(p, v, f, ec, q >> 1);
        if ((int64_t)f >= p.split_col) {   // straddling tile: transposed part, bias only
#pragma unroll
          for (int e = 0; e < 4; ++e) p.yt[(int64_t)(f + e - p.split_col) * p.ldyt + t] = static_cast<bf16>(v[e]);
          continue;
        }
        epilogue4<EPI>(p, v, t, f);
        *reinterpret_cast<u32x2*>(p.y + (int64_t)t * p.ldy + f) = pack4(v);
      } else {
        const int t0 = tok0 + a_row0 + ai;
        const int f = feat0 + b_row0 + jb * 32 + br;
        if (f >= p.n || t0 >= p.m) continue;
        float sc, bb;
        bias_scale1<W8, PRE>(p, f, ec, 2 * jb + (q & 1), bb, sc);
        u32x2 out;
        bf16* oe = reinterpret_cast<bf16*>(&out);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          oe[e] = static_cast<bf16>(W8 ? __builtin_fmaf(v[e], sc, bb) : v[e] + bb);
        }
        bf16* dst = p.yt + (int64_t)(f - p.split_col) * p.ldyt + t0;
        if (t0 + 3 < p.m) {
          *reinterpret_cast<u32x2*>(dst) = out;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (t0 + e < p.m) dst[e] = oe[e];
        }
      }
    }
}

// The same epilogue for a tile that lies wholly on one side of split_col,
// staged through LDS so that the global stores are whole 128-byte row
// segments.  The wave's sub-tile, finished in registers as above, goes to
// `stage` (idle operand-ring LDS) in rounds of JR 32-row blocks, each as
// [32 JR B-rows][64 A-values] bf16 (4 JR KiB), 16-byte chunk c of row r at
// chunk c ^ ((r ^ r/8) % 8); each lane then stores 16 bytes, 8 lanes per
// row.  Row-major output: B-rows are tokens and the 64 A-values features;
// transposed output (V^T): B-rows are features and the A-values tokens.
template <int EPI, bool W8, bool PRE, int JR, typename AccT>
__device__ __forceinline__ void store_tile_staged(const GemmParams& p, const AccT& acc, int a_row0, int b_row0,
                                                  int tok0, int feat0, bool trans, int lane, char* stage,
                                                  const EpiConsts& ec, const float2* rope_tab = nullptr) {
  auto swz = [](int r) { return (r ^ (r >> 3)) & 7; };
  // The orientation is the same for the whole tile, so each gets its own
  // unrolled copy of the loops, with no per-quad branch on it.  With the
  // constants in registers, the bias and GELU epilogues read no memory and
  // run on every quad (rows >= m and features >= n are computed from the
  // zero-filled operands and never stored); the rotary and residual ones,
  // and the memory-read constants, keep the bounds test.
  constexpr bool kAll = PRE && (EPI == kEpiBias || EPI == kEpiGelu);
  auto run = [&](auto tr) {
    constexpr bool TR = decltype(tr)::value;
#pragma unroll
    for (int rnd = 0; rnd < 4 / JR; ++rnd) {
#pragma unroll
      for (int jj = 0; jj < JR; ++jj)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int j = rnd * JR + jj;
          float v[4];
          int ai, br;
          quad(acc, j, q, lane, v, ai, br);
          const int brow = jj * 32 + br;
          if constexpr (!TR) {
            const int f = feat0 + a_row0 + ai, t = tok0 + b_row0 + j * 32 + br;
            if (kAll || (t < p.m && f < p.n)) {
              scale_bias4c<W8, PRE>(p, v, f, ec, q >> 1);
              epilogue4<EPI>(p, v, t, f, rope_tab);
            }
          } else {
            const int f = feat0 + b_row0 + j * 32 + br;
            if (PRE || f < p.n) {
              float sc, bb;
              bias_scale1<W8, PRE>(p, f, ec, 2 * j + (q & 1), bb, sc);
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = W8 ? __builtin_fmaf(v[e], sc, bb) : v[e] + bb;
            }
          }
          *reinterpret_cast<u32x2*>(stage + brow * 128 + (((ai >> 3) ^ swz(brow)) << 4) + ((ai >> 2) & 1) * 8) =
              pack4(v);
        }
#pragma unroll
      for (int s8 = 0; s8 < 4 * JR; ++s8) {
        const int row = s8 * 8 + (lane >> 3), c = lane & 7;
        const int brow = rnd * JR * 32 + row;
        const u32x4 val = *reinterpret_cast<const u32x4*>(stage + row * 128 + ((c ^ swz(row)) << 4));
        if constexpr (!TR) {
          const int t = tok0 + b_row0 + brow, f = feat0 + a_row0 + 8 * c;
          if (t < p.m && f < p.n) *reinterpret_cast<u32x4*>(p.y + (int64_t)t * p.ldy + f) = val;
        } else {
          const int f = feat0 + b_row0 + brow, t0 = tok0 + a_row0 + 8 * c;
          if (f < p.n && t0 < p.m) {
            bf16* dst = p.yt + (int64_t)(f - p.split_col) * p.ldyt + t0;
            if (t0 + 7 < p.m) {
              *reinterpret_cast<u32x4*>(dst) = val;
            } else {
              const bf16* ve = reinterpret_cast<const bf16*>(&val);
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (t0 + e < p.m) dst[e] = ve[e];
            }
          }
        }
      }
    }
  };
  if (trans) run(std::true_type{});
  else run(std::false_type{});
}

// Gated residual, row-major: the residual is read in the same coalesced
// pattern as the output is written, so the wave stages z = acc (x scale) +
// bias in fp32 instead, in rounds of JR 32-row blocks (8 JR KiB): row r
// holds 64 fp32 values, 16-byte chunk c at chunk c ^ (r % 16).  Each lane
// then finishes 8 consecutive features of one token: y = r + g * z, one
// rounding.
template <bool W8, bool PRE, int JR, typename AccT>
__device__ __forceinline__ void store_tile_staged_residual(const GemmParams& p, const AccT& acc, int a_row0,
                                                           int b_row0, int tok0, int feat0, int lane, char* stage,
                                                           const EpiConsts& ec) {
  // the lane's 8 gate values, and each round's residual pieces, are read
  // before they are needed, all at once (rows and features clamped into
  // range; what lies outside is never stored)
  const int fg = min(feat0 + a_row0 + 8 * (lane & 7), p.n - 8);
  const f32x4 g0 = *reinterpret_cast<const f32x4*>(p.gate + fg);
  const f32x4 g1 = *reinterpret_cast<const f32x4*>(p.gate + fg + 4);
#pragma unroll
  for (int rnd = 0; rnd < 4 / JR; ++rnd) {
    // one round's residual pieces in registers at a time
    __builtin_amdgcn_sched_barrier(0);
    u32x4 rres[4 * JR];
#pragma unroll
    for (int s8 = 0; s8 < 4 * JR; ++s8) {
      const int t = min(tok0 + b_row0 + rnd * JR * 32 + s8 * 8 + (lane >> 3), p.m - 1);
      rres[s8] = *reinterpret_cast<const u32x4*>(p.residual + (int64_t)t * p.ldr + fg);
    }
#pragma unroll
    for (int jj = 0; jj < JR; ++jj)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = rnd * JR + jj;
        float v[4];
        int ai, br;
        quad(acc, j, q, lane, v, ai, br);
        const int brow = jj * 32 + br;
        const int f = feat0 + a_row0 + ai, t = tok0 + b_row0 + j * 32 + br;
        if (PRE || (t < p.m && f < p.n)) scale_bias4c<W8, PRE>(p, v, f, ec, q >> 1);
        f32x4 z = {v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(stage + brow * 256 + (((ai >> 2) ^ (brow & 15)) << 4)) = z;
      }
#pragma unroll
    for (int s8 = 0; s8 < 4 * JR; ++s8) {
      const int row = s8 * 8 + (lane >> 3), c = lane & 7;
      const int t = tok0 + b_row0 + rnd * JR * 32 + row, f = feat0 + a_row0 + 8 * c;
      const f32x4 z0 = *reinterpret_cast<const f32x4*>(stage + row * 256 + (((2 * c) ^ (row & 15)) << 4));
      const f32x4 z1 = *reinterpret_cast<const f32x4*>(stage + row * 256 + (((2 * c + 1) ^ (row & 15)) << 4));
      if (t < p.m && f < p.n) {
        const bf16* re = reinterpret_cast<const bf16*>(&rres[s8]);
        u32x4 out;
        bf16* oe = reinterpret_cast<bf16*>(&out);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          oe[e] = static_cast<bf16>(__builtin_fmaf(g0[e], z0[e], static_cast<float>(re[e])));
          oe[4 + e] = static_cast<bf16>(__builtin_fmaf(g1[e], z1[e], static_cast<float>(re[4 + e])));
        }
        *reinterpret_cast<u32x4*>(p.y + (int64_t)t * p.ldy + f) = out;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Ring kernel.  bf16 operands arrive by direct-to-LDS loads (buffer_load ...
// lds): no staging registers and no LDS store instructions.  An operand's k-tile is
// [256 rows][128 B], 16-byte chunk c of row r stored at chunk c ^ rswz(r).
// The swizzle is applied on the source side: lane l of a load writes row
// r0 + l/8, chunk l%8, and so fetches logical chunk (l%8) ^ rswz(row).
//
// The swizzle fits the 16x16 fragment reads (lane l: row l%16, chunk
// selected by l/16), measured conflict-free on MI355X (ds_read_b128
// throughput per access pattern) where (r ^ r/8) % 8, conflict-free for
// 32x32 fragments, leaves two-way conflicts.  It is linear in the row bits
// and zero at every multiple of 16 rows.
__device__ __forceinline__ int rswz(int r) { return (r >> 1) & 7; }
constexpr int kSlot = 256 * 128;   // one operand's k-tile of 64: [256 rows][128 B]
constexpr int kSlots = 5;          // 160 KiB
// m-tiles per group in this kernel's tile order (the 32 workgroups resident
// on one XCD then cover 2 m-tiles x 16 n-tiles); measured best of 1..32
constexpr int kRingGroupM = 2;

// Tile `lin` of that order: groups of kRingGroupM m-tiles, m fastest.
__device__ __forceinline__ void tile_origin(const GemmParams& p, int lin, int& tok0, int& feat0) {
  const int per_group = kRingGroupM * p.tiles_n;
  const int group = lin / per_group;
  const int first_m = group * kRingGroupM;
  const int gm = min(p.tiles_m - first_m, kRingGroupM);
  const int in_group = lin - group * per_group;
  tok0 = (first_m + in_group % gm) * BM;
  feat0 = (in_group / gm) * BN;
}

// SC: bf16 weights that are int8 weights widened beforehand (dequant_int8_kernel):
// 1 with per-channel scales (w_scale applied in the epilogue, as for W8), 2
// with group scales (already in the widened values).  The same code as SC = 0
// otherwise; the value only tells the two apart (and in a kernel trace).
template <int EPI, bool I8, bool W8 = false, bool GRP = false, int SC = 0>
__global__ __launch_bounds__(512) void gemm_ring_kernel(GemmParams p) {
  static_assert(!(I8 && W8), "int8 activations take the int8 MFMA path");
  // bf16 MFMA 16x16x32, int8 MFMA 16x16x64: both take a 16-byte chunk of a
  // 128-byte k-tile row per lane, so slots, swizzle and fragment reads are shared
  auto sw = [](int r) { return rswz(r); };
  __shared__ __attribute__((aligned(1024))) char lds[kSlots * kSlot];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // a k-tile is 128 bytes of every operand row: 64 bf16 or 128 int8 values
  constexpr int ES = I8 ? 1 : 2;
  const int nblk = p.tiles_m * p.tiles_n;
  // Whole tiles come first, in the XCD-aware order; with a tail split, block
  // full_tiles + s * tail + j takes k-tiles [s KT / S, (s + 1) KT / S) of tail
  // tile j (S = tail_split ways) and stores its partial tile part_idx.
  int lin, kt0 = 0, KT = p.k / (128 / ES), part_idx = -1;
  if (I8 || W8 || (int)blockIdx.x < p.full_tiles) {
    lin = xcd_remap(blockIdx.x, I8 || W8 ? nblk : p.full_tiles);
  } else {
    const int tail = nblk - p.full_tiles, q = (int)blockIdx.x - p.full_tiles;
    const int j = q % tail, sp = q / tail;
    lin = p.full_tiles + j;
    kt0 = sp * KT / p.tail_split;
    KT = (sp + 1) * KT / p.tail_split - kt0;
    part_idx = j * p.tail_split + sp;
  }
  int tok0, feat0;
  tile_origin(p, lin, tok0, feat0);
  const bool trans = (int64_t)feat0 >= p.split_col;

  // Ring of 5 operand slots; position q holds operand q&1 (0: activations,
  // 1: weights) of k-tile q>>1, in slot q%5.  Loads: instruction j (0..3)
  // of wave w covers rows (8 j + w) * 8 .. +8; sw(lrow + 64 j) == sw(lrow).
  const __amdgpu_buffer_rsrc_t rsx = make_rsrc(p.x, (uint32_t)((uint64_t)p.m * p.ldx * ES));
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(p.w, (uint32_t)((uint64_t)p.n * p.ldw * (W8 ? 1 : ES)));
  const int lrow = wave * 8 + (lane >> 3);
  const uint32_t c16 = (uint32_t)(((lane & 7) ^ sw(lrow)) * 16);
  const uint32_t xo0 = (uint32_t)(tok0 + lrow) * (uint32_t)p.ldx * ES + c16 + (uint32_t)kt0 * 128u;
  const uint32_t wo0 = (uint32_t)(feat0 + lrow) * (uint32_t)p.ldw * ES + c16 + (uint32_t)kt0 * 128u;
  const uint32_t xstep = 64u * (uint32_t)p.ldx * ES, wstep = 64u * (uint32_t)p.ldw * ES;
  // half h (0/1) of position q: instructions 2h, 2h+1; past the end the last
  // k-tile is re-loaded into the (unread) slot so the load counts stay uniform
  auto issue = [&](int q, int h) {
    int kt = q >> 1;
    kt = kt < KT ? kt : KT - 1;
    char* st = lds + (q % kSlots) * kSlot + wave * 1024;
    const uint32_t kb = (uint32_t)kt * 128u;
    const bool isw = q & 1;
    const __amdgpu_buffer_rsrc_t r = isw ? rsw : rsx;
    const uint32_t o0 = (isw ? wo0 : xo0) + kb, step = isw ? wstep : xstep;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * h + jj;
      lds_dma16(r, st + j * 8192, o0 + j * step);
    }
  };

  // int8 weights (W8): global -> registers, widened to bf16 (times the
  // group scale with GRP) on the way into the weight slot, which then holds
  // the same bf16 layout as a direct-to-LDS slot.  Load j (0..3) of a lane:
  // tile row w8_row + 8 j, int8 values 8 (lane%8) .. +8 (logical bf16 chunk
  // lane%8).  Each LDS store then writes 8 whole 128-byte rows, like a
  // direct-to-LDS load: measured on MI355X, ds_write_b128 runs without bank
  // conflicts when every 4 consecutive lanes fill one aligned 64-byte block,
  // and takes 8 extra cycles per instruction when they write 16-byte pieces
  // 32 bytes apart.
  const int w8_row = wave * 32 + (lane >> 3), w8_c = lane & 7;
  const uint32_t w8_off = (uint32_t)(feat0 + w8_row) * (uint32_t)p.ldw + w8_c * 8;
  const uint32_t w8_step = 8u * (uint32_t)p.ldw;
  const int n_groups = GRP ? (p.k >> p.group_shift) : 0;
  const __amdgpu_buffer_rsrc_t rss = make_rsrc(p.w_scale, GRP ? (uint32_t)((uint64_t)p.n * n_groups * 4) : 0u);
  const uint32_t s_off = GRP ? (uint32_t)(feat0 + w8_row) * (uint32_t)n_groups * 4u : 0u;
  const uint32_t s_step = GRP ? 8u * (uint32_t)n_groups * 4u : 0u;
  u32x2 wq[4];
  float wsc[4];
  auto wload = [&](int kt) {
    kt = kt < KT ? kt : KT - 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) wq[j] = __builtin_amdgcn_raw_buffer_load_b64(rsw, w8_off + j * w8_step + kt * 64u, 0, 0);
    if constexpr (GRP) {
      const uint32_t g4 = (uint32_t)((kt * 64 + w8_c * 8) >> p.group_shift) * 4u;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wsc[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rss, s_off + j * s_step + g4, 0, 0));
    }
  };
  auto wput = [&](int kt) {
    char* st = lds + ((2 * kt + 1) % kSlots) * kSlot;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = w8_row + 8 * j;
      *reinterpret_cast<u32x4*>(st + r * 128 + ((w8_c ^ sw(r)) << 4)) = i8x8_to_bf16<GRP>(wq[j], GRP ? wsc[j] : 1.0f);
    }
  };
  // vector-memory loads of one wload (four int8 pieces, and their four group scales)
  constexpr int kW8Loads = GRP ? 8 : 4;

  const int a_row0 = (wave & 3) * 64;
  const int b_row0 = (wave >> 2) * 128;
  // A is the weight (row-major output) or the activation (transposed output)
  const int a_op = trans ? 0 : 1;

  // int32 accumulators (exact) for int8 operands, fp32 for bf16
  using Acc16 = typename std::conditional<I8, i32x4, f32x4>::type;
  Acc16 acc16[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc16[i][j] = Acc16{};

  // 16x16 fragments: 16-row block at row R (a multiple of 16), k-step ks
  // (32 bf16 or 64 int8 values): lane l reads row R + l%16, logical chunk 4 ks + l/16, at
  // physical chunk (4 ks + l/16) ^ sw(l%16) ^ sw(R); sw(R) = sw(16 (block % 4))
  // for the wave's A blocks (a_row0 % 64 == 0) and B blocks (b_row0 % 128 == 0).
  const int xl = lane & 15;
  int lo16[2][4];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int b = 0; b < 4; ++b) lo16[ks][b] = xl * 128 + ((((4 * ks + (lane >> 4)) ^ sw(xl)) ^ sw(16 * b)) << 4);
  // A fragments of k-step ks (4 blocks of 16 rows), B fragments of k-step ks,
  // blocks 4 hb .. 4 hb + 3
  auto load_a16 = [&](int t, int ks, bf16x8 (&fa)[4]) {
    const char* sa = lds + ((2 * t + a_op) % kSlots) * kSlot + a_row0 * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(sa + i * 2048 + lo16[ks][i]);
  };
  auto load_b16 = [&](int t, int ks, int hb, bf16x8 (&fb)[4]) {
    const char* sb = lds + ((2 * t + 1 - a_op) % kSlots) * kSlot + b_row0 * 128 + hb * 8192;
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(sb + j * 2048 + lo16[ks][j]);
  };
  auto mfmas16 = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[4], int hb) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if constexpr (I8)
          acc16[i][4 * hb + j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
              __builtin_bit_cast(i32x4, fa[i]), __builtin_bit_cast(i32x4, fb[j]), acc16[i][4 * hb + j], 0, 0, 0);
        else
          acc16[i][4 * hb + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc16[i][4 * hb + j], 0, 0, 0);
  };

  bf16x8 g0a[4], g1a[4], g0b[4], g1b[4];
  if constexpr (W8) {
    // prologue: k-tile 0 in LDS; the activations (position 2) and the
    // weights of k-tile 1 in flight
    issue(0, 0);
    issue(0, 1);
    wload(0);
    wait_vmcnt<0>();
    wput(0);
    issue(2, 0);
    issue(2, 1);
    wload(1);
    wait_lgkm0();
    wg_barrier();
    // Widening step: the weights of t+1 (loaded a step earlier) go from
    // registers to the slot of the activations of t-1 while MFMAs of t run,
    // and the registers take the weights of t+2.  It runs in the second
    // group of MFMAs, or in the third with group scales (more vector work,
    // measured faster there).  Loads issued after the weights of t+1: the
    // activation loads of one step (4).
    auto widen = [&](int t) {
      wait_vmcnt<4>();
      wput(t + 1);
      wload(t + 2);
    };
    // loads issued after the activations of t+1 by the end of step t: one
    // wload and 4 activation loads, or (group scales) two wloads and 4
    constexpr int kAfterActs = GRP ? 2 * kW8Loads + 4 : kW8Loads + 4;
    for (int t = 0; t < KT; ++t) {
      // the activations of t+2 load into the slot of the weights of t-1 and
      // the widened weights of t+1 go to the slot of the activations of t-1:
      // both slots' readers passed the last barrier
      load_a16(t, 0, g0a);
      load_b16(t, 0, 0, g0b);
      load_b16(t, 0, 1, g1b);
      issue(2 * t + 4, 0);
      mfmas16(g0a, g0b, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!GRP) widen(t);
      load_a16(t, 1, g1a);
      load_b16(t, 1, 0, g0b);
      issue(2 * t + 4, 1);
      mfmas16(g0a, g1b, 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (GRP) widen(t);
      load_b16(t, 1, 1, g1b);
      mfmas16(g1a, g0b, 0);
      __builtin_amdgcn_sched_barrier(0);
      mfmas16(g1a, g1b, 1);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<kAfterActs>();   // activations of t+1 landed; this step's loads may fly
      wait_lgkm0();               // this wave's widened weights of t+1 are in LDS
      wg_barrier();
    }
  } else {
  // prologue: positions 0, 1, 2 in flight; 0 and 1 (k-tile 0) must be complete
  for (int q = 0; q < 3; ++q) {
    issue(q, 0);
    issue(q, 1);
  }
  wait_vmcnt<4>();
  wg_barrier();
  for (int t = 0; t < KT; ++t) {
    // positions 2t+3 (weights of t+1) and 2t+4 (activations of t+2) go to the
    // slots of k-tile t-1, whose readers all passed the last barrier
    load_a16(t, 0, g0a);
    load_b16(t, 0, 0, g0b);
    issue(2 * t + 3, 0);
    load_b16(t, 0, 1, g1b);
    issue(2 * t + 3, 1);
    mfmas16(g0a, g0b, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_a16(t, 1, g1a);
    load_b16(t, 1, 0, g0b);
    issue(2 * t + 4, 0);
    mfmas16(g0a, g1b, 1);
    __builtin_amdgcn_sched_barrier(0);
    load_b16(t, 1, 1, g1b);
    issue(2 * t + 4, 1);
    mfmas16(g1a, g0b, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas16(g1a, g1b, 1);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<4>();   // own loads of k-tile t+1 have landed; activations of t+2 may fly
    wg_barrier();
  }
  }
  // the epilogue's bias and channel scales, read now so that they overlap the
  // last loads' wait (the in-GEMM widening kernels, whose epilogue has no
  // registers to spare for them, read them per quad)
  constexpr bool kScale = W8 ? !GRP : (I8 || SC == 1);
  constexpr bool kPre = !W8;
  EpiConsts ec;
  if constexpr (kPre) load_epi_consts<kScale>(p, feat0, a_row0, b_row0, trans, lane, ec);
  wait_vmcnt<0>();
  if constexpr (!I8 && !W8) {
    if (part_idx >= 0) {   // same for the whole workgroup
      // raw fp32 accumulators: wave w, quad (i, j) and lane l at float4 index
      // part_idx * 16384 + w * 2048 + (8 i + j) * 64 + l (1 KiB per store)
      f32x4* dst = reinterpret_cast<f32x4*>(p.part) + ((int64_t)part_idx << 14) + wave * 2048 + lane;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[(8 * i + j) * 64] = acc16[i][j];
      return;
    }
  }
  // a tile wholly on one side of split_col (features >= n are never stored)
  // stages its epilogue in the ring:
  // every wave's loads (including the clamped re-loads past the last k-tile)
  // have landed once all waves pass this barrier
  const bool staged = trans || (int64_t)feat0 + BN <= p.split_col || p.split_col >= p.n;
  if (staged) wg_barrier();
  char* const stage = lds + wave * 16384;
  // rotary epilogue: (cos, sin) per axis position and pair in the ring's
  // fifth slot, which the staging (slots 0-3) leaves free
  const float2* rope_tab = nullptr;
  if constexpr (EPI == kEpiBiasRope) {
    const int frames = p.m / (p.rope.height * p.rope.width);
    const int n_ent = rope_table_size(p.rope, frames);
    if (staged && !trans && n_ent * (int)sizeof(float2) <= kSlot) {
      float2* tab = reinterpret_cast<float2*>(lds + 4 * kSlot);
      for (int e = tid; e < n_ent; e += 512) tab[e] = rope_table_entry(e, p.rope, frames);
      wait_lgkm0();
      wg_barrier();
      rope_tab = tab;
    }
  }
  if constexpr (I8) {
    // int32 -> fp32 (one rounding), times the activation row scale; the
    // weight channel scale, bias and epilogue follow in store_tile.  The
    // int8 path has no transposed part, so B-rows are tokens: quad j8 of a
    // lane is token b_row0 + 16 j8 + lane%16.
    f32x4 accf[4][8];
#pragma unroll
    for (int j8 = 0; j8 < 8; ++j8) {
      const int t = tok0 + b_row0 + j8 * 16 + (lane & 15);
      const float xs0 = p.x_scale[min(t, p.m - 1)];   // unconditional: the reads go out together
      const float xs = t < p.m ? xs0 : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) accf[i][j8][r] = static_cast<float>(acc16[i][j8][r]) * xs;
    }
    if (staged && EPI == kEpiGatedResidual)
      store_tile_staged_residual<true, true, 2>(p, accf, a_row0, b_row0, tok0, feat0, lane, stage, ec);
    else if (staged) store_tile_staged<EPI, true, true, 4>(p, accf, a_row0, b_row0, tok0, feat0, false, lane, stage, ec);
    else store_tile<EPI, true, true>(p, accf, a_row0, b_row0, tok0, feat0, false, lane, ec);
  } else {
    auto finish = [&](const auto& ac) {
      if (staged && EPI == kEpiGatedResidual && !trans)
        store_tile_staged_residual<kScale, kPre, 2>(p, ac, a_row0, b_row0, tok0, feat0, lane, stage, ec);
      else if (staged)
        store_tile_staged<EPI, kScale, kPre, 4>(p, ac, a_row0, b_row0, tok0, feat0, trans, lane, stage, ec, rope_tab);
      else store_tile<EPI, kScale, kPre>(p, ac, a_row0, b_row0, tok0, feat0, trans, lane, ec);
    };
    finish(acc16);
  }
}

// ---------------------------------------------------------------------------
// Second kernel of a tail split: each thread sums the S partial values of one
// accumulator quad (4 consecutive features of one token) in split order, then
// applies the ring kernel's epilogue (scale_bias4, epilogue4, one rounding).
// Row-major output only (the launcher splits no tile with a transposed part).
template <int EPI, int SC>
__global__ __launch_bounds__(256) void gemm_tail_kernel(GemmParams p) {
  const int tail = p.tiles_m * p.tiles_n - p.full_tiles, S = p.tail_split;
  const int idx = blockIdx.x * 256 + threadIdx.x;   // quad index over the tail tiles
  const int j = idx >> 14, e4 = idx & 16383;
  if (j >= tail) return;
  int tok0, feat0;
  tile_origin(p, p.full_tiles + j, tok0, feat0);
  // the layout the ring kernel stored: wave w, quad (i, jb), lane l
  const int w = e4 >> 11, i = (e4 >> 9) & 3, jb = (e4 >> 6) & 7, l = e4 & 63;
  const int f = feat0 + (w & 3) * 64 + 16 * i + 4 * (l >> 4);
  const int t = tok0 + (w >> 2) * 128 + 16 * jb + (l & 15);
  const f32x4* src = reinterpret_cast<const f32x4*>(p.part) + ((int64_t)j * S << 14) + e4;
  f32x4 a = __builtin_nontemporal_load(src);
  for (int sp = 1; sp < S; ++sp) a += __builtin_nontemporal_load(src + ((int64_t)sp << 14));
  if (t >= p.m || f >= p.n) return;
  float v[4] = {a[0], a[1], a[2], a[3]};
  scale_bias4<SC == 1>(p, v, f);
  epilogue4<EPI>(p, v, t, f);
  *reinterpret_cast<u32x2*>(p.y + (int64_t)t * p.ldy + f) = pack4(v);
}

// int8 weights [rows, cols] -> bf16 [rows, cols] (dense), 16 values per
// thread: with group scales (group_shift > 0) bf16(q * s[row, col / group]),
// the value the W8A16 ring kernel widens to with group scales; else bf16(q),
// exact, the per-row scale being applied in the GEMM epilogue.  cols is a
// multiple of 16 (of 128 for the GEMM).
__global__ __launch_bounds__(256) void dequant_int8_kernel(const int8_t* __restrict__ q, int64_t ldq,
                                                           const float* __restrict__ s, int64_t rows, int64_t cols,
                                                           int group_shift, bf16* __restrict__ out) {
  const int64_t i16 = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 16-value chunk
  const int64_t per_row = cols >> 4;
  if (i16 >= rows * per_row) return;
  const int64_t r = i16 / per_row, c0 = (i16 - r * per_row) << 4;
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q + r * ldq + c0));
  const u32x2 lo = {v[0], v[1]}, hi = {v[2], v[3]};
  u32x4 o0, o1;
  if (group_shift > 0) {
    const float sc = s[r * (cols >> group_shift) + (c0 >> group_shift)];   // 16 values lie in one group
    o0 = i8x8_to_bf16<true>(lo, sc);
    o1 = i8x8_to_bf16<true>(hi, sc);
  } else {
    o0 = i8x8_to_bf16<false>(lo, 1.0f);
    o1 = i8x8_to_bf16<false>(hi, 1.0f);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(out + r * cols + c0);
  __builtin_nontemporal_store(o0, dst);
  __builtin_nontemporal_store(o1, dst + 1);
}


// ---------------------------------------------------------------------------
// fp32 SIMT GEMM: 64x64 tile, k-steps of 16, 4x4 outputs per thread.
struct GemmParamsF {
  const float* x; int64_t ldx;
  const float* w; int64_t ldw;
  const float* bias;
  const float* residual; int64_t ldr;
  const float* gate;
  float* y; int64_t ldy;
  float* yt; int64_t ldyt;
  int64_t split_col;
  int m, n, k;
};

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParamsF p) {
  __shared__ float sX[16][64 + 4];
  __shared__ float sW[16][64 + 4];
  const int tid = threadIdx.x;
  const int tok0 = blockIdx.y * 64, feat0 = blockIdx.x * 64;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  const int lr = tid / 4, lk = (tid % 4) * 4;
  for (int k0 = 0; k0 < p.k; k0 += 16) {
    {
      const int t = tok0 + lr;
      f32x4 v = (t < p.m) ? *reinterpret_cast<const f32x4*>(p.x + (int64_t)t * p.ldx + k0 + lk) : f32x4{0, 0, 0, 0};
      const int f = feat0 + lr;
      f32x4 u = (f < p.n) ? *reinterpret_cast<const f32x4*>(p.w + (int64_t)f * p.ldw + k0 + lk) : f32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) { sX[lk + e][lr] = v[e]; sW[lk + e][lr] = u[e]; }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) { a[e] = sX[kk][ty * 4 + e]; b[e] = sW[kk][tx * 4 + e]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = tok0 + ty * 4 + i;
    if (t >= p.m) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f = feat0 + tx * 4 + j;
      if (f >= p.n) continue;
      float v = acc[i][j] + (p.bias ? p.bias[f] : 0.0f);
      if ((int64_t)f >= p.split_col) {
        p.yt[(int64_t)(f - p.split_col) * p.ldyt + t] = v;
        continue;
      }
      if constexpr (EPI == kEpiGelu) v = gelu_tanh(v);
      if constexpr (EPI == kEpiGatedResidual) v = p.residual[(int64_t)t * p.ldr + f] + p.gate[f] * v;
      p.y[(int64_t)t * p.ldy + f] = v;
    }
  }
}

// ---------------------------------------------------------------------------
template <int EPI, bool W8, int SC = 0>
static void launch_bf16(const LinearArgs& a, hipStream_t stream, int* kernels) {
  GemmParams p;
  p.x = a.x; p.ldx = a.ldx;
  p.x_scale = a.x_scale;
  p.w = a.w; p.ldw = a.ldw;
  p.w_scale = a.w_scale;
  p.bias = (const bf16*)a.bias;
  p.residual = (const bf16*)a.residual; p.ldr = a.ldr;
  p.gate = a.gate;
  p.y = (bf16*)a.y; p.ldy = a.ldy;
  p.yt = (bf16*)a.yt; p.ldyt = a.ldyt;
  p.split_col = a.split_col;
  p.scale_cols = a.scale_cols;
  p.col_scale = a.col_scale;
  p.m = (int)a.m; p.n = (int)a.n; p.k = (int)a.k;
  p.tiles_m = (p.m + BM - 1) / BM;
  p.tiles_n = (p.n + BN - 1) / BN;
  p.group_shift = a.group > 0 ? __builtin_ctz((unsigned)a.group) : 0;
  p.rope = RopeGeom{a.rope_hd, a.rope_h, a.rope_w, a.rope_spatial};
  const int nblk = p.tiles_m * p.tiles_n;
  p.full_tiles = nblk;
  p.tail_split = 0;
  p.part = nullptr;
  *kernels = 1;
  if (a.act == kINT8) {
    gemm_ring_kernel<EPI, true><<<dim3(nblk), dim3(512), 0, stream>>>(p);
    return;
  }
  if constexpr (W8) {
    if (a.group > 0)
      gemm_ring_kernel<EPI, false, true, true><<<dim3(nblk), dim3(512), 0, stream>>>(p);
    else
      gemm_ring_kernel<EPI, false, true><<<dim3(nblk), dim3(512), 0, stream>>>(p);
  } else {
    int S = 0;
    if constexpr (EPI != kEpiBiasRope) {   // row-major outputs only: no transposed or rotated part
      const int cus = (a.part && a.split_col >= a.n) ? device_compute_units() : 0;
      if (cus > 0) S = tail_split_ways(nblk, p.k / 64, cus, a.part_bytes / kPartTileBytes);
      if (S) {
        p.full_tiles = nblk - nblk % cus;
        p.tail_split = S;
        p.part = a.part;
      }
    }
    const int grid = p.full_tiles + (nblk - p.full_tiles) * S;
    gemm_ring_kernel<EPI, false, false, false, SC><<<dim3(grid), dim3(512), 0, stream>>>(p);
    if (S) {
      gemm_tail_kernel<EPI, SC><<<dim3((nblk - p.full_tiles) * 64), dim3(256), 0, stream>>>(p);
      *kernels = 2;
    }
  }
}

// int8 weights with a staging buffer (bf16 activations): the weights are
// widened to bf16 there (with group scales, times the scale), then the bf16
// ring kernel runs on them with the per-channel scale (if any) in its
// epilogue.  The same MFMA operands in the same order as the W8A16 ring
// kernel, so the same bits, at the bf16 kernel's speed plus one pass over the
// weights.
template <int EPI>
static void launch_w8_staged(const LinearArgs& a, hipStream_t stream, int* kernels) {
  const int64_t chunks = a.n * (a.k / 16);
  const int gs = a.group > 0 ? __builtin_ctz((unsigned)a.group) : 0;
  dequant_int8_kernel<<<dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream>>>(
      (const int8_t*)a.w, a.ldw, a.w_scale, a.n, a.k, gs, (bf16*)a.wstage);
  LinearArgs b = a;
  b.weight = kBF16;
  b.w = a.wstage;
  b.ldw = a.k;
  b.group = 0;
  b.wstage = nullptr;
  b.wstage_bytes = 0;
  int nk = 0;
  if (a.group > 0) {
    b.w_scale = nullptr;
    launch_bf16<EPI, false, 2>(b, stream, &nk);
  } else {
    launch_bf16<EPI, false, 1>(b, stream, &nk);
  }
  *kernels = 1 + nk;
}

template <int EPI>
static void launch_f32(const LinearArgs& a, hipStream_t stream) {
  GemmParamsF p;
  p.x = (const float*)a.x; p.ldx = a.ldx;
  p.w = (const float*)a.w; p.ldw = a.ldw;
  p.bias = (const float*)a.bias;
  p.residual = (const float*)a.residual; p.ldr = a.ldr;
  p.gate = a.gate;
  p.y = (float*)a.y; p.ldy = a.ldy;
  p.yt = (float*)a.yt; p.ldyt = a.ldyt;
  p.split_col = a.split_col;
  p.m = (int)a.m; p.n = (int)a.n; p.k = (int)a.k;
  const dim3 grid((p.n + 63) / 64, (p.m + 63) / 64);
  gemm_f32_kernel<EPI><<<grid, dim3(256), 0, stream>>>(p);
}

hipError_t launch_linear(const LinearArgs& a, hipStream_t stream, int* kernels) {
  int dummy = 0;
  if (!kernels) kernels = &dummy;
  *kernels = 0;
  if (a.m == 0 || a.n == 0) return hipSuccess;
  *kernels = 1;
  if (a.act == kF32) {
    switch (a.epi) {
      case kEpiBias: launch_f32<kEpiBias>(a, stream); break;
      case kEpiGelu: launch_f32<kEpiGelu>(a, stream); break;
      case kEpiGatedResidual: launch_f32<kEpiGatedResidual>(a, stream); break;
      default: return hipErrorInvalidValue;   // no rotary epilogue on the fp32 path
    }
  } else if (a.weight == kINT8 && a.act == kBF16 && a.wstage && a.wstage_bytes >= a.n * a.k * 2) {
    switch (a.epi) {
      case kEpiBias: launch_w8_staged<kEpiBias>(a, stream, kernels); break;
      case kEpiGelu: launch_w8_staged<kEpiGelu>(a, stream, kernels); break;
      case kEpiGatedResidual: launch_w8_staged<kEpiGatedResidual>(a, stream, kernels); break;
      default: launch_w8_staged<kEpiBiasRope>(a, stream, kernels); break;
    }
  } else if (a.weight == kINT8) {
    switch (a.epi) {
      case kEpiBias: launch_bf16<kEpiBias, true>(a, stream, kernels); break;
      case kEpiGelu: launch_bf16<kEpiGelu, true>(a, stream, kernels); break;
      case kEpiGatedResidual: launch_bf16<kEpiGatedResidual, true>(a, stream, kernels); break;
      default: launch_bf16<kEpiBiasRope, true>(a, stream, kernels); break;
    }
  } else {
    switch (a.epi) {
      case kEpiBias: launch_bf16<kEpiBias, false>(a, stream, kernels); break;
      case kEpiGelu: launch_bf16<kEpiGelu, false>(a, stream, kernels); break;
      case kEpiGatedResidual: launch_bf16<kEpiGatedResidual, false>(a, stream, kernels); break;
      default: launch_bf16<kEpiBiasRope, false>(a, stream, kernels); break;
    }
  }
  return hipGetLastError();
}

}  // namespace h3k
