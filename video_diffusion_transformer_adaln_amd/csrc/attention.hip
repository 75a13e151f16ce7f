// Full (non-causal) multi-head self-attention over all video-latent tokens,
// the middle stage of the block (h3.c memory-techniques page, technique 2).
//
// bf16 path (flash-style, fp32 online softmax, v_mfma_f32_16x16x32_bf16,
// whose streams hold a 10-14 % higher clock under the power limit than the
// 32x32x16 form on MI355X):
//   * one workgroup = NW waves x 16 QB queries of one head (d = 128: 8 waves
//     of two 16-query blocks; d = 64: 4 waves of two); each wave keeps its
//     queries' Q fragments in registers and walks all keys in tiles of 32.
//     Measured on MI355X: 4 waves of three or four blocks (one wave per
//     SIMD, so that each LDS fragment feeds more products) ran 25 % slower,
//     and 4 waves of two blocks (two workgroups per CU) 3 % slower at 22680
//     tokens x 40 heads (they serve short sequences; see the launcher);
//   * scores are computed transposed, S^T = K Q^T, so that the accumulator's
//     lane index is the query: a query's 32 keys per tile lie in the four
//     lanes l%16 + 16 g (8 keys each), which share its running reference;
//   * K rows are read through a fixed key permutation, so that the eight
//     probabilities a lane holds per query block are eight consecutive keys;
//     they then serve directly as the B operand of O^T = V^T P^T;
//   * V arrives transposed (V^T [H*d, ldvt], written so by the QKV projection),
//     so the A operand of O^T = V^T P^T is a 16-byte read along the key axis;
//   * the softmax scale is folded into q: q arrives multiplied by
//     log2(e)/sqrt(d) (the QKV projection's epilogue writes it so), and each
//     score product starts from the accumulator value -m, so the scores come
//     out as s - m, the exponent of v_exp_f32 (exp2).  Unscaled q (the
//     standalone entry point's default) takes one fma per score instead;
//   * a query's sum over a tile's 32 keys comes from the matrix cores: one
//     MFMA of a ones fragment with the bf16 probabilities (the values the
//     product with V uses), which also reduces over the four lanes;
//   * software pipeline: the step for tile t runs the scores of tile t+1 and
//     the product with V of tile t-1 on the matrix cores while the vector
//     ALUs take the exponentials of tile t.  The three are independent; the
//     step is written as chunks (an LDS read two chunks ahead, the MFMAs of
//     that fragment, a share of the exponentials) kept in order by
//     sched_barrier, so that each wave alternates the two units;
//   * lazy online softmax without a per-tile maximum: probabilities are
//     exp2(s - m) against the running reference m.  When a query's tile sum
//     exceeds 2^48 or is not finite (or on the first tile) the tile is
//     redone: m moves to the maximum so far, O and the row sum l (which hold
//     tiles up to t-1, all relative to the old m) are scaled by
//     exp2(m_old - m_new), the pending scores of the next tile shift with
//     the reference, and the exponentials are recomputed.  The result is the
//     usual online-softmax recurrence with the reference updated only when
//     the probabilities would otherwise grow large.  The bound keeps every
//     accepted tile's sum, and so l and |O| / max|V|, below 2^48 per tile
//     (2^58 over 1024 tiles), far from fp32's (and bf16's) range; the rounding
//     of P to bf16 is relative, so its size does not change the precision.
//     With block-like logits (q.k/sqrt(d) of std 9) the reference then moves
//     only on the first tile or two: measured on MI355X, 2.3-4.2 % faster at
//     22680 tokens x 40 heads and 2.8-4.6 % at 6144 x 24 than a bound of
//     2^16 (which was itself 1.8 % faster than 2^10);
//   * two tiles per workgroup barrier: K tiles and full V^T tiles arrive
//     with direct-to-LDS loads, the V^T tiles of the last passes through
//     registers (keys beyond N are zeroed there), all in rings of four
//     32-key slots; a pass over tiles (t0, t0+1) loads
//     K_{t0+3}, K_{t0+4}, V_{t0+1}, V_{t0+2} into the slots the previous pass
//     read, then waits for them and meets the other waves.  The barrier
//     carries no fence: each wave waits for its own loads first.  Keys
//     beyond N contribute exactly zero (their K rows load as zero, their
//     scores are set to -inf and their V^T entries to zero).
//   * key split of the last round (with a caller scratch, head_dim 128): when
//     the last round of workgroups would leave at least half the slots idle,
//     each of its workgroups becomes S workgroups over S key ranges, each
//     storing its unnormalised O, m and l; attention_combine_kernel merges
//     them (attn_shape128 / attn_split_ways give the shape and S).
// fp32 path: one thread per query, K/V tiles in LDS, for the small fp32
// workload.
#include "common.hpp"
#include "kernels.hpp"

namespace h3k {

struct AttnParams {
  const bf16* q; int64_t ldq;
  const bf16* k; int64_t ldk;
  const bf16* vt; int64_t ldvt;
  bf16* o; int64_t ldo;
  int n, n_heads, q_tiles;
  float scale_log2;   // log2(e) / sqrt(d)
  // Key split: workgroups full_blocks .. of the order below are each split
  // into kv_split key ranges whose unnormalised results go to part
  // (attention_combine_kernel finishes them).
  int full_blocks, kv_split;
  float* part;
};

// a tile is redone when a query's probability sum over the tile's 32 keys exceeds this
constexpr float kLazyBound = 0x1p48f;
// bf16 kernel for head_dim 128: waves per workgroup, and 16-query blocks per
// wave (head_dim 64 uses 4 waves of 2 blocks)
constexpr int kAttnWaves128 = 8;
constexpr int kAttnQBlocks128 = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
}
// Key permutation inside a 32-key tile: the 16x16 score block kb of the
// wave takes as its A-row x the key 8 (x/4) + 4 kb + x%4, so that the four
// scores lane l holds per block (rows 4 (l/16) .. +3) are, over the two
// blocks, the eight consecutive keys 8 (l/16) .. +7: the B operand of the
// V^T P^T product that lane supplies.
__device__ __forceinline__ int kperm(int kb, int x) { return 8 * (x >> 2) + 4 * kb + (x & 3); }
// Chunk swizzle of a K row of CPR 16-byte chunks (CPR = 16 for d = 128, 8 for
// d = 64).  Measured on MI355X (ds_read_b128 throughput per access pattern),
// the 16x16 fragment reads of the permuted rows are conflict-free with it.
template <int CPR> __device__ __forceinline__ int kswz(int r) { return (r ^ (r >> 2)) & (CPR - 1); }

template <int HD, int NW, int QB, bool QPRE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(QB > 2 ? 1 : 2, QB > 2 ? 1 : 2)))
void attention_bf16_kernel(AttnParams p) {
  constexpr int KT = 32;                       // keys per tile
  constexpr int KS = HD / 32;                  // k-steps of the score product (16x16x32)
  constexpr int DB = HD / 16;                  // 16-row blocks of O^T
  // K stage: [32 keys][HD dims] (HD*2-byte rows), 16-byte chunk c of row r at
  // chunk c ^ kswz(r).  V^T stage: 2 planes (one per 16 keys) of
  // [HD rows][32 B].  Four slots of each; tile j lives in slot j % 4.
  constexpr int KROW = HD * 2, KBYTES = KT * KROW;
  constexpr int VPL = HD * 32, VBYTES = 2 * VPL;
  constexpr int LPW = HD / (16 * NW);          // K (and V^T) load instructions per wave and tile
  static_assert(LPW >= 1 && KBYTES == NW * LPW * 1024, "whole 1 KiB K load instructions per wave and tile");
  static_assert(HD == NW * LPW * 16, "whole V^T loads per lane and tile");
  __shared__ __attribute__((aligned(1024))) char lds[4 * KBYTES + 4 * VBYTES];
  char* const kbuf = lds;                      // slot u at kbuf + u * KBYTES
  char* const vbuf = lds + 4 * KBYTES;         // slot u at vbuf + u * VBYTES

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, x16 = lane & 15;
  const int nblk = p.q_tiles * p.n_heads;
  // Whole workgroups first, in the XCD-aware order; with a key split, block
  // full_blocks + s * tail + j takes key tiles [s TA / S, (s + 1) TA / S) of
  // tail workgroup j (TA tiles in all, S = kv_split) and stores partial unit
  // j S + s.  The workgroup then sees the keys of its range as a sequence of
  // NK keys (K and V^T addressed from the range's first key).
  const int TA = (p.n + KT - 1) / KT;
  int lin, unit = -1, key_first = 0, key_end = p.n;
  if ((int)blockIdx.x < p.full_blocks) {
    lin = xcd_remap(blockIdx.x, p.full_blocks);
  } else {
    const int tail = nblk - p.full_blocks, qb_ = (int)blockIdx.x - p.full_blocks;
    const int j = qb_ % tail, sp = qb_ / tail;
    lin = p.full_blocks + j;
    key_first = sp * TA / p.kv_split * KT;
    key_end = min(p.n, (sp + 1) * TA / p.kv_split * KT);
    unit = j * p.kv_split + sp;
  }
  const int head = lin / p.q_tiles;
  const int qtile = lin - head * p.q_tiles;
  const int N = p.n;                           // queries
  const int NK = key_end - key_first;          // keys of this workgroup
  const int T = (NK + KT - 1) / KT;
  const bf16* const kp = p.k + (int64_t)key_first * p.ldk;
  const bf16* const vtp = p.vt + key_first;
  constexpr int QW = 16 * QB;                  // queries per wave
  const int q0 = qtile * (NW * QW) + wave * QW;
  const float sc = p.scale_log2;

  // ---- Q fragments (B operand of S^T = K Q^T) of the wave's two 16-query
  // blocks: lane l holds query q0 + 16 qb + l%16, dims 32 ks + 8 (l/16) .. +8;
  // queries >= N load as zero
  bf16x8 qf[QB][KS];
  {
    const __amdgpu_buffer_rsrc_t rq = rsrc(p.q, (uint32_t)((uint64_t)N * p.ldq * 2));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t off = (uint32_t)(q0 + 16 * qb + x16) * (uint32_t)p.ldq * 2u + (head * HD + ks * 32 + g * 8) * 2;
        const u32x4 v = bload16(rq, off);
        qf[qb][ks] = *reinterpret_cast<const bf16x8*>(&v);
      }
  }

  // ---- K tiles: direct-to-LDS loads, LPW 1 KiB instructions per wave;
  // instruction u = wave + NW j: lane l -> row u*RPI + l/CPR, physical chunk
  // l%CPR, fetching logical chunk phys ^ kswz(row).  Rows >= N load as zero
  // (buffer bounds); tiles past the last one re-load the last tile so that
  // the load counts stay uniform.
  constexpr int CPR = KROW / 16;               // chunks per K row
  constexpr int RPI = 64 / CPR;                // rows per load instruction
  const __amdgpu_buffer_rsrc_t rk = rsrc(kp, (uint32_t)((uint64_t)NK * p.ldk * 2));
  uint32_t kdma_off[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int row = (wave + NW * j) * RPI + lane / CPR;
    const int c = (lane % CPR) ^ kswz<CPR>(row);
    kdma_off[j] = (uint32_t)row * (uint32_t)p.ldk * 2u + (head * HD + c * 8) * 2;
  }
  const uint32_t ktile_bytes = (uint32_t)KT * (uint32_t)p.ldk * 2u;
  auto kdma = [&](int t) {
    const int tt = t < T ? t : T - 1;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      lds_dma16(rk, kbuf + (t & 3) * KBYTES + (wave + NW * j) * 1024, kdma_off[j], (uint32_t)tt * ktile_bytes);
  };

  // ---- V^T tiles of the last passes, through registers: LPW 16-byte loads
  // per lane; piece j: plane lane/32, row (wave + NW j)*16 + (lane%32)/2,
  // half lane&1 (keys 16 plane + 8 half .. +8)
  const int st_pl = lane >> 5, st_h = lane & 1;
  const __amdgpu_buffer_rsrc_t rvt = rsrc(vtp, (uint32_t)(((uint64_t)p.n_heads * HD * p.ldvt - key_first) * 2));
  auto st_row = [&](int j) { return (wave + NW * j) * 16 + ((lane & 31) >> 1); };
  auto vload_masked = [&](int t, u32x4 (&v)[LPW]) {   // zero for keys >= NK
    const int key0 = t * KT + st_pl * 16 + st_h * 8;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      v[j] = u32x4{0, 0, 0, 0};
      if (key0 < NK) {
        const uint32_t off = ((uint32_t)(head * HD + st_row(j)) * (uint32_t)p.ldvt + st_pl * 16 + st_h * 8) * 2u;
        v[j] = bload16(rvt, off, (uint32_t)t * (KT * 2));
        uint16_t* e = reinterpret_cast<uint16_t*>(&v[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (key0 + i >= NK) e[i] = 0;
      }
    }
  };
  auto vstore = [&](int t, const u32x4 (&v)[LPW]) {
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      *reinterpret_cast<u32x4*>(vbuf + (t & 3) * VBYTES + st_pl * VPL + st_row(j) * 32 + (st_h << 4)) = v[j];
  };
  // full V^T tiles: direct-to-LDS, LPW 1 KiB instructions per wave;
  // instruction u = wave + NW j -> plane u / (HD/32), rows 32 (u % (HD/32)) +
  // lane/2, half lane&1
  constexpr int RB = HD / 32;
  uint32_t vdma_off[LPW];
  int vdma_dst[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int u = wave + NW * j;
    const int vd_row = 32 * (u % RB) + (lane >> 1);
    vdma_off[j] = ((uint32_t)(head * HD + vd_row) * (uint32_t)p.ldvt + (u / RB) * 16 + (lane & 1) * 8) * 2u;
    vdma_dst[j] = (u / RB) * VPL + 32 * (u % RB) * 32;
  }
  auto vdma = [&](int t) {
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      lds_dma16(rvt, vbuf + (t & 3) * VBYTES + vdma_dst[j], vdma_off[j], (uint32_t)t * (KT * 2));
  };

  // ---- fragment addresses.  K block kb, k-step ks: row kperm(kb, l%16),
  // logical chunk 4 ks + l/16.  V^T block db: row 16 db + l%16, keys
  // 8 (l/16) .. +8 = plane (l/16)/2, half (l/16)%2.
  int k_off[2][KS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kr = kperm(kb, x16);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k_off[kb][ks] = kr * KROW + (((4 * ks + g) ^ kswz<CPR>(kr)) << 4);
  }
  const int v_frag = (g >> 1) * VPL + x16 * 32 + ((g & 1) << 4);

  // O^T block (db, qb): lane l holds dims 16 db + 4 (l/16) .. +4 of query
  // q0 + 16 qb + l%16.  S block (kb, qb) likewise holds keys
  // 8 (l/16) + 4 kb .. +4 of the tile.  Element r (0..15) of a lane's tile
  // scores is query block r/8, key 8 (l/16) + r%8.
  f32x4 O[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) O[db][qb] = f32x4{};
  // Running references m (log2 units).  With QPRE, q arrives multiplied by
  // log2(e)/sqrt(d) and every score product starts from the accumulator
  // value -m (minit), so the scores already are s - m and feed the
  // exponential directly; a moved reference shifts the pending scores of the
  // next tile by the same amount.  Without QPRE the scores are raw q.k and
  // one fma per element applies the scale and the reference.
  float m_ref[QB], l_run[QB];
  f32x4 minit[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = QPRE ? 0.f : -INFINITY;
    l_run[qb] = 0.f;
    minit[qb] = f32x4{};
  }
  f32x4 S[2][2][QB];                           // [tile parity][kb][qb]
  u32x4 P[2][QB];                              // [tile parity][qb]: eight bf16 probabilities, in pairs
  auto sel = [&](const f32x4 (&s)[2][QB], int r) __attribute__((always_inline)) -> float { return s[(r >> 2) & 1][r >> 3][r & 3]; };
  // exponent of element r: s - m in log2 units
  auto xval = [&](const f32x4 (&s)[2][QB], int r) __attribute__((always_inline)) -> float {
    if constexpr (QPRE) return sel(s, r);
    else return fmaf(sel(s, r), sc, -m_ref[r >> 3]);
  };
  auto mfma16 = [](const bf16x8& a, const bf16x8& b, const f32x4& c) __attribute__((always_inline)) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  };
  auto pb = [](const u32x4& w) __attribute__((always_inline)) { return __builtin_bit_cast(bf16x8, w); };
  auto sinit = [&](int qb) __attribute__((always_inline)) -> f32x4 {
    if constexpr (QPRE) return minit[qb];
    else return f32x4{};
  };

  auto scores = [&](const char* kb_, f32x4 (&s)[2][QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = sinit(qb);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb_ + k_off[kb][ks]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma16(a, qf[qb][ks], s[kb][qb]);
      }
    }
  };
  auto pv = [&](const char* vb, const u32x4 (&pp)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(vb + db * 512 + v_frag);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) O[db][qb] = mfma16(a, pb(pp[qb]), O[db][qb]);
    }
  };
  // keys >= NK of tile t
  auto mask_tail = [&](f32x4 (&s)[2][QB], int t) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (t * KT + 8 * g + 4 * kb + j >= NK) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[kb][qb][j] = -INFINITY;
        }
  };
  // a query's sum over the tile's 32 keys, from the matrix cores: ones (A) times P^T (B),
  // every lane of the query gets the full sum
  const u32x4 ones8 = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  auto tile_sums = [&](const u32x4 (&pp)[QB], float (&ls)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) ls[qb] = mfma16(pb(ones8), pb(pp[qb]), f32x4{})[0];
  };
  // probabilities against the current references, rounded to bf16 in
  // pairs; the lane's per-query-block sums are taken from the rounded pairs
  // (v_dot2 with (1, 1)), the values the product with V uses
  auto expo = [&](const f32x4 (&s)[2][QB], u32x4 (&pp)[QB], float (&ls)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(xval(s, 8 * qb + e));
        const float p1 = __builtin_amdgcn_exp2f(xval(s, 8 * qb + e + 1));
        const bf16x2 pr = {static_cast<bf16>(p0), static_cast<bf16>(p1)};
        pp[qb][e >> 1] = __builtin_bit_cast(uint32_t, pr);
      }
    }
    tile_sums(pp, ls);
  };
  // move each query's reference to its maximum so far (over the four lanes
  // holding its keys), rescale O and l, recompute.  `first`: the first tile,
  // whose maximum becomes the reference (O and l are still zero).  With
  // QPRE the scores are relative to the reference, so the current tile's
  // and, when `fix_next`, the next tile's pending scores shift with it.
  auto redo = [&](f32x4 (&s)[2][QB], f32x4 (&sn)[2][QB], bool fix_next, u32x4 (&pp)[QB], float (&ls)[QB],
                  bool first) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, s[e >> 2][qb][e & 3]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      if constexpr (QPRE) {
        const float delta = first ? mx : fmaxf(0.f, mx);
        if (!first) {
          const float alpha = __builtin_amdgcn_exp2f(-delta);
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) O[db][qb] *= alpha;
        }
        m_ref[qb] += delta;
        minit[qb] = f32x4{-m_ref[qb], -m_ref[qb], -m_ref[qb], -m_ref[qb]};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[kb][qb] -= delta;
          if (fix_next) sn[kb][qb] -= delta;
        }
      } else {
        const float m_new = fmaxf(m_ref[qb], mx * sc);
        const float alpha = __builtin_amdgcn_exp2f(m_ref[qb] - m_new);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) O[db][qb] *= alpha;
        m_ref[qb] = m_new;
      }
    }
    expo(s, pp, ls);
  };

  // ---- one tile's work, t with K_{t+1} in K slot KSL and V_{t-1} in V slot
  // VSL: the scores of tile t+1 and the product with V of tile t-1 on the
  // matrix cores, the exponentials of tile t on the vector ALUs.  Chunk i
  // issues an LDS read two chunks ahead, the two MFMAs (one per query block)
  // of fragment i (even: K block and k-step i/2, odd: V^T block i/2) and its
  // of the exponentials; sched_barrier keeps the chunks in this order, so
  // that each wave alternates the two units.
  auto step = [&](int t, auto u_c, auto ksl_c, auto vsl_c, bool mask) __attribute__((always_inline)) {
    constexpr int U = decltype(u_c)::value;
    const char* kb_ = kbuf + decltype(ksl_c)::value * KBYTES;
    const char* vb = vbuf + decltype(vsl_c)::value * VBYTES;
    if (mask) mask_tail(S[U], t);
    constexpr int NCH = 2 * KS + DB;           // chunks (fragments) per tile (16 or 8)
    constexpr int NE = 8 * QB;                 // scores per lane and tile
    // chunk i takes the exponentials of elements NE i / NCH .. NE (i+1) / NCH - 1
    auto frag = [&](int i) __attribute__((always_inline)) {
      const int j = i >> 1;
      const char* a = (i & 1) ? vb + j * 512 + v_frag : kb_ + k_off[j / KS][j % KS];
      return *reinterpret_cast<const bf16x8*>(a);
    };
    bf16x8 fr[NCH];
    fr[0] = frag(0);
    fr[1] = frag(1);
    // The exponential chain is skewed by one: chunk i takes the exponent of
    // element r + 1, the exponential of element r (whose exponent the
    // previous chunk took) and rounds and sums element r - 1 (exponentiated
    // in the previous chunk), so no instruction waits on a result from its
    // own chunk.  Elements are rounded to bf16 in pairs and the pair summed
    // with one v_dot2 against (1, 1).
    float xa[NE + 1], pe[NE];
    auto sum_cvt = [&](int q) __attribute__((always_inline)) {
      if (q & 1) {
        const bf16x2 pr = {static_cast<bf16>(pe[q - 1]), static_cast<bf16>(pe[q])};
        P[U][q >> 3][(q & 7) >> 1] = __builtin_bit_cast(uint32_t, pr);
      }
    };
    xa[0] = xval(S[U], 0);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (i + 2 < NCH) fr[i + 2] = frag(i + 2);
      const int j = i >> 1;
      if (i & 1) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) O[j][qb] = mfma16(fr[i], pb(P[1 - U][qb]), O[j][qb]);
      } else {
        const int kb = j / KS, ks = j % KS;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          S[1 - U][kb][qb] = mfma16(fr[i], qf[qb][ks], ks == 0 ? sinit(qb) : S[1 - U][kb][qb]);
      }
#pragma unroll
      for (int r = NE * i / NCH; r < NE * (i + 1) / NCH; ++r) {
        if (r + 1 < NE) xa[r + 1] = xval(S[U], r + 1);
        pe[r] = __builtin_amdgcn_exp2f(xa[r]);
        if (r >= 1) sum_cvt(r - 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    sum_cvt(NE - 1);
    float lt[QB];
    tile_sums(P[U], lt);
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) over = over || !(lt[qb] <= kLazyBound);
    if (__any(over)) redo(S[U], S[1 - U], true, P[U], lt, false);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += lt[qb];
  };

  // ---- two tiles per barrier.  Pass (t0, t0+1), t0 odd, with SL = t0 % 4:
  // entry: S_{t0}, P_{t0-1} in registers; K_{t0+1}, K_{t0+2}, V_{t0-1}, V_{t0}
  // in LDS.  It loads K_{t0+3}, K_{t0+4}, V_{t0+1}, V_{t0+2} (into the slots
  // of the tiles read by the previous pass) and waits for them before the
  // barrier.  TAIL passes mask the last tile and its V^T, and skip tiles >= T.
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C3 = std::integral_constant<int, 3>;
  auto pass = [&](int t0, auto sl_c, auto tail_c) {
    constexpr int SL = decltype(sl_c)::value;  // 1 or 3
    constexpr bool TAIL = decltype(tail_c)::value;
    using K1 = std::integral_constant<int, (SL + 1) & 3>;
    using K2 = std::integral_constant<int, (SL + 2) & 3>;
    using V0 = std::integral_constant<int, (SL + 3) & 3>;
    using V1 = std::integral_constant<int, SL>;
    kdma(t0 + 3);
    kdma(t0 + 4);
    u32x4 va[LPW], vb[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) va[j] = vb[j] = u32x4{0, 0, 0, 0};
    if constexpr (!TAIL) {
      vdma(t0 + 1);
      vdma(t0 + 2);
    } else {
      if (t0 + 1 < T) vload_masked(t0 + 1, va);
      if (t0 + 2 < T) vload_masked(t0 + 2, vb);
    }
    step(t0, C1{}, K1{}, V0{}, TAIL && t0 == T - 1);
    if (!TAIL || t0 + 1 < T) step(t0 + 1, C0{}, K2{}, V1{}, TAIL && t0 + 1 == T - 1);
    wait_vmcnt<0>();
    if constexpr (TAIL) {
      vstore(t0 + 1, va);
      vstore(t0 + 2, vb);
    }
    wait_lgkm0();
    wg_barrier();
  };

  // ---- prologue: K_0..K_3 and V_0, V_1 staged; S_0 -> P_0 (always through
  // redo, the reference being -inf); S_1 computed
  kdma(0);
  kdma(1);
  kdma(2);
  kdma(3);
  {
    u32x4 v0[LPW], v1[LPW];
    vload_masked(0, v0);
#pragma unroll
    for (int j = 0; j < LPW; ++j) v1[j] = u32x4{0, 0, 0, 0};
    if (T > 1) vload_masked(1, v1);
    wait_vmcnt<0>();
    vstore(0, v0);
    vstore(1, v1);
  }
  wait_lgkm0();
  wg_barrier();
  scores(kbuf, S[0]);
  if (T == 1) mask_tail(S[0], 0);
  {
    float ls[QB];
    redo(S[0], S[1], false, P[0], ls, true);   // before S_1 is computed: it starts from the new reference
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += ls[qb];
  }
  if (T > 1) scores(kbuf + KBYTES, S[1]);
  wg_barrier();                                // K slots 0 and 1 are refilled next

  using Full = std::integral_constant<bool, false>;
  using Tail = std::integral_constant<bool, true>;
  int t0 = 1;
  for (; (t0 + 5) * KT <= NK; t0 += 4) {       // V^T tiles up to t0+4 are full
    pass(t0, C1{}, Full{});
    pass(t0 + 2, C3{}, Full{});
  }
  // t0 % 4 == 1 here and fewer than six tiles remain
  if (t0 < T) pass(t0, C1{}, Tail{});
  if (t0 + 2 < T) pass(t0 + 2, C3{}, Tail{});
  if (t0 + 4 < T) pass(t0 + 4, C1{}, Tail{});
  // the last tile's product with V
  {
    const char* vl = vbuf + ((T - 1) & 3) * VBYTES;
    if ((T - 1) & 1) pv(vl, P[1]);
    else pv(vl, P[0]);
  }
  wait_vmcnt<0>();                             // no load left in flight at exit

  if (unit >= 0) {   // same for the whole workgroup
    // a key range's partial result: O unnormalised (relative to 2^m), then
    // the reference m and the row sum l, for the workgroup's NW QW queries
    constexpr int QWG = NW * QW;
    float* const po = p.part + (int64_t)unit * (QWG * (HD + 2));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int ql = wave * QW + 16 * qb + x16;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(po + ql * HD + 16 * db + 4 * g) = O[db][qb];
      if (g == 0) {
        po[QWG * HD + ql] = m_ref[qb];
        po[QWG * HD + QWG + ql] = l_run[qb];
      }
    }
    return;
  }

  // ---- normalise and store (every lane holds its query's full row sum)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float inv = 1.0f / l_run[qb];
    const int q = q0 + 16 * qb + x16;
    if (q < N) {
      bf16* orow = p.o + (int64_t)q * p.ldo + head * HD + 4 * g;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        u32x2 out;
        bf16* oe = reinterpret_cast<bf16*>(&out);
#pragma unroll
        for (int e = 0; e < 4; ++e) oe[e] = static_cast<bf16>(O[db][qb][e] * inv);
        *reinterpret_cast<u32x2*>(orow + db * 16) = out;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32: one thread per query (64 per workgroup), 32-key tiles of K and V in
// LDS (V gathered from V^T), online softmax with expf.
struct AttnParamsF {
  const float* q; int64_t ldq;
  const float* k; int64_t ldk;
  const float* vt; int64_t ldvt;
  float* o; int64_t ldo;
  int n;
  float scale;
};

template <int HD>
__global__ __launch_bounds__(64) void attention_f32_kernel(AttnParamsF p) {
  constexpr int TK = 32;
  __shared__ float sK[TK][HD];
  __shared__ float sV[TK][HD];
  const int head = blockIdx.y;
  const int qi = blockIdx.x * 64 + threadIdx.x;
  const bool valid = qi < p.n;
  float q[HD], o[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    q[d] = valid ? p.q[(int64_t)qi * p.ldq + head * HD + d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int k0 = 0; k0 < p.n; k0 += TK) {
    for (int idx = threadIdx.x; idx < TK * HD; idx += 64) {
      const int j = idx / HD, d = idx % HD;
      const bool kv = k0 + j < p.n;
      sK[j][d] = kv ? p.k[(int64_t)(k0 + j) * p.ldk + head * HD + d] : 0.f;
      const int jv = idx % TK, dv = idx / TK;
      sV[jv][dv] = (k0 + jv < p.n) ? p.vt[(int64_t)(head * HD + dv) * p.ldvt + k0 + jv] : 0.f;
    }
    __syncthreads();
    float s[TK];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < HD; ++d) acc = fmaf(q[d], sK[j][d], acc);
      s[j] = (k0 + j < p.n) ? acc * p.scale : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float m_new = fmaxf(m, mt);
    const float alpha = expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < HD; ++d) o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      const float pr = expf(s[j] - m_new);
      l += pr;
#pragma unroll
      for (int d = 0; d < HD; ++d) o[d] = fmaf(pr, sV[j][d], o[d]);
    }
    m = m_new;
    __syncthreads();
  }
  if (!valid) return;
  const float inv = 1.0f / l;
#pragma unroll
  for (int d = 0; d < HD; ++d) p.o[(int64_t)qi * p.ldo + head * HD + d] = o[d] * inv;
}

// ---------------------------------------------------------------------------
// Second kernel of a key split: each thread merges the S partial results of 4
// dims of one query, the usual way: with M the largest reference, O = sum_s
// 2^(m_s - M) O_s and l = sum_s 2^(m_s - M) l_s, out = O / l (as in the main
// kernel, times the reciprocal), one bf16 rounding.
template <int HD, int QWG>
__global__ __launch_bounds__(256) void attention_combine_kernel(AttnParams p) {
  constexpr int C4 = HD / 4, UF = QWG * (HD + 2);
  const int tail = p.q_tiles * p.n_heads - p.full_blocks, S = p.kv_split;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int j = idx / (QWG * C4);
  if (j >= tail) return;
  const int r = idx - j * (QWG * C4), ql = r / C4, c = r - ql * C4;
  const int lin = p.full_blocks + j, head = lin / p.q_tiles, qtile = lin - head * p.q_tiles;
  const int q = qtile * QWG + ql;
  if (q >= p.n) return;
  const float* const base = p.part + (int64_t)j * S * UF;
  float M = -INFINITY;
  for (int sp = 0; sp < S; ++sp) M = fmaxf(M, base[sp * UF + QWG * HD + ql]);
  float l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < S; ++sp) {
    const float* u = base + sp * UF;
    const float w = __builtin_amdgcn_exp2f(u[QWG * HD + ql] - M);
    l += w * u[QWG * HD + QWG + ql];
    o += w * *reinterpret_cast<const f32x4*>(u + ql * HD + 4 * c);
  }
  const float inv = 1.0f / l;
  u32x2 out;
  bf16* oe = reinterpret_cast<bf16*>(&out);
#pragma unroll
  for (int e = 0; e < 4; ++e) oe[e] = static_cast<bf16>(o[e] * inv);
  *reinterpret_cast<u32x2*>(p.o + (int64_t)q * p.ldo + head * HD + 4 * c) = out;
}


// ---------------------------------------------------------------------------
// S: key split of the last round (0: none; head_dim 128 only)
template <int HD, int NW, int QB, bool QPRE>
static void launch_bf16_attn_nw(const AttentionArgs& a, hipStream_t stream, int* kernels, int S, int cus) {
  AttnParams p;
  p.q = (const bf16*)a.q; p.ldq = a.ldq;
  p.k = (const bf16*)a.k; p.ldk = a.ldk;
  p.vt = (const bf16*)a.vt; p.ldvt = a.ldvt;
  p.o = (bf16*)a.o; p.ldo = a.ldo;
  p.n = a.n; p.n_heads = a.n_heads;
  p.q_tiles = (a.n + NW * 16 * QB - 1) / (NW * 16 * QB);
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  const int nblk = p.q_tiles * p.n_heads;
  p.full_blocks = nblk;
  p.kv_split = 0;
  p.part = nullptr;
  if (S) {
    // one 8-wave workgroup or two 4-wave ones per CU (256 VGPRs per wave, 64 KiB of LDS each)
    const int64_t slots = (int64_t)cus * (NW == 4 ? 2 : 1);
    p.full_blocks = nblk - (int)(nblk % slots);
    p.kv_split = S;
    p.part = a.part;
  }
  const int grid = p.full_blocks + (nblk - p.full_blocks) * S;
  attention_bf16_kernel<HD, NW, QB, QPRE><<<dim3(grid), dim3(NW * 64), 0, stream>>>(p);
  *kernels = 1;
  if (S) {
    constexpr int QWG = NW * 16 * QB;
    const int64_t threads = (int64_t)(nblk - p.full_blocks) * QWG * (HD / 4);
    attention_combine_kernel<HD, QWG><<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(p);
    *kernels = 2;
  }
}
// head_dim 128: 8-wave workgroups (256 queries), or 4-wave ones (128 queries,
// two per CU) for short sequences with few workgroups, where the last round
// of workgroups is then spread over twice as many CUs, unless the caller's
// scratch lets 8-wave workgroups split their last round (attn_shape128).
// Measured on MI355X (same bits): 6144 tokens x 24 heads 452 -> 417 us, 2000
// x 40 108 -> 91 us; but 22680 tokens x 5 heads (as few workgroups, a long
// key loop) 1055 -> 1177 us, so the long sequences keep 8 waves.
template <int HD, bool QPRE>
static void launch_bf16_attn(const AttentionArgs& a, hipStream_t stream, int* kernels) {
  if constexpr (HD == 128) {
    static_assert(kAttnWaves128 == 8 && kAttnQBlocks128 == 2, "attn_shape128 assumes 8 waves of two blocks");
    const int cus = a.part ? device_compute_units() : 0;
    int S = 0;
    if (attn_shape128(a.n, a.n_heads, cus, a.part ? a.part_bytes : 0, &S) == 4)
      launch_bf16_attn_nw<128, 4, kAttnQBlocks128, QPRE>(a, stream, kernels, S, cus);
    else
      launch_bf16_attn_nw<128, kAttnWaves128, kAttnQBlocks128, QPRE>(a, stream, kernels, S, cus);
  } else {
    launch_bf16_attn_nw<HD, 4, 2, QPRE>(a, stream, kernels, 0, 0);
  }
}

template <int HD>
static void launch_f32_attn(const AttentionArgs& a, hipStream_t stream) {
  AttnParamsF p;
  p.q = (const float*)a.q; p.ldq = a.ldq;
  p.k = (const float*)a.k; p.ldk = a.ldk;
  p.vt = (const float*)a.vt; p.ldvt = a.ldvt;
  p.o = (float*)a.o; p.ldo = a.ldo;
  p.n = a.n;
  p.scale = 1.0f / sqrtf((float)HD);
  attention_f32_kernel<HD><<<dim3((a.n + 63) / 64, a.n_heads), dim3(64), 0, stream>>>(p);
}

hipError_t launch_attention(const AttentionArgs& a, hipStream_t stream, int* kernels) {
  int dummy = 0;
  if (!kernels) kernels = &dummy;
  *kernels = 0;
  if (a.n == 0) return hipSuccess;
  *kernels = 1;
  if (a.dt == kF32) {
    if (a.head_dim == 64) launch_f32_attn<64>(a, stream);
    else launch_f32_attn<128>(a, stream);
  } else {
    if (a.q_prescaled) {
      if (a.head_dim == 64) launch_bf16_attn<64, true>(a, stream, kernels);
      else launch_bf16_attn<128, true>(a, stream, kernels);
    } else {
      if (a.head_dim == 64) launch_bf16_attn<64, false>(a, stream, kernels);
      else launch_bf16_attn<128, false>(a, stream, kernels);
    }
  }
  return hipGetLastError();
}

}  // namespace h3k
