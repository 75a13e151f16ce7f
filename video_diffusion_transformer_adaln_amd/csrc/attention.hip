// Full (non-causal) multi-head self-attention over all video-latent tokens,
// the middle stage of the block (h3.c memory-techniques page, technique 2).
//
// bf16 path (flash-style, fp32 online softmax, v_mfma_f32_32x32x16_bf16):
//   * one workgroup = NW waves x 32 queries of one head (NW = 8 for d = 128,
//     4 for d = 64); each wave keeps its queries' Q fragments in registers and
//     walks all keys in tiles of 32;
//   * scores are computed transposed, S^T = K Q^T, so that the accumulator's
//     lane index is the query: every lane owns its query's running reference
//     and sum, and rescaling needs no cross-lane traffic except one xor-32
//     exchange for a tile maximum;
//   * K rows are read through a fixed key permutation (bits 2 and 3 of the
//     key index swapped inside each 32-key block), so that the eight
//     probabilities a lane holds per 16-key step are eight consecutive keys;
//     they then serve directly as the B operand of O^T = V^T P^T;
//   * V arrives transposed (V^T [H*d, ldvt], written so by the QKV projection),
//     so the A operand of O^T = V^T P^T is a 16-byte read along the key axis;
//   * software pipeline: the step for tile t runs the scores of tile t+1 and
//     the product with V of tile t-1 on the matrix cores while the vector
//     ALUs take the exponentials of tile t.  The three are independent; the
//     step is written as chunks (an LDS read two chunks ahead, one MFMA, a
//     share of the exponentials) kept in order by sched_barrier, so that
//     each wave alternates the two units;
//   * lazy online softmax without a per-tile maximum: probabilities are
//     exp2(s - m) against the running reference m.  When some lane's tile sum
//     exceeds 2^8 (a probability above 2^8, or the first tile, where m is
//     still -inf) the tile is redone: m moves to the maximum so far, O and the
//     row sum l (which hold tiles up to t-1, all relative to the old m) are
//     scaled by exp2(m_old - m_new), and the exponentials are recomputed.
//     The result is the usual online-softmax recurrence with the reference
//     updated only when a probability would otherwise exceed 2^8;
//   * two tiles per workgroup barrier: K tiles and full V^T tiles arrive
//     with direct-to-LDS loads, the V^T tiles of the last passes through
//     registers (keys beyond N are zeroed there), all in rings of four
//     32-key slots; a pass over tiles (t0, t0+1) loads
//     K_{t0+3}, K_{t0+4}, V_{t0+1}, V_{t0+2} into the slots the previous pass
//     read, then waits for them and meets the other waves.  The barrier
//     carries no fence: each wave waits for its own loads first.  Keys
//     beyond N contribute exactly zero (their K rows load as zero, their
//     scores are set to -inf and their V^T entries to zero).
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
};

constexpr float kLazyBound = 256.0f;   // a tile is redone when a lane's probability sum exceeds this

__device__ __forceinline__ f32x16 mfma32a(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
}
// Row halves are swapped when bit 2 xor bit 3 of the row is set (LDS banks).
__device__ __forceinline__ int hswap(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }
// Key permutation inside a 32-key block: swap bits 2 and 3.
__device__ __forceinline__ int kperm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
// Chunk swizzle of a K row of CPR 16-byte chunks (CPR = 16 for d = 128, 8 for
// d = 64): the fragment reads of rows kperm(0..7), kperm(8..15) and of any 16
// consecutive rows each land on distinct banks.
template <int CPR> __device__ __forceinline__ int kswz(int r);
template <> __device__ __forceinline__ int kswz<16>(int r) { return (r & 15) ^ (((r >> 3) & 1) << 2); }
template <> __device__ __forceinline__ int kswz<8>(int r) { return (r & 7) ^ (((r >> 3) & 1) * 5); }

template <int HD, int NW>
__global__ __launch_bounds__(NW * 64) void attention_bf16_kernel(AttnParams p) {
  constexpr int KT = 32;                       // keys per tile
  constexpr int KS = HD / 16;                  // k-steps of the score product
  constexpr int DB = HD / 32;                  // 32-row blocks of O^T
  // K stage: [32 keys][HD dims] (HD*2-byte rows), 16-byte chunk c of row r at
  // chunk c ^ kswz(r).  V^T stage: 2 planes (one per 16-key step) of
  // [HD rows][32 B], the two 16-byte halves of row r swapped when hswap(r).
  // Four slots of each; tile j lives in slot j % 4.
  constexpr int KROW = HD * 2, KBYTES = KT * KROW;
  constexpr int VPL = HD * 32, VBYTES = 2 * VPL;
  static_assert(KBYTES == NW * 1024, "one K load instruction per wave and tile");
  static_assert(HD == NW * 16, "one V^T load per lane and tile");
  __shared__ __attribute__((aligned(1024))) char lds[4 * KBYTES + 4 * VBYTES];
  char* const kbuf = lds;                      // slot u at kbuf + u * KBYTES
  char* const vbuf = lds + 4 * KBYTES;         // slot u at vbuf + u * VBYTES

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int nblk = p.q_tiles * p.n_heads;
  const int lin = xcd_remap(blockIdx.x, nblk);
  const int head = lin / p.q_tiles;
  const int qtile = lin - head * p.q_tiles;
  const int N = p.n;
  const int T = (N + KT - 1) / KT;
  const int q0 = qtile * (NW * 32) + wave * 32;
  const float sc = p.scale_log2;

  // ---- Q fragments (B operand of S^T = K Q^T); queries >= N load as zero
  bf16x8 qf[KS];
  {
    const __amdgpu_buffer_rsrc_t rq = rsrc(p.q, (uint32_t)((uint64_t)N * p.ldq * 2));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t off = (uint32_t)(q0 + l32) * (uint32_t)p.ldq * 2u + (head * HD + ks * 16 + h * 8) * 2;
      const u32x4 v = bload16(rq, off);
      qf[ks] = *reinterpret_cast<const bf16x8*>(&v);
    }
  }

  // ---- K tiles: direct-to-LDS loads, one 1 KiB instruction per wave: lane l
  // -> row wave*RPI + l/CPR, physical chunk l%CPR, fetching logical chunk
  // phys ^ kswz(row).  Rows >= N load as zero (buffer bounds); tiles past the
  // last one re-load the last tile so that the load counts stay uniform.
  constexpr int CPR = KROW / 16;               // chunks per K row
  constexpr int RPI = 64 / CPR;                // rows per load instruction
  const __amdgpu_buffer_rsrc_t rk = rsrc(p.k, (uint32_t)((uint64_t)N * p.ldk * 2));
  uint32_t kdma_off;
  {
    const int row = wave * RPI + lane / CPR;
    const int c = (lane % CPR) ^ kswz<CPR>(row);
    kdma_off = (uint32_t)row * (uint32_t)p.ldk * 2u + (head * HD + c * 8) * 2;
  }
  const uint32_t ktile_bytes = (uint32_t)KT * (uint32_t)p.ldk * 2u;
  auto kdma = [&](int t) {
    const int tt = t < T ? t : T - 1;
    lds_dma16(rk, kbuf + (t & 3) * KBYTES + wave * 1024, kdma_off, (uint32_t)tt * ktile_bytes);
  };

  // ---- V^T tiles of the last passes, through registers: one 16-byte load
  // per lane: plane lane/32, row wave*16 + (lane%32)/2, half lane&1 (keys
  // 16 plane + 8 half .. +8)
  const int st_pl = lane >> 5, st_row = wave * 16 + ((lane & 31) >> 1), st_h = lane & 1;
  const __amdgpu_buffer_rsrc_t rvt = rsrc(p.vt, (uint32_t)((uint64_t)p.n_heads * HD * p.ldvt * 2));
  const uint32_t vld_off = ((uint32_t)(head * HD + st_row) * (uint32_t)p.ldvt + st_pl * 16 + st_h * 8) * 2u;
  const int vst_off = st_pl * VPL + st_row * 32 + ((st_h ^ hswap(st_row)) << 4);
  auto vload_masked = [&](int t) {             // zero for keys >= N
    const int key0 = t * KT + st_pl * 16 + st_h * 8;
    u32x4 v = {0, 0, 0, 0};
    if (key0 < N) {
      v = bload16(rvt, vld_off, (uint32_t)t * (KT * 2));
      uint16_t* e = reinterpret_cast<uint16_t*>(&v);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (key0 + j >= N) e[j] = 0;
    }
    return v;
  };
  auto vstore = [&](int t, const u32x4& v) { *reinterpret_cast<u32x4*>(vbuf + (t & 3) * VBYTES + vst_off) = v; };
  // full V^T tiles: direct-to-LDS, one 1 KiB instruction per wave: wave ->
  // plane wave / (HD/32), rows 32 (wave % (HD/32)) + lane/2, physical half
  // lane&1 (holding logical half (lane&1) ^ hswap(row))
  constexpr int RB = HD / 32;
  const int vd_row = 32 * (wave % RB) + (lane >> 1);
  const uint32_t vdma_off = ((uint32_t)(head * HD + vd_row) * (uint32_t)p.ldvt + (wave / RB) * 16 +
                             (((lane & 1) ^ hswap(vd_row)) * 8)) * 2u;
  const int vdma_dst = (wave / RB) * VPL + 32 * (wave % RB) * 32;
  auto vdma = [&](int t) { lds_dma16(rvt, vbuf + (t & 3) * VBYTES + vdma_dst, vdma_off, (uint32_t)t * (KT * 2)); };

  // ---- fragment addresses.  K: row kperm(l32), logical chunk 2ks+h;
  // V^T: row l32 (+ db*32), plane = 16-key step.
  const int kr = kperm(l32);
  const int kq = kswz<CPR>(kr);
  int k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = kr * KROW + (((2 * ks + h) ^ kq) << 4);
  const int v_frag = l32 * 32 + ((h ^ hswap(l32)) << 4);

  f32x16 O[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) O[db] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;
  f32x16 S[2];
  bf16x8 P[2][2];

  auto scores = [&](const char* kb, f32x16& s) {
    s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = mfma32a(*reinterpret_cast<const bf16x8*>(kb + k_off[ks]), qf[ks], s);
  };
  auto pv = [&](const char* vb, const bf16x8 (&pp)[2]) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        O[db] = mfma32a(*reinterpret_cast<const bf16x8*>(vb + m * VPL + db * 1024 + v_frag), pp[m], O[db]);
  };
  // keys >= N of tile t: lane half h, register r holds key 16*(r/8) + 8h + r%8
  auto mask_tail = [&](f32x16& s, int t) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (t * KT + 16 * (r >> 3) + 8 * h + (r & 7) >= N) s[r] = -INFINITY;
  };
  // probabilities against the current reference; returns the lane's sum
  auto expo = [&](const f32x16& s, bf16x8 (&pp)[2]) {
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[8 * m + j], sc, -m_ref));
        if (j & 1) ls1 += pr; else ls0 += pr;
        pp[m][j] = static_cast<bf16>(pr);
      }
    return ls0 + ls1;
  };
  // move the reference to the maximum so far, rescale O and l, recompute
  auto redo = [&](const f32x16& s, bf16x8 (&pp)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * sc;
    const float m_new = fmaxf(m_ref, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) O[db] *= alpha;
    m_ref = m_new;
    return expo(s, pp);
  };

  // ---- one tile's work, t with K_{t+1} in K slot KSL and V_{t-1} in V slot
  // VSL: the scores of tile t+1 and the product with V of tile t-1 on the
  // matrix cores, the exponentials of tile t on the vector ALUs.  Chunk i
  // issues an LDS read two chunks ahead, MFMA i (even: score k-step i/2,
  // odd: 16-key step m and row block db of the V product) and EPM of the
  // exponentials; sched_barrier keeps the chunks in this order, so that each
  // wave alternates the two units.
  auto step = [&](int t, auto u_c, auto ksl_c, auto vsl_c, bool mask) {
    constexpr int U = decltype(u_c)::value;
    const char* kb = kbuf + decltype(ksl_c)::value * KBYTES;
    const char* vb = vbuf + decltype(vsl_c)::value * VBYTES;
    if (mask) mask_tail(S[U], t);
    constexpr int NMF = KS + 2 * DB;           // MFMAs per tile (16 or 8)
    constexpr int EPM = 16 / NMF;              // exponentials per MFMA
    auto frag = [&](int i) {
      const int j = i >> 1;
      const char* a = (i & 1) ? vb + (j / DB) * VPL + (j % DB) * 1024 + v_frag : kb + k_off[j];
      return *reinterpret_cast<const bf16x8*>(a);
    };
    bf16x8 fr[NMF];
    fr[0] = frag(0);
    fr[1] = frag(1);
    // The exponential chain is skewed by one: chunk i takes the scaled score
    // of element r + 1, the exponential of element r (scaled in the previous
    // chunk) and sums element r - 1 (exponentiated in the previous chunk), so
    // no instruction waits on a result from its own chunk.
    float xa[17], pe[16];
    float ls0 = 0.f, ls1 = 0.f;
    auto sum_cvt = [&](int q) {
      if (q & 1) {
        ls1 += pe[q];
        P[U][q >> 3][(q & 7) - 1] = static_cast<bf16>(pe[q - 1]);
        P[U][q >> 3][q & 7] = static_cast<bf16>(pe[q]);
      } else {
        ls0 += pe[q];
      }
    };
    xa[0] = fmaf(S[U][0], sc, -m_ref);
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      if (i + 2 < NMF) fr[i + 2] = frag(i + 2);
      if (i & 1) {
        const int j = i >> 1;
        O[j % DB] = mfma32a(fr[i], P[1 - U][j / DB], O[j % DB]);
      } else {
        S[1 - U] = mfma32a(fr[i], qf[i >> 1], i == 0 ? f32x16{} : S[1 - U]);
      }
#pragma unroll
      for (int e = 0; e < EPM; ++e) {
        const int r = i * EPM + e;
        if (r + 1 < 16) xa[r + 1] = fmaf(S[U][r + 1], sc, -m_ref);
        pe[r] = __builtin_amdgcn_exp2f(xa[r]);
        if (r >= 1) sum_cvt(r - 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    sum_cvt(15);
    float ls = ls0 + ls1;
    if (__any(!(ls <= kLazyBound))) ls = redo(S[U], P[U]);
    l_run += ls;
  };

  // ---- two tiles per barrier.  Pass (t0, t0+1), t0 odd, with SL = t0 % 4:
  // entry: S_{t0}, P_{t0-1} in registers; K_{t0+1}, K_{t0+2}, V_{t0-1}, V_{t0}
  // in LDS.  It loads K_{t0+3}, K_{t0+4}, V_{t0+1}, V_{t0+2} (into the slots
  // of the tiles read by the previous pass) and waits for them before the
  // barrier.  TAIL passes mask the last tile and its V^T, and skip tiles >= T.
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
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
    u32x4 va = {0, 0, 0, 0}, vb = {0, 0, 0, 0};
    if constexpr (!TAIL) {
      vdma(t0 + 1);
      vdma(t0 + 2);
    } else {
      if (t0 + 1 < T) va = vload_masked(t0 + 1);
      if (t0 + 2 < T) vb = vload_masked(t0 + 2);
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
    const u32x4 v0 = vload_masked(0);
    const u32x4 v1 = T > 1 ? vload_masked(1) : u32x4{0, 0, 0, 0};
    wait_vmcnt<0>();
    vstore(0, v0);
    vstore(1, v1);
  }
  wait_lgkm0();
  wg_barrier();
  scores(kbuf, S[0]);
  if (T == 1) mask_tail(S[0], 0);
  l_run += redo(S[0], P[0]);
  if (T > 1) scores(kbuf + KBYTES, S[1]);
  wg_barrier();                                // K slots 0 and 1 are refilled next

  using Full = std::integral_constant<bool, false>;
  using Tail = std::integral_constant<bool, true>;
  int t0 = 1;
  for (; (t0 + 5) * KT <= N; t0 += 4) {        // V^T tiles up to t0+4 are full
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

  // ---- normalise and store: register r of block db holds dv = db*32 + 8*(r/4) + 4h + r%4
  {
    const int q = q0 + l32;
    const float lt = l_run + __shfl_xor(l_run, 32, kWave);
    const float inv = 1.0f / lt;
    if (q < N) {
      bf16* orow = p.o + (int64_t)q * p.ldo + head * HD;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 out;
          bf16* oe = reinterpret_cast<bf16*>(&out);
#pragma unroll
          for (int e = 0; e < 4; ++e) oe[e] = static_cast<bf16>(O[db][4 * g + e] * inv);
          *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * g + 4 * h) = out;
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
template <int HD>
static void launch_bf16_attn(const AttentionArgs& a, hipStream_t stream) {
  constexpr int NW = HD / 16;
  AttnParams p;
  p.q = (const bf16*)a.q; p.ldq = a.ldq;
  p.k = (const bf16*)a.k; p.ldk = a.ldk;
  p.vt = (const bf16*)a.vt; p.ldvt = a.ldvt;
  p.o = (bf16*)a.o; p.ldo = a.ldo;
  p.n = a.n; p.n_heads = a.n_heads;
  p.q_tiles = (a.n + NW * 32 - 1) / (NW * 32);
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  attention_bf16_kernel<HD, NW><<<dim3(p.q_tiles * p.n_heads), dim3(NW * 64), 0, stream>>>(p);
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

hipError_t launch_attention(const AttentionArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  if (a.dt == kF32) {
    if (a.head_dim == 64) launch_f32_attn<64>(a, stream);
    else launch_f32_attn<128>(a, stream);
  } else {
    if (a.head_dim == 64) launch_bf16_attn<64>(a, stream);
    else launch_bf16_attn<128>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace h3k
