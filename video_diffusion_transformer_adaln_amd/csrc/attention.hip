// Full (non-causal) multi-head self-attention over all video-latent tokens,
// the middle stage of the block (h3.c memory-techniques page, technique 2).
//
// bf16 path (flash-style, fp32 online softmax, v_mfma_f32_32x32x16_bf16):
//   * one workgroup = 4 waves = 4*QB*32 queries of one head; each wave keeps
//     its queries' Q fragments in registers and loops over all keys in tiles
//     of 64, staged (double-buffered) in LDS;
//   * scores are computed transposed, S^T = K Q^T, so that the accumulator's
//     lane index is the query: every lane owns its query's running max and
//     sum, and rescaling the output needs no cross-lane traffic except one
//     xor-32 exchange for the tile maximum;
//   * K rows are read through a fixed key permutation (bits 2 and 3 of the
//     key index swapped inside each 32-key block), so that the eight
//     probabilities a lane holds per 16-key step are eight consecutive keys;
//     they then serve directly as the B operand of O^T = V^T P^T;
//   * V arrives transposed (V^T [H*d, ldvt], written so by the QKV projection),
//     so the A operand of O^T = V^T P^T is a 16-byte read along the key axis;
//   * keys beyond N contribute exactly zero: their K rows load as zero, their
//     scores are set to -inf and their V^T entries to zero.
// fp32 path: one thread per query, K/V tiles in LDS, for the small fp32
// workload.
#include "common.hpp"
#include "kernels.hpp"
#ifndef H3K_ATTN_KT
#define H3K_ATTN_KT 64
#endif
#ifndef H3K_QB
#define H3K_QB 1
#endif
#ifndef H3K_NW
#define H3K_NW 8
#endif

namespace h3k {

struct AttnParams {
  const bf16* q; int64_t ldq;
  const bf16* k; int64_t ldk;
  const bf16* vt; int64_t ldvt;
  bf16* o; int64_t ldo;
  int n, n_heads, q_tiles;
  float scale_log2;   // log2(e) / sqrt(d)
};

constexpr float kRescaleLog2 = 8.0f;   // lazy-rescale threshold (log2 units)

__device__ __forceinline__ f32x16 mfma32a(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// 16-byte direct-to-LDS buffer load: lane l's 16 bytes land at lds_dst + 16 l.
// (A plain device function: host compilation never instantiates its body.)
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, char* lds_dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, 0, 0, 0);
}
// Row halves are swapped when bit 2 xor bit 3 of the row is set (LDS banks).
__device__ __forceinline__ int hswap(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }
// Key permutation inside a 32-key block: swap bits 2 and 3.
__device__ __forceinline__ int kperm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
// Chunk swizzle of a K row of CPR 16-byte chunks (CPR = 16 for d = 128, 8 for
// d = 64): the fragment reads of rows kperm(0..7), kperm(8..15) and of any 16
// consecutive rows each land on distinct banks (checked exhaustively offline).
template <int CPR> __device__ __forceinline__ int kswz(int r);
template <> __device__ __forceinline__ int kswz<16>(int r) { return (r & 15) ^ (((r >> 3) & 1) << 2); }
template <> __device__ __forceinline__ int kswz<8>(int r) { return (r & 7) ^ (((r >> 3) & 1) * 5); }

template <int HD, int KT, int QB, int NW>
__global__ __launch_bounds__(NW * 64) void attention_bf16_kernel(AttnParams p) {
  constexpr int KB = KT / 32;                  // 32-key blocks per tile
  // K stage: [64 keys][HD dims] (HD*2-byte rows), 16-byte chunk c of row r at
  // chunk c ^ kswz(r).  V^T stage: 4 planes (one per 16-key step) of [HD rows][32 B].
  constexpr int KROW = HD * 2, KBYTES = KT * KROW;
  constexpr int VPL = HD * 32, VBYTES = (KT / 16) * VPL;
  __shared__ __attribute__((aligned(1024))) char lds[2 * KBYTES + 2 * VBYTES];
  char* const kbuf0 = lds;
  char* const kbuf1 = lds + KBYTES;
  char* const vbuf0 = lds + 2 * KBYTES;
  char* const vbuf1 = lds + 2 * KBYTES + VBYTES;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int nblk = p.q_tiles * p.n_heads;
  const int lin = xcd_remap(blockIdx.x, nblk);
  const int head = lin / p.q_tiles;
  const int qtile = lin - head * p.q_tiles;
  const int N = p.n;
  const int T = (N + KT - 1) / KT;
  const int q0 = qtile * (NW * QB * 32) + wave * (QB * 32);

  // ---- Q fragments (B operand of S^T = K Q^T)
  bf16x8 qf[QB][HD / 16];
  {
    const __amdgpu_buffer_rsrc_t rq = rsrc(p.q, (uint32_t)((uint64_t)N * p.ldq * 2));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ks = 0; ks < HD / 16; ++ks) {
        const uint32_t off = (uint32_t)(q0 + qb * 32 + l32) * (uint32_t)p.ldq * 2u + (head * HD + ks * 16 + h * 8) * 2;
        const u32x4 v = bload16(rq, off);
        qf[qb][ks] = *reinterpret_cast<const bf16x8*>(&v);
      }
  }

  // ---- K tiles: direct-to-LDS loads.  A wave instruction fills 1 KiB =
  // KT*KROW/1024 ... rows (HD*2 bytes each); lane l -> row r0 + l/(KROW/16),
  // physical chunk l%(KROW/16), fetching logical chunk phys ^ kswz(row).
  constexpr int CPR = KROW / 16;               // chunks per K row
  constexpr int RPI = 64 / CPR;                // rows per DMA instruction
  constexpr int KDMA = KT / RPI / NW;          // DMA instructions per wave per tile
  static_assert(KDMA >= 1 && KDMA * RPI * NW == KT, "K tile does not split over the waves");
  const __amdgpu_buffer_rsrc_t rk = rsrc(p.k, (uint32_t)((uint64_t)N * p.ldk * 2));
  uint32_t kdma_off[KDMA];
#pragma unroll
  for (int j = 0; j < KDMA; ++j) {
    const int row = (j * NW + wave) * RPI + lane / CPR;
    const int c = (lane % CPR) ^ kswz<CPR>(row);
    kdma_off[j] = (uint32_t)row * (uint32_t)p.ldk * 2u + (head * HD + c * 8) * 2;
  }
  auto kdma = [&](int t, char* dst) {
    const uint32_t kofs = (uint32_t)t * KT * (uint32_t)p.ldk * 2u;
#pragma unroll
    for (int j = 0; j < KDMA; ++j)
      lds_dma16(rk, dst + (j * NW + wave) * RPI * KROW, kdma_off[j] + kofs);
  };

  // ---- V^T tiles: register staging (keys >= N are zeroed here)
  // a wave instruction covers (KT/16) planes x (64/(KT/16)/2) rows x 2 halves
  constexpr int VPLN = KT / 16;                // planes per tile
  constexpr int VRPW = 32 / VPLN;              // V^T rows per wave instruction
  const int st_pl = lane / (64 / VPLN), st_row = (lane % (64 / VPLN)) >> 1, st_h = lane & 1;
  constexpr int VLOADS = (HD * KT / 8) / (NW * 64);
  static_assert(VLOADS >= 1 && VLOADS * NW * VRPW == HD, "V^T tile does not split over the waves");
  u32x4 rv_[VLOADS];
  auto vload = [&](int t) {
    const int k0 = t * KT;
    const bool full = k0 + KT <= N;
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int row = i * (NW * VRPW) + wave * VRPW + st_row;
      const int key0 = k0 + st_pl * 16 + st_h * 8;
      const bf16* src = p.vt + (int64_t)(head * HD + row) * p.ldvt + key0;
      if (full) {
        rv_[i] = *reinterpret_cast<const u32x4*>(src);
      } else {
        u32x4 v = {0, 0, 0, 0};
        if (key0 < N) {
          v = *reinterpret_cast<const u32x4*>(src);
          uint16_t* e = reinterpret_cast<uint16_t*>(&v);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (key0 + j >= N) e[j] = 0;
        }
        rv_[i] = v;
      }
    }
  };
  auto vstore = [&](char* base) {
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int row = i * (NW * VRPW) + wave * VRPW + st_row;
      *reinterpret_cast<u32x4*>(base + st_pl * VPL + row * 32 + ((st_h ^ hswap(row)) << 4)) = rv_[i];
    }
  };

  // ---- fragment addresses.  K: row kperm(l32) (+ kb*32), chunk 2ks+h;
  // V^T: row l32 (+ db*32), plane = 16-key step.
  const int kr = kperm(l32);
  const int kq = kswz<CPR>(kr);
  int k_off[HD / 16];
#pragma unroll
  for (int ks = 0; ks < HD / 16; ++ks) k_off[ks] = kr * KROW + (((2 * ks + h) ^ kq) << 4);
  const int v_frag = l32 * 32 + ((h ^ hswap(l32)) << 4);

  f32x16 O[HD / 32][QB];
#pragma unroll
  for (int db = 0; db < HD / 32; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) O[db][qb] = f32x16{};
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m_run[qb] = -INFINITY; l_run[qb] = 0.f; }

  auto scores = [&](const char* kb_base, f32x16 (&S)[KB][QB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) S[kb][qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb_base + kb * 32 * KROW + k_off[ks]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) S[kb][qb] = mfma32a(a, qf[qb][ks], S[kb][qb]);
      }
  };

  // keys >= N of the last tile: lane half h, register r of key block kb holds
  // key kb*32 + 16*(r/8) + 8h + r%8
  auto mask_tail = [&](f32x16 (&S)[KB][QB], int t) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool out = t * KT + kb * 32 + 16 * (r >> 3) + 8 * h + (r & 7) >= N;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) S[kb][qb][r] = out ? -INFINITY : S[kb][qb][r];
      }
  };
  // softmax of one tile (scores S) -> P; rescales O and l when the reference max moves
  auto softmax = [&](const f32x16 (&S)[KB][QB], bf16x8 (&P)[KB][2][QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][qb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * p.scale_log2;
      if (__any(mx > m_run[qb] + kRescaleLog2)) {
        const float m_new = fmaxf(m_run[qb], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        l_run[qb] *= alpha;
        m_run[qb] = m_new;
#pragma unroll
        for (int db = 0; db < HD / 32; ++db) {   // one 16-register tile at a time
          O[db][qb] *= alpha;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const float m_ref = m_run[qb];
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float pr = __builtin_amdgcn_exp2f(fmaf(S[kb][qb][8 * m + j], p.scale_log2, -m_ref));
            ls += pr;
            P[kb][m][qb][j] = static_cast<bf16>(pr);
          }
      l_run[qb] += ls;
    }
  };

  auto pv = [&](const char* vb, const bf16x8 (&P)[KB][2][QB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int db = 0; db < HD / 32; ++db) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vb + (2 * kb + m) * VPL + db * 1024 + v_frag);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) O[db][qb] = mfma32a(a, P[kb][m][qb], O[db][qb]);
        }
  };

  // ---- prologue: K_0, K_1 and V_0 in LDS, S_0 computed
  kdma(0, kbuf0);
  if (T > 1) kdma(1, kbuf1);
  vload(0);
  vstore(vbuf0);
  __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt = 0: the K loads have landed
  __syncthreads();
  f32x16 Sa[KB][QB], Sb[KB][QB];
  bf16x8 P[KB][2][QB];
  scores(kbuf0, Sa);
  __syncthreads();                             // kbuf0 is refilled in iteration 0

  // ---- iteration t: S_{t+1} = K_{t+1} Q^T runs alongside softmax(S_t);
  // then O += V_t P_t.  K_{t+2} and V_{t+1} are staged meanwhile.  Past the
  // last tile these loads and scores are harmless extra work (K rows >= N
  // load as zero, V^T past N is zeroed, stale LDS stays finite) and keep the
  // loop body free of branches.
  auto step = [&](int t, f32x16 (&Scur)[KB][QB], f32x16 (&Snext)[KB][QB]) {
    char* kdst = (t & 1) ? kbuf1 : kbuf0;       // held K_t (consumed in iteration t-1)
    const char* ksrc = (t & 1) ? kbuf0 : kbuf1; // K_{t+1}
    const char* vsrc = (t & 1) ? vbuf1 : vbuf0; // V_t
    char* vdst = (t & 1) ? vbuf0 : vbuf1;       // V_{t+1}
    kdma(t + 2, kdst);
    vload(t + 1);
    scores(ksrc, Snext);
    softmax(Scur, P);
    pv(vsrc, P);
    vstore(vdst);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };
  int t = 0;
  for (; t + 2 < T; t += 2) {                  // all but the last one or two tiles
    step(t, Sa, Sb);
    step(t + 1, Sb, Sa);
  }
  if (T - t == 2) {
    step(t, Sa, Sb);
    mask_tail(Sb, t + 1);
    step(t + 1, Sb, Sa);
  } else {
    mask_tail(Sa, t);
    step(t, Sa, Sb);
  }

  // ---- normalise and store: register r of tile db holds dv = db*32 + 8*(r/4) + 4h + r%4
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = q0 + qb * 32 + l32;
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32, kWave);
    const float inv = 1.0f / lt;
    if (q >= N) continue;
    bf16* orow = p.o + (int64_t)q * p.ldo + head * HD;
#pragma unroll
    for (int db = 0; db < HD / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 out;
        bf16* oe = reinterpret_cast<bf16*>(&out);
#pragma unroll
        for (int e = 0; e < 4; ++e) oe[e] = static_cast<bf16>(O[db][qb][4 * g + e] * inv);
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * g + 4 * h) = out;
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
template <int HD, int KT, int QB, int NW>
static void launch_bf16_attn(const AttentionArgs& a, hipStream_t stream) {
  AttnParams p;
  p.q = (const bf16*)a.q; p.ldq = a.ldq;
  p.k = (const bf16*)a.k; p.ldk = a.ldk;
  p.vt = (const bf16*)a.vt; p.ldvt = a.ldvt;
  p.o = (bf16*)a.o; p.ldo = a.ldo;
  p.n = a.n; p.n_heads = a.n_heads;
  p.q_tiles = (a.n + NW * QB * 32 - 1) / (NW * QB * 32);
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  attention_bf16_kernel<HD, KT, QB, NW><<<dim3(p.q_tiles * p.n_heads), dim3(NW * 64), 0, stream>>>(p);
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
    if (a.head_dim == 64) launch_bf16_attn<64, 64, H3K_QB, H3K_NW>(a, stream);
    else launch_bf16_attn<128, H3K_ATTN_KT, H3K_QB, H3K_NW>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace h3k
