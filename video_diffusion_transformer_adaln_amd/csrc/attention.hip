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

namespace h3k {

struct AttnParams {
  const bf16* q; int64_t ldq;
  const bf16* k; int64_t ldk;
  const bf16* vt; int64_t ldvt;
  bf16* o; int64_t ldo;
  int n, n_heads, q_tiles;
  float scale_log2;   // log2(e) / sqrt(d)
};

constexpr int KT = 64;   // keys per tile
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
// Row halves are swapped when bit 2 xor bit 3 of the row is set (LDS banks).
__device__ __forceinline__ int hswap(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }
// Key permutation inside a 32-key block: swap bits 2 and 3.
__device__ __forceinline__ int kperm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

template <int HD, int QB>
__global__ __launch_bounds__(256) void attention_bf16_kernel(AttnParams p) {
  // K tile: HD/16 planes (one per 16-wide d-step) of [64 keys][32 B];
  // V^T tile: 4 planes (one per 16-key step) of [HD rows][32 B].
  constexpr int KPL = KT * 32, KBYTES = (HD / 16) * KPL;
  constexpr int VPL = HD * 32, VBYTES = 4 * VPL;
  constexpr int STAGE = KBYTES + VBYTES;
  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int nblk = p.q_tiles * p.n_heads;
  const int lin = xcd_remap(blockIdx.x, nblk);
  const int head = lin / p.q_tiles;          // all q-tiles of a head on one XCD range
  const int qtile = lin - head * p.q_tiles;
  const int N = p.n;
  const int q0 = qtile * (4 * QB * 32) + wave * (QB * 32);

  // ---- Q fragments (B operand of S^T = K Q^T): query q0+qb*32+l32, dims ks*16+h*8..+7
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

  // ---- staging assignment (conflict-free LDS stores: 16 lanes fill 8 rows x 32 B of one plane)
  const __amdgpu_buffer_rsrc_t rk = rsrc(p.k, (uint32_t)((uint64_t)N * p.ldk * 2));
  const int st_pl = lane >> 4, st_row = (lane & 15) >> 1, st_h = lane & 1;
  constexpr int KLOADS = (KT * HD / 8) / 256;   // 16-byte chunks per thread per K tile
  constexpr int VLOADS = (HD * KT / 8) / 256;
  u32x4 rk_[KLOADS], rv_[VLOADS];

  auto gload = [&](int t) {
    const int k0 = t * KT;
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      // plane group (i % (HD/64)) * 4 + st_pl, key block (i / (HD/64)) * 32 + wave * 8 + st_row
      const int pl = (i % (HD / 64)) * 4 + st_pl;
      const int key = (i / (HD / 64)) * 32 + wave * 8 + st_row;
      const uint32_t off = (uint32_t)(k0 + key) * (uint32_t)p.ldk * 2u + (head * HD + pl * 16 + st_h * 8) * 2;
      rk_[i] = bload16(rk, off);
    }
    const bool full = k0 + KT <= N;
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int row = i * 32 + wave * 8 + st_row;             // dv
      const int key0 = k0 + st_pl * 16 + st_h * 8;            // first key of the chunk
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
  auto lstore = [&](char* base) {
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int pl = (i % (HD / 64)) * 4 + st_pl;
      const int key = (i / (HD / 64)) * 32 + wave * 8 + st_row;
      *reinterpret_cast<u32x4*>(base + pl * KPL + key * 32 + ((st_h ^ hswap(key)) << 4)) = rk_[i];
    }
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int row = i * 32 + wave * 8 + st_row;
      *reinterpret_cast<u32x4*>(base + KBYTES + st_pl * VPL + row * 32 + ((st_h ^ hswap(row)) << 4)) = rv_[i];
    }
  };

  // fragment addresses: K row kperm(l32) (+ kb*32), V^T row l32 (+ db*32)
  const int kr = kperm(l32);
  const int k_frag = kr * 32 + ((h ^ hswap(kr)) << 4);
  const int v_frag = KBYTES + l32 * 32 + ((h ^ hswap(l32)) << 4);

  f32x16 O[HD / 32][QB];
#pragma unroll
  for (int db = 0; db < HD / 32; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) O[db][qb] = f32x16{};
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m_run[qb] = -INFINITY; l_run[qb] = 0.f; }

  const int T = (N + KT - 1) / KT;
  gload(0);
  lstore(lds);
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    const char* cur = lds + (t & 1) * STAGE;
    if (t + 1 < T) gload(t + 1);

    // ---- S^T[key][query] for 64 keys x QB*32 queries
    f32x16 S[2][QB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) S[kb][qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(cur + ks * KPL + kb * 1024 + k_frag);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) S[kb][qb] = mfma32a(a, qf[qb][ks], S[kb][qb]);
      }
    }
    // ---- mask keys >= N (last tile only).  Lane half h, register r of key
    // block kb holds key kb*32 + 16*(r/8) + 8h + r%8.
    if ((t + 1) * KT > N) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t * KT + kb * 32 + 16 * (r >> 3) + 8 * h + (r & 7);
          if (key >= N) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) S[kb][qb][r] = -INFINITY;
          }
        }
    }
    // ---- online softmax (log2 domain), P rounded to bf16 for the MFMA.
    // The reference max m_run is raised (and O, l rescaled) only when some
    // lane's tile maximum exceeds it by more than kRescaleLog2; otherwise the
    // old reference is kept and p <= 2^kRescaleLog2.  O / l at the end is the
    // same either way.
    bf16x8 P[2][2][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][qb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * p.scale_log2;
      if (__any(mx > m_run[qb] + kRescaleLog2)) {
        const float m_new = fmaxf(m_run[qb], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        l_run[qb] *= alpha;
        m_run[qb] = m_new;
#pragma unroll
        for (int db = 0; db < HD / 32; ++db) O[db][qb] *= alpha;
      }
      const float m_ref = m_run[qb];
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
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
    // ---- O^T[dv][query] += V^T[dv][keys] P^T[keys][query]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int db = 0; db < HD / 32; ++db) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(cur + (2 * kb + m) * VPL + db * 1024 + v_frag);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) O[db][qb] = mfma32a(a, P[kb][m][qb], O[db][qb]);
        }

    if (t + 1 < T) lstore(lds + ((t + 1) & 1) * STAGE);
    __syncthreads();
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
template <int HD, int QB>
static void launch_bf16_attn(const AttentionArgs& a, hipStream_t stream) {
  AttnParams p;
  p.q = (const bf16*)a.q; p.ldq = a.ldq;
  p.k = (const bf16*)a.k; p.ldk = a.ldk;
  p.vt = (const bf16*)a.vt; p.ldvt = a.ldvt;
  p.o = (bf16*)a.o; p.ldo = a.ldo;
  p.n = a.n; p.n_heads = a.n_heads;
  p.q_tiles = (a.n + 4 * QB * 32 - 1) / (4 * QB * 32);
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  attention_bf16_kernel<HD, QB><<<dim3(p.q_tiles * p.n_heads), dim3(256), 0, stream>>>(p);
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
    // Two query blocks per wave when there is enough work to fill the chip
    // several times over; one otherwise (shorter tail).
    const int64_t wg2 = (int64_t)((a.n + 255) / 256) * a.n_heads;
    const bool qb2 = wg2 >= 4 * 256;
    if (a.head_dim == 64) {
      if (qb2) launch_bf16_attn<64, 2>(a, stream); else launch_bf16_attn<64, 1>(a, stream);
    } else {
      if (qb2) launch_bf16_attn<128, 2>(a, stream); else launch_bf16_attn<128, 1>(a, stream);
    }
  }
  return hipGetLastError();
}

}  // namespace h3k
