// Host stand-ins for the kernel launchers and the few HIP runtime calls of the
// C-ABI layer (h3k_api.cpp), for an AddressSanitizer / UBSan build of that
// layer on the CPU.  The driver passes host buffers as "device" memory; each
// launcher stand-in touches the first and last byte of every row it would read
// (and writes those of every row it would write), so that a planner offset or
// a validation gap that lets a kernel reach outside a buffer shows up as an
// ASan report.  It also checks the launch preconditions the real kernels rely
// on (32-bit buffer offsets, tile multiples).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kernels.hpp"

namespace {

volatile unsigned char g_sink;
int64_t g_launches = 0;

[[noreturn]] void die(const char* what) {
  std::fprintf(stderr, "launch precondition violated: %s\n", what);
  std::abort();
}
void need(bool ok, const char* what) {
  if (!ok) die(what);
}

int64_t es(h3k::DType d) { return d == h3k::kF32 ? 4 : d == h3k::kBF16 ? 2 : 1; }

// rows x cols elements of `esz` bytes at pitch ld (elements)
void touch_read(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t esz) {
  if (rows <= 0 || cols <= 0) return;
  need(p != nullptr, "read of a NULL operand");
  const unsigned char* b = static_cast<const unsigned char*>(p);
  for (int64_t r = 0; r < rows; ++r) {
    g_sink = b[r * ld * esz];
    g_sink = b[(r * ld + cols) * esz - 1];
  }
}
void touch_write(void* p, int64_t rows, int64_t cols, int64_t ld, int64_t esz) {
  if (rows <= 0 || cols <= 0) return;
  need(p != nullptr, "write to a NULL operand");
  unsigned char* b = static_cast<unsigned char*>(p);
  for (int64_t r = 0; r < rows; ++r) {
    b[r * ld * esz] = 0;
    b[(r * ld + cols) * esz - 1] = 0;
  }
}
bool fits31(int64_t bytes) { return bytes >= 0 && bytes < (int64_t(1) << 31); }

}  // namespace

extern "C" int64_t h3k_stub_launches() { return g_launches; }

namespace h3k {

hipError_t launch_adaln_gemv(DType dt, int rows, int cols, const void* w, const void* b, const void* c, float* mod,
                             hipStream_t) {
  ++g_launches;
  touch_read(w, rows, cols, cols, es(dt));
  if (b) touch_read(b, 1, rows, rows, es(dt));
  touch_read(c, 1, cols, cols, es(dt));
  touch_write(mod, 1, rows, rows, 4);
  return hipSuccess;
}

hipError_t launch_ln_modulate(DType dt, int n, int D, float, const void* x, int64_t ldx, const float* shift,
                              const float* scale, void* out, int64_t ldo, hipStream_t) {
  ++g_launches;
  touch_read(x, n, D, ldx, es(dt));
  touch_read(shift, 1, D, D, 4);
  touch_read(scale, 1, D, D, 4);
  touch_write(out, n, D, ldo, es(dt));
  return hipSuccess;
}

hipError_t launch_linear(const LinearArgs& a, hipStream_t, int* kernels) {
  ++g_launches;
  if (kernels) *kernels = 1;
  // int8 weights widened into the staging buffer first (one more kernel),
  // then a bf16 GEMM
  const bool staged = a.weight == kINT8 && a.act == kBF16 && a.wstage && a.wstage_bytes >= a.n * a.k * 2;
  if (staged) {
    touch_write(a.wstage, a.n, a.k, a.k, 2);
    touch_read(a.wstage, a.n, a.k, a.k, 2);
    ++g_launches;
    if (kernels) *kernels = 2;
  }
  // the tail split as the bf16 launcher takes it on 256 compute units: the
  // partial tiles it writes must lie inside the scratch it was given
  if (a.part && a.act == kBF16 && (a.weight == kBF16 || staged) && a.epi != kEpiBiasRope && a.split_col >= a.n) {
    const int64_t tiles = ((a.m + 255) / 256) * ((a.n + 255) / 256);
    const int S = tail_split_ways(tiles, a.k / 64, 256, a.part_bytes / kPartTileBytes);
    if (S) {
      const int64_t used = (tiles % 256) * S * kPartTileBytes;
      need(used <= a.part_bytes, "k-split partial tiles inside their scratch");
      touch_write(a.part, 1, used, used, 1);
      touch_read(a.part, 1, used, used, 1);
      ++g_launches;
      if (kernels) ++*kernels;
    }
  }
  const int64_t ex = es(a.act), ew = es(a.weight), ey = a.act == kINT8 ? 2 : es(a.act);
  if (a.act != kF32) {
    need(a.k % (a.act == kINT8 ? 128 : 64) == 0, "k-tile multiple");
    need(fits31((a.m + 256) * a.ldx * ex) && fits31((a.n + 256) * a.ldw * ew), "32-bit operand offsets");
  }
  touch_read(a.x, a.m, a.k, a.ldx, ex);
  touch_read(a.w, a.n, a.k, a.ldw, ew);
  if (a.weight == kINT8) {
    if (a.group) touch_read(a.w_scale, a.n, a.k / a.group, a.k / a.group, 4);
    else touch_read(a.w_scale, 1, a.n, a.n, 4);
  }
  if (a.act == kINT8) touch_read(a.x_scale, 1, a.m, a.m, 4);
  if (a.bias) touch_read(a.bias, 1, a.n, a.n, ey);
  if (a.epi == kEpiGatedResidual) {
    touch_read(a.residual, a.m, a.split_col, a.ldr, ey);
    touch_read(a.gate, 1, a.split_col, a.split_col, 4);
  }
  if (a.scale_cols) need(a.scale_cols <= a.split_col, "scaled columns inside the row-major part");
  touch_write(a.y, a.m, a.split_col, a.ldy, ey);
  if (a.split_col < a.n) touch_write(a.yt, a.n - a.split_col, a.m, a.ldyt, ey);
  return hipSuccess;
}

hipError_t launch_attention(const AttentionArgs& a, hipStream_t, int* kernels) {
  ++g_launches;
  if (kernels) *kernels = 1;
  const int64_t e = es(a.dt), D = (int64_t)a.n_heads * a.head_dim;
  need(a.ldvt >= (a.n + 7) / 8 * 8, "V^T pitch covers the 8-padded keys");
  touch_read(a.q, a.n, D, a.ldq, e);
  touch_read(a.k, a.n, D, a.ldk, e);
  touch_read(a.vt, D, a.n, a.ldvt, e);
  touch_write(a.o, a.n, D, a.ldo, e);
  // the key split as the bf16 launcher takes it on 256 compute units: the
  // partial results it writes must lie inside the scratch it was given
  if (a.part && a.dt == kBF16 && a.head_dim == 128 && a.n > 0) {
    int S = 0;
    const int nw = attn_shape128(a.n, a.n_heads, 256, a.part_bytes, &S);
    const int64_t slots = 256 * (nw == 4 ? 2 : 1);
    const int64_t blocks = (a.n + nw * 32 - 1) / (nw * 32) * a.n_heads;
    if (S) {
      const int64_t used = (blocks % slots) * S * attn_unit_bytes(nw);
      need(used <= a.part_bytes, "key-split partial results inside their scratch");
      touch_write(a.part, 1, used, used, 1);
      touch_read(a.part, 1, used, used, 1);
      ++g_launches;
      if (kernels) *kernels = 2;
    }
  }
  return hipSuccess;
}

hipError_t launch_token_merge(DType dt, int64_t n, int64_t D, const void* x, int64_t ldx, void* xm, int64_t ldm,
                              hipStream_t) {
  ++g_launches;
  touch_read(x, n, D, ldx, es(dt));
  touch_write(xm, n / 2, D, ldm, es(dt));
  return hipSuccess;
}

hipError_t launch_token_unmerge(DType dt, int64_t n, int64_t D, const void* entry, int64_t lde, const void* xm,
                                int64_t ldm, void* out, int64_t ldo, hipStream_t) {
  ++g_launches;
  touch_read(entry, n, D, lde, es(dt));
  touch_read(xm, n / 2, D, ldm, es(dt));
  touch_write(out, n, D, ldo, es(dt));
  return hipSuccess;
}

hipError_t launch_rope(int64_t n, int64_t cols, int, int, int, float, void* x, int64_t ldx, hipStream_t) {
  ++g_launches;
  touch_read(x, n, cols, ldx, 2);
  touch_write(x, n, cols, ldx, 2);
  return hipSuccess;
}

hipError_t launch_quantize_int8(DType dt, const void* w, int64_t rows, int64_t cols, int8_t* q, float* scales,
                                hipStream_t) {
  ++g_launches;
  touch_read(w, rows, cols, cols, es(dt));
  touch_write(q, rows, cols, cols, 1);
  touch_write(scales, 1, rows, rows, 4);
  return hipSuccess;
}

hipError_t launch_quantize_int8_groups(DType dt, const void* w, int64_t rows, int64_t cols, int group, int8_t* q,
                                       float* scales, hipStream_t) {
  ++g_launches;
  touch_read(w, rows, cols, cols, es(dt));
  touch_write(q, rows, cols, cols, 1);
  touch_write(scales, rows, cols / group, cols / group, 4);
  return hipSuccess;
}

}  // namespace h3k

// ---- the HIP runtime calls h3k_api.cpp makes: a device is present, events are
// host tokens with a fixed 1 ms between any two
extern "C" {
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub HIP runtime"; }
hipError_t hipEventCreate(hipEvent_t* event) {
  *event = reinterpret_cast<hipEvent_t>(new char[1]);
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t event) {
  delete[] reinterpret_cast<char*>(event);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 1.0f;
  return hipSuccess;
}
// one device with MI355X-like properties
hipError_t hipGetDeviceCount(int* count) {
  *count = 1;
  return hipSuccess;
}
hipError_t hipGetDeviceProperties(hipDeviceProp_t* prop, int device) {
  if (device != 0) return hipErrorInvalidDevice;
  std::memset(prop, 0, sizeof(*prop));
  prop->multiProcessorCount = 256;
  prop->clockRate = 2400000;
  prop->maxSharedMemoryPerMultiProcessor = 160 * 1024;
  prop->warpSize = 64;
  prop->totalGlobalMem = size_t(288) << 30;
  std::snprintf(prop->gcnArchName, sizeof(prop->gcnArchName), "gfx950:sramecc+:xnack-");
  return hipSuccess;
}
}
