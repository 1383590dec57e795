// Streaming-read ceiling: the rate at which this GPU reads a buffer once
// from HBM with the load shape of the GEMVs (16-byte non-temporal vector
// loads, several in flight per lane, every CU busy). A GEMV cannot move its
// weights faster than this at the same size, so the measurement pages drill
// down to exactly this kind of single-kernel read test ("01 · Phase
// overview: from 2B to 8B to MoE", icman.com.cn, issue ledger: isolate the
// access pattern in a microbenchmark). It is a measurement export, not part
// of the GEMV path.
#include "common.cuh"
#include "internal.h"

namespace qg {

namespace {

constexpr int kThreads = 256;
// 16-byte loads per lane per piece. Measured on MI355X at 9 MB .. 570 MB:
// one load per lane and piece, with enough resident waves, reads faster than
// 2, 4 or 8 loads per lane, and faster than a grid stride, from 28 MB up.
constexpr int kUnroll = 1;
constexpr uint32_t kNever = 0x9E3779B9u;

// Each wave reads contiguous pieces of kUnroll KB (kUnroll loads of 1 KB,
// all in flight together), piece w, w + waves, ...; the last partial piece
// is read by all threads with a grid stride.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                               uint32_t* __restrict__ out) {
  constexpr int kPiece = 64 * kUnroll;  // 16-byte units per piece
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t full = n16 / kPiece * kPiece;
  uint32_t acc = 0;
  for (int64_t c = wave * kPiece; c < full; c += waves * kPiece) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + c + 64 * u + lane);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int64_t i = full + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += (int64_t)gridDim.x * kThreads) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // The loaded values decide whether anything is stored, so the loads stay;
  // with real data the store practically never happens.
  if (acc == kNever) atomicXor(out, acc);
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t s) {
  if (!buf || !out || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15)) return hipErrorInvalidValue;
  if (bytes == 0) return hipSuccess;
  int per_cu = 0, cus = 0;
  hipError_t e = kernel_residency(reinterpret_cast<const void*>(stream_read_kernel), kThreads, 0, false, &per_cu,
                                  &cus);
  if (e != hipSuccess) return e;
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t grid = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
  const int64_t pieces = (n16 + 64 * kUnroll - 1) / (64 * kUnroll);
  const int64_t need = (pieces + kThreads / 64 - 1) / (kThreads / 64);
  if (grid > need) grid = need;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s,
                     reinterpret_cast<const u32x4*>(buf), n16, out);
  return hipGetLastError();
}

}  // namespace qg
