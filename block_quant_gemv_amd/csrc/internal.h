// Host-side launchers shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qg {

enum Fmt { kF32 = 0, kQ4_0 = 1, kQ8_0 = 2, kQ4_K = 3, kQ6_K = 4, kIQ4_NL = 5, kQ5_K = 6, kIQ4_XS = 7 };

// Elements and bytes of one block of each format (0 for F32).
int fmt_block_elems(int fmt);
int fmt_block_bytes(int fmt);
int64_t fmt_row_bytes(int fmt, int64_t k);  // -1 if k is not a multiple of the block

// One GEMV launch: y[t, r] = sum_k W[r, k] x_hat[t, k] for t < m, r < n.
// Activations are already quantized (xq int8, token stride xs elements; dx
// fp32, token stride xs/32).
//
// Grouped mode (tbl != nullptr, used by the MoE layer): grid.y runs over up
// to `nprob` table entries; tbl[0] holds the number of entries in use. Entry
// e is stored at tbl + 1 + e * tbl_stride as {expert, count, rows[count]}
// with count <= kGroupTokens: expert >= 0 uses matrix w + expert *
// w_stride, expert == -1 the shared matrix w_shared. Token j of an entry
// reads activation row rows[j] / act_div and writes output row rows[j].
// Tokens per grouped entry. Measured on MI355X at 16 tokens x top-8 of 256
// experts: one token per entry (the leanest kernel, 8 waves per SIMD) beats
// grouping 2 or 4 tokens per entry, whose token slots cost registers and
// occupancy, even though an expert chosen by several tokens is then read
// once per token (often from the last-level cache).
#ifndef QG_GROUP_TOKENS
#define QG_GROUP_TOKENS 1
#endif
constexpr int kGroupTokens = QG_GROUP_TOKENS;

struct GemvProblem {
  const uint8_t* w = nullptr;
  const int8_t* xq = nullptr;
  const float* dx = nullptr;
  int64_t xs = 0;
  // Fused quantization: with xf set, each workgroup quantizes the fp32
  // activations xf (token stride xs) itself instead of reading xq/dx; the
  // first workgroup also writes the codes to xq_out/dx_out/sx_out if set.
  const float* xf = nullptr;
  int8_t* xq_out = nullptr;
  float* dx_out = nullptr;
  int32_t* sx_out = nullptr;
  float* y = nullptr;
  int64_t ldy = 0;
  int32_t* dots = nullptr;  // checking epilogue output (int32)
  int64_t n = 0;
  int64_t k = 0;
  int m = 1;
  uint32_t cb[4] = {0, 0, 0, 0};  // IQ4_NL / IQ4_XS codebook as two byte-permute pools
  const int32_t* tbl = nullptr;
  int tbl_stride = 0;
  int nprob = 1;
  int64_t w_stride = 0;
  const uint8_t* w_shared = nullptr;
  int act_div = 1;
};

// Second copy of at most 32 tokens' quantized activations for the batched
// matrix-core path, block-major so that one block's 32 tokens are contiguous:
// codes [block][g][t % 16][t / 16][8] (g = element / 8: the 16 bytes of
// tokens t and t + 16 for elements 8 g .. 8 g + 7 sit together), the block
// scales dx [block][32] and the products dx * (block code sum) c [block][32].
// Token slots m..31 are not written.
struct TiledAct {
  int8_t* codes = nullptr;
  float* dx = nullptr;
  float* c = nullptr;
  int kblocks = 0;
};
__host__ __device__ inline int64_t tiled_code_offset(int64_t b, int t, int e) {
  return b * 1024 + (((e >> 3) * 16 + (t & 15)) * 2 + (t >> 4)) * 8 + (e & 7);
}

// Q8 quantizer over nblocks 32-element blocks (token-major). With tiled set
// it also writes the block-major copy for the matrix-core path (at most 32
// tokens of tiled->kblocks blocks each).
hipError_t launch_quant_q8(const float* x, int8_t* xq, float* dx, int32_t* sx,
                           int64_t nblocks, hipStream_t s, const TiledAct* tiled = nullptr);

// Row GEMV over packed blocks for m <= 16 tokens (chunks larger m on the
// host). dots_epilogue selects the integer-store checking epilogue.
hipError_t launch_gemv(int fmt, const GemvProblem& p, bool dots_epilogue, hipStream_t s);

// Codes xq [m, k] (m <= 32) copied to the block-major layout of TiledAct::codes.
hipError_t launch_tile_codes(const int8_t* xq, int8_t* xqt, int m, int kblocks, hipStream_t s);

// Single-token Q4_K / Q5_K GEMV that loads the 16-byte-aligned super-block
// fields straight into registers (no LDS); applies when kdirect_ok(fmt, p):
// m == 1, quantized activations given, no grouping, K a multiple of 2048 up
// to 8192. dots selects the integer-store checking epilogue (p.dots, int32
// [n, K/32]).
bool kdirect_ok(int fmt, const GemvProblem& p, bool dots);
hipError_t launch_kdirect(int fmt, const GemvProblem& p, bool dots, hipStream_t s);

// Launch facts of the current device (launch_cache.cpp), looked up and
// filled under one lock, keyed by device: safe from several threads at once.
constexpr int kLdsBytes = 160 * 1024;  // LDS per CU on gfx950
int device_cus();
// Resident workgroups per CU of kernel `kern` launched with `threads` threads
// and `lds` bytes of dynamic LDS (at least 1); with raise_lds the kernel's
// dynamic-LDS limit is first raised to kLdsBytes (once per kernel and
// device). cus (optional) receives the device's compute-unit count.
hipError_t kernel_residency(const void* kern, int threads, size_t lds, bool raise_lds, int* per_cu,
                            int* cus = nullptr);
// Forgets every cached fact (the next launch of each kernel queries again).
void clear_launch_cache();

// Streaming-read measurement (stream.hip): reads bytes (a multiple of 16,
// buf 16-byte aligned) once with 16-byte non-temporal loads over every CU.
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t s);

// Bytes of the fixed device scratch behind the allocation-free GEMV entry
// point (noalloc.hip), and the address of the current device's copy of it
// (looked up once per device with that device current).
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
hipError_t noalloc_scratch(void** out);

// Largest token count one GEMV launch handles.
constexpr int kGemvMaxTokens = 16;
// From this many tokens on, Q4_K and Q6_K GEMVs run on int8 MFMA (the VALU
// dot-product kernel's cost grows with the token count, the MFMA one's not).
constexpr int kMfmaMinTokens = 9;

}  // namespace qg
