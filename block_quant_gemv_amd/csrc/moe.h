#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qg {

// Buffers and shapes of one MoE layer call (all device pointers).
struct MoeCall {
  const float* router = nullptr;  // fp32 [n_experts, hidden]
  const uint8_t *gu = nullptr, *dn = nullptr, *gu_shared = nullptr, *dn_shared = nullptr;
  int64_t gu_stride = 0, dn_stride = 0;  // bytes between experts
  const float* x = nullptr;              // fp32 [m, hidden]
  float* y = nullptr;                    // fp32 [m, hidden]
  int m = 1;
  int64_t hidden = 0, inter = 0;
  int n_experts = 0, top_k = 0, fmt = 0;
  uint32_t cb[4] = {0, 0, 0, 0};
  // workspace regions
  float* logits = nullptr;   // [m, n_experts]
  int32_t* ids = nullptr;    // [m, top_k]
  float* wts = nullptr;      // [m, top_k]
  int8_t* xq = nullptr;      // [m, hidden]
  float* dx = nullptr;       // [m, hidden/32]
  int32_t* sx = nullptr;
  float* gu_out = nullptr;   // [m*(top_k+1), 2*inter] (slot rows)
  float* h = nullptr;        // [m*(top_k+1), inter]
  int8_t* hq = nullptr;
  float* hd = nullptr;
  int32_t* hs = nullptr;
  float* out = nullptr;      // [m*(top_k+1), hidden]
  int32_t* tbl = nullptr;    // grouping table, moe_table_ints(m, top_k) ints
  // 16-bit activation variant (Q4_0 experts): when set, x and h are
  // quantized to int16 codes here (dx/sx and hd/hs then hold their scales
  // and sums) and the expert GEMVs run on them.
  int16_t* xq16 = nullptr;   // [m, hidden]
  int16_t* hq16 = nullptr;   // [m*(top_k+1), inter]
};

// int32 entries of the expert grouping table for m tokens and top_k slots.
int64_t moe_table_ints(int m, int top_k);

hipError_t launch_moe(const MoeCall& c, hipStream_t s);

// The expert stage (after the router launch has written logits and the Q8
// codes of x) in two launches: routing + gate|up + SwiGLU + re-quantization,
// then down + weighted combine (moe_fused.hip). moe_fused_ok tells whether the
// call's shapes fit it: 1..16 tokens, top_k <= 15, at most 1024 experts,
// hidden a multiple of 2048 up to 8192 with m * hidden <= 65536, inter in
// {512, 1024, 2048, 4096}, row bytes a multiple of 16, and rows short enough
// for one load per wave (and the up workgroup's LDS).
bool moe_fused_ok(const MoeCall& c);
hipError_t launch_moe_fused(const MoeCall& c, hipStream_t s);

}  // namespace qg
