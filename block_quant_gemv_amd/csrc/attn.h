// Host-side launchers of the decode-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qg {

struct AttnShape {
  int n_heads = 0;     // query heads
  int n_kv = 0;        // key/value heads (n_heads % n_kv == 0)
  int head_dim = 0;    // 128 or 256
  int64_t n_ctx = 0;   // cached tokens
};

// Chunking chosen for a shape: tokens per chunk and number of chunks (one
// chunk means the single-pass path, no merge).
struct AttnPlan {
  int64_t chunk = 0;
  int64_t nchunks = 0;
};

bool attn_supported(const AttnShape& a);
// Whether stage 1 runs its scores on matrix cores (head dimension 256, 8
// query heads per key/value head).
bool attn_uses_mfma(const AttnShape& a);
AttnPlan attn_plan(const AttnShape& a);
// Workspace bytes for the chunk partials (0 when one chunk suffices).
size_t attn_workspace_bytes(const AttnShape& a);
hipError_t launch_attn(const AttnShape& a, const float* q, const uint16_t* k, const uint16_t* v, float* out,
                       void* ws, hipStream_t s);

}  // namespace qg
