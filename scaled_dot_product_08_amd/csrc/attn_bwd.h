// Internal interface between the C ABI layer and the backward kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa08 {

struct BwdParams {
  const uint16_t* q;          // (B, S, H, D) or (T, H, D), like the forward
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;          // forward output
  const uint16_t* dout;       // gradient of the loss with respect to o
  const float* lse;           // forward log-sum-exp, (B, H, S) or (H, T), natural log
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;               // workspace: rowsum(dO * O), same layout as lse
  float* lse2;                // workspace: lse * log2(e), same layout
  const int32_t* cu_seqlens;  // packed mode offsets, or nullptr
  int B, H, S;
  int n_tiles;                // 128-row tiles per (sequence, head), set by the launcher
  float c_log2;               // scale * log2(e), any sign
  float scale;
};

// Rows of one workgroup's query tile (dQ kernel) or key tile (dK/dV kernel).
constexpr int kBwdTileRows = 128;

hipError_t launch_bwd(const BwdParams& p, int D, bool bf16, bool causal, bool varlen,
                      hipStream_t stream);

}  // namespace sdpa08
