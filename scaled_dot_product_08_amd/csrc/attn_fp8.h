// Internal interface between the C ABI layer and the FP8 forward kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa08 {

struct Fp8Params {
  const uint8_t* q;           // E4M3 codes, (B, S, H, 128) or (T, H, 128)
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;                // bf16 or fp16 output, same layout
  float* lse;                 // (B, H, S) or (H, T), natural log, or nullptr
  const int32_t* cu_seqlens;  // packed mode offsets, or nullptr
  int B, H, S;
  int n_qtiles;               // set by the launcher
  float c_log2;               // |scale * descale_q * descale_k| * log2(e)
  int q_mode;                 // 0: as is, 1: negate Q (negative scale), 2: zero Q
  float v_descale;            // descale_v
};

hipError_t launch_fwd_fp8(const Fp8Params& p, bool out_bf16, bool causal, bool varlen,
                          hipStream_t stream);

}  // namespace sdpa08
