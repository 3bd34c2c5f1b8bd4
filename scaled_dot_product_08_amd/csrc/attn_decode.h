// Internal interface between the C ABI layer and the KV-cache decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa08 {

struct DecodeParams {
  const uint16_t* q;        // (B, Sq, H, D)
  const uint16_t* k;        // (B, H, S_max, D) cache
  const uint16_t* v;        // (B, H, S_max, D) cache
  const int32_t* seqlens;   // (B) valid cache rows, or nullptr (all S_max)
  uint16_t* o;              // (B, Sq, H, D)
  float* lse;               // (B, H, Sq) natural log, or nullptr
  float* part_o;            // (B*H*Sq, n_splits, D) normalised partial outputs (n_splits > 1)
  float* part_lse;          // (B*H*Sq, n_splits) log2-domain partial LSE (n_splits > 1)
  int B, H, Sq, S_max;
  int n_splits;             // key splits per query row
  int chunk;                // keys per split (multiple of the per-workgroup step)
  float c_log2;             // scale * log2(e), any sign
  int causal;
};

// How a decode call is split: n_splits workgroups per query row, each
// covering `chunk` consecutive cache rows.
struct DecodePlan {
  int n_splits;
  int chunk;
};

// `ragged`: per-sequence lengths are given (finer splits). A ragged plan
// never has fewer splits than the full-cache plan of the same shapes.
DecodePlan decode_plan(int B, int H, int Sq, int S_max, int D, int num_splits_req, bool ragged);

hipError_t launch_decode(const DecodeParams& p, int D, bool bf16, hipStream_t stream);

// Size of the library's own per-GPU scratch array that attn_decode_noalloc
// keeps the split partials in (instead of a caller's workspace).
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;

// Device address of that array on the device `stream` belongs to (the current
// device for the null stream). The first call on a device looks it up with
// that device current and keeps it; later calls return the kept address.
hipError_t decode_scratch(hipStream_t stream, float** ptr);

}  // namespace sdpa08
