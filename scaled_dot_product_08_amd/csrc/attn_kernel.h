// Internal interface between the C ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa08 {

struct FwdParams {
  const uint16_t* q;        // (B,S,H,D) or (T,H,D), 16-bit elements
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;               // (B,H,S) or (H,T) fp32, may be null
  const int32_t* cu_seqlens;  // packed mode only (device)
  int B;                    // batch (padded) or number of sequences (packed)
  int H;
  int S;                    // sequence length (padded) or total tokens T (packed)
  int n_qtiles;             // query tiles per (batch, head), or virtual tiles (packed); set at launch
  int head_group;           // heads whose query tiles one XCD interleaves; set at launch
  float c_log2;             // |scale| * log2(e), or log2(e) when scale == 0
  int q_mode;               // 0: scale > 0, 1: scale < 0 (use -Q), 2: scale == 0 (Q := 0)
  int window;               // sliding-window width in keys (0: none)
  int n_global;             // leading query rows of each sequence that see every key
  const float* alibi;       // per-head ALiBi slopes (device), or null
};

// Largest / smallest query tile (rows per workgroup) the launcher may pick.
int max_query_tile_rows();
int min_query_tile_rows();

// Launch shape chosen by the caller instead of by problem size (0 = automatic).
struct FwdTuning {
  int tile_rows = 0;        // query rows per workgroup: 128 or 256
  int head_group = 0;       // heads whose query tiles one XCD interleaves
  int key_split = 0;        // 1: one wave per 32 rows; 2: two wave groups split the keys (128-row tiles)
};

// Launch the kernel instance for (D, dtype, causal, packed) on `stream`; picks
// the workgroup size, fills n_qtiles and head_group and sizes the grid.
hipError_t launch_fwd(const FwdParams& p, int D, bool bf16, bool causal, bool varlen,
                      const FwdTuning& tuning, hipStream_t stream);

}  // namespace sdpa08
