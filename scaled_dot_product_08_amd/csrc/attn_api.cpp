// C ABI of the attention-forward library: argument validation, kernel
// instance selection, grid sizing and launch on the caller's stream.
// Validation is pure host logic and returns before any HIP call.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/attn.h"
#include "attn_bwd.h"
#include "attn_clock.h"
#include "attn_decode.h"
#include "attn_fp8.h"
#include "attn_kernel.h"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ATTN_DEBUG=1 (read once, at the first call that could use it) makes the
// packed-mode entry points validate cu_seqlens first, synchronizing.
bool debug_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("ATTN_DEBUG");
    return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
  }();
  return on;
}

// The HIP error of this thread's most recent launch (attn_last_hip_error).
thread_local int g_last_hip_error = 0;

// A stale error that an earlier runtime call of the caller's thread left
// behind would otherwise be read back as this call's launch error.
void clear_stale_error() { (void)hipGetLastError(); }

int launch_status(hipError_t e) {
  g_last_hip_error = (int)e;
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Validation shared by attn_fwd; no HIP call. Fills the grid size on success.
int validate(const void* q, const void* k, const void* v, void* out, const float* lse, int B,
             int H, int S, int D, float scale, int dtype, const int32_t* cu, long long* grid) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return ATTN_ERR_NULL;
  if (dtype != ATTN_DTYPE_FP16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_DTYPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  const bool packed = cu != nullptr;
  if (H < 1 || H > 65535 || S < 0) return ATTN_ERR_SHAPE;
  if (packed ? (B < 0) : (B < 1)) return ATTN_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return ATTN_ERR_ALIGN;
  if (lse != nullptr && !aligned(lse, 4)) return ATTN_ERR_ALIGN;
  // Element count must fit in int64 (it always does for int inputs, but the
  // product of four ints is checked explicitly).
  const long double elems = (long double)(packed ? 1 : B) * S * H * D;
  if (elems > (long double)LLONG_MAX / 2) return ATTN_ERR_SHAPE;
  // The grid is largest with the smallest query tile; check that bound.
  const long long bm = sdpa08::min_query_tile_rows();
  long long tiles;
  if (packed) {
    tiles = (long long)S / bm + B;                // virtual tiles of the packed batch
    *grid = tiles * H;
  } else {
    tiles = ((long long)S + bm - 1) / bm;
    *grid = tiles * B * H;
  }
  if (*grid > INT_MAX) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

// Validation of attn_decode's arguments; no HIP call. Fills the split plan.
int validate_decode(const void* q, const void* k, const void* v, void* out, const float* lse,
                    int B, int H, int Sq, int S_max, int D, float scale, int dtype,
                    int num_splits, bool ragged, sdpa08::DecodePlan* plan) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return ATTN_ERR_NULL;
  if (dtype != ATTN_DTYPE_FP16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_DTYPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if (B < 0 || H < 1 || H > 65535 || Sq < 0 || S_max < 0 || num_splits < 0) return ATTN_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return ATTN_ERR_ALIGN;
  if (lse != nullptr && !aligned(lse, 4)) return ATTN_ERR_ALIGN;
  // Byte offsets inside one (batch, head) cache slice are 32-bit, with room
  // for the last partial step past the end.
  if ((long long)S_max * D * 2 + (1LL << 20) > (long long)UINT32_MAX) return ATTN_ERR_SHAPE;
  const long double elems = (long double)B * H * ((long double)S_max + Sq) * D;
  if (elems > (long double)LLONG_MAX / 2) return ATTN_ERR_SHAPE;
  *plan = sdpa08::decode_plan(B, H, Sq, S_max, D, num_splits, ragged);
  const long long rows = (long long)B * H * Sq;
  if (rows * plan->n_splits > INT_MAX) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

size_t decode_workspace_bytes(long long rows, const sdpa08::DecodePlan& plan, int D) {
  if (plan.n_splits <= 1) return 0;
  return (size_t)rows * plan.n_splits * (size_t)(D + 1) * sizeof(float);
}

}  // namespace

extern "C" {

int attn_version(void) { return kVersion; }

int attn_last_hip_error(void) { return g_last_hip_error; }

int attn_clock_sample(uint64_t* dst, void* stream) {
  if (dst == nullptr) return ATTN_ERR_NULL;
  if (!aligned(dst, 8)) return ATTN_ERR_ALIGN;
  clear_stale_error();
  return launch_status(sdpa08::launch_clock_sample(dst, reinterpret_cast<hipStream_t>(stream)));
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, H or S out of range (or the problem is too large)";
    case ATTN_ERR_DTYPE: return "unknown dtype (expected ATTN_DTYPE_FP16 or ATTN_DTYPE_BF16)";
    case ATTN_ERR_SCALE: return "scale is not finite";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension (expected 64 or 128)";
    case ATTN_ERR_LAUNCH: return "HIP runtime error at launch";
    case ATTN_ERR_SEQLENS: return "cu_seqlens is not a valid prefix-offset array";
    case ATTN_ERR_ALIGN: return "tensor pointer misaligned (q/k/v/out need 16 bytes, lse 4)";
    case ATTN_ERR_WORKSPACE: return "workspace missing or smaller than attn_decode_workspace_size";
    case ATTN_ERR_SCRATCH:
      return "the requested split count needs more than the library's 16 MiB per-GPU scratch array";
    default: return "unknown status";
  }
}

int attn_check_cu_seqlens(const int32_t* cu_seqlens, int B, int T, void* stream) {
  if (cu_seqlens == nullptr) return ATTN_ERR_NULL;
  if (B < 0 || T < 0) return ATTN_ERR_SHAPE;
  std::vector<int32_t> h((size_t)B + 1);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(h.data(), cu_seqlens, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
      hipSuccess) {
    return ATTN_ERR_LAUNCH;
  }
  if (hipStreamSynchronize(st) != hipSuccess) return ATTN_ERR_LAUNCH;
  if (h[0] != 0 || h[B] != T) return ATTN_ERR_SEQLENS;
  for (int i = 0; i < B; ++i) {
    if (h[i + 1] < h[i]) return ATTN_ERR_SEQLENS;
  }
  return ATTN_OK;
}

static int fwd_common(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                      int H, int S, int D, int causal, float scale, int dtype,
                      const int32_t* cu_seqlens, int window, int n_global, const float* alibi,
                      const sdpa08::FwdTuning& tuning, void* stream) {
  long long grid = 0;
  const int st = validate(q, k, v, out, lse, B, H, S, D, scale, dtype, cu_seqlens, &grid);
  if (st != ATTN_OK) return st;
  if (window < 0 || n_global < 0) return ATTN_ERR_SHAPE;
  const bool packed = cu_seqlens != nullptr;
  if (S == 0 || (packed && B == 0)) return ATTN_OK;
  if (packed && debug_enabled()) {
    const int c = attn_check_cu_seqlens(cu_seqlens, B, S, stream);
    if (c != ATTN_OK) return c;
  }
  sdpa08::FwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.B = B;
  p.H = H;
  p.S = S;
  p.n_qtiles = 0;   // set by the launcher for the workgroup size it picks
  p.head_group = 0;  // set by the launcher
  const float log2e = 1.4426950408889634f;
  if (scale > 0.0f) {
    p.c_log2 = scale * log2e;
    p.q_mode = 0;
  } else if (scale < 0.0f) {
    p.c_log2 = -scale * log2e;
    p.q_mode = 1;
  } else {
    p.c_log2 = log2e;
    p.q_mode = 2;
  }
  p.window = window;
  p.n_global = n_global;
  p.alibi = alibi;
  clear_stale_error();
  return launch_status(sdpa08::launch_fwd(p, D, dtype == ATTN_DTYPE_BF16, causal != 0, packed,
                                          tuning, reinterpret_cast<hipStream_t>(stream)));
}

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
             int S, int D, int causal, float scale, int dtype, const int32_t* cu_seqlens,
             void* stream) {
  return fwd_common(q, k, v, out, lse, B, H, S, D, causal, scale, dtype, cu_seqlens, 0, 0,
                    nullptr, sdpa08::FwdTuning{}, stream);
}

int attn_fwd_tuned(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                   int H, int S, int D, int causal, float scale, int dtype,
                   const int32_t* cu_seqlens, int tile_rows, int key_split, int head_group,
                   void* stream) {
  if (tile_rows != 0 && tile_rows != 128 && tile_rows != 256) return ATTN_ERR_UNSUPPORTED;
  if (key_split < 0 || key_split > 2 || (key_split == 2 && tile_rows == 256)) {
    return ATTN_ERR_UNSUPPORTED;
  }
  if (head_group < 0) return ATTN_ERR_SHAPE;
  sdpa08::FwdTuning t;
  t.tile_rows = tile_rows;
  t.key_split = key_split;
  t.head_group = head_group;
  return fwd_common(q, k, v, out, lse, B, H, S, D, causal, scale, dtype, cu_seqlens, 0, 0,
                    nullptr, t, stream);
}

int attn_fwd_ext(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                 int H, int S, int D, int causal, float scale, int dtype,
                 const int32_t* cu_seqlens, int window, int n_global,
                 const float* alibi_slopes, void* stream) {
  if (alibi_slopes != nullptr && !aligned(alibi_slopes, 4)) return ATTN_ERR_ALIGN;
  return fwd_common(q, k, v, out, lse, B, H, S, D, causal, scale, dtype, cu_seqlens, window,
                    n_global, alibi_slopes, sdpa08::FwdTuning{}, stream);
}

int attn_fwd_ext_tuned(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                       int H, int S, int D, int causal, float scale, int dtype,
                       const int32_t* cu_seqlens, int window, int n_global,
                       const float* alibi_slopes, int tile_rows, int head_group, void* stream) {
  if (tile_rows != 0 && tile_rows != 128 && tile_rows != 256) return ATTN_ERR_UNSUPPORTED;
  if (tile_rows == 256 && (window != 0 || n_global != 0 || alibi_slopes == nullptr || D != 128)) {
    return ATTN_ERR_UNSUPPORTED;
  }
  if (head_group < 0) return ATTN_ERR_SHAPE;
  if (alibi_slopes != nullptr && !aligned(alibi_slopes, 4)) return ATTN_ERR_ALIGN;
  sdpa08::FwdTuning t;
  t.tile_rows = tile_rows;
  t.key_split = 1;
  t.head_group = head_group;
  return fwd_common(q, k, v, out, lse, B, H, S, D, causal, scale, dtype, cu_seqlens, window,
                    n_global, alibi_slopes, t, stream);
}

size_t attn_decode_workspace_size(int B, int H, int Sq, int S_max, int D, int num_splits) {
  if (B < 0 || H < 1 || Sq < 0 || S_max < 0 || num_splits < 0 || (D != 64 && D != 128)) return 0;
  // Sized for the ragged plan, which has at least as many splits as the
  // full-cache one: one size serves calls with and without seqlens_k.
  const sdpa08::DecodePlan plan = sdpa08::decode_plan(B, H, Sq, S_max, D, num_splits, true);
  return decode_workspace_bytes((long long)B * H * Sq, plan, D);
}

// Shared by attn_decode (caller's workspace) and attn_decode_noalloc (the
// library's per-GPU scratch array; ws == nullptr and noalloc set).
static int decode_common(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* seqlens_k, void* out, float* lse, int B, int H, int Sq,
                         int S_max, int D, int causal, float scale, int dtype, int num_splits,
                         void* workspace, size_t workspace_bytes, bool noalloc, void* stream) {
  sdpa08::DecodePlan plan{1, 0};
  const bool ragged = seqlens_k != nullptr;
  const int st = validate_decode(q, k_cache, v_cache, out, lse, B, H, Sq, S_max, D, scale, dtype,
                                 num_splits, ragged, &plan);
  if (st != ATTN_OK) return st;
  if (seqlens_k != nullptr && !aligned(seqlens_k, 4)) return ATTN_ERR_ALIGN;
  const long long rows = (long long)B * H * Sq;
  size_t need = decode_workspace_bytes(rows, plan, D);
  if (noalloc && need > sdpa08::kDecodeScratchBytes) {
    // An explicit split count is honoured or refused; the automatic choice
    // shrinks to what the scratch array holds (one split needs none).
    if (num_splits > 0) return ATTN_ERR_SCRATCH;
    const long long per_split = rows * (long long)(D + 1) * (long long)sizeof(float);
    long long fit = (long long)sdpa08::kDecodeScratchBytes / per_split;
    if (fit < 1) fit = 1;
    plan = sdpa08::decode_plan(B, H, Sq, S_max, D, (int)fit, ragged);
    need = decode_workspace_bytes(rows, plan, D);
    if (need > sdpa08::kDecodeScratchBytes) return ATTN_ERR_SCRATCH;   // cannot happen
  }
  if (!noalloc) {
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 16)) return ATTN_ERR_ALIGN;
  }
  if (rows == 0) return ATTN_OK;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  float* part = need > 0 ? static_cast<float*>(workspace) : nullptr;
  if (noalloc && need > 0) {
    clear_stale_error();
    const hipError_t es = sdpa08::decode_scratch(hs, &part);
    if (es != hipSuccess) return launch_status(es);
  }
  sdpa08::DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k_cache);
  p.v = static_cast<const uint16_t*>(v_cache);
  p.seqlens = seqlens_k;
  p.o = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.part_o = part;
  p.part_lse = need > 0 ? p.part_o + (size_t)rows * plan.n_splits * D : nullptr;
  p.B = B;
  p.H = H;
  p.Sq = Sq;
  p.S_max = S_max;
  p.n_splits = plan.n_splits;
  p.chunk = plan.chunk;
  p.c_log2 = scale * 1.4426950408889634f;
  p.causal = causal != 0;
  clear_stale_error();
  return launch_status(sdpa08::launch_decode(p, D, dtype == ATTN_DTYPE_BF16, hs));
}

int attn_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* seqlens_k, void* out, float* lse, int B, int H, int Sq,
                int S_max, int D, int causal, float scale, int dtype, int num_splits,
                void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(q, k_cache, v_cache, seqlens_k, out, lse, B, H, Sq, S_max, D, causal,
                       scale, dtype, num_splits, workspace, workspace_bytes, false, stream);
}

int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seqlens_k, void* out, float* lse, int B, int H, int Sq,
                        int S_max, int D, int causal, float scale, int dtype, int num_splits,
                        void* stream) {
  return decode_common(q, k_cache, v_cache, seqlens_k, out, lse, B, H, Sq, S_max, D, causal,
                       scale, dtype, num_splits, nullptr, 0, true, stream);
}

size_t attn_bwd_workspace_size(int B, int H, int S, int packed) {
  if (H < 1 || S < 0 || B < 0) return 0;
  const long long rows = packed ? (long long)S : (long long)B * S;
  return 2 * (size_t)rows * H * sizeof(float);   // rowsum(dO * O) and LSE * log2(e)
}

int attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int B, int H, int S, int D,
             int causal, float scale, int dtype, const int32_t* cu_seqlens, void* workspace,
             size_t workspace_bytes, void* stream) {
  long long grid = 0;
  // q, k, v and out are checked like the forward's (out is an input here).
  const int st = validate(q, k, v, const_cast<void*>(out), lse, B, H, S, D, scale, dtype,
                          cu_seqlens, &grid);
  if (st != ATTN_OK) return st;
  if (lse == nullptr || dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr) {
    return ATTN_ERR_NULL;
  }
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16)) {
    return ATTN_ERR_ALIGN;
  }
  const bool packed = cu_seqlens != nullptr;
  const size_t need = attn_bwd_workspace_size(B, H, S, packed ? 1 : 0);
  if (S == 0 || (packed && B == 0)) return ATTN_OK;
  if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return ATTN_ERR_ALIGN;
  if (packed && debug_enabled()) {
    const int c = attn_check_cu_seqlens(cu_seqlens, B, S, stream);
    if (c != ATTN_OK) return c;
  }
  sdpa08::BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(out);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.delta = static_cast<float*>(workspace);
  p.lse2 = p.delta + need / (2 * sizeof(float));
  p.cu_seqlens = cu_seqlens;
  p.B = B;
  p.H = H;
  p.S = S;
  p.n_tiles = 0;
  p.c_log2 = scale * 1.4426950408889634f;
  p.scale = scale;
  clear_stale_error();
  return launch_status(sdpa08::launch_bwd(p, D, dtype == ATTN_DTYPE_BF16, causal != 0, packed,
                                          reinterpret_cast<hipStream_t>(stream)));
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                 int H, int S, int D, int causal, float scale, float descale_q, float descale_k,
                 float descale_v, int out_dtype, const int32_t* cu_seqlens, void* stream) {
  long long grid = 0;
  const int st = validate(q, k, v, out, lse, B, H, S, D, scale, out_dtype, cu_seqlens, &grid);
  if (st != ATTN_OK) return st;
  if (D != 128) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(descale_q) || !std::isfinite(descale_k) || !std::isfinite(descale_v)) {
    return ATTN_ERR_SCALE;
  }
  const float eff = scale * descale_q * descale_k;
  if (!std::isfinite(eff)) return ATTN_ERR_SCALE;
  const bool packed = cu_seqlens != nullptr;
  if (S == 0 || (packed && B == 0)) return ATTN_OK;
  if (packed && debug_enabled()) {
    const int c = attn_check_cu_seqlens(cu_seqlens, B, S, stream);
    if (c != ATTN_OK) return c;
  }
  sdpa08::Fp8Params p;
  p.q = static_cast<const uint8_t*>(q);
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.o = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.B = B;
  p.H = H;
  p.S = S;
  p.n_qtiles = 0;
  const float log2e = 1.4426950408889634f;
  if (eff > 0.0f) {
    p.c_log2 = eff * log2e;
    p.q_mode = 0;
  } else if (eff < 0.0f) {
    p.c_log2 = -eff * log2e;
    p.q_mode = 1;
  } else {
    p.c_log2 = log2e;
    p.q_mode = 2;
  }
  p.v_descale = descale_v;
  clear_stale_error();
  return launch_status(sdpa08::launch_fwd_fp8(p, out_dtype == ATTN_DTYPE_BF16, causal != 0,
                                              packed, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
