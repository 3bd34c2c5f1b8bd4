// Attention against a KV cache (decode) for gfx950: split-KV streaming on the VALU.
//
// A decode step has a handful of query rows per (sequence, head) and a long
// cache of keys and values laid out [batch, heads, seq_len, head_dim] (the
// cache layout of lnrk.cn/news/11729 §2.2). Every cached byte is used for
// one multiply-add per query row, so the step is bound by HBM bandwidth, not
// by the matrix cores: a 32x32 MFMA tile would leave 31 of its 32 query
// columns empty. The kernels therefore stream the cache through registers
// and do the arithmetic on the VALU:
//
//   * Split: each query row's cache rows are cut into `chunk`-row splits,
//     one workgroup (4 waves) per (row, split), so even B*H = 128 rows fill
//     the 256 CUs many times over.
//   * Inside a workgroup a cache row (D 16-bit values) is read by D/8 lanes,
//     16 bytes each, so one wave-wide 16-byte load covers 64/(D/8) whole rows
//     and the four waves together read one contiguous stretch of the cache.
//     Each lane keeps sixteen loads of K and sixteen of V in flight, marked
//     non-temporal (the cache is read once; measured 12 % faster than
//     default-policy loads on MI355X).
//   * Score: four packed dot2 operations per lane, then a butterfly sum over
//     the D/8 lanes of the row (DPP quad permutations and row mirrors, no LDS).
//     Every lane of the group ends with the full score.
//   * Online softmax (jianying88.com/news/49672 §3) per lane group: running
//     maximum m and sum l in the log2 domain, refreshed lazily (the stale
//     maximum is kept until the new one exceeds it by more than 8), and
//     O += p * V on the lane's eight columns in fp32.
//   * The 16 partial results of a workgroup (4 waves x 4 lane groups for
//     D = 128) merge through LDS: O = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p.
//   * With one split per row that result is final. Otherwise each split
//     stores its normalised output and log2-sum-exp, and a second kernel
//     merges the splits of a row: O = sum_s 2^(lse_s - LSE) O_s with
//     LSE = log2 sum_s 2^lse_s, the same log-sum-exp combination that lets
//     attention over key shards be merged exactly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "attn_decode.h"
#include "gfx950_util.h"

namespace sdpa08 {
namespace {

constexpr int NWAVE = 4;          // waves per workgroup
constexpr int UNROLL = 16;        // cache-row steps per wave per iteration (loads in flight)
constexpr int LOAD_AUX = 2;       // cache policy bits of the cache loads: non-temporal, streamed once
constexpr float LAZY_RESCALE_LOG2 = 8.0f;
constexpr int MAX_SPLITS = 256;

template <int D>
struct Geo {
  static constexpr int KL = D / 8;                 // lanes per cache row
  static constexpr int KPW = 64 / KL;              // cache rows per wave-wide load
  static constexpr int ROWB = D * 2;               // bytes per cache row
  static constexpr int KEYS_WAVE = KPW * UNROLL;   // rows per wave per iteration
  static constexpr int KEYS_WG = KEYS_WAVE * NWAVE;
  static constexpr int NPART = NWAVE * KPW;        // partial results per workgroup
};

// x + (x from the lane given by a DPP pattern), within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float add_dpp(float x) {
  const int y = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true);
  return x + __builtin_bit_cast(float, y);
}

// Sum over the KL lanes that hold one cache row; every lane gets the sum.
// Quad permutations [1,0,3,2] and [2,3,0,1] sum each quad; the half-row
// mirror (lane i <-> 7-i) adds the other quad of the eight; the row mirror
// (i <-> 15-i) adds the other eight of the sixteen.
template <int KL>
__device__ __forceinline__ float group_sum(float x) {
  x = add_dpp<0xB1>(x);
  x = add_dpp<0x4E>(x);
  x = add_dpp<0x141>(x);
  if constexpr (KL == 16) x = add_dpp<0x140>(x);
  return x;
}

template <bool BF16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                  false);
  }
}

// Element e (0 or 1) of a packed pair, widened to fp32 exactly.
template <bool BF16>
__device__ __forceinline__ float widen(uint32_t w, int e) {
  if constexpr (BF16) {
    return __builtin_bit_cast(float, e == 0 ? (w << 16) : (w & 0xffff0000u));
  } else {
    const f16x2 h = __builtin_bit_cast(f16x2, w);
    return (float)h[e];
  }
}

template <bool BF16>
__device__ __forceinline__ uint16_t narrow(float x) {
  if constexpr (BF16) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  } else {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(NWAVE * 64) void attn_decode_split_kernel(DecodeParams p) {
  using G = Geo<D>;
  __shared__ float s_o[G::NPART][D];
  __shared__ float s_m[G::NPART];
  __shared__ float s_l[G::NPART];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane / G::KL;       // which cache row of a wave-wide load
  const int sub = lane % G::KL;       // which 16-byte column chunk of that row

  // Workgroup i runs on XCD i % 8. With per-batch cache lengths, and when the
  // (batch, head) pairs divide evenly among the XCDs, XCD x takes pairs x,
  // x + 8, x + 16, ... with all their (split, query row) items: heads of one
  // batch share its length, so every XCD then holds the same share of each
  // batch's cache (exactly so when H is a multiple of 8), where contiguous
  // runs of pairs would hand an XCD whole batches and so unequal amounts of
  // cache. Otherwise (full caches: equal work per pair, and contiguous runs
  // measured faster there) each XCD owns a contiguous run of items. Either
  // way the Sq query rows that share a split are neighbours, so their
  // repeated cache reads meet in one L2.
  const int per_bh = p.n_splits * p.Sq;
  const int n_bh = (int)gridDim.x / per_bh;
  int logical;
  if (p.seqlens != nullptr && n_bh % NXCD == 0) {
    const int xcd = blockIdx.x % NXCD, local = blockIdx.x / NXCD;
    logical = ((local / per_bh) * NXCD + xcd) * per_bh + local % per_bh;
  } else {
    logical = xcd_logical(blockIdx.x, gridDim.x);
  }
  const int qi = logical % p.Sq;
  const int rest = logical / p.Sq;
  const int split = rest % p.n_splits;
  const int bh = rest / p.n_splits;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int row = bh * p.Sq + qi;     // (b, h, qi) in the partial-result layout

  int L = p.seqlens != nullptr ? p.seqlens[b] : p.S_max;
  L = min(max(L, 0), p.S_max);
  // Query row qi sits at position L - Sq + qi; under causality it sees keys
  // up to and including that position.
  const int kv_end = p.causal ? min(L, max(0, L - p.Sq + qi + 1)) : L;
  const int k_begin = split * p.chunk;
  const int k_stop = min(k_begin + p.chunk, kv_end);

  const u32x4 qv = *reinterpret_cast<const u32x4*>(
      p.q + (((size_t)b * p.Sq + qi) * p.H + h) * D + sub * 8);

  float m_run = -INFINITY;   // running maximum (log2 domain) of this lane group
  float l_run = 0.0f;        // running sum of 2^(t - m_run)
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;

  const size_t kvbase = ((size_t)b * p.H + h) * (size_t)p.S_max * D;
  // Rows at or past k_stop read as zeros (buffer range check) and are masked.
  const uint32_t nbytes = (uint32_t)max(k_stop, 0) * G::ROWB;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + kvbase, nbytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + kvbase, nbytes);

  for (int kb = k_begin + wave * G::KEYS_WAVE; kb < k_stop; kb += G::KEYS_WG) {
    u32x4 kr[UNROLL], vr[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint32_t off = (uint32_t)(kb + u * G::KPW + grp) * G::ROWB + sub * 16;
      kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, LOAD_AUX);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint32_t off = (uint32_t)(kb + u * G::KPW + grp) * G::ROWB + sub * 16;
      vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, LOAD_AUX);
    }

    float t[UNROLL];
    float mc = -INFINITY;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float d = dot2<BF16>(kr[u][0], qv[0], 0.0f);
      d = dot2<BF16>(kr[u][1], qv[1], d);
      d = dot2<BF16>(kr[u][2], qv[2], d);
      d = dot2<BF16>(kr[u][3], qv[3], d);
      d = group_sum<G::KL>(d);
      const int key = kb + u * G::KPW + grp;
      t[u] = key < k_stop ? d * p.c_log2 : -INFINITY;
      mc = fmaxf(mc, t[u]);
    }

    const bool bump = mc > m_run + LAZY_RESCALE_LOG2;
    if (__builtin_amdgcn_ballot_w64(bump)) {
      const float m_new = bump ? mc : m_run;
      const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    // A group that has seen no visible row keeps m = -inf; its t are -inf too.
    const float m_sub = (m_run == -INFINITY) ? 0.0f : m_run;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const float pu = __builtin_amdgcn_exp2f(t[u] - m_sub);
      l_run += pu;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(pu, widen<BF16>(vr[u][e >> 1], e & 1), acc[e]);
    }
  }

  // Merge the lane groups of all waves.
  const int part = wave * G::KPW + grp;
#pragma unroll
  for (int e = 0; e < 8; ++e) s_o[part][sub * 8 + e] = acc[e];
  if (sub == 0) {
    s_m[part] = m_run;
    s_l[part] = l_run;
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < G::NPART; ++q) M = fmaxf(M, s_m[q]);
    float lsum = 0.0f, o = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int q = 0; q < G::NPART; ++q) {
        const float w = __builtin_amdgcn_exp2f(s_m[q] - M);
        lsum = fmaf(s_l[q], w, lsum);
        o = fmaf(s_o[q][d], w, o);
      }
    }
    const bool any = lsum > 0.0f;
    const float out = any ? o / lsum : 0.0f;
    const float lse2 = any ? M + __builtin_amdgcn_logf(lsum) : -INFINITY;
    if (p.n_splits == 1) {
      p.o[(((size_t)b * p.Sq + qi) * p.H + h) * D + d] = narrow<BF16>(out);
      if (d == 0 && p.lse != nullptr) {
        p.lse[((size_t)b * p.H + h) * p.Sq + qi] = lse2 * 0.69314718055994531f;
      }
    } else {
      p.part_o[((size_t)row * p.n_splits + split) * D + d] = out;
      if (d == 0) p.part_lse[(size_t)row * p.n_splits + split] = lse2;
    }
  }
}

// One workgroup of D threads per query row: combine the row's splits.
template <int D, bool BF16>
__global__ __launch_bounds__(D) void attn_decode_merge_kernel(DecodeParams p) {
  const int row = blockIdx.x;        // (b*H + h)*Sq + qi
  const int d = threadIdx.x;
  const float* pl = p.part_lse + (size_t)row * p.n_splits;
  const float* po = p.part_o + (size_t)row * p.n_splits * D;
  float M = -INFINITY;
  for (int s = 0; s < p.n_splits; ++s) M = fmaxf(M, pl[s]);
  float wsum = 0.0f, o = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < p.n_splits; ++s) {
      const float w = __builtin_amdgcn_exp2f(pl[s] - M);
      wsum += w;
      o = fmaf(w, po[(size_t)s * D + d], o);
    }
  }
  const bool any = wsum > 0.0f;
  const int qi = row % p.Sq;
  const int bh = row / p.Sq;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  p.o[(((size_t)b * p.Sq + qi) * p.H + h) * D + d] = narrow<BF16>(any ? o / wsum : 0.0f);
  if (d == 0 && p.lse != nullptr) {
    p.lse[(size_t)bh * p.Sq + qi] =
        any ? (M + __builtin_amdgcn_logf(wsum)) * 0.69314718055994531f : -INFINITY;
  }
}

template <int D, bool BF16>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  const long long rows = (long long)p.B * p.H * p.Sq;
  hipLaunchKernelGGL((attn_decode_split_kernel<D, BF16>), dim3((unsigned)(rows * p.n_splits)),
                     dim3(NWAVE * 64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_splits == 1) return e;
  hipLaunchKernelGGL((attn_decode_merge_kernel<D, BF16>), dim3((unsigned)rows), dim3(D), 0, stream,
                     p);
  return hipGetLastError();
}

}  // namespace

DecodePlan decode_plan(int B, int H, int Sq, int S_max, int D, int num_splits_req, bool ragged) {
  const int keys_wg = (D == 64) ? Geo<64>::KEYS_WG : Geo<128>::KEYS_WG;
  const long long rows = (long long)B * H * Sq;
  long long n;
  if (num_splits_req > 0) {
    n = num_splits_req;
  } else {
    // Full caches: about 2048 workgroups (8 per CU). Ragged lengths (known
    // only on the device): 8x finer splits, so the splits past a short
    // sequence's end exit at once and the long ones do not leave a tail.
    // Every split covers at least two iterations of the workgroup loop.
    const long long target = ragged ? 16384 : 2048;
    const long long min_keys = 2LL * keys_wg;
    const long long by_size = ((long long)S_max + min_keys - 1) / min_keys;
    const long long want = rows > 0 ? (target + rows - 1) / rows : 1;
    n = want < by_size ? want : by_size;
  }
  if (n < 1) n = 1;
  if (n > MAX_SPLITS) n = MAX_SPLITS;
  long long chunk = ((long long)S_max + n - 1) / n;
  chunk = ((chunk + keys_wg - 1) / keys_wg) * keys_wg;
  if (chunk < keys_wg) chunk = keys_wg;
  n = ((long long)S_max + chunk - 1) / chunk;
  if (n < 1) n = 1;
  return DecodePlan{(int)n, (int)chunk};
}

// The split partials of attn_decode_noalloc: one array per GPU (each device
// holds its own copy at its own address), kept until the process ends. In host
// code `scratch` names a host-side stand-in, never a device address: kernels
// get the address decode_scratch looked up.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(hipStream_t stream, float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const int current = dev;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    if (dev != current && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (dev != current) {
      const hipError_t e2 = hipSetDevice(current);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (a == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = static_cast<float*>(a);
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, int D, bool bf16, hipStream_t stream) {
  if (D == 64) return bf16 ? launch_d<64, true>(p, stream) : launch_d<64, false>(p, stream);
  return bf16 ? launch_d<128, true>(p, stream) : launch_d<128, false>(p, stream);
}

}  // namespace sdpa08
