// Fused attention forward for gfx950 (CDNA4): MFMA + LDS-tiled online softmax.
//
// One workgroup of 4 waves (256 lanes) owns a tile of BM = 128 query rows of
// one (sequence, head); wave w owns rows 32w..32w+31 of the tile. The kernel
// streams the visible keys in tiles of BN = 64 rows through double-buffered
// LDS and, per tile, runs the fused chain of mlqm.cn/news/343191 §3.1
// (Q K^T -> scale -> mask -> softmax -> P V) with the online softmax of
// jianying88.com/news/49672 §3: a running row maximum m and exponential sum l
// per query row, so no score ever leaves registers.
//
// Orientation (what makes the softmax cheap on a 64-lane wave):
//   * Scores are produced transposed, S^T = K Q^T, by v_mfma_f32_32x32x16
//     with A = a 32-key block of K (from LDS) and B = Q^T (registers). The
//     accumulator column index is the lane (mod 32), so each lane holds one
//     query row and 16 of its 32 keys; the other 16 sit in lane ^ 32. A row
//     max / sum is 15 in-lane ops plus one exchange with lane ^ 32.
//   * The output is accumulated transposed too, O^T += V^T P^T, with B = the
//     probabilities straight out of the score accumulator (cast to 16 bit)
//     and A = V^T read from LDS. Each lane again owns one query row, so the
//     rescale by exp(m_old - m_new) is a per-lane scalar.
//   * V is transposed once per tile on its way into LDS (in registers), and
//     its key columns and head-dim rows are permuted so that every MFMA
//     operand is one 16-byte LDS read and every O store is 16 bytes.
//
// Exponentials use exp2 on logits pre-multiplied by scale*log2(e). The row
// maximum is refreshed lazily: the stale maximum is kept until the new one
// exceeds it by more than 2^8 (probabilities are then at most 256, exact in
// the normalisation because the same maximum enters numerator and
// denominator), which saves most of the accumulator rescales.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_kernel.h"

namespace sdpa08 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;       // query rows per workgroup
constexpr int BN = 64;        // keys per LDS tile
constexpr int NWAVES = 4;
constexpr int NTHREADS = NWAVES * 64;
constexpr float LAZY_RESCALE_LOG2 = 8.0f;

// 32x32x16 MFMA, fp32 accumulate; a/b carry eight 16-bit values each.
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Two floats -> two 16-bit values (round to nearest even), low half first.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  f32x2 v = {x, y};
  if constexpr (BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
}

// acc + lo(p) + hi(p): sums the 16-bit probabilities exactly as they enter P V.
template <bool BF16>
__device__ __forceinline__ float add_pair(uint32_t p, float acc) {
  if constexpr (BF16) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), one, acc, false);
  } else {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), one, acc, false);
  }
}

// Swap bits 2 and 3 of a small index. Used twice:
//  * V^T column of key j inside a 64-key tile, so that the eight keys one
//    lane contributes to a P V step are adjacent;
//  * V^T row read by MFMA row p, so that each lane ends up with runs of
//    eight consecutive head-dim outputs.
__device__ __forceinline__ int swap23(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

__device__ __forceinline__ float wave_xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

template <int D, bool BF16, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NTHREADS, 2) void attn_fwd_kernel(FwdParams p) {
  constexpr int KSTR = D + 8;          // K tile row stride in LDS (elements)
  constexpr int VSTR = BN + 8;         // V^T tile row stride in LDS (elements)
  constexpr int DCH = D / 16;          // 16-deep contraction chunks of Q K^T
  constexpr int DB = D / 32;           // 32-row blocks of O^T
  constexpr int KCH = D / 8;           // 16-byte chunks per K/V row
  constexpr int K_LD = BN * KCH / NTHREADS;   // K chunks per lane per tile
  constexpr int KG = (D == 128) ? 4 : 2;      // keys per lane in the V transpose
  static_assert((BN / KG) * KCH == NTHREADS, "V transpose mapping must cover the tile");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][D * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;     // query row inside the wave's 32 / MFMA row
  const int hh = lane >> 5;     // which half of the contraction this lane feeds

  // ---- which (sequence, head, query tile) this workgroup owns -------------
  // Linear id: the query-tile rank is the slowest index and is taken in
  // reverse, so the longest causal tiles start first; (batch, head) is the
  // fastest index, so consecutive workgroups (which land on different XCDs)
  // carry different heads and every query tile of one head lands on the
  // same XCD whenever the head count is a multiple of 8.
  const int nbh = VARLEN ? p.H : p.B * p.H;
  const int rank = blockIdx.x / nbh;
  const int bh = blockIdx.x - rank * nbh;
  const int h = bh % p.H;
  const int b = VARLEN ? 0 : bh / p.H;
  const int vt = p.n_qtiles - 1 - rank;
  int seq_start = 0, L = p.S, q0;
  if constexpr (VARLEN) {
    // Virtual tile space: sequence s owns tiles [cu[s]/BM + s, ... + ceil(L_s/BM)).
    // These ranges are disjoint and lie in [0, T/BM + B); gaps are idle.
    int lo = 0, hi = p.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.cu_seqlens[mid] / BM + mid <= vt) lo = mid; else hi = mid - 1;
    }
    seq_start = p.cu_seqlens[lo];
    L = p.cu_seqlens[lo + 1] - seq_start;
    q0 = (vt - (seq_start / BM + lo)) * BM;
    if (q0 >= L) return;        // idle virtual tile (uniform over the workgroup)
  } else {
    q0 = vt * BM;
  }

  const size_t tok_stride = (size_t)p.H * D;
  const size_t base = ((size_t)b * p.S + seq_start) * tok_stride + (size_t)h * D;
  const uint16_t* __restrict__ qg = p.q + base;
  const uint16_t* __restrict__ kg = p.k + base;
  const uint16_t* __restrict__ vg = p.v + base;
  uint16_t* __restrict__ og = p.o + base;

  const int kv_end = CAUSAL ? min(q0 + BM, L) : L;
  const int n_kv = (kv_end + BN - 1) / BN;
  const int wq0 = q0 + wave * 32;        // first query row of this wave
  const int qi = wq0 + li;               // this lane's query row

  // ---- Q^T operand, resident in registers for the whole key loop ----------
  // Rows past the sequence end load the last row instead (never stored).
  const int qi_ld = min(qi, L - 1);
  u32x4 qreg[DCH];
#pragma unroll
  for (int c = 0; c < DCH; ++c) {
    qreg[c] = *reinterpret_cast<const u32x4*>(qg + (size_t)qi_ld * tok_stride + c * 16 + hh * 8);
    if (p.q_mode == 1) qreg[c] ^= 0x80008000u;          // negative scale: use -Q, |scale|
    else if (p.q_mode == 2) qreg[c] = u32x4{0u, 0u, 0u, 0u};  // zero scale: all scores 0
  }
  const float c_log2 = p.c_log2;          // |scale| * log2(e) (> 0)

  // ---- K / V tile staging ---------------------------------------------------
  u32x4 kpre[K_LD];
  u32x4 vpre[KG];
  const int v_grp = tid / KCH;           // key group (KG keys) of this lane
  const int v_dc = tid - v_grp * KCH;    // 8-wide head-dim chunk of this lane

  auto load_tile = [&](int j) {
    const int key0 = j * BN;
#pragma unroll
    for (int u = 0; u < K_LD; ++u) {
      const int c = tid + u * NTHREADS;
      const int row = c / KCH, col = (c - row * KCH) * 8;
      const int r = min(key0 + row, L - 1);
      kpre[u] = *reinterpret_cast<const u32x4*>(kg + (size_t)r * tok_stride + col);
    }
#pragma unroll
    for (int u = 0; u < KG; ++u) {
      const int row = v_grp * KG + u;
      const int r = min(key0 + row, L - 1);
      vpre[u] = *reinterpret_cast<const u32x4*>(vg + (size_t)r * tok_stride + v_dc * 8);
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < K_LD; ++u) {
      const int c = tid + u * NTHREADS;
      const int row = c / KCH, col = (c - row * KCH) * 8;
      *reinterpret_cast<u32x4*>(&k_lds[buf][row * KSTR + col]) = kpre[u];
    }
    // Transpose KG keys x 8 dims into 8 rows of V^T (KG adjacent columns each).
    const int col = swap23(v_grp * KG);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int w = dd >> 1;
      const bool odd = dd & 1;
      uint32_t pair[KG / 2];
#pragma unroll
      for (int u = 0; u < KG / 2; ++u) {
        const uint32_t a = vpre[2 * u][w], c2 = vpre[2 * u + 1][w];
        pair[u] = odd ? ((a >> 16) | (c2 & 0xffff0000u)) : ((a & 0xffffu) | (c2 << 16));
      }
      uint16_t* dst = &vt_lds[buf][(v_dc * 8 + dd) * VSTR + col];
      if constexpr (KG == 4) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(pair[0], pair[1]);
      } else {
        *reinterpret_cast<uint32_t*>(dst) = pair[0];
      }
    }
  };

  // ---- running statistics and accumulator --------------------------------
  f32x16 acc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) acc[d] = f32x16{};
  float m_run = -INFINITY;     // running max of the log2-scaled logits
  float l_run = 0.0f;          // this lane's half of the running exp-sum

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_kv; ++j) {
    const int buf = j & 1;
    const int key0 = j * BN;
    if (j + 1 < n_kv) load_tile(j + 1);

    // A wave whose rows all precede the tile's first key has nothing to do.
    const bool active = !CAUSAL || key0 <= wq0 + 31;
    if (active) {
      // S^T = K Q^T for two 32-key blocks.
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const uint16_t* krow = &k_lds[buf][(kb * 32 + li) * KSTR + hh * 8];
#pragma unroll
        for (int c = 0; c < DCH; ++c) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(krow + c * 16);
          s[kb] = mfma32<BF16>(a, qreg[c], s[kb]);
        }
      }

      // Mask keys past the sequence end and, under causality, keys after the
      // query (only tiles that reach those positions pay for it).
      const bool need_mask = (key0 + BN > L) || (CAUSAL && key0 + BN - 1 > wq0);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
            const bool ok = (key < L) && (!CAUSAL || key <= qi);
            s[kb][r] = ok ? s[kb][r] : -INFINITY;
          }
        }
      }

      // Row maximum over this tile (16 + 16 values here, the rest in lane ^ 32).
      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float mx2 = (mx == -INFINITY) ? -INFINITY : mx * c_log2;

      // Lazy refresh of the running maximum.
      const bool bump = mx2 > m_run + LAZY_RESCALE_LOG2;
      if (__builtin_amdgcn_ballot_w64(bump)) {
        const float m_new = bump ? mx2 : m_run;
        const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int d = 0; d < DB; ++d) acc[d] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }

      // P = exp2(s * c - m), packed to 16 bit for P V.
      // l: bf16 keeps 8 significant bits, so a row with few visible keys
      // would carry up to 2^-9 relative error into ln(l) if l summed the
      // rounded values; it sums the fp32 values instead. fp16 (11 bits) keeps
      // that error below 2.5e-4 and sums the rounded pairs with one dot2.
      uint32_t pk[2][8];
      float tile_l = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * t], c_log2, -m_run));
          const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * t + 1], c_log2, -m_run));
          pk[kb][t] = pack2<BF16>(e0, e1);
          if constexpr (BF16) {
            tile_l += e0 + e1;
          } else {
            tile_l = add_pair<false>(pk[kb][t], tile_l);
          }
        }
      }
      l_run += tile_l;

      // O^T += V^T P^T over four 16-key steps.
      const int vrow = swap23(li);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const int kb = kc >> 1, e = kc & 1;
        const u32x4 bop = {pk[kb][e * 4 + 0], pk[kb][e * 4 + 1], pk[kb][e * 4 + 2], pk[kb][e * 4 + 3]};
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(
              &vt_lds[buf][(d * 32 + vrow) * VSTR + kc * 16 + hh * 8]);
          acc[d] = mfma32<BF16>(a, bop, acc[d]);
        }
      }
    }

    if (j + 1 < n_kv) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = ln(l) + m -------------------------------
  const float l_tot = l_run + wave_xor32(l_run);
  if (qi < L) {
    const float inv = 1.0f / l_tot;
    uint16_t* orow = og + (size_t)qi * tok_stride;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 w;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          w[t] = pack2<BF16>(acc[d][half * 8 + 2 * t] * inv, acc[d][half * 8 + 2 * t + 1] * inv);
        }
        *reinterpret_cast<u32x4*>(orow + d * 32 + half * 16 + hh * 8) = w;
      }
    }
    if (p.lse != nullptr && hh == 0) {
      // __builtin_amdgcn_logf is the hardware base-2 logarithm.
      const float lse = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
      p.lse[((size_t)b * p.H + h) * p.S + seq_start + qi] = lse;
    }
  }
}

template <int D, bool BF16, bool CAUSAL, bool VARLEN>
static hipError_t launch_one(const FwdParams& p, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, CAUSAL, VARLEN>), dim3(grid), dim3(NTHREADS), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_d(const FwdParams& p, bool causal, bool varlen, unsigned grid,
                           hipStream_t stream) {
  if (causal) {
    return varlen ? launch_one<D, BF16, true, true>(p, grid, stream)
                  : launch_one<D, BF16, true, false>(p, grid, stream);
  }
  return varlen ? launch_one<D, BF16, false, true>(p, grid, stream)
                : launch_one<D, BF16, false, false>(p, grid, stream);
}

int query_tile_rows() { return BM; }

hipError_t launch_fwd(const FwdParams& p, int D, bool bf16, bool causal, bool varlen,
                      unsigned grid, hipStream_t stream) {
  if (D == 64) {
    return bf16 ? launch_d<64, true>(p, causal, varlen, grid, stream)
                : launch_d<64, false>(p, causal, varlen, grid, stream);
  }
  return bf16 ? launch_d<128, true>(p, causal, varlen, grid, stream)
              : launch_d<128, false>(p, causal, varlen, grid, stream);
}

}  // namespace sdpa08
