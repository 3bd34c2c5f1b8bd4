// Attention forward on FP8 (OCP E4M3) Q, K, V for gfx950, head dimension 128.
//
// Same method and tiling as the 16-bit forward (online softmax over 64-key
// tiles streamed through a two-stage LDS ring, jianying88.com/news/49672 §3),
// with both products on the 8-bit matrix core:
// v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, unit block scales) takes
// 64 contraction steps per instruction, so Q K^T of a 32x32 block is two
// instructions and P V of a 64-key tile is one per 32 output columns.
//
// Operand layout of that instruction (measured on the device): lane l holds
// row (A) or column (B) l % 32 and 32 of the 64 contraction indices, as 32
// bytes; byte b of lane-half hh of A meets byte b of lane-half hh of B. Any
// assignment of contraction indices to (hh, b) works if both operands use it.
//   * Q K^T: half hh holds head dimensions [32 hh, 32 hh + 32) of each
//     64-wide step, read as two 16-byte pieces of a row.
//   * P V: the probabilities come out of the score accumulator with lane =
//     query and registers = keys; byte b = 16 kb + r of half hh is key
//     32 kb + 8 (r / 4) + 4 hh + r % 4 (block kb, register r). V^T is read
//     with ds_read_b64_tr_b8 (in each 16-lane block, lane i receives byte
//     i % 8 of the 8-byte pieces addressed by lanes 2 j + i / 8, j = 0..7),
//     with each lane pointing at the key row that the byte order needs.
// The 128-byte tile rows are stored with their 16-byte chunks permuted by
// chunk ^ f(row), f(r) = 2 ((r>>1)&1) + 4 ((r>>3)&1) + ((r>>2)&1), which
// keeps the 16-byte K reads and the transposing V reads free of bank
// conflicts on the 64-bank LDS.
//
// P is quantised to E4M3 after scaling by 2^4 (probabilities relative to
// the lazily refreshed maximum stay below 2^4, so P * 2^4 < 2^8 < 448, and
// values down to 2^-13 of the maximum keep a code); the same factor is in
// the row sum, so it cancels in O and is taken out of the LSE. After the
// first tile the exponentials are first taken against the running maximum
// without a row maximum; they are kept when the lane's row sum (a bound on
// every P * 2^4) is at most 448.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fp8.h"
#include "gfx950_util.h"

namespace sdpa08 {
namespace {

constexpr int D = 128;
constexpr int NW = 4;             // waves per workgroup
constexpr int BM = 32 * NW;       // query rows per workgroup
constexpr int BN = 64;            // keys per tile
constexpr int ROWB = D;           // bytes per K/V row
constexpr int TILEB = BN * ROWB;  // 8 KB
constexpr int STAGEB = 2 * TILEB; // K tile + V tile
constexpr int LDW = TILEB / 1024 / NW;
constexpr int DB = D / 32;        // 32-column blocks of O^T
constexpr int HEAD_GROUP = 4;
constexpr float LAZY_RESCALE_LOG2 = 4.0f;
constexpr float E4M3_MAX = 448.0f;       // largest finite E4M3 value
constexpr float P_SHIFT_LOG2 = 4.0f;   // P is quantised as P * 2^4
constexpr int E8M0_ONE = 127;          // block scale 2^0

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, E8M0_ONE, 0, E8M0_ONE);
}

// 16-byte chunk permutation of a 128-byte LDS row (see the header comment).
__device__ __forceinline__ int swz8(int r) {
  return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2) | ((r >> 2) & 1);
}


template <bool OUT_BF16, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_fp8_kernel(Fp8Params p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[STAGEB];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[STAGEB];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar)
  const int li = lane & 31;
  const int hh = lane >> 5;

  // ---- (sequence, head, query tile) of this workgroup, as the 16-bit kernel
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int nbh = VARLEN ? p.H : p.B * p.H;
  const int nt = p.n_qtiles;
  const int grp = logical / (HEAD_GROUP * nt);
  const int in_grp = min(HEAD_GROUP, nbh - grp * HEAD_GROUP);
  const int rem = logical - grp * (HEAD_GROUP * nt);
  const int rank = rem / in_grp;
  const int bh = grp * HEAD_GROUP + (rem - rank * in_grp);
  const int h = bh % p.H;
  const int b = VARLEN ? 0 : bh / p.H;
  const int vt = nt - 1 - rank;
  int seq_start = 0, L = p.S, q0;
  if constexpr (VARLEN) {
    int lo = 0, hi = p.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.cu_seqlens[mid] / BM + mid <= vt) lo = mid; else hi = mid - 1;
    }
    seq_start = p.cu_seqlens[lo];
    L = p.cu_seqlens[lo + 1] - seq_start;
    q0 = (vt - (seq_start / BM + lo)) * BM;
    if (q0 >= L) return;
  } else {
    q0 = vt * BM;
  }

  const uint32_t tok_bytes = (uint32_t)p.H * ROWB;        // input bytes between tokens
  const uint32_t out_tok = (uint32_t)p.H * D * 2;          // output bytes between tokens
  const size_t base = (((size_t)b * p.S + seq_start) * p.H + h) * D;   // elements
  const uint8_t* kg = p.k + base;
  const uint8_t* vg = p.v + base;

  const int kv_hi = CAUSAL ? min(q0 + BM, L) : L;
  const int n_kv = (kv_hi + BN - 1) / BN;
  const int wq0 = q0 + wave * 32;
  const int qi = wq0 + li;
  const uint32_t q_rows = (uint32_t)min(L - q0, BM);

  // ---- Q^T operand: 32 bytes per 64-wide step, half hh = dims [32 hh, +32)
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(p.q + base + (size_t)q0 * p.H * D, q_rows * tok_bytes);
  const uint32_t q_voff = (uint32_t)(wave * 32 + li) * tok_bytes + hh * 32;
  const uint32_t q_xor = (p.q_mode == 1) ? 0x80808080u : 0u;
  const uint32_t q_and = (p.q_mode == 2) ? 0u : 0xffffffffu;
  i32x8 qreg[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, q_voff + c * 64, 0, 0));
    const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, q_voff + c * 64 + 16, 0, 0));
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      qreg[c][t] = (int)((lo[t] ^ q_xor) & q_and);
      qreg[c][4 + t] = (int)((hi[t] ^ q_xor) & q_and);
    }
  }
  const float c_log2 = p.c_log2;

  // ---- per-lane LDS offsets ------------------------------------------------
  uint32_t ld_voff[LDW];
#pragma unroll
  for (int u = 0; u < LDW; ++u) {
    const int byte = (wave * LDW + u) * 1024 + lane * 16;
    const int r = byte / ROWB, pc = (byte % ROWB) / 16;
    ld_voff[u] = (uint32_t)r * tok_bytes + (uint32_t)((pc ^ swz8(r)) * 16);
  }
  // K operand: row li (+32 per key block), chunks 4c + 2hh and 4c + 2hh + 1.
  uint32_t k_off[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int e = 0; e < 2; ++e) k_off[c][e] = li * ROWB + (((4 * c + 2 * hh + e) ^ swz8(li)) << 4);
  }
  // V^T operand: read t (0..3) of column block db; this lane points at key
  // 16 t + 8 (j / 4) + 4 hh + j % 4 with j = (lane % 16) / 2, at the 8 bytes
  // of columns 32 db + 16 ((lane / 16) % 2) + 8 (lane % 2).
  uint32_t v_off[DB];
  {
    const int j = (lane & 15) >> 1;
    const int key = 8 * (j >> 2) + 4 * hh + (j & 3);      // + 16 t
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int ch = 2 * db + ((lane >> 4) & 1);
      v_off[db] = key * ROWB + ((ch ^ swz8(key)) << 4) + 8 * (lane & 1);
    }
  }

  auto issue_tile = [&](int j, int st) {
    const int key0 = j * BN;
    const uint32_t rows = (uint32_t)min(L - key0, BN);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kg + (size_t)key0 * p.H * D, rows * tok_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vg + (size_t)key0 * p.H * D, rows * tok_bytes);
    uint8_t* kdst = (st ? smem1 : smem0) + wave * LDW * 1024;
    uint8_t* vdst = kdst + TILEB;
#pragma unroll
    for (int u = 0; u < LDW; ++u) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kdst + u * 1024), 16, (int)ld_voff[u], 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < LDW; ++u) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vdst + u * 1024), 16, (int)ld_voff[u], 0, 0, 0);
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) acc[d] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.0f;

  auto compute_tile = [&](int j, const uint8_t* ks) {
    const uint8_t* vs = ks + TILEB;
    const int key0 = j * BN;
    if (CAUSAL && key0 > wq0 + 31) return;

    // S^T = K Q^T: two 32-key blocks, two 64-wide steps each.
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint8_t* row = ks + kb * 32 * ROWB;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(row + k_off[c][0]);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(row + k_off[c][1]);
        const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        s[kb] = mfma_fp8(a, qreg[c], s[kb]);
      }
    }

    const bool need_mask = (key0 + BN > L) || (CAUSAL && key0 + BN - 1 > wq0);
    if (need_mask) {
      // Register r of block kb holds key key0 + 4 hh + c, c = 32 kb + 8 (r / 4) + r % 4
      // (a constant): visible iff key < L and, causal, key <= qi, i.e. c <= T.
      const int T = (CAUSAL ? min(L - 1, qi) : L - 1) - key0 - hh * 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
          s[kb][r] = c <= T ? s[kb][r] : -INFINITY;
        }
      }
    }

    // P * 2^4 = exp2(s c - m + 4): E4M3 bytes for P V, fp32 for the row sum.
    uint32_t pk[8];
    auto exps = [&](float m) {
      const float m_sub = m - P_SHIFT_LOG2;
      float tl = -0.0f;   // -0 + x folds to x
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = w >> 2, r0 = 4 * (w & 3);
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[i] = __builtin_amdgcn_exp2f(fmaf(s[kb][r0 + i], c_log2, -m_sub));
          tl += e[i];
        }
        // The first conversion writes the low half and keeps the high half of
        // its third operand, which the second overwrites: any register serves
        // (a constant 0 there cost one v_mov per word).
        uint32_t x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], __builtin_bit_cast(int, e[0]), false);
        x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], (int)x, true);
        pk[w] = x;
      }
      return tl;
    };
    // Optimistic pass (as in the 16-bit kernel): exponentials against the
    // running maximum as it stands; a lane sum within E4M3_MAX bounds every
    // scaled probability of the tile, so each keeps an exact-range code.
    // Otherwise (or on the first tile) the row maximum is taken, refreshed
    // lazily and the exponentials redone.
    float tile_l = 0.0f;
    bool redo = true;
    if (j != 0) {
      tile_l = exps(m_run);
      redo = __builtin_amdgcn_ballot_w64(!(tile_l <= E4M3_MAX)) != 0;
    }
    if (redo) {
      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
      mx = half_max(mx);
      const float mx2 = (mx == -INFINITY) ? -INFINITY : mx * c_log2;
      const bool bump = mx2 > m_run + LAZY_RESCALE_LOG2;
      if (__builtin_amdgcn_ballot_w64(bump)) {
        const float m_new = bump ? mx2 : m_run;
        const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int d = 0; d < DB; ++d) acc[d] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      tile_l = exps(m_run);
    }
    l_run += tile_l;

    // O^T += V^T P^T: one 64-key instruction per 32-column block.
    const i32x8 bop = {(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3],
                       (int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]};
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      i32x8 a;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vs + v_off[db] + t * 16 * ROWB));
        a[2 * t] = r[0];
        a[2 * t + 1] = r[1];
      }
      acc[db] = mfma_fp8(a, bop, acc[db]);
    }
  };

  issue_tile(0, 0);
  wait_vmem_all();
  __syncthreads();
#pragma unroll 1
  for (int j = 0; j < n_kv; j += 2) {
    if (j + 1 < n_kv) issue_tile(j + 1, 1);
    compute_tile(j, smem0);
    wait_vmem_all();
    __syncthreads();
    if (j + 1 >= n_kv) break;
    if (j + 2 < n_kv) issue_tile(j + 2, 0);
    compute_tile(j + 1, smem1);
    wait_vmem_all();
    __syncthreads();
  }

  // ---- epilogue: O = descale_v * acc / l, LSE = (m - 4 + log2 l) ln 2 --------
  const float l_tot = half_sum(l_run);
  const float f = p.v_descale / l_tot;
  // Register r of block d holds column 32 d + 8 (r / 4) + 4 hh + r % 4: runs
  // of four consecutive columns, stored 8 bytes at a time.
  const __amdgpu_buffer_rsrc_t o_rsrc = make_rsrc(p.o + base + (size_t)q0 * p.H * D, q_rows * out_tok);
  const uint32_t o_voff = (uint32_t)(wave * 32 + li) * out_tok + hh * 8;
#pragma unroll
  for (int d = 0; d < DB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 w = {pack2<OUT_BF16>(acc[d][4 * g] * f, acc[d][4 * g + 1] * f),
                       pack2<OUT_BF16>(acc[d][4 * g + 2] * f, acc[d][4 * g + 3] * f)};
      __builtin_amdgcn_raw_buffer_store_b64(w, o_rsrc, o_voff + (uint32_t)(d * 64 + g * 16), 0, 0);
    }
  }
  if (p.lse != nullptr && hh == 0 && qi < L) {
    const float lse = (m_run - P_SHIFT_LOG2 + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
    p.lse[((size_t)b * p.H + h) * p.S + seq_start + qi] = lse;
  }
}

template <bool OUT_BF16, bool CAUSAL, bool VARLEN>
hipError_t launch_one(Fp8Params p, hipStream_t stream) {
  const long long tiles = VARLEN ? (long long)p.S / BM + p.B : ((long long)p.S + BM - 1) / BM;
  p.n_qtiles = (int)tiles;
  const long long grid = tiles * (VARLEN ? p.H : (long long)p.B * p.H);
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<OUT_BF16, CAUSAL, VARLEN>), dim3((unsigned)grid),
                     dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <bool OUT_BF16>
hipError_t launch_o(const Fp8Params& p, bool causal, bool varlen, hipStream_t stream) {
  if (causal) {
    return varlen ? launch_one<OUT_BF16, true, true>(p, stream) : launch_one<OUT_BF16, true, false>(p, stream);
  }
  return varlen ? launch_one<OUT_BF16, false, true>(p, stream) : launch_one<OUT_BF16, false, false>(p, stream);
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Params& p, bool out_bf16, bool causal, bool varlen,
                          hipStream_t stream) {
  return out_bf16 ? launch_o<true>(p, causal, varlen, stream) : launch_o<false>(p, causal, varlen, stream);
}

}  // namespace sdpa08
