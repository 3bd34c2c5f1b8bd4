// Attention backward for gfx950: dQ, dK and dV from the saved log-sum-exp.
//
// The forward keeps only O and the per-row LSE; the backward recomputes the
// probabilities P = exp(scale * Q K^T - LSE) tile by tile and applies the
// chain rule through the three steps of the forward (scores, row softmax,
// weighted sum of V):
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - delta),
//     dQ = scale * dS K,   dK = scale * dS^T Q,
// with delta_i = rowsum(dO_i * O_i) (which equals rowsum(P * dP)). Neither
// P nor dS ever reaches HBM. Two kernels, no atomics, so results are
// deterministic:
//   * dQ kernel: one workgroup per 128-row query tile, like the forward.
//     Each wave keeps Q^T and dO^T of its 32 rows in registers and streams
//     64-key K and V tiles through a two-stage LDS ring. It also computes
//     delta for its rows and stores it for the second kernel.
//   * dK/dV kernel: one workgroup per 128-key tile. Each wave keeps K^T and
//     V^T of its 32 keys in registers and streams 64-row Q and dO tiles
//     (with their LSE, in log2 units, and delta) through the ring.
// Orientation follows the forward: every MFMA's output column is the lane
// (mod 32). In the dQ kernel the lane owns a query row, so LSE and delta
// are one value per lane; in the dK/dV kernel the lane owns a key and the
// per-row LSE and delta come from LDS. The second operand of every
// "accumulate over rows" product (dQ^T += K^T dS^T, dV^T += dO^T P,
// dK^T += Q^T dS) is the packed score block straight from registers, and
// its first operand is read transposed from the row-major LDS tile with
// ds_read_b64_tr_b16, as the forward reads V^T.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_bwd.h"
#include "gfx950_util.h"

namespace sdpa08 {
namespace {

constexpr int NW = 4;           // waves per workgroup
constexpr int BM = kBwdTileRows; // rows owned by a workgroup (32 per wave)
constexpr int BN = 64;          // rows per streamed LDS tile
static_assert(BM == 2 * BN, "a workgroup's rows span two streamed tiles");
// Compile-time flag of a tile body: the tile may hold positions some row must
// not see (a diagonal or a sequence end); without it the mask code is left out.
template <bool B> struct MaskTag { static constexpr bool value = B; };
constexpr int HEAD_GROUP = 4;   // heads whose tiles are interleaved on one XCD
constexpr float LOG2E = 1.4426950408889634f;

// Which (sequence, head, 128-row tile) a workgroup owns. Workgroup i runs on
// XCD i % 8; each XCD gets a contiguous run of the logical order, which walks
// heads HEAD_GROUP at a time with their tiles interleaved. `ascending`:
// tile 0 first (the dK/dV kernel's longest causal tiles), else the last.
struct Item {
  int b, h, seq_start, L, t0;
};

template <bool VARLEN>
__device__ __forceinline__ bool map_item(const BwdParams& p, bool ascending, Item& it) {
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int nbh = VARLEN ? p.H : p.B * p.H;
  const int nt = p.n_tiles;
  const int grp = logical / (HEAD_GROUP * nt);
  const int in_grp = min(HEAD_GROUP, nbh - grp * HEAD_GROUP);
  const int rem = logical - grp * (HEAD_GROUP * nt);
  const int rank = rem / in_grp;
  const int bh = grp * HEAD_GROUP + (rem - rank * in_grp);
  it.h = bh % p.H;
  it.b = VARLEN ? 0 : bh / p.H;
  const int vt = ascending ? rank : nt - 1 - rank;
  it.seq_start = 0;
  it.L = p.S;
  if constexpr (VARLEN) {
    // Virtual tile space: sequence s owns tiles [cu[s]/BM + s, ... + ceil(L_s/BM)).
    int lo = 0, hi = p.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.cu_seqlens[mid] / BM + mid <= vt) lo = mid; else hi = mid - 1;
    }
    it.seq_start = p.cu_seqlens[lo];
    it.L = p.cu_seqlens[lo + 1] - it.seq_start;
    it.t0 = (vt - (it.seq_start / BM + lo)) * BM;
    return it.t0 < it.L;
  } else {
    it.t0 = vt * BM;
    return true;
  }
}

// Per-lane LDS offsets shared by both kernels.
template <int D>
struct Offsets {
  static constexpr int ROWB = D * 2;
  static constexpr int TILEB = BN * ROWB;
  static constexpr int LDW = TILEB / 1024 / NW;
  static constexpr int DCH = D / 16;
  static constexpr int DB = D / 32;
  uint32_t ld_voff[LDW];      // direct loads: global offset of this lane's 16 bytes
  uint32_t a_off[DCH];        // A operand (32 rows x 16 d) of a row-major tile
  uint32_t t_off[2][DB];      // transposing reads (32 d x 16 rows)

  __device__ __forceinline__ Offsets(int wave, int lane, uint32_t tok_bytes) {
    const int li = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int u = 0; u < LDW; ++u) {
      const int byte = (wave * LDW + u) * 1024 + lane * 16;
      const int r = byte / ROWB, pc = (byte % ROWB) / 16;
      ld_voff[u] = (uint32_t)r * tok_bytes + (uint32_t)((pc ^ swz<D>(r)) * 16);
    }
#pragma unroll
    for (int c = 0; c < DCH; ++c) a_off[c] = li * ROWB + (((2 * c + hh) ^ swz<D>(li)) << 4);
    const int blk = li >> 4, s = li & 15;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int row = t2 * 8 + hh * 4 + (s >> 2);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = db * 32 + blk * 16 + swap23(4 * (s & 3));
        t_off[t2][db] = row * ROWB + ((((col >> 3) ^ swz<D>(row)) << 4) | ((col & 7) * 2));
      }
    }
  }
};

// A operand from a transposing read: 32 columns (d) x 16 rows, rows
// [16 kc, 16 kc + 16) of the tile in the order the packed scores use.
template <int D>
__device__ __forceinline__ u32x4 read_t(const uint8_t* tile, const Offsets<D>& o, int kc, int db) {
  const uint8_t* base = tile + kc * 16 * Offsets<D>::ROWB;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + o.t_off[0][db]));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + o.t_off[1][db]));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
}

// Store the 32 x D block a wave accumulated transposed (lane = row) as
// 16-bit rows, times `f`. Rows past the descriptor's range are dropped.
template <int D, bool BF16>
__device__ __forceinline__ void store_rows(const f32x16* acc, float f, __amdgpu_buffer_rsrc_t r,
                                           uint32_t voff) {
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 w;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        w[t] = pack2<BF16>(acc[d][half * 8 + 2 * t] * f, acc[d][half * 8 + 2 * t + 1] * f);
      }
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), r,
                                             voff + (uint32_t)(d * 64 + half * 32), 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// dQ (and delta): one workgroup per 128 query rows.
template <int D, bool BF16, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NW * 64, 2) void attn_bwd_dq_kernel(BwdParams p) {
  using O = Offsets<D>;
  constexpr int ROWB = O::ROWB, TILEB = O::TILEB, LDW = O::LDW, DCH = O::DCH, DB = O::DB;
  constexpr int STAGEB = 2 * TILEB;   // K tile + V tile
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[STAGEB];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[STAGEB];

  const int lane = threadIdx.x & 63;
  // Wave-uniform (scalar) at D = 128; at D = 64 the scalar form measured 6 %
  // slower on B4 H12 S2048.
  const int wave = D == 128 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : (int)(threadIdx.x >> 6);
  const int li = lane & 31;
  const int hh = lane >> 5;

  Item it;
  if (!map_item<VARLEN>(p, false, it)) return;
  const int b = it.b, h = it.h, L = it.L, q0 = it.t0;

  const uint32_t tok_bytes = (uint32_t)p.H * ROWB;
  const size_t base = (((size_t)b * p.S + it.seq_start) * p.H + h) * D;
  const size_t qbase = base + (size_t)q0 * p.H * D;
  const uint16_t* kg = p.k + base;
  const uint16_t* vg = p.v + base;
  const size_t row_base = ((size_t)b * p.H + h) * p.S + it.seq_start;   // lse / delta rows

  const int kv_hi = CAUSAL ? min(q0 + BM, L) : L;
  const int n_kv = (kv_hi + BN - 1) / BN;
  const int wq0 = q0 + wave * 32;
  const int qi = wq0 + li;
  const uint32_t q_rows = (uint32_t)min(L - q0, BM);

  // Q^T and dO^T of this wave's rows stay in registers; O is read once for delta.
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(p.q + qbase, q_rows * tok_bytes);
  const __amdgpu_buffer_rsrc_t do_rsrc = make_rsrc(p.dout + qbase, q_rows * tok_bytes);
  const __amdgpu_buffer_rsrc_t o_rsrc = make_rsrc(p.o + qbase, q_rows * tok_bytes);
  const uint32_t row_voff = (uint32_t)(wave * 32 + li) * tok_bytes + hh * 16;
  u32x4 qreg[DCH], doreg[DCH];
  float dpart = 0.0f;
#pragma unroll
  for (int c = 0; c < DCH; ++c) {
    qreg[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, row_voff + c * 32, 0, 0));
    doreg[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(do_rsrc, row_voff + c * 32, 0, 0));
    const u32x4 ov = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(o_rsrc, row_voff + c * 32, 0, 0));
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x2 a = unpack2<BF16>(doreg[c][t]), o2 = unpack2<BF16>(ov[t]);
      dpart = fmaf(a[0], o2[0], dpart);
      dpart = fmaf(a[1], o2[1], dpart);
    }
  }
  const float delta = half_sum(dpart);
  const float lse2 = (qi < L) ? p.lse[row_base + qi] * LOG2E : 0.0f;
  if (hh == 0 && qi < L) {
    // For the dK/dV kernel: delta, and the LSE in log2 units (saves a multiply per score there).
    p.delta[row_base + qi] = delta;
    p.lse2[row_base + qi] = lse2;
  }
  const float c_log2 = p.c_log2;

  const O off(wave, lane, tok_bytes);

  auto issue_tile = [&](int j, int st) {
    const int key0 = j * BN;
    const uint32_t rows = (uint32_t)min(L - key0, BN);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kg + (size_t)key0 * p.H * D, rows * tok_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vg + (size_t)key0 * p.H * D, rows * tok_bytes);
    uint8_t* kdst = (st ? smem1 : smem0) + wave * LDW * 1024;
    uint8_t* vdst = kdst + TILEB;
#pragma unroll
    for (int u = 0; u < LDW; ++u) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kdst + u * 1024), 16, (int)off.ld_voff[u], 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < LDW; ++u) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vdst + u * 1024), 16, (int)off.ld_voff[u], 0, 0, 0);
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) acc[d] = f32x16{};

  auto compute_tile = [&](auto masked_c, int j, const uint8_t* ks) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const uint8_t* vs = ks + TILEB;
    const int key0 = j * BN;
    if (MASKED && CAUSAL && key0 > wq0 + 31) return;     // no row of this wave sees the tile

    // S^T = K Q^T and dP^T = V dO^T, two 32-key blocks each.
    f32x16 s[2] = {f32x16{}, f32x16{}};
    f32x16 dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int c = 0; c < DCH; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(ks + kb * 32 * ROWB + off.a_off[c]);
        s[kb] = mfma32<BF16>(ka, qreg[c], s[kb]);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 va = *reinterpret_cast<const u32x4*>(vs + kb * 32 * ROWB + off.a_off[c]);
        dp[kb] = mfma32<BF16>(va, doreg[c], dp[kb]);
      }
    }

    // P^T = exp2(s * c - lse2), dS^T = P^T (dP^T - delta), packed to 16 bit.
    const bool need_mask = MASKED && ((key0 + BN > L) || (CAUSAL && key0 + BN - 1 > wq0));
    // Register r of block kb holds key key0 + 4 hh + c, c = 32 kb + 8 (r / 4) + r % 4
    // (a constant): visible iff key < L and, causal, key <= qi, i.e. c <= T.
    const int T = (CAUSAL ? min(L - 1, qi) : L - 1) - key0 - hh * 4;
    uint32_t pk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float ds[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * t + e;
          float pr = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c_log2, -lse2));
          if (need_mask && !(kb * 32 + (r >> 2) * 8 + (r & 3) <= T)) pr = 0.0f;
          ds[e] = pr * (dp[kb][r] - delta);
        }
        pk[kb][t] = pack2<BF16>(ds[0], ds[1]);
      }
    }

    // dQ^T += K^T dS^T over four 16-key steps (K^T by transposing reads).
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int kb = kc >> 1, e = kc & 1;
      const u32x4 bop = {pk[kb][e * 4 + 0], pk[kb][e * 4 + 1], pk[kb][e * 4 + 2], pk[kb][e * 4 + 3]};
#pragma unroll
      for (int d = 0; d < DB; ++d) acc[d] = mfma32<BF16>(read_t<D>(ks, off, kc, d), bop, acc[d]);
    }
  };

  // Key tiles before j_plain hold no key that any row of the workgroup must not
  // see: they run without the mask code, in a loop of their own (the mask's
  // lane-dependent condition would otherwise cost every tile its exec-mask
  // handling). Their count is kept even so the masked loop starts on stage 0.
  int j_plain = min(n_kv, L / BN);
  if (CAUSAL) j_plain = min(j_plain, (q0 + 1) / BN);
  j_plain &= ~1;
  constexpr MaskTag<true> masked_t{};
  constexpr MaskTag<false> plain_t{};
  issue_tile(0, 0);
  wait_vmem_all();
  __syncthreads();
#pragma unroll 1
  for (int j = 0; j < j_plain; j += 2) {
    issue_tile(j + 1, 1);
    compute_tile(plain_t, j, smem0);
    wait_vmem_all();
    __syncthreads();
    if (j + 2 < n_kv) issue_tile(j + 2, 0);
    compute_tile(plain_t, j + 1, smem1);
    wait_vmem_all();
    __syncthreads();
  }
#pragma unroll 1
  for (int j = j_plain; j < n_kv; j += 2) {
    if (j + 1 < n_kv) issue_tile(j + 1, 1);
    compute_tile(masked_t, j, smem0);
    wait_vmem_all();
    __syncthreads();
    if (j + 1 >= n_kv) break;
    if (j + 2 < n_kv) issue_tile(j + 2, 0);
    compute_tile(masked_t, j + 1, smem1);
    wait_vmem_all();
    __syncthreads();
  }

  const __amdgpu_buffer_rsrc_t dq_rsrc = make_rsrc(p.dq + qbase, q_rows * tok_bytes);
  store_rows<D, BF16>(acc, p.scale, dq_rsrc, row_voff);
}

// ---------------------------------------------------------------------------
// dK and dV: one workgroup per 128 keys. MODE 0 computes both. With D = 128
// a wave would hold K^T, V^T (64 registers) and both accumulators (128)
// besides the score blocks, more than the 256 registers that two waves per
// SIMD allow; there the work is split over two launches instead, MODE 1
// (dV only: S, P, dO^T P; no V^T, no dS) and MODE 2 (dK only: S, dP, dS,
// Q^T dS), each fitting two waves per SIMD, at the price of computing Q K^T
// twice.
enum { DKDV_BOTH = 0, DKDV_V = 1, DKDV_K = 2 };
#ifndef SDPA_BWD_SPLIT_128
#define SDPA_BWD_SPLIT_128 1
#endif
template <int D, bool BF16, bool CAUSAL, bool VARLEN, int MODE>
__global__ __launch_bounds__(NW * 64, (D == 128 && MODE == DKDV_BOTH) ? 1 : 2) void attn_bwd_dkdv_kernel(BwdParams p) {
  constexpr bool DO_V = MODE != DKDV_K;
  constexpr bool DO_K = MODE != DKDV_V;
  using O = Offsets<D>;
  constexpr int ROWB = O::ROWB, TILEB = O::TILEB, LDW = O::LDW, DCH = O::DCH, DB = O::DB;
  constexpr int STAGEB = 2 * TILEB + 2048;   // Q tile + dO tile + 1 KB LSE + 1 KB delta
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[STAGEB];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[STAGEB];

  const int lane = threadIdx.x & 63;
  // Wave-uniform (scalar) at D = 128, except in the dK launch, whose registers
  // are full (the scalar form spilled 27 there); at D = 64 the scalar form
  // measured 6 % slower on B4 H12 S2048.
  const int wave = (D == 128 && MODE != DKDV_K) ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)
                                                : (int)(threadIdx.x >> 6);
  const int li = lane & 31;
  const int hh = lane >> 5;

  Item it;
  if (!map_item<VARLEN>(p, true, it)) return;
  const int b = it.b, h = it.h, L = it.L, k0 = it.t0;

  const uint32_t tok_bytes = (uint32_t)p.H * ROWB;
  const size_t base = (((size_t)b * p.S + it.seq_start) * p.H + h) * D;
  const size_t kbase = base + (size_t)k0 * p.H * D;
  const uint16_t* qg = p.q + base;
  const uint16_t* dog = p.dout + base;
  const size_t row_base = ((size_t)b * p.H + h) * p.S + it.seq_start;

  const int wk0 = k0 + wave * 32;           // first key of this wave
  const int ki = wk0 + li;                   // this lane's key
  const uint32_t k_rows = (uint32_t)min(L - k0, BM);
  const int j_lo = CAUSAL ? k0 / BN : 0;     // first query tile that sees a key here
  const int n_q = (L + BN - 1) / BN;

  const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(p.k + kbase, k_rows * tok_bytes);
  const __amdgpu_buffer_rsrc_t v_rsrc = make_rsrc(p.v + kbase, k_rows * tok_bytes);
  const uint32_t row_voff = (uint32_t)(wave * 32 + li) * tok_bytes + hh * 16;
  u32x4 kreg[DCH], vreg[DCH];
#pragma unroll
  for (int c = 0; c < DCH; ++c) {
    kreg[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, row_voff + c * 32, 0, 0));
    if constexpr (DO_K) {
      vreg[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(v_rsrc, row_voff + c * 32, 0, 0));
    }
  }
  const float c_log2 = p.c_log2;
  const O off(wave, lane, tok_bytes);

  auto issue_tile = [&](int j, int st) {
    const int row0 = j * BN;
    const uint32_t rows = (uint32_t)min(L - row0, BN);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qg + (size_t)row0 * p.H * D, rows * tok_bytes);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(dog + (size_t)row0 * p.H * D, rows * tok_bytes);
    uint8_t* stage = st ? smem1 : smem0;
    uint8_t* qdst = stage + wave * LDW * 1024;
    uint8_t* ddst = qdst + TILEB;
#pragma unroll
    for (int u = 0; u < LDW; ++u) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void*)(qdst + u * 1024), 16, (int)off.ld_voff[u], 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < LDW; ++u) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(dr, (lds_void*)(ddst + u * 1024), 16, (int)off.ld_voff[u], 0, 0, 0);
    }
    if (wave == 0) {
      // 64 LSE and 64 delta values: lanes 0-15 fetch 16 bytes each, the
      // rest fall outside the descriptor and write zeros.
      const __amdgpu_buffer_rsrc_t lr = make_rsrc(p.lse2 + row_base + row0, rows * 4);
      const __amdgpu_buffer_rsrc_t er = make_rsrc(p.delta + row_base + row0, rows * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lr, (lds_void*)(stage + 2 * TILEB), 16, lane * 16, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(er, (lds_void*)(stage + 2 * TILEB + 1024), 16, lane * 16, 0, 0, 0);
    }
  };

  f32x16 acc_k[DB], acc_v[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    acc_k[d] = f32x16{};
    acc_v[d] = f32x16{};
  }

  auto compute_tile = [&](auto masked_c, int j, const uint8_t* qs) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const uint8_t* dos = qs + TILEB;
    const float* lse_t = reinterpret_cast<const float*>(qs + 2 * TILEB);
    const float* del_t = reinterpret_cast<const float*>(qs + 2 * TILEB + 1024);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int qb0 = j * BN + kb * 32;      // first query row of this block
      if (MASKED && qb0 >= L) continue;
      if (MASKED && CAUSAL && qb0 + 31 < wk0) continue;  // every row precedes every key of the wave

      // S = Q K^T and dP = dO V^T: lane = key, registers = query rows.
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < DCH; ++c) {
        const u32x4 qa = *reinterpret_cast<const u32x4*>(qs + kb * 32 * ROWB + off.a_off[c]);
        s = mfma32<BF16>(qa, kreg[c], s);
        if constexpr (DO_K) {
          const u32x4 da = *reinterpret_cast<const u32x4*>(dos + kb * 32 * ROWB + off.a_off[c]);
          dp = mfma32<BF16>(da, vreg[c], dp);
        }
      }

      const bool need_mask = MASKED && ((qb0 + 32 > L) || (CAUSAL && qb0 < wk0 + 31));
      uint32_t pp[8], pd[8];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // registers 4g..4g+3 hold query rows qb0 + 8g + 4hh + {0..3}
        const int rl = kb * 32 + 8 * g + 4 * hh;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_t + rl);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(del_t + rl);
        float pv[4], dv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pr = __builtin_amdgcn_exp2f(fmaf(s[r], c_log2, -l4[e]));
          if (need_mask) {
            const int qrow = qb0 + 8 * g + 4 * hh + e;
            if (!(qrow < L && (!CAUSAL || qrow >= ki))) pr = 0.0f;
          }
          pv[e] = pr;
          if constexpr (DO_K) dv[e] = pr * (dp[r] - d4[e]);
        }
        if constexpr (DO_V) {
          pp[2 * g] = pack2<BF16>(pv[0], pv[1]);
          pp[2 * g + 1] = pack2<BF16>(pv[2], pv[3]);
        }
        if constexpr (DO_K) {
          pd[2 * g] = pack2<BF16>(dv[0], dv[1]);
          pd[2 * g + 1] = pack2<BF16>(dv[2], dv[3]);
        }
      }

      // dV^T += dO^T P and dK^T += Q^T dS over two 16-row steps.
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int kc = 2 * kb + e;
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          if constexpr (DO_V) {
            const u32x4 bp = {pp[e * 4 + 0], pp[e * 4 + 1], pp[e * 4 + 2], pp[e * 4 + 3]};
            acc_v[d] = mfma32<BF16>(read_t<D>(dos, off, kc, d), bp, acc_v[d]);
          }
          if constexpr (DO_K) {
            const u32x4 bd = {pd[e * 4 + 0], pd[e * 4 + 1], pd[e * 4 + 2], pd[e * 4 + 3]};
            acc_k[d] = mfma32<BF16>(read_t<D>(qs, off, kc, d), bd, acc_k[d]);
          }
        }
      }
    }
  };

  // Query tiles in [j_pl, j_ph) see every key of the workgroup from their
  // first row on and lie inside the sequence: they run without the mask code in
  // a loop of their own. Before them come the diagonal tiles (two: the
  // workgroup's 128 keys span two 64-row tiles), after them the tail; the
  // plain count is kept even so each loop starts on stage 0.
  int j_pl = CAUSAL ? min(n_q, j_lo + 2) : j_lo;
  int j_ph = max(j_pl, min(n_q, L / BN));
  j_ph = j_pl + ((j_ph - j_pl) & ~1);
  constexpr MaskTag<true> masked_t{};
  constexpr MaskTag<false> plain_t{};
  auto walk = [&](auto masked_c, int ja, int jb) __attribute__((always_inline)) {
#pragma unroll 1
    for (int j = ja; j < jb; j += 2) {
      if (j + 1 < n_q) issue_tile(j + 1, 1);
      compute_tile(masked_c, j, smem0);
      wait_vmem_all();
      __syncthreads();
      if (j + 1 >= jb) break;
      if (j + 2 < n_q) issue_tile(j + 2, 0);
      compute_tile(masked_c, j + 1, smem1);
      wait_vmem_all();
      __syncthreads();
    }
  };
  if (j_lo < n_q) {
    issue_tile(j_lo, 0);
    wait_vmem_all();
    __syncthreads();
    walk(masked_t, j_lo, j_pl);
    walk(plain_t, j_pl, j_ph);
    walk(masked_t, j_ph, n_q);
  }

  const __amdgpu_buffer_rsrc_t dk_rsrc = make_rsrc(p.dk + kbase, k_rows * tok_bytes);
  const __amdgpu_buffer_rsrc_t dv_rsrc = make_rsrc(p.dv + kbase, k_rows * tok_bytes);
  if constexpr (DO_K) store_rows<D, BF16>(acc_k, p.scale, dk_rsrc, row_voff);
  if constexpr (DO_V) store_rows<D, BF16>(acc_v, 1.0f, dv_rsrc, row_voff);
}

template <int D, bool BF16, bool CAUSAL, bool VARLEN>
hipError_t launch_one(BwdParams p, hipStream_t stream) {
  const long long tiles = VARLEN ? (long long)p.S / BM + p.B : ((long long)p.S + BM - 1) / BM;
  p.n_tiles = (int)tiles;
  const long long grid = tiles * (VARLEN ? p.H : (long long)p.B * p.H);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, BF16, CAUSAL, VARLEN>), dim3((unsigned)grid),
                     dim3(NW * 64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (D == 128 && SDPA_BWD_SPLIT_128) {
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, BF16, CAUSAL, VARLEN, DKDV_V>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, BF16, CAUSAL, VARLEN, DKDV_K>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, stream, p);
  } else {
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, BF16, CAUSAL, VARLEN, DKDV_BOTH>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, stream, p);
  }
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_d(const BwdParams& p, bool causal, bool varlen, hipStream_t stream) {
  if (causal) {
    return varlen ? launch_one<D, BF16, true, true>(p, stream) : launch_one<D, BF16, true, false>(p, stream);
  }
  return varlen ? launch_one<D, BF16, false, true>(p, stream) : launch_one<D, BF16, false, false>(p, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int D, bool bf16, bool causal, bool varlen,
                      hipStream_t stream) {
  if (D == 64) {
    return bf16 ? launch_d<64, true>(p, causal, varlen, stream) : launch_d<64, false>(p, causal, varlen, stream);
  }
  return bf16 ? launch_d<128, true>(p, causal, varlen, stream) : launch_d<128, false>(p, causal, varlen, stream);
}

}  // namespace sdpa08
