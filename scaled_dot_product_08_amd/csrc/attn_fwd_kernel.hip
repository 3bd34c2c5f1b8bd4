// Fused attention forward for gfx950 (CDNA4): MFMA + LDS-tiled online softmax.
//
// One workgroup of NW waves (NW = 4 or 8) owns a tile of BM = 32*NW query rows
// of one (sequence, head); wave w owns rows 32w..32w+31 of the tile. The kernel
// streams the visible keys in tiles of BN rows (64; 128 for D = 64, 4 waves) through a
// two-stage LDS ring and, per tile, runs the fused chain of mlqm.cn/news/343191 §3.1
// (Q K^T -> scale -> mask -> softmax -> P V) with the online softmax of
// jianying88.com/news/49672 §3: a running row maximum m and exponential sum l
// per query row, so no score ever leaves registers.
//
// Data movement:
//   * K and V tiles go from HBM straight into LDS (buffer_load ... lds, 16
//     bytes per lane): no registers, no LDS store instructions. Each 16-byte
//     chunk of a row is placed at chunk ^ swz(row), which makes every LDS
//     access pattern below conflict-free on the 64-bank LDS.
//   * Rows past the end of a sequence come back as zeros from the buffer
//     descriptor's range check, so ragged tails need no branches.
//
// Orientation (what makes the softmax cheap on a 64-lane wave):
//   * Scores are produced transposed, S^T = K Q^T, by v_mfma_f32_32x32x16
//     with A = a 32-key block of K (ds_read_b128) and B = Q^T (registers).
//     The accumulator column index is the lane (mod 32), so each lane holds
//     one query row and 16 of its 32 keys; the other 16 sit in lane ^ 32.
//   * The output is accumulated transposed too, O^T += V^T P^T, with B = the
//     probabilities straight out of the score accumulator (cast to 16 bit)
//     and A = V^T read from the row-major V tile by the transposing LDS read
//     ds_read_b64_tr_b16. Each lane owns one query row, so rescaling the
//     accumulator is a per-lane scalar multiply.
//
// Exponentials use exp2 on logits pre-multiplied by scale*log2(e). After a
// wave's first tile, a tile's exponentials are first taken against the
// running maximum as it stands, without computing the tile's row maximum:
// softmax does not depend on the constant subtracted, and a row sum within
// OPT_LIMIT bounds every probability of the tile. Only when that bound fails
// is the row maximum taken and refreshed, lazily: the stale maximum is kept
// until the new one exceeds it by more than 8 (log2 units), which skips most
// accumulator rescales.
//
// A second kernel (attn_fwd_w64_kernel, below) gives each wave 64 query rows
// so that every K and V^T operand read from LDS feeds two MFMAs, runs one wave
// per SIMD with the output accumulators in AGPRs (their MFMAs are inline
// assembly, guarded by explicit wait states that the build verifies on the
// emitted code), and software-pipelines the 32-key blocks of a three-stage LDS
// ring so that every group of MFMAs has softmax work beside it. It halves the
// LDS reads but, with a single wave per SIMD, exposes every latency the second
// wave used to hide; under sustained load it is slower than the 32-row kernel
// on every benchmark workload and runs only when ATTN_WAVES=w64 asks for it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>
#include <type_traits>

#ifndef SDPA_SCHED_QK
#define SDPA_SCHED_QK 1
#endif

#include "attn_kernel.h"

namespace sdpa08 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int HEAD_GROUP = 4; // heads whose query tiles are interleaved on one XCD
constexpr int NXCD = 8;       // accelerator complex dies; workgroups go round-robin over them
constexpr float LAZY_RESCALE_LOG2 = 8.0f;
constexpr float OPT_LIMIT = 32768.0f;   // largest probability the optimistic pass accepts (fp16-safe)
constexpr int BUF_FLAGS = 0x00020000;   // raw buffer descriptor word 3 (32-bit dwords)

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

// The same MFMA with the accumulator held in the accumulation registers
// (AGPRs), for kernels whose accumulators do not fit beside the working set in
// the 256 VGPRs. Written as assembly because the compiler otherwise places
// every MFMA result of such a kernel in AGPRs, scores included. The compiler's
// hazard model does not see these instructions; callers keep the rules:
// an operand written by a VALU instruction is at least 2 wait states old
// (operand_fence), and the accumulators are read or written by anything but
// these MFMAs only across acc_fence.
template <bool BF16>
__device__ __forceinline__ void mfma32_acc(f32x16& acc, u32x4 a, u32x4 b) {
  if constexpr (BF16) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  } else {
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  }
}
// 16 wait states between the last MFMA writing or reading an accumulator and
// a VALU access to it (gfx950 needs 12 after an 8-pass XDL write), and more
// than the 2 that a VALU write needs before an MFMA reads it.
__device__ __forceinline__ void acc_fence(f32x16& a) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+a"(a));
}
// 2 wait states after VALU writes of MFMA operands (the probabilities, packed
// by VALU instructions), applied to the assembled operand registers.
__device__ __forceinline__ void operand_fence(u32x4& a, u32x4& b) {
  asm volatile("s_nop 1" : "+v"(a), "+v"(b));
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

// acc + lo(p) + hi(p) for a pair of fp16 values (one v_dot2).
__device__ __forceinline__ float add_pair_f16(uint32_t p, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), one, acc, false);
}

// Swap bits 2 and 3 of a small index (orders head-dim outputs so that every
// lane ends with runs of eight consecutive columns).
__device__ __forceinline__ int swap23(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

// 16-byte chunk swizzle of an LDS tile row. Chunk c of row r lives at
// chunk c ^ swz(r). Chosen so that (a) 16 consecutive rows read at one
// logical chunk hit 16 different bank groups (K operand reads) and (b) 4
// consecutive rows read over 64 contiguous bytes hit 16 different bank
// groups (transposing V reads), on 64 banks x 4 bytes.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
}

// Combine the two halves of a wave: lane i gets op(x[i % 32], x[i % 32 + 32]).
// v_permlane32_swap_b32 a, b exchanges the upper half of a with the lower
// half of b; with a = b = x, afterwards {a, b} = {x[i % 32], x[i % 32 + 32]}
// at every lane (measured), in some order, and max and + are symmetric. It is
// written in assembly because the compiler's model of the builtin's second
// result folds it into the first; the s_nops on either side cover the
// VALU-to-permlane and permlane-to-VALU hazards.
__device__ __forceinline__ void swap_halves(float x, float& a, float& b) {
  a = x;
  b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float half_max(float x) {
  float a, b;
  swap_halves(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float half_sum(float x) {
  float a, b;
  swap_halves(x, a, b);
  return a + b;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, BUF_FLAGS);
}

__device__ __forceinline__ void wait_vmem_all() {
  // vmcnt(0), other counters untouched (gfx9 encoding).
  __builtin_amdgcn_s_waitcnt(0x0f70);
}

// EXT: the mask/bias variants (sliding window, global query rows, ALiBi);
// the plain instances compile none of that code.
template <int D, bool BF16, bool CAUSAL, bool VARLEN, int NW, bool EXT>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_fwd_kernel(FwdParams p) {
  constexpr int NWAVES = NW;
  constexpr int BM = 32 * NW;                  // query rows per workgroup
  // Keys per LDS tile: 128 for D = 64 with 4 waves (the same 16 KB as 64 keys
  // of D = 128, twice the matrix work per barrier and per softmax pass;
  // measured 2-7 % faster on B4 H12 S2048, 7 % slower with 8 waves), else 64.
  constexpr int BN = (D == 64 && !EXT && NW == 4) ? 128 : 64;
  constexpr int NKB = BN / 32;                 // 32-key blocks per tile
  constexpr int ROWB = D * 2;                  // bytes per K/V row
  constexpr int TILEB = BN * ROWB;             // bytes per K (or V) tile
  constexpr int STAGEB = 2 * TILEB;            // K tile + V tile
  constexpr int LDW = TILEB / 1024 / NWAVES;   // 1 KB direct loads per wave per tile
  constexpr int DCH = D / 16;                  // 16-deep contraction chunks of Q K^T
  constexpr int DB = D / 32;                   // 32-row blocks of O^T
  static_assert(LDW >= 1, "tile must give every wave a 1 KB load");

  // Two separate arrays, one per stage: the compiler can then tell that LDS
  // reads of one stage never alias the in-flight direct loads into the other
  // and does not wait for those loads before every read.
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[STAGEB];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[STAGEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;     // query row inside the wave / MFMA row index
  const int hh = lane >> 5;     // which half of the contraction this lane feeds

  // ---- which (sequence, head, query tile) this workgroup owns -------------
  // Workgroup i runs on XCD i % 8. Undo that interleave so each XCD owns a
  // contiguous run of the logical order, then walk heads in groups of
  // HEAD_GROUP with the query tiles of a group interleaved, longest (causal)
  // tiles first. An XCD then works on a few heads at a time, whose K/V stay
  // in its L2, and the longest tiles start first.
  const int G = gridDim.x;
  const int xcd = blockIdx.x % NXCD;
  const int local = blockIdx.x / NXCD;
  const int gq = G / NXCD, gr = G % NXCD;
  const int logical = (xcd < gr) ? xcd * (gq + 1) + local : gr * (gq + 1) + (xcd - gr) * gq + local;
  const int nbh = VARLEN ? p.H : p.B * p.H;
  const int nt = p.n_qtiles;
  // Heads per group: chosen by the launcher for the plain 128-row tiles (see
  // head_group_128), HEAD_GROUP otherwise.
  const int HGRP = (NW == 4 && !EXT) ? p.head_group : HEAD_GROUP;
  const int grp = logical / (HGRP * nt);
  const int in_grp = min(HGRP, nbh - grp * HGRP);
  const int rem = logical - grp * (HGRP * nt);
  const int rank = rem / in_grp;
  const int bh = grp * HGRP + (rem - rank * in_grp);
  const int h = bh % p.H;
  const int b = VARLEN ? 0 : bh / p.H;
  int vt = nt - 1 - rank;
  if constexpr (EXT && !VARLEN) {
    // Tiles holding global rows see every key: they are by far the longest,
    // so they start first.
    const int gt = min((p.n_global + BM - 1) / BM, nt);
    vt = rank < gt ? rank : nt - 1 - (rank - gt);
  }
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

  const uint32_t tok_bytes = (uint32_t)p.H * ROWB;             // bytes between tokens
  const size_t base = (((size_t)b * p.S + seq_start) * p.H + h) * D;   // elements
  const uint16_t* qg = p.q + base + (size_t)q0 * p.H * D;
  const uint16_t* kg = p.k + base;
  const uint16_t* vg = p.v + base;
  uint16_t* og = p.o + base + (size_t)q0 * p.H * D;

  // Key range [kv_lo, kv_hi) any row of this workgroup may see.
  int kv_lo = 0, kv_hi = CAUSAL ? min(q0 + BM, L) : L;
  if constexpr (EXT) {
    if (q0 < p.n_global) {
      kv_hi = L;                                   // global rows see every key
    } else if (p.window > 0) {
      kv_lo = max(0, q0 - p.window + 1);
      if (!CAUSAL) kv_hi = min(L, q0 + BM - 1 + p.window);
    }
  }
  const int j_lo = kv_lo / BN;
  const int n_kv = (kv_hi + BN - 1) / BN;          // one past the last tile
  const int wq0 = q0 + wave * 32;        // first query row of this wave
  const int qi = wq0 + li;               // this lane's query row
  // Mask-variant state of this wave (EXT only).
  const int win = EXT ? p.window : 0;
  const int n_glob = EXT ? p.n_global : 0;
  const bool w_any_glob = EXT && wq0 < n_glob;          // some row of the wave is global
  const bool w_all_glob = EXT && wq0 + 31 < n_glob;     // every row of the wave is global
  const float slope2 = (EXT && p.alibi != nullptr) ? p.alibi[h] * 1.4426950408889634f : 0.0f;
  const bool use_alibi = EXT && p.alibi != nullptr;
  const uint32_t q_rows = (uint32_t)min(L - q0, BM);

  // ---- Q^T operand, resident in registers for the whole key loop ----------
  // Rows past the sequence end read as zeros (buffer range check).
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(qg, q_rows * tok_bytes);
  const uint32_t q_voff = (uint32_t)(wave * 32 + li) * tok_bytes + hh * 16;
  // Sign handling of the scale: negative scale uses -Q and |scale|; zero
  // scale zeroes Q so every visible score is exactly 0.
  const uint32_t q_xor = (p.q_mode == 1) ? 0x80008000u : 0u;
  const uint32_t q_and = (p.q_mode == 2) ? 0u : 0xffffffffu;
  u32x4 qreg[DCH];
#pragma unroll
  for (int c = 0; c < DCH; ++c) {
    qreg[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, q_voff + c * 32, 0, 0));
  }
#pragma unroll
  for (int c = 0; c < DCH; ++c) qreg[c] = (qreg[c] ^ q_xor) & q_and;
  const float c_log2 = p.c_log2;          // |scale| * log2(e) (> 0)

  // ---- per-lane constant offsets --------------------------------------------
  // Direct loads: load u of this wave fills LDS bytes [(wave*LDW+u)*1 KB, +1 KB)
  // of a tile; lane l writes 16 bytes at +16 l, i.e. row r, physical chunk pc,
  // and so fetches logical chunk pc ^ swz(r) of key row r.
  uint32_t ld_voff[LDW];
#pragma unroll
  for (int u = 0; u < LDW; ++u) {
    const int byte = (wave * LDW + u) * 1024 + lane * 16;
    const int r = byte / ROWB, pc = (byte % ROWB) / 16;
    ld_voff[u] = (uint32_t)r * tok_bytes + (uint32_t)((pc ^ swz<D>(r)) * 16);
  }
  // K operand: row li (+32 for the second key block), logical chunk 2c+hh.
  uint32_t k_off[DCH];
#pragma unroll
  for (int c = 0; c < DCH; ++c) k_off[c] = li * ROWB + (((2 * c + hh) ^ swz<D>(li)) << 4);
  // V^T operand via the transposing read: in each 16-lane block, lane s points
  // at key row (s / 4) of a 4-key group and at a 4-column group; the read
  // hands lane i the 4 keys of column (group(i/4) + i%4). Column groups are
  // ordered so that output rows come out as runs of 8 consecutive columns.
  uint32_t v_off[2][DB];
  {
    const int blk = li >> 4, s = li & 15;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int key = t2 * 8 + hh * 4 + (s >> 2);        // + 16 * (16-key step)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = db * 32 + blk * 16 + swap23(4 * (s & 3));
        v_off[t2][db] = key * ROWB + ((((col >> 3) ^ swz<D>(key)) << 4) | ((col & 7) * 2));
      }
    }
  }

  // Issue the direct loads of key tile j into stage `st`.
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

  // ---- running statistics and accumulator --------------------------------
  f32x16 acc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) acc[d] = f32x16{};
  float m_run = -INFINITY;     // running max of the log2-scaled logits
  float l_run = 0.0f;          // this lane's half of the running exp-sum

  auto compute_tile = [&](int j, const uint8_t* ks) {
    const uint8_t* vs = ks + TILEB;
    const int key0 = j * BN;
    // A wave none of whose rows sees a key of this tile has nothing to do.
    if constexpr (EXT) {
      if (!w_any_glob) {
        if (CAUSAL && key0 > wq0 + 31) return;
        if (win > 0 && key0 + BN - 1 <= wq0 - win) return;
        if (win > 0 && !CAUSAL && key0 >= wq0 + 31 + win) return;
      }
    } else {
      if (CAUSAL && key0 > wq0 + 31) return;
    }

    // S^T = K Q^T for two 32-key blocks. The two accumulation chains
    // alternate (a chain's next MFMA waits for its previous result) and the
    // K operands are read two contraction steps ahead of their MFMAs.
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
    {
      auto kread = [&](int kb, int c) {
        return *reinterpret_cast<const u32x4*>(ks + kb * 32 * ROWB + k_off[c]);
      };
      u32x4 ka[2][NKB];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) ka[c][kb] = kread(kb, c);
      }
#pragma unroll
      for (int c = 0; c < DCH; ++c) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma32<BF16>(ka[c & 1][kb], qreg[c], s[kb]);
        if (c + 2 < DCH) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) ka[c & 1][kb] = kread(kb, c + 2);
        }
      }
#if SDPA_SCHED_QK
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * NKB, 0);
#pragma unroll
      for (int c = 0; c < DCH; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x008, NKB, 0);
        if (c + 2 < DCH) __builtin_amdgcn_sched_group_barrier(0x100, NKB, 0);
      }
#endif
    }

    // Mask keys past the sequence end and, under causality, keys after the
    // query (only tiles that reach those positions pay for it).
    bool need_mask = (key0 + BN > L) || (CAUSAL && key0 + BN - 1 > wq0);
    if constexpr (EXT) {
      // every row of the wave sees every key of the tile, or not
      bool all_vis = key0 + BN <= L;
      if (!w_all_glob) {
        if (CAUSAL && key0 + BN - 1 > wq0) all_vis = false;
        if (win > 0 && key0 <= wq0 + 31 - win) all_vis = false;
        if (win > 0 && !CAUSAL && key0 + BN - 1 >= wq0 + win) all_vis = false;
        if (w_any_glob && !all_vis) all_vis = false;
      }
      need_mask = !all_vis;
    }
    if constexpr (EXT) {
      const bool glob_row = qi < n_glob;
      if (use_alibi) {
        // Work in the log2-scaled domain: t = s * c - slope * |i - j|.
        // slope * (j - i) = slope * (key0 + 4 hh - i) + slope * (offset of
        // the register), and -|x| = min(x, -x).
        const float bl = slope2 * (float)(key0 + hh * 4 - qi);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float u = fmaf(slope2, (float)(kb * 32 + (r >> 2) * 8 + (r & 3)), bl);
            s[kb][r] = fmaf(s[kb][r], c_log2, fminf(u, -u));
          }
        }
      }
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
            bool ok = key < L;
            if (!glob_row) {
              if (CAUSAL) ok = ok && key <= qi;
              if (win > 0) ok = ok && key > qi - win && (CAUSAL || key < qi + win);
            }
            s[kb][r] = ok ? s[kb][r] : -INFINITY;
          }
        }
      }
    } else if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
          const bool ok = (key < L) && (!CAUSAL || key <= qi);
          s[kb][r] = ok ? s[kb][r] : -INFINITY;
        }
      }
    }

    // With ALiBi the scores are already log2-scaled.
    const bool prescaled = EXT && use_alibi;
    const float c_mul = prescaled ? 1.0f : c_log2;
    // P = exp2(s * c - m), packed to 16 bit for P V; returns this lane's half
    // of the tile's row sum.
    // l: bf16 keeps 8 significant bits, so a row with few visible keys would
    // carry up to 2^-9 relative error into ln(l) if l summed the rounded
    // values; it sums the fp32 values instead. fp16 (11 bits) keeps that
    // error below 2.5e-4 and sums the rounded pairs with one dot2.
    uint32_t pk[NKB][8];
    auto exps = [&](float m_sub) {
      float tl = 0.0f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * t], c_mul, -m_sub));
          const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * t + 1], c_mul, -m_sub));
          pk[kb][t] = pack2<BF16>(e0, e1);
          if constexpr (BF16) {
            tl += e0 + e1;
          } else {
            tl = add_pair_f16(pk[kb][t], tl);
          }
        }
      }
      return tl;
    };

    // Optimistic pass: exponentials against the running maximum as it stands,
    // with no row maximum of the tile at all. Every probability is at most
    // the row sum, so a sum within OPT_LIMIT proves that none exceeded it
    // (and none overflowed); only otherwise (or on a wave's first tile) is the
    // maximum taken, refreshed and the exponentials redone. Softmax does not
    // depend on which constant is subtracted, so this changes rounding only.
    float tile_l = 0.0f;
    bool redo = true;
    if (j != j_lo) {
      tile_l = exps(m_run);
      redo = __builtin_amdgcn_ballot_w64(!(tile_l <= OPT_LIMIT)) != 0;
    }
    if (redo) {
      // Row maximum over this tile (16 + 16 values here, the rest in lane ^ 32).
      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int kb = 1; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      }
      mx = half_max(mx);
      const float mx2 = prescaled ? mx : ((mx == -INFINITY) ? -INFINITY : mx * c_log2);
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
      // A row that has seen no visible key yet keeps m = -inf (its scores here
      // are all -inf too): subtract 0 instead, which gives exp2(-inf) = 0.
      tile_l = exps((EXT && m_run == -INFINITY) ? 0.0f : m_run);
    }
    l_run += tile_l;

    // O^T += V^T P^T over four 16-key steps. Step (kb, e) uses score
    // registers 8e..8e+7 of block kb, i.e. keys kb*32 + 16e + {0..3, 8..11}
    // (+4 in the upper half-wave); the V reads fetch the same keys.
#pragma unroll
    for (int kc = 0; kc < 2 * NKB; ++kc) {
      const int kb = kc >> 1, e = kc & 1;
      const u32x4 bop = {pk[kb][e * 4 + 0], pk[kb][e * 4 + 1], pk[kb][e * 4 + 2], pk[kb][e * 4 + 3]};
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const uint8_t* vb = vs + kc * 16 * ROWB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + v_off[0][d]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + v_off[1][d]));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 a = {lo2[0], lo2[1], hi2[0], hi2[1]};
        acc[d] = mfma32<BF16>(a, bop, acc[d]);
      }
    }
  };

  // ---- main loop: two-stage LDS ring, unrolled by two ----------------------
  issue_tile(j_lo, 0);
  wait_vmem_all();
  __syncthreads();
#pragma unroll 1
  for (int j = j_lo; j < n_kv; j += 2) {
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

  // ---- epilogue: O = acc / l, LSE = ln(l) + m -------------------------------
  const float l_tot = half_sum(l_run);
  const float inv = 1.0f / l_tot;
  // Stores past the sequence end fall outside the descriptor and are dropped.
  const __amdgpu_buffer_rsrc_t o_rsrc = make_rsrc(og, q_rows * tok_bytes);
  const uint32_t o_voff = (uint32_t)(wave * 32 + li) * tok_bytes + hh * 16;
#pragma unroll
  for (int d = 0; d < DB; ++d) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 w;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        w[t] = pack2<BF16>(acc[d][half * 8 + 2 * t] * inv, acc[d][half * 8 + 2 * t + 1] * inv);
      }
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), o_rsrc,
                                             o_voff + (uint32_t)(d * 64 + half * 32), 0, 0);
    }
  }
  if (p.lse != nullptr && hh == 0 && qi < L) {
    // __builtin_amdgcn_logf is the hardware base-2 logarithm.
    const float lse = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
    p.lse[((size_t)b * p.H + h) * p.S + seq_start + qi] = lse;
  }
}

// ---------------------------------------------------------------------------
// Two-block waves: 64 query rows per wave (two 32-row blocks), 4 waves and 256
// rows per workgroup, one wave per SIMD. Every K and V^T operand a wave reads
// from LDS feeds two MFMAs, one per row block, so LDS read traffic per matrix
// operation is half that of the 32-row waves above (whose eight waves per CU
// read 256 KB of K and V per 64-key tile, about what LDS delivers in the time
// the matrix cores take for the tile). With 512 registers per lane available
// at one wave per SIMD, the 2*D/32 output accumulators sit in the
// accumulation registers. The 32-key blocks of consecutive tiles form a
// software pipeline over a three-stage LDS ring (see the main loop) so that a
// single wave has softmax work beside every group of matrix operations. The
// per-row arithmetic (optimistic exponentials, lazy maximum, row sums) is that
// of the 32-row kernel, applied per 32-key block instead of per 64-key tile.
// Slower than the 32-row kernel under sustained load (one wave per SIMD
// exposes the latencies a second wave hides); reachable with ATTN_WAVES=w64.
template <int D, bool BF16, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, 1) void attn_fwd_w64_kernel(FwdParams p) {
  constexpr int NWAVES = 4;
  constexpr int BM = 256;                      // query rows per workgroup
  constexpr int BN = 64;                       // keys per LDS tile
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BN * ROWB;
  constexpr int STAGEB = 2 * TILEB;
  constexpr int LDW = TILEB / 1024 / NWAVES;
  constexpr int DCH = D / 16;
  constexpr int DB = D / 32;
  static_assert(LDW >= 1, "tile must give every wave a 1 KB load");

  __shared__ __attribute__((aligned(1024))) uint8_t smem0[STAGEB];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[STAGEB];
  __shared__ __attribute__((aligned(1024))) uint8_t smem2[STAGEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;
  const int hh = lane >> 5;

  // Same XCD-aware order as the 32-row kernel: contiguous runs of the logical
  // order per XCD, heads in groups of HEAD_GROUP, longest tiles first.
  const int G = gridDim.x;
  const int xcd = blockIdx.x % NXCD;
  const int local = blockIdx.x / NXCD;
  const int gq = G / NXCD, gr = G % NXCD;
  const int logical = (xcd < gr) ? xcd * (gq + 1) + local : gr * (gq + 1) + (xcd - gr) * gq + local;
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

  const uint32_t tok_bytes = (uint32_t)p.H * ROWB;
  const size_t base = (((size_t)b * p.S + seq_start) * p.H + h) * D;
  const uint16_t* qg = p.q + base + (size_t)q0 * p.H * D;
  const uint16_t* kg = p.k + base;
  const uint16_t* vg = p.v + base;
  uint16_t* og = p.o + base + (size_t)q0 * p.H * D;

  const int kv_hi = CAUSAL ? min(q0 + BM, L) : L;
  const int n_kv = (kv_hi + BN - 1) / BN;
  const int wq0 = q0 + wave * 64;               // first query row of this wave
  const uint32_t q_rows = (uint32_t)min(L - q0, BM);

  // Q^T operands of both row blocks, resident for the whole key loop.
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(qg, q_rows * tok_bytes);
  const uint32_t q_xor = (p.q_mode == 1) ? 0x80008000u : 0u;
  const uint32_t q_and = (p.q_mode == 2) ? 0u : 0xffffffffu;
  u32x4 qreg[2][DCH];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const uint32_t q_voff = (uint32_t)(wave * 64 + rb * 32 + li) * tok_bytes + hh * 16;
#pragma unroll
    for (int c = 0; c < DCH; ++c) {
      qreg[rb][c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, q_voff + c * 32, 0, 0));
      qreg[rb][c] = (qreg[rb][c] ^ q_xor) & q_and;
    }
  }
  const float c_log2 = p.c_log2;

  uint32_t ld_voff[LDW];
#pragma unroll
  for (int u = 0; u < LDW; ++u) {
    const int byte = (wave * LDW + u) * 1024 + lane * 16;
    const int r = byte / ROWB, pc = (byte % ROWB) / 16;
    ld_voff[u] = (uint32_t)r * tok_bytes + (uint32_t)((pc ^ swz<D>(r)) * 16);
  }
  uint32_t k_off[DCH];
#pragma unroll
  for (int c = 0; c < DCH; ++c) k_off[c] = li * ROWB + (((2 * c + hh) ^ swz<D>(li)) << 4);
  uint32_t v_off[2][DB];
  {
    const int blk = li >> 4, s = li & 15;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int key = t2 * 8 + hh * 4 + (s >> 2);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = db * 32 + blk * 16 + swap23(4 * (s & 3));
        v_off[t2][db] = key * ROWB + ((((col >> 3) ^ swz<D>(key)) << 4) | ((col & 7) * 2));
      }
    }
  }

  auto issue_tile = [&](int j, int st) __attribute__((always_inline)) {
    const int key0 = j * BN;
    const uint32_t rows = (uint32_t)min(L - key0, BN);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kg + (size_t)key0 * p.H * D, rows * tok_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vg + (size_t)key0 * p.H * D, rows * tok_bytes);
    uint8_t* kdst = (st == 0 ? smem0 : (st == 1 ? smem1 : smem2)) + wave * LDW * 1024;
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

  f32x16 acc[2][DB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      acc[rb][d] = f32x16{};
      acc_fence(acc[rb][d]);
    }
  }
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.0f, 0.0f};

  // S^T of one 32-key block for both row blocks: each K operand feeds two
  // MFMAs; the two chains alternate and K is read two steps ahead.
  auto qk_block = [&](const uint8_t* ks, int kb, f32x16 (&s)[2]) __attribute__((always_inline)) {
    s[0] = f32x16{};
    s[1] = f32x16{};
    auto kread = [&](int c) __attribute__((always_inline)) { return *reinterpret_cast<const u32x4*>(ks + kb * 32 * ROWB + k_off[c]); };
    constexpr int KP = 2;                         // K operands read ahead
    u32x4 ka[KP];
#pragma unroll
    for (int c = 0; c < KP; ++c) ka[c] = kread(c);
#pragma unroll
    for (int c = 0; c < DCH; ++c) {
      s[0] = mfma32<BF16>(ka[c % KP], qreg[0][c], s[0]);
      s[1] = mfma32<BF16>(ka[c % KP], qreg[1][c], s[1]);
      if (c + KP < DCH) ka[c % KP] = kread(c + KP);
    }
  };
  auto mask_block = [&](int key0, int kb, f32x16 (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int qi = wq0 + rb * 32 + li;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + kb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
        const bool ok = (key < L) && (!CAUSAL || key <= qi);
        s[rb][r] = ok ? s[rb][r] : -INFINITY;
      }
    }
  };
  // P = exp2(s * c - m) of one row block and key block, packed to 16 bit;
  // returns this lane's half of the block's row sum (fp32 sums for bf16, one
  // dot2 per rounded pair for fp16, as in the 32-row kernel).
  auto exps = [&](const f32x16& s, uint32_t (&pk)[8], float m_sub) __attribute__((always_inline)) {
    float tl = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[2 * t], c_log2, -m_sub));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[2 * t + 1], c_log2, -m_sub));
      pk[t] = pack2<BF16>(e0, e1);
      if constexpr (BF16) {
        tl += e0 + e1;
      } else {
        tl = add_pair_f16(pk[t], tl);
      }
    }
    return tl;
  };
  // Accept the optimistic exponentials of a key block, or take the row
  // maximum, refresh the running maximum lazily and redo them. A wave's first
  // block always lands here (m = -inf makes the optimistic sums inf or NaN).
  auto settle = [&](const f32x16 (&s)[2], uint32_t (&pk)[2][8], float (&tl)[2]) __attribute__((always_inline)) {
    const bool bad = !(tl[0] <= OPT_LIMIT) || !(tl[1] <= OPT_LIMIT);
    if (__builtin_amdgcn_ballot_w64(bad)) {
      float mx2[2];
      bool bump[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float mx = s[rb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[rb][r]);
        mx = half_max(mx);
        mx2[rb] = (mx == -INFINITY) ? -INFINITY : mx * c_log2;
        bump[rb] = mx2[rb] > m_run[rb] + LAZY_RESCALE_LOG2;
      }
      if (__builtin_amdgcn_ballot_w64(bump[0] || bump[1])) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const float m_new = bump[rb] ? mx2[rb] : m_run[rb];
          const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
#pragma unroll
          for (int d = 0; d < DB; ++d) {
            acc_fence(acc[rb][d]);
            acc[rb][d] *= alpha;
            acc_fence(acc[rb][d]);
          }
          l_run[rb] *= alpha;
          m_run[rb] = m_new;
        }
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) tl[rb] = exps(s[rb], pk[rb], (m_run[rb] == -INFINITY) ? 0.0f : m_run[rb]);
    }
    l_run[0] += tl[0];
    l_run[1] += tl[1];
  };
  // The B operands (probabilities) of one key block: [16-key step][row block].
  auto p_operands = [&](const uint32_t (&pk)[2][8], u32x4 (&bo)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        bo[e][rb] = u32x4{pk[rb][e * 4 + 0], pk[rb][e * 4 + 1], pk[rb][e * 4 + 2], pk[rb][e * 4 + 3]};
      }
    }
    operand_fence(bo[0][0], bo[0][1]);
    operand_fence(bo[1][0], bo[1][1]);
  };
  // P V over key block kb of the stage at vs (both row blocks, 2*2*DB MFMAs),
  // interleaved by hand with the exponentials of one row block of another key
  // block (8 pairs, spread evenly over the MFMAs). The accumulator MFMAs are
  // assembly, which the compiler does not schedule, hence the fences; the V^T
  // operands are read two steps ahead.
  auto pv_with_exps = [&](const uint8_t* vs, int kb, const uint32_t (&pkA)[2][8], const f32x16& s,
                          uint32_t (&pkB)[8], float& tl, float m_sub) __attribute__((always_inline)) {
    constexpr int NSTEP = 2 * DB;                 // (16-key step, 32-column block) pairs
    constexpr int NM = 2 * NSTEP;                 // MFMAs
    auto vread = [&](int st) __attribute__((always_inline)) {
      const int e = st / DB, d = st % DB;
      const uint8_t* vb = vs + (kb * 2 + e) * 16 * ROWB;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + v_off[0][d]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + v_off[1][d]));
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
      return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
    };
    const float m_neg = -m_sub;
    float t_acc = 0.0f;
    auto exp_pair = [&](int t) __attribute__((always_inline)) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[2 * t], c_log2, m_neg));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[2 * t + 1], c_log2, m_neg));
      pkB[t] = pack2<BF16>(e0, e1);
      if constexpr (BF16) {
        t_acc += e0 + e1;
      } else {
        t_acc = add_pair_f16(pkB[t], t_acc);
      }
    };
    u32x4 bo[2][2];
    p_operands(pkA, bo);
    constexpr int VP = 2;                         // V^T steps read ahead
    u32x4 va[VP + 1];
#pragma unroll
    for (int st = 0; st < VP; ++st) va[st] = vread(st);
    int pair = 0;
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      if (st + VP < NSTEP) va[(st + VP) % (VP + 1)] = vread(st + VP);
      const int e = st / DB, d = st % DB;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int m = 2 * st + rb;
        __builtin_amdgcn_sched_barrier(0);
        mfma32_acc<BF16>(acc[rb][d], va[st % (VP + 1)], bo[e][rb]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (; pair < 8 && pair * NM < (m + 1) * 8; ++pair) exp_pair(pair);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    tl = t_acc;
  };

  // ---- main loop: a three-stage LDS ring and a software pipeline over the
  // 32-key blocks ("units") of the tiles. Tile j's body runs, for this wave:
  //   g1: S of unit (j,1)                      | exponentials of unit (j,0), row block 1
  //       settle unit (j,0)
  //   g2: P V of unit (j,0)                    | exponentials of unit (j,1), row block 0
  //       barrier (tile j+1 resident); loads of tile j+2 into the stage of tile j-1
  //   g3: S of unit (j+1,0)                    | exponentials of unit (j,1), row block 1
  //       settle unit (j,1)
  //   g4: P V of unit (j,1)                    | exponentials of unit (j+1,0), row block 0
  // so every group of matrix operations has softmax work beside it. One barrier
  // per tile; each stage is its own array and the loop is unrolled by three, so
  // the compiler can tell LDS reads from the in-flight direct loads apart.
  // Tiles past this wave's causal range are skipped (the wave still joins the
  // barriers and issues its share of the loads); on a wave's last tile, g3/g4
  // work on stale LDS and their results are never used.
  f32x16 s_c[2];                 // scores of unit (j, 0)
  uint32_t pk_c[2][8];
  float tl_c[2];
  const int nw = CAUSAL ? min(n_kv, (wq0 + 63) / BN + 1) : n_kv;   // tiles this wave computes
  auto need_mask = [&](int jj) __attribute__((always_inline)) {
    return (jj * BN + BN > L) || (CAUSAL && jj * BN + BN - 1 > wq0);
  };
  auto stage = [&](int st) __attribute__((always_inline)) -> uint8_t* {
    return st == 0 ? smem0 : (st == 1 ? smem1 : smem2);
  };
  auto body = [&](int jj, auto st_tag) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_tag)::value;
    const uint8_t* ks = stage(ST);
    const uint8_t* vs = ks + TILEB;
    const uint8_t* ks_next = stage((ST + 1) % 3);
    const bool act = jj < nw;
    const int key0 = jj * BN;
    f32x16 s_n[2];
    uint32_t pk_n[2][8];
    float tl_n[2];
    if (act) {
      qk_block(ks, 1, s_n);
      tl_c[1] = exps(s_c[1], pk_c[1], m_run[1]);
      settle(s_c, pk_c, tl_c);
      if (need_mask(jj)) mask_block(key0, 1, s_n);
      pv_with_exps(vs, 0, pk_c, s_n[0], pk_n[0], tl_n[0], m_run[0]);
    }
    wait_vmem_all();
    __syncthreads();
    if (jj + 2 < n_kv) issue_tile(jj + 2, (ST + 2) % 3);
    if (act) {
      qk_block(ks_next, 0, s_c);
      tl_n[1] = exps(s_n[1], pk_n[1], m_run[1]);
      settle(s_n, pk_n, tl_n);
      if (need_mask(jj + 1)) mask_block(key0 + BN, 0, s_c);
      pv_with_exps(vs, 1, pk_n, s_c[0], pk_c[0], tl_c[0], m_run[0]);
    }
  };

  issue_tile(0, 0);
  if (n_kv > 1) issue_tile(1, 1);
  wait_vmem_all();
  __syncthreads();
  if (0 < nw) {
    qk_block(smem0, 0, s_c);
    if (need_mask(0)) mask_block(0, 0, s_c);
    tl_c[0] = exps(s_c[0], pk_c[0], m_run[0]);
  }
#pragma unroll 1
  for (int j = 0; j < n_kv; j += 3) {
    body(j, std::integral_constant<int, 0>{});
    if (j + 1 < n_kv) body(j + 1, std::integral_constant<int, 1>{});
    if (j + 2 < n_kv) body(j + 2, std::integral_constant<int, 2>{});
  }

  const __amdgpu_buffer_rsrc_t o_rsrc = make_rsrc(og, q_rows * tok_bytes);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int d = 0; d < DB; ++d) acc_fence(acc[rb][d]);
    const float l_tot = half_sum(l_run[rb]);
    const float inv = 1.0f / l_tot;
    const uint32_t o_voff = (uint32_t)(wave * 64 + rb * 32 + li) * tok_bytes + hh * 16;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 w;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          w[t] = pack2<BF16>(acc[rb][d][half * 8 + 2 * t] * inv, acc[rb][d][half * 8 + 2 * t + 1] * inv);
        }
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), o_rsrc,
                                               o_voff + (uint32_t)(d * 64 + half * 32), 0, 0);
      }
    }
    const int qi = wq0 + rb * 32 + li;
    if (p.lse != nullptr && hh == 0 && qi < L) {
      const float lse = (m_run[rb] + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
      p.lse[((size_t)b * p.H + h) * p.S + seq_start + qi] = lse;
    }
  }
}

// Workgroup size: 8 waves (256 query rows, one workgroup per CU) when the
// problem has enough 256-row tiles to fill the chip several times over; else
// 4 waves (128 rows, two workgroups per CU), which balances small problems
// better. Both share every per-row arithmetic step, so results are identical.
constexpr long long kBigProblemTiles = 2048;

// Returns 4 or 8 (32-row waves) or 64 (the 64-row-wave kernel). The 64-row
// waves are never chosen by default: under sustained load they measured
// slower on every benchmark workload (LLaMA-shaped layer about -9 %,
// B4 H12 S2048 D64 -4 % without and -27 % with causality), so they are only
// reachable through ATTN_WAVES=w64.
static int choose_waves(const FwdParams& p, bool varlen) {
  // ATTN_WAVES=4, 8 or w64 overrides the choice (used by tests to cover all three).
  if (const char* e = std::getenv("ATTN_WAVES")) {
    if (e[0] == '4' && e[1] == '\0') return 4;
    if (e[0] == '8' && e[1] == '\0') return 8;
    if (e[0] == 'w' && e[1] == '6' && e[2] == '4' && e[3] == '\0') return 64;
  }
  const long long bh = varlen ? p.H : (long long)p.B * p.H;
  const long long tiles256 = varlen ? (long long)p.S / 256 + p.B : ((long long)p.S + 255) / 256;
  return tiles256 * bh >= kBigProblemTiles ? 8 : 4;
}

int max_query_tile_rows() { return 256; }
int min_query_tile_rows() { return 128; }

// Heads per XCD group for the plain 128-row tiles. Each XCD owns a contiguous
// run of about nbh / 8 heads; when the K and V of that whole run fit in the
// XCD's 4 MB L2, one group spans it, so the XCD starts the longest causal
// tiles of all its heads first (B4 H12 S2048 D64: 6 heads of 0.5 MB, causal
// +11 % over groups of 2 and +17 % over 4, non-causal unchanged; groups of 8,
// which straddle XCDs, gained nothing). Otherwise groups of 2 (16 heads of
// 2 MB measured clearly slower).
static int head_group_128(const FwdParams& p, int D, bool varlen) {
  const long long nbh = varlen ? p.H : (long long)p.B * p.H;
  const long long per_xcd = (nbh + NXCD - 1) / NXCD;
  const long long kv_bytes_head = (long long)p.S * D * 2 * 2;   // K and V, 16-bit (S = T when packed)
  const long long l2_bytes = 4LL << 20;
  long long g = (per_xcd * kv_bytes_head <= l2_bytes) ? per_xcd : 2;
  if (g > nbh) g = nbh;
  return g < 1 ? 1 : (int)g;
}

template <int D, bool BF16, bool CAUSAL, bool VARLEN, int NW, bool EXT>
static hipError_t launch_one(FwdParams p, hipStream_t stream) {
  constexpr long long BM = 32 * NW;
  const long long tiles = VARLEN ? (long long)p.S / BM + p.B : ((long long)p.S + BM - 1) / BM;
  p.n_qtiles = (int)tiles;
  p.head_group = head_group_128(p, D, VARLEN);
  const long long grid = tiles * (VARLEN ? p.H : (long long)p.B * p.H);
  hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, CAUSAL, VARLEN, NW, EXT>), dim3((unsigned)grid),
                     dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool BF16, bool CAUSAL, bool VARLEN>
static hipError_t launch_w64(FwdParams p, hipStream_t stream) {
  constexpr long long BM = 256;
  const long long tiles = VARLEN ? (long long)p.S / BM + p.B : ((long long)p.S + BM - 1) / BM;
  p.n_qtiles = (int)tiles;
  const long long grid = tiles * (VARLEN ? p.H : (long long)p.B * p.H);
  hipLaunchKernelGGL((attn_fwd_w64_kernel<D, BF16, CAUSAL, VARLEN>), dim3((unsigned)grid), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D, bool BF16, bool CAUSAL, bool VARLEN>
static hipError_t launch_nw(const FwdParams& p, hipStream_t stream) {
  // The mask/bias variants run with 4-wave workgroups only.
  if (p.window > 0 || p.n_global > 0 || p.alibi != nullptr) {
    return launch_one<D, BF16, CAUSAL, VARLEN, 4, true>(p, stream);
  }
  const int w = choose_waves(p, VARLEN);
  if (w == 64) return launch_w64<D, BF16, CAUSAL, VARLEN>(p, stream);
  return w == 8 ? launch_one<D, BF16, CAUSAL, VARLEN, 8, false>(p, stream)
                : launch_one<D, BF16, CAUSAL, VARLEN, 4, false>(p, stream);
}

template <int D, bool BF16>
static hipError_t launch_d(const FwdParams& p, bool causal, bool varlen, hipStream_t stream) {
  if (causal) {
    return varlen ? launch_nw<D, BF16, true, true>(p, stream)
                  : launch_nw<D, BF16, true, false>(p, stream);
  }
  return varlen ? launch_nw<D, BF16, false, true>(p, stream)
                : launch_nw<D, BF16, false, false>(p, stream);
}

hipError_t launch_fwd(const FwdParams& p, int D, bool bf16, bool causal, bool varlen,
                      hipStream_t stream) {
  if (D == 64) {
    return bf16 ? launch_d<64, true>(p, causal, varlen, stream)
                : launch_d<64, false>(p, causal, varlen, stream);
  }
  return bf16 ? launch_d<128, true>(p, causal, varlen, stream)
              : launch_d<128, false>(p, causal, varlen, stream);
}

}  // namespace sdpa08
